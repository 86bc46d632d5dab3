// K-cache pack: fp16 keys -> 2-bit thumbnail (codes + fp16 scale/zero) and
// int8 residual (+ fp16 residual scale), per token and 32-channel group.
//
// Follows "Faster Than Flash" (gist.science summary of arXiv 2609.00097),
// Method section 1: the K cache is split into a 2-bit quantized thumbnail used
// to estimate scores and 8-bit residuals that rebuild K close to fp16.  The
// page gives no quantizer; the convention implemented here is documented in
// include/ffd.h.  Every decision is an exact fp64 comparison: fp16 inputs,
// their differences, code*scale products and (k +- 1/2)*scale thresholds are
// all exactly representable in fp64, and the two divisions are correctly
// rounded in fp64 and then rounded once more to fp16 with integer logic (the
// fp64 quotient is never close enough to an fp16 rounding midpoint for that
// double rounding to differ from rounding the exact quotient).
//
// Launch: grid (ceil(n/64), Hkv, B), 256 threads; thread = (token, group),
// 4 threads per token, 64 tokens per work-group.  The decode-loop append takes
// the same decisions for one token per (sequence, KV head), spread over a wave.
#include "ffd_device.h"
#include "ffd_launch.h"

namespace ffd {

// round a finite double (|x| < 65520) to fp16 bits, nearest-even
__device__ inline uint16_t f64_to_f16_rne(double x) {
  const uint64_t bits = __builtin_bit_cast(uint64_t, x);
  const uint16_t sign = (uint16_t)((bits >> 48) & 0x8000u);
  const uint64_t mag = bits & 0x7fffffffffffffffull;
  if (mag == 0) return sign;
  const int e = (int)(mag >> 52) - 1023;  // inputs here are normal doubles
  const uint64_t m = (mag & ((1ull << 52) - 1)) | (1ull << 52);
  const int shift = (e >= -14) ? 42 : 42 + (-14 - e);
  if (shift >= 54) return sign;  // below 2^-25: rounds to zero
  uint64_t kept = m >> shift;
  const uint64_t rem = m & ((1ull << shift) - 1);
  const uint64_t half = 1ull << (shift - 1);
  if (rem > half || (rem == half && (kept & 1))) ++kept;
  if (e >= -14) {
    int ee = e;
    if (kept == 2048) { kept = 1024; ++ee; }
    if (ee > 15) return (uint16_t)(sign | 0x7c00u);
    return (uint16_t)(sign | ((ee + 15) << 10) | (uint16_t)(kept - 1024));
  }
  return (uint16_t)(sign | (uint16_t)kept);  // subnormal (kept == 1024 is the smallest normal)
}

__device__ inline double f16bits_to_f64(uint16_t b) {
  return (double)__builtin_bit_cast(_Float16, b);
}

// Quantize one (token, group) -- 32 fp16 keys at `src` -- and store its code
// bits, (scale, zero), residual bytes and residual scale at token t of head
// `head`.  The code word of a token is shared by the groups g and g ^ 1, which
// must sit in the lanes lane and lane ^ 1 of the same wave (both lanes active,
// same token); `store` = false computes and takes part in that exchange but
// writes nothing.
__device__ inline void pack_group(const uint16_t* __restrict__ src, size_t head, int nblk_cap, int t, int g,
                                  bool store, uint32_t* __restrict__ codes, uint32_t* __restrict__ sz,
                                  int8_t* __restrict__ res, uint16_t* __restrict__ rsc) {
  const uint4* s4 = reinterpret_cast<const uint4*>(src);
  uint32_t w[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 v = s4[i];
    w[4 * i + 0] = v.x; w[4 * i + 1] = v.y; w[4 * i + 2] = v.z; w[4 * i + 3] = v.w;
  }
  double x[32];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    x[2 * i] = f16bits_to_f64((uint16_t)(w[i] & 0xffffu));
    x[2 * i + 1] = f16bits_to_f64((uint16_t)(w[i] >> 16));
  }
  double mn = x[0], mx = x[0];
#pragma unroll
  for (int i = 1; i < 32; ++i) { mn = fmin(mn, x[i]); mx = fmax(mx, x[i]); }
  mn = mn + 0.0;  // -0 -> +0
  const uint16_t zb = f64_to_f16_rne(mn);
  const uint16_t sb = f64_to_f16_rne((mx - mn) / 3.0 + 0.0);
  const double s = f16bits_to_f64(sb);

  int c[32];
  double amax = 0.0;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const double d = x[i] - mn;
    int ci = 0;
    if (s > 0.0) ci = (d >= 0.5 * s) + (d >= 1.5 * s) + (d >= 2.5 * s);
    c[i] = ci;
    x[i] = x[i] - (mn + ci * s);  // residual, exact
    amax = fmax(amax, fabs(x[i]));
  }
  const uint16_t s8b = f64_to_f16_rne(amax / 127.0);
  const double s8 = f16bits_to_f64(s8b);

  uint32_t rw[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) rw[i] = 0;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    int e = 0;
    if (s8 > 0.0) {
      const double a = fabs(x[i]);
      double kf = floor(a / s8 + 0.5);
      if (a >= (kf + 0.5) * s8) kf += 1.0;
      if (kf > 0.0 && a < (kf - 0.5) * s8) kf -= 1.0;
      kf = fmin(kf, 127.0);
      e = (int)kf;
      if (x[i] < 0.0) e = -e;
    }
    rw[i >> 2] |= ((uint32_t)(e & 0xff)) << (8 * (i & 3));
  }

  // code fragments of this group for the four channel slices kq
  uint32_t frag[4];
#pragma unroll
  for (int kq = 0; kq < 4; ++kq) {
    uint32_t f = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) f |= (uint32_t)c[8 * kq + j] << code_bit(g, j);
    frag[kq] = f;
  }
  uint32_t other[4];
#pragma unroll
  for (int kq = 0; kq < 4; ++kq) other[kq] = (uint32_t)__shfl_xor((int)frag[kq], 1, 64);

  if (!store) return;
  const int blk = t >> 6, tb = t & 63;
  const size_t blk_idx = head * nblk_cap + blk;
  uint8_t* cbase = reinterpret_cast<uint8_t*>(codes) + blk_idx * kCodesBytes;
  const int p = g >> 1;
  // even group writes slices 0,1; odd group writes slices 2,3 of the shared words
  const int kq0 = (g & 1) ? 2 : 0;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int kq = kq0 + u;
    *reinterpret_cast<uint32_t*>(cbase + codes_word_off(tb, kq, p)) = frag[kq] | other[kq];
  }
  uint8_t* zbase = reinterpret_cast<uint8_t*>(sz) + blk_idx * kSzBytes;
  *reinterpret_cast<uint32_t*>(zbase + sz_off(tb, g)) = (uint32_t)sb | ((uint32_t)zb << 16);
  int8_t* rbase = res + blk_idx * kResBytes;
  *reinterpret_cast<uint4*>(rbase + res_off(tb, 32 * g)) = make_uint4(rw[0], rw[1], rw[2], rw[3]);
  *reinterpret_cast<uint4*>(rbase + res_off(tb, 32 * g + 16)) = make_uint4(rw[4], rw[5], rw[6], rw[7]);
  uint8_t* sbase = reinterpret_cast<uint8_t*>(rsc) + blk_idx * kRscBytes;
  *reinterpret_cast<uint16_t*>(sbase + rsc_off(tb, g)) = s8b;
}

__global__ __launch_bounds__(256) void pack_kernel(const uint16_t* __restrict__ k, int L_cap,
                                                   int t_begin, int t_end,
                                                   uint32_t* __restrict__ codes,
                                                   uint32_t* __restrict__ sz,
                                                   int8_t* __restrict__ res,
                                                   uint16_t* __restrict__ rsc) {
  const int tid = threadIdx.x;
  const int g = tid & 3;
  const int t = t_begin + blockIdx.x * 64 + (tid >> 2);
  const bool active = t < t_end;
  const size_t head = (size_t)blockIdx.z * gridDim.y + blockIdx.y;
  const int tc = active ? t : t_begin;  // inactive threads read a valid row and store nothing
  pack_group(k + (head * L_cap + tc) * kHeadDim + g * kGroup, head, L_cap >> 6, tc, g, active, codes, sz, res,
             rsc);
}

// Decode-loop append: one new token per (sequence, KV head), written at the
// sequence's own position pos[b] read on the device (so the append can sit in a
// captured graph beside the decode step).  One wave per (b, kv head); lane l
// owns channels 2l and 2l+1 of the key (group l / 16) and of the value.  The
// decisions are those of pack_group, spread over the lanes: group minimum,
// maximum and largest residual by exact reductions over the group's 16 lanes,
// scales by the same roundings, codes and residual bytes per channel.  A
// position outside [0, L_cap) skips the sequence.
__device__ inline double shfl_xor_f64(double v, int m) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)u, m, 64);
  const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(u >> 32), m, 64);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

__global__ __launch_bounds__(64) void append_kernel(const uint16_t* __restrict__ k_new,
                                                    const uint16_t* __restrict__ v_new,
                                                    const int32_t* __restrict__ pos, int L_cap,
                                                    uint32_t* __restrict__ codes, uint32_t* __restrict__ sz,
                                                    int8_t* __restrict__ res, uint16_t* __restrict__ rsc,
                                                    uint16_t* __restrict__ vt) {
  const int lane = threadIdx.x;
  const int b = blockIdx.y;
  const size_t head = (size_t)b * gridDim.x + blockIdx.x;
  const int t = pos[b];
  if (t < 0 || t >= L_cap) return;  // uniform over the work-group
  const int g = lane >> 4, li = lane & 15;
  const uint32_t kw = *reinterpret_cast<const uint32_t*>(k_new + head * kHeadDim + 2 * lane);
  const double x[2] = {f16bits_to_f64((uint16_t)(kw & 0xffffu)), f16bits_to_f64((uint16_t)(kw >> 16))};
  double mn = fmin(x[0], x[1]), mx = fmax(x[0], x[1]);
#pragma unroll
  for (int m = 1; m < 16; m <<= 1) {
    mn = fmin(mn, shfl_xor_f64(mn, m));
    mx = fmax(mx, shfl_xor_f64(mx, m));
  }
  mn = mn + 0.0;  // -0 -> +0
  const uint16_t zb = f64_to_f16_rne(mn);
  const uint16_t sb = f64_to_f16_rne((mx - mn) / 3.0 + 0.0);
  const double s = f16bits_to_f64(sb);
  int c[2];
  double r[2], amax = 0.0;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const double d = x[i] - mn;
    c[i] = s > 0.0 ? (d >= 0.5 * s) + (d >= 1.5 * s) + (d >= 2.5 * s) : 0;
    r[i] = x[i] - (mn + c[i] * s);  // exact
    amax = fmax(amax, fabs(r[i]));
  }
#pragma unroll
  for (int m = 1; m < 16; m <<= 1) amax = fmax(amax, shfl_xor_f64(amax, m));
  const uint16_t s8b = f64_to_f16_rne(amax / 127.0);
  const double s8 = f16bits_to_f64(s8b);
  int e[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    e[i] = 0;
    if (s8 > 0.0) {
      const double a = fabs(r[i]);
      double kf = floor(a / s8 + 0.5);
      if (a >= (kf + 0.5) * s8) kf += 1.0;
      if (kf > 0.0 && a < (kf - 0.5) * s8) kf -= 1.0;
      kf = fmin(kf, 127.0);
      e[i] = (int)kf;
      if (r[i] < 0.0) e[i] = -e[i];
    }
  }
  // code word (kq, p) holds channels 8kq..8kq+7 of groups 2p and 2p+1: the
  // lanes 32p + 4kq + {0..3} and 16 lanes above them
  const int kq = li >> 2, j0 = 2 * (li & 3);
  uint32_t bits = ((uint32_t)c[0] << code_bit(g, j0)) | ((uint32_t)c[1] << code_bit(g, j0 + 1));
  bits |= (uint32_t)__shfl_xor((int)bits, 1, 64);
  bits |= (uint32_t)__shfl_xor((int)bits, 2, 64);
  bits |= (uint32_t)__shfl_xor((int)bits, 16, 64);

  const int blk = t >> 6, tb = t & 63;
  const size_t blk_idx = head * (size_t)(L_cap >> 6) + blk;
  if ((lane & 0x13) == 0)
    *reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(codes) + blk_idx * kCodesBytes +
                                 codes_word_off(tb, kq, g >> 1)) = bits;
  if (li == 0) {
    *reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(sz) + blk_idx * kSzBytes + sz_off(tb, g)) =
        (uint32_t)sb | ((uint32_t)zb << 16);
    *reinterpret_cast<uint16_t*>(reinterpret_cast<uint8_t*>(rsc) + blk_idx * kRscBytes + rsc_off(tb, g)) = s8b;
  }
  *reinterpret_cast<uint16_t*>(reinterpret_cast<uint8_t*>(res) + blk_idx * kResBytes + res_off(tb, 2 * lane)) =
      (uint16_t)((uint32_t)(e[0] & 0xff) | ((uint32_t)(e[1] & 0xff) << 8));
  const uint32_t vv = *reinterpret_cast<const uint32_t*>(v_new + head * kHeadDim + 2 * lane);
  uint16_t* dst = vt + (head * L_cap + (size_t)(t & ~3)) * kHeadDim + 8 * lane + (t & 3);
  dst[0] = (uint16_t)(vv & 0xffffu);  // channel 2*lane
  dst[4] = (uint16_t)(vv >> 16);      // channel 2*lane + 1
}

// V pack: natural fp16 rows -> the token-quad tiled layout the refine's
// P.V MFMA reads (element ((t/4)*128 + ch)*4 + t%4 of the head's array), so a
// lane's A fragment (4 tokens of one channel) is 8 contiguous bytes.  Thread =
// (token quad, channel pair): 4 quads x 64 pairs per work-group.  A quad
// entirely inside [t_begin, t_end) is stored with one 16-byte write; the
// partial quads at the ends of the range store only their in-range tokens.
__global__ __launch_bounds__(256) void pack_v_kernel(const uint16_t* __restrict__ v, int L_cap, int t_begin,
                                                     int t_end, uint16_t* __restrict__ vt) {
  const int tid = threadIdx.x;
  const int cp = tid & 63;
  const int tq = (t_begin >> 2) + blockIdx.x * 4 + (tid >> 6);
  const size_t head = (size_t)blockIdx.z * gridDim.y + blockIdx.y;
  const int t0 = 4 * tq;
  if (t0 >= t_end) return;
  uint32_t w[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int t = t0 + j;
    const bool in = t >= t_begin && t < t_end;
    w[j] = in ? *reinterpret_cast<const uint32_t*>(v + (head * L_cap + t) * kHeadDim + 2 * cp) : 0u;
  }
  // channel 2cp: low halves of w[0..3]; channel 2cp+1: high halves
  const uint32_t a0 = (w[0] & 0xffffu) | (w[1] << 16), a1 = (w[2] & 0xffffu) | (w[3] << 16);
  const uint32_t b0 = (w[0] >> 16) | (w[1] & 0xffff0000u), b1 = (w[2] >> 16) | (w[3] & 0xffff0000u);
  uint16_t* dst = vt + (head * L_cap + (size_t)t0) * kHeadDim + 8 * cp;
  if (t0 >= t_begin && t0 + 4 <= t_end) {
    *reinterpret_cast<uint4*>(dst) = make_uint4(a0, a1, b0, b1);
  } else {
    const uint32_t lo[4] = {a0 & 0xffffu, a0 >> 16, a1 & 0xffffu, a1 >> 16};
    const uint32_t hi[4] = {b0 & 0xffffu, b0 >> 16, b1 & 0xffffu, b1 >> 16};
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (t0 + j >= t_begin && t0 + j < t_end) {
        dst[j] = (uint16_t)lo[j];
        dst[4 + j] = (uint16_t)hi[j];
      }
  }
}

hipError_t launch_pack_v(const void* v, int B, int Hkv, int L_cap, int t_begin, int t_end, void* vt,
                         hipStream_t stream) {
  const int nq = (t_end + 3) / 4 - t_begin / 4;
  if (t_end <= t_begin || nq <= 0) return hipSuccess;
  dim3 grid((nq + 3) / 4, Hkv, B);
  hipLaunchKernelGGL(pack_v_kernel, grid, dim3(256), 0, stream, static_cast<const uint16_t*>(v), L_cap, t_begin,
                     t_end, static_cast<uint16_t*>(vt));
  return hipGetLastError();
}

hipError_t launch_pack(const void* k, int B, int Hkv, int L_cap, int t_begin, int t_end, void* codes,
                       void* sz, void* res, void* rsc, hipStream_t stream) {
  const int n = t_end - t_begin;
  if (n <= 0) return hipSuccess;
  dim3 grid((n + 63) / 64, Hkv, B);
  hipLaunchKernelGGL(pack_kernel, grid, dim3(256), 0, stream, static_cast<const uint16_t*>(k), L_cap,
                     t_begin, t_end, static_cast<uint32_t*>(codes), static_cast<uint32_t*>(sz),
                     static_cast<int8_t*>(res), static_cast<uint16_t*>(rsc));
  return hipGetLastError();
}

hipError_t launch_append(const void* k_new, const void* v_new, const int32_t* pos, int B, int Hkv, int L_cap,
                         void* codes, void* sz, void* res, void* rsc, void* vt, hipStream_t stream) {
  hipLaunchKernelGGL(append_kernel, dim3(Hkv, B), dim3(64), 0, stream, static_cast<const uint16_t*>(k_new),
                     static_cast<const uint16_t*>(v_new), pos, L_cap, static_cast<uint32_t*>(codes),
                     static_cast<uint32_t*>(sz), static_cast<int8_t*>(res), static_cast<uint16_t*>(rsc),
                     static_cast<uint16_t*>(vt));
  return hipGetLastError();
}

}  // namespace ffd
