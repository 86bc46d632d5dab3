// FFD decode attention, one step: pseudo-max, fused Top-delta scan + refine,
// log-sum-exp merge; plus the dense flash-decode baseline.
//
// Page: "Faster Than Flash" (gist.science summary of arXiv 2609.00097).
//   Method 2 (Top-delta): keep when s >= m~ - delta, m~ from sink + local tokens.
//   Method 3 stage 1: pseudo-max estimation      -> pseudomax_kernel
//   Method 3 stage 2: stream the 2-bit keys, provisional scores, block filter
//   Method 3 stage 3: residuals + values of the kept blocks, exact attention
//                                                 -> attend_kernel (stages 2+3
//                                                    fused per chunk of blocks,
//                                                    reusing the stage-2 scores)
//   split partials combined with a log-sum-exp merge -> merge_kernel
//
// Work decomposition (all kernels): one work-group per (chunk of `cb` 64-token
// blocks, KV head, sequence); one wave64 per work-group.  Each chunk writes one
// un-normalised partial (o[128], m, l) per query head.
#include "ffd_device.h"
#include "ffd_launch.h"

namespace ffd {



__device__ inline int clamp_len(const DecodeParams& p, int b) {
  const int L = p.seq_lens[b];
  return L < 1 ? 1 : (L > p.L_cap ? p.L_cap : L);
}

// ---------------------------------------------------------------------------
// Stage 1: pseudo-max over support tokens [0, min(S,L)) U [max(0,L-W), L).
// Exact scores use K-hat = zero + code*scale + res*rscale, evaluated per group
// as scale*(q.c) + zero*sum(q) + rscale*(q.e).  Grid (Hkv, B), 256 threads.
// ---------------------------------------------------------------------------
template <int G>
__global__ __launch_bounds__(256) void pseudomax_kernel(DecodeParams p) {
  __shared__ float qs[G][kHeadDim];
  __shared__ float qsum[G][kGroups];
  __shared__ float red[G][4];
  const int tid = threadIdx.x;
  const int hkv = blockIdx.x, b = blockIdx.y;
  const size_t head = (size_t)b * p.Hkv + hkv;
  const int L = clamp_len(p, b);
  const int qh0 = hkv * G;
  for (int i = tid; i < G * kHeadDim; i += 256)
    qs[i >> 7][i & 127] = h2f(p.q[((size_t)b * p.Hq + qh0 + (i >> 7)) * kHeadDim + (i & 127)]);
  __syncthreads();
  if (tid < G * kGroups) {
    const int h = tid >> 2, g = tid & 3;
    float s = 0.f;
    for (int k = 0; k < kGroup; ++k) s += qs[h][32 * g + k];
    qsum[h][g] = s;
  }
  __syncthreads();

  const int n_s = min(p.sink, L);
  const int lo = max(n_s, L - p.local);
  const int n = n_s + (L - lo);
  float m[G];
#pragma unroll
  for (int h = 0; h < G; ++h) m[h] = -INFINITY;

  for (int j = tid; j < n; j += 256) {
    const int t = j < n_s ? j : lo + (j - n_s);
    const int tb = t & 63;
    const size_t bi = head * p.nblk_cap + (t >> 6);
    const uint8_t* cb = p.codes + bi * kCodesBytes;
    const uint8_t* zb = p.sz + bi * kSzBytes;
    const int8_t* rb = p.res + bi * kResBytes;
    const uint8_t* sb = p.rsc + bi * kRscBytes;
    float sc[G];
#pragma unroll
    for (int h = 0; h < G; ++h) sc[h] = 0.f;
#pragma unroll 1
    for (int g = 0; g < kGroups; ++g) {
      const uint32_t zw = *reinterpret_cast<const uint32_t*>(zb + sz_off(tb, g));
      const float s = lo_h(zw), z = hi_h(zw);
      const float s8 = h2f(*reinterpret_cast<const uint16_t*>(sb + rsc_off(tb, g)));
      float A[G], E[G];
#pragma unroll
      for (int h = 0; h < G; ++h) { A[h] = 0.f; E[h] = 0.f; }
#pragma unroll 1
      for (int kq = 0; kq < 4; ++kq) {
        const uint32_t w = *reinterpret_cast<const uint32_t*>(cb + codes_word_off(tb, kq, g >> 1));
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          const float c = (float)((w >> code_bit(g, jj)) & 3u);
#pragma unroll
          for (int h = 0; h < G; ++h) A[h] = fmaf(qs[h][32 * g + 8 * kq + jj], c, A[h]);
        }
      }
#pragma unroll 1
      for (int half = 0; half < 2; ++half) {
        const uint4 rv = *reinterpret_cast<const uint4*>(rb + res_off(tb, 32 * g + 16 * half));
        const uint32_t rw[4] = {rv.x, rv.y, rv.z, rv.w};
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float e = (float)(int8_t)((rw[i >> 2] >> (8 * (i & 3))) & 0xffu);
#pragma unroll
          for (int h = 0; h < G; ++h) E[h] = fmaf(qs[h][32 * g + 16 * half + i], e, E[h]);
        }
      }
#pragma unroll
      for (int h = 0; h < G; ++h) sc[h] += s * A[h] + z * qsum[h][g] + s8 * E[h];
    }
#pragma unroll
    for (int h = 0; h < G; ++h) m[h] = fmaxf(m[h], sc[h] * p.sm_scale);
  }
  const int wave = tid >> 6, lane = tid & 63;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float r = wave_max(m[h]);
    if (lane == 0) red[h][wave] = r;
  }
  __syncthreads();
  if (tid < G) {
    const float mt = fmaxf(fmaxf(red[tid][0], red[tid][1]), fmaxf(red[tid][2], red[tid][3]));
    const size_t o = (size_t)b * p.Hq + qh0 + tid;
    p.thr[o] = mt - p.delta;
    if (p.dbg_mt) p.dbg_mt[o] = mt;
  }
}

// ---------------------------------------------------------------------------
// shared softmax update + P.V for one 64-token block (one wave)
//   sc[h]   exact score of token `lane` for head h (-inf when invalid)
//   Vr[i]   V[row tp + 4i][8co .. 8co+7] of the block, lane = (tp, co)
// ---------------------------------------------------------------------------
template <int G>
struct SoftmaxState {
  float m[G];
  float l[G];
  float acc[G][8];
};

template <int G, int PG>
__device__ inline void softmax_pv(SoftmaxState<G>& st, float (&sc)[G], const uint4 (&Vr)[16],
                                  float (*pw)[PG], int lane, int n_valid) {
  float alpha[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float mb = wave_max(sc[h]);
    const float mn = fmaxf(st.m[h], mb);
    alpha[h] = exp2f((st.m[h] - mn) * kLog2e);
    const float pt = exp2f((sc[h] - mn) * kLog2e);
    st.l[h] = st.l[h] * alpha[h] + wave_sum(pt);
    st.m[h] = mn;
    pw[lane][h] = pt;
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int k = 0; k < 8; ++k) st.acc[h][k] *= alpha[h];
  const int tp = lane >> 4;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int t = tp + 4 * i;
    if (t < n_valid) {
      float pp[G];
#pragma unroll
      for (int h = 0; h < G; ++h) pp[h] = pw[t][h];
      const uint32_t vw[4] = {Vr[i].x, Vr[i].y, Vr[i].z, Vr[i].w};
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float vk = (k & 1) ? hi_h(vw[k >> 1]) : lo_h(vw[k >> 1]);
#pragma unroll
        for (int h = 0; h < G; ++h) st.acc[h][k] = fmaf(pp[h], vk, st.acc[h][k]);
      }
    }
  }
  __syncthreads();
}

template <int G>
__device__ inline void write_partial(const DecodeParams& p, SoftmaxState<G>& st, int b, int qh0,
                                     int chunk, int lane) {
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      float a = st.acc[h][k];
      a += xor_lane(a, 16);
      a += xor_lane(a, 32);
      st.acc[h][k] = a;
    }
  const bool any = st.l[0] > 0.f;
  if (lane < 16 && any) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float* o = p.part_o + (((size_t)b * p.Hq + qh0 + h) * p.nchunk + chunk) * kHeadDim + 8 * lane;
      *reinterpret_cast<float4*>(o) = make_float4(st.acc[h][0], st.acc[h][1], st.acc[h][2], st.acc[h][3]);
      *reinterpret_cast<float4*>(o + 4) = make_float4(st.acc[h][4], st.acc[h][5], st.acc[h][6], st.acc[h][7]);
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h)
      p.part_ml[((size_t)b * p.Hq + qh0 + h) * p.nchunk + chunk] = make_float2(st.m[h], st.l[h]);
  }
}

// 2-bit code word -> MFMA A fragment of 8 fp16 values 1 + c/4 (channels j = 0..7)
__device__ inline h8 unpack_even(uint32_t w) {
  const uint32_t M = 0x03000300u, BIAS = 0x3C003C00u;
  uint4 d;
  d.x = (w & M) | BIAS;
  d.y = ((w >> 2) & M) | BIAS;
  d.z = ((w >> 4) & M) | BIAS;
  d.w = ((w >> 6) & M) | BIAS;
  return __builtin_bit_cast(h8, d);
}
__device__ inline h8 unpack_odd(uint32_t w) {
  const uint32_t M = 0x03000300u, BIAS = 0x3C003C00u;
  uint4 d;
  d.x = ((w << 8) & M) | BIAS;
  d.y = ((w << 6) & M) | BIAS;
  d.z = ((w << 4) & M) | BIAS;
  d.w = ((w << 2) & M) | BIAS;
  return __builtin_bit_cast(h8, d);
}

// ---------------------------------------------------------------------------
// Stages 2 + 3 fused per chunk of blocks.
//
// Scan (MFMA): per 16-token tile, A = codes as fp16 (1 + c/4), tokens on rows;
// B = q with column n = 4*h + g holding head h restricted to group g (zero
// elsewhere), so one accumulator collects the per-group products
// C[t][(h,g)] = sum_{k in g} (1 + c_k/4) q_hk; starting it at -sum_{k in g} q_hk
// leaves (q_g . c_g)/4.  The fp32 epilogue adds zero*sum(q) with the group's
// scale, a quad sum over g gives the estimate; a block max per head against the
// head's threshold decides the block (union over the GQA group).
//
// Refine (VALU, lane = token): exact score = estimate (kept in LDS) +
// rscale * (q . res) per group, online softmax, P.V with lanes over channels.
// ---------------------------------------------------------------------------
template <int G>
__global__ __launch_bounds__(64) void attend_kernel(DecodeParams p) {
  constexpr int NT = (G + 3) / 4;
  constexpr int PG = (G + 3) & ~3;
  const int chunk = blockIdx.x, hkv = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x;
  const int L = clamp_len(p, b);
  const int nblk = (L + 63) >> 6;
  const int blk0 = chunk * p.cb;
  if (blk0 >= nblk) return;
  const int blk1 = min(nblk, blk0 + p.cb);
  const size_t head = (size_t)b * p.Hkv + hkv;
  const int qh0 = hkv * G;

  __shared__ h2 q2[G][64];
  __shared__ float qg[G][kGroups];
  __shared__ float est[G][64];
  __shared__ float pw[64][PG];

#pragma unroll
  for (int h = 0; h < G; ++h)
    q2[h][lane] = __builtin_bit_cast(h2, *reinterpret_cast<const uint32_t*>(
                                            p.q + ((size_t)b * p.Hq + qh0 + h) * kHeadDim + 2 * lane));
  __syncthreads();
  if (lane < G * kGroups) {
    const int h = lane >> 2, g = lane & 3;
    float s = 0.f;
    for (int k = 0; k < 16; ++k) { const h2 v = q2[h][16 * g + k]; s += (float)v.x + (float)v.y; }
    qg[h][g] = s;
  }
  __syncthreads();

  // scan-side lane roles
  const int col = lane & 15, hc = col >> 2, gc = col & 3, ks = lane >> 4;
  h8 Bf[NT][kGroups];
  float cinit[NT], qq[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int h = 4 * nt + hc;
    const bool live = h < G;
#pragma unroll
    for (int g = 0; g < kGroups; ++g) {
      h8 f;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        h2 pr = {(_Float16)0.f, (_Float16)0.f};
        if (live && g == gc) pr = q2[h][16 * g + 4 * ks + d];
        f[2 * d] = pr.x;
        f[2 * d + 1] = pr.y;
      }
      Bf[nt][g] = f;
    }
    cinit[nt] = live ? -qg[h][gc] : 0.f;
    qq[nt] = live ? 0.25f * qg[h][gc] : 0.f;
  }
  float thr[G];
#pragma unroll
  for (int h = 0; h < G; ++h) thr[h] = p.thr[(size_t)b * p.Hq + qh0 + h];
  const float scale4 = 4.f * p.sm_scale;
  const int sink_end = p.sink > 0 ? ((min(p.sink, L) + 63) >> 6) : 0;
  const int local_beg = p.local > 0 ? (max(0, L - p.local) >> 6) : nblk;

  SoftmaxState<G> st;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    st.m[h] = -INFINITY;
    st.l[h] = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) st.acc[h][k] = 0.f;
  }

  for (int blk = blk0; blk < blk1; ++blk) {
    const size_t bi = head * p.nblk_cap + blk;
    const uint8_t* cbp = p.codes + bi * kCodesBytes + (col * 4 + ks) * 32;
    const uint4 cw0 = *reinterpret_cast<const uint4*>(cbp);
    const uint4 cw1 = *reinterpret_cast<const uint4*>(cbp + 16);
    const uint8_t* zbp = p.sz + bi * kSzBytes + (gc * 4 + ks) * 64;
    uint4 szw[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) szw[tt] = *reinterpret_cast<const uint4*>(zbp + 16 * tt);
    const int n_valid = min(64, L - blk * 64);

    float vmax[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) vmax[nt] = -INFINITY;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      const uint4 cw = tt < 2 ? cw0 : cw1;
      const uint32_t w0 = (tt & 1) ? cw.z : cw.x;
      const uint32_t w1 = (tt & 1) ? cw.w : cw.y;
      const h8 a0 = unpack_even(w0), a1 = unpack_odd(w0), a2 = unpack_even(w1), a3 = unpack_odd(w1);
      const uint32_t zs[4] = {szw[tt].x, szw[tt].y, szw[tt].z, szw[tt].w};
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        f4 c = {cinit[nt], cinit[nt], cinit[nt], cinit[nt]};
        c = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, Bf[nt][0], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, Bf[nt][1], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x32_f16(a2, Bf[nt][2], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x32_f16(a3, Bf[nt][3], c, 0, 0, 0);
        float v4[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float v = fmaf(lo_h(zs[i]), c[i], hi_h(zs[i]) * qq[nt]);
          v += dpp<kQuadXor1>(v);
          v += dpp<kQuadXor2>(v);
          v = (tt * 16 + 4 * ks + i < n_valid) ? v : -INFINITY;
          vmax[nt] = fmaxf(vmax[nt], v);
          v4[i] = v * scale4;
        }
        const int h = 4 * nt + hc;
        if (gc == 0 && h < G)
          *reinterpret_cast<float4*>(&est[h][tt * 16 + 4 * ks]) = make_float4(v4[0], v4[1], v4[2], v4[3]);
      }
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      vmax[nt] = fmaxf(vmax[nt], xor_lane(vmax[nt], 16));
      vmax[nt] = fmaxf(vmax[nt], xor_lane(vmax[nt], 32));
    }
    bool keep = blk < sink_end || blk >= local_beg;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float bm = uniform_lane(vmax[h >> 2], 4 * (h & 3)) * scale4;
      keep = keep || (bm >= thr[h]);
      if (p.dbg_bmax && lane == 0) p.dbg_bmax[((size_t)b * p.Hq + qh0 + h) * p.nblk_cap + blk] = bm;
    }
    if (p.dbg_keep && lane == 0) p.dbg_keep[bi] = keep ? 1 : 0;
    __syncthreads();
    if (!keep) continue;

    // ---- refine the kept block ----
    const int8_t* rbp = p.res + bi * kResBytes + lane * 16;
    uint4 R[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) R[c] = *reinterpret_cast<const uint4*>(rbp + c * 1024);
    const uint2 s8w = *reinterpret_cast<const uint2*>(p.rsc + bi * kRscBytes + lane * 8);
    const int co = lane & 15, tp = lane >> 4;
    const uint16_t* vbp = p.v + ((head * p.L_cap + (size_t)blk * 64 + tp) * kHeadDim + 8 * co);
    uint4 Vr[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) Vr[i] = *reinterpret_cast<const uint4*>(vbp + (size_t)(4 * i) * kHeadDim);

    float sc[G];
#pragma unroll
    for (int h = 0; h < G; ++h) sc[h] = est[h][lane];
    const uint32_t s8h[2] = {s8w.x, s8w.y};
#pragma unroll
    for (int g = 0; g < kGroups; ++g) {
      float E[G];
#pragma unroll
      for (int h = 0; h < G; ++h) E[h] = 0.f;
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        const int c = 2 * g + cc;
        const uint32_t rw[4] = {R[c].x, R[c].y, R[c].z, R[c].w};
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t x = rw[w] ^ 0x80808080u;  // offset binary: byte = e + 128
          const uint32_t pa = (__builtin_amdgcn_perm(x, x, 0x0C010C00u) << 2) | 0x5C005C00u;  // 384 + e
          const uint32_t pb = (__builtin_amdgcn_perm(x, x, 0x0C030C02u) << 2) | 0x5C005C00u;
          const int pi = 8 * c + 2 * w;
#pragma unroll
          for (int h = 0; h < G; ++h) {
            E[h] = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, pa), q2[h][pi], E[h], false);
            E[h] = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, pb), q2[h][pi + 1], E[h], false);
          }
        }
      }
      const float s8 = ((g & 1) ? hi_h(s8h[g >> 1]) : lo_h(s8h[g >> 1])) * p.sm_scale;
#pragma unroll
      for (int h = 0; h < G; ++h) sc[h] = fmaf(s8, fmaf(-384.f, qg[h][g], E[h]), sc[h]);
    }
    if (lane >= n_valid) {
#pragma unroll
      for (int h = 0; h < G; ++h) sc[h] = -INFINITY;
    }
    softmax_pv<G, PG>(st, sc, Vr, pw, lane, n_valid);
  }
  write_partial<G>(p, st, b, qh0, chunk, lane);
}

// ---------------------------------------------------------------------------
// Dense flash-decode over fp16 K/V (speed baseline), same chunking + merge.
// ---------------------------------------------------------------------------
template <int G>
__global__ __launch_bounds__(64) void dense_kernel(DecodeParams p) {
  constexpr int PG = (G + 3) & ~3;
  const int chunk = blockIdx.x, hkv = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x;
  const int L = clamp_len(p, b);
  const int nblk = (L + 63) >> 6;
  const int blk0 = chunk * p.cb;
  if (blk0 >= nblk) return;
  const int blk1 = min(nblk, blk0 + p.cb);
  const size_t head = (size_t)b * p.Hkv + hkv;
  const int qh0 = hkv * G;
  __shared__ h2 q2[G][64];
  __shared__ float pw[64][PG];
#pragma unroll
  for (int h = 0; h < G; ++h)
    q2[h][lane] = __builtin_bit_cast(h2, *reinterpret_cast<const uint32_t*>(
                                            p.q + ((size_t)b * p.Hq + qh0 + h) * kHeadDim + 2 * lane));
  __syncthreads();
  SoftmaxState<G> st;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    st.m[h] = -INFINITY;
    st.l[h] = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) st.acc[h][k] = 0.f;
  }
  for (int blk = blk0; blk < blk1; ++blk) {
    const int n_valid = min(64, L - blk * 64);
    const uint16_t* krow = p.k + (head * p.L_cap + (size_t)blk * 64 + lane) * kHeadDim;
    const int co = lane & 15, tp = lane >> 4;
    const uint16_t* vbp = p.v + ((head * p.L_cap + (size_t)blk * 64 + tp) * kHeadDim + 8 * co);
    uint4 Vr[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) Vr[i] = *reinterpret_cast<const uint4*>(vbp + (size_t)(4 * i) * kHeadDim);
    float sc[G];
#pragma unroll
    for (int h = 0; h < G; ++h) sc[h] = 0.f;
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      const uint4 kv = *reinterpret_cast<const uint4*>(krow + 8 * c);
      const uint32_t kw[4] = {kv.x, kv.y, kv.z, kv.w};
#pragma unroll
      for (int w = 0; w < 4; ++w)
#pragma unroll
        for (int h = 0; h < G; ++h)
          sc[h] = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, kw[w]), q2[h][4 * c + w], sc[h], false);
    }
#pragma unroll
    for (int h = 0; h < G; ++h) sc[h] = lane < n_valid ? sc[h] * p.sm_scale : -INFINITY;
    softmax_pv<G, PG>(st, sc, Vr, pw, lane, n_valid);
  }
  write_partial<G>(p, st, b, qh0, chunk, lane);
}

// ---------------------------------------------------------------------------
// Log-sum-exp merge of the chunk partials -> fp16 out.  Grid (Hq, B), 128 threads.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(128) void merge_kernel(DecodeParams p) {
  const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int L = clamp_len(p, b);
  const int nblk = (L + 63) >> 6;
  const int nch = (nblk + p.cb - 1) / p.cb;
  const size_t row = (size_t)b * p.Hq + h;
  const float2* ml = p.part_ml + row * p.nchunk;
  const float* po = p.part_o + row * p.nchunk * kHeadDim;
  __shared__ float red[2];
  float m = -INFINITY;
  for (int c = tid; c < nch; c += 128) {
    const float2 v = ml[c];
    if (v.y > 0.f) m = fmaxf(m, v.x);
  }
  m = wave_max(m);
  if ((tid & 63) == 0) red[tid >> 6] = m;
  __syncthreads();
  const float M = fmaxf(red[0], red[1]);
  __syncthreads();
  float lsum = 0.f;
  for (int c = tid; c < nch; c += 128) {
    const float2 v = ml[c];
    if (v.y > 0.f) lsum += v.y * exp2f((v.x - M) * kLog2e);
  }
  lsum = wave_sum(lsum);
  if ((tid & 63) == 0) red[tid >> 6] = lsum;
  __syncthreads();
  const float Lsum = red[0] + red[1];
  float o = 0.f;
  for (int c = 0; c < nch; ++c) {
    const float2 v = ml[c];
    if (v.y > 0.f) o = fmaf(po[(size_t)c * kHeadDim + tid], exp2f((v.x - M) * kLog2e), o);
  }
  p.out[row * kHeadDim + tid] = __builtin_bit_cast(uint16_t, (_Float16)(o / Lsum));
}

// ---------------------------------------------------------------------------
// host-side launchers
// ---------------------------------------------------------------------------
template <int G>
static void launch_ffd_g(const DecodeParams& p, hipStream_t s) {
  hipLaunchKernelGGL(pseudomax_kernel<G>, dim3(p.Hkv, p.B), dim3(256), 0, s, p);
  if (p.ev_start) (void)hipEventRecord(p.ev_start, s);
  hipLaunchKernelGGL(attend_kernel<G>, dim3(p.nchunk, p.Hkv, p.B), dim3(64), 0, s, p);
  if (p.ev_stop) (void)hipEventRecord(p.ev_stop, s);
  hipLaunchKernelGGL(merge_kernel, dim3(p.Hq, p.B), dim3(128), 0, s, p);
}
template <int G>
static void launch_dense_g(const DecodeParams& p, hipStream_t s) {
  hipLaunchKernelGGL(dense_kernel<G>, dim3(p.nchunk, p.Hkv, p.B), dim3(64), 0, s, p);
  hipLaunchKernelGGL(merge_kernel, dim3(p.Hq, p.B), dim3(128), 0, s, p);
}

#define FFD_DISPATCH_G(FN, G_, P_, S_) \
  switch (G_) {                        \
    case 1: FN<1>(P_, S_); break;      \
    case 2: FN<2>(P_, S_); break;      \
    case 3: FN<3>(P_, S_); break;      \
    case 4: FN<4>(P_, S_); break;      \
    case 5: FN<5>(P_, S_); break;      \
    case 6: FN<6>(P_, S_); break;      \
    case 7: FN<7>(P_, S_); break;      \
    case 8: FN<8>(P_, S_); break;      \
    default: return hipErrorInvalidValue; \
  }

hipError_t launch_ffd_decode(const DecodeParams& p, hipStream_t s) {
  const int G = p.Hq / p.Hkv;
  FFD_DISPATCH_G(launch_ffd_g, G, p, s);
  return hipGetLastError();
}

hipError_t launch_dense_decode(const DecodeParams& p, hipStream_t s) {
  const int G = p.Hq / p.Hkv;
  FFD_DISPATCH_G(launch_dense_g, G, p, s);
  return hipGetLastError();
}

}  // namespace ffd
