// FFD decode attention, one step: pseudo-max, then one fused kernel that scans
// the 2-bit thumbnail, refines the kept blocks and merges the partials; plus the
// dense flash-decode baseline built from the same pieces.
//
// Page: "Faster Than Flash" (gist.science summary of arXiv 2609.00097).
//   Method 2 (Top-delta): keep when s >= m~ - delta, m~ from sink + local tokens.
//   Method 3 stage 1, pseudo-max estimation               -> pseudomax_kernel
//   Method 3 stage 2, stream the 2-bit keys, provisional
//            scores, filter blocks against the threshold   -> attend_kernel phase A
//   Method 3 stage 3, residuals + values of the selected
//            blocks, exact attention (reusing the stage-2
//            scores kept on chip)                          -> attend_kernel phase B
//   log-sum-exp merge of the per-chunk partials            -> merge_kernel
//
// Work decomposition of attend/dense: one work-group (4 wave64) per chunk of `cb`
// 64-token blocks of one (sequence, KV head).  Wave w owns token tile
// [16w, 16w+16) of every block of the chunk, so the four waves do identical work
// and each keeps its own online-softmax state; the states are combined in LDS
// into one partial per chunk, which merge_kernel combines.
#include "ffd_device.h"
#include "ffd_launch.h"

namespace ffd {

__device__ inline int clamp_len(const DecodeParams& p, int b) {
  const int L = p.seq_lens[b];
  return L < 1 ? 1 : (L > p.L_cap ? p.L_cap : L);
}

// quad (4 adjacent lanes) sum, result in every lane of the quad
__device__ inline float quad_sum(float v) {
  v += dpp<kQuadXor1>(v);
  v += dpp<kQuadXor2>(v);
  return v;
}

// ---------------------------------------------------------------------------
// Stage 1: pseudo-max over support tokens [0, min(S,L)) U [max(0,L-W), L).
// Grid (npart, Hkv, B), 256 threads; work-group `part` takes support tokens
// [64*part, 64*part + 64); thread = (token, group).  Exact score of a token:
// sum over groups of scale*(q.c) + zero*sum(q) + rscale*(q.e) with K-hat =
// zero + c*scale + e*rscale.  Writes the part's maximum per query head; the
// attend kernel takes the maximum over parts.
// ---------------------------------------------------------------------------
template <int G>
__global__ __launch_bounds__(256) void pseudomax_kernel(DecodeParams p) {
  __shared__ float qs[G][kHeadDim];
  __shared__ float qsum[G][kGroups];
  __shared__ float red[4][G];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int part = blockIdx.x, hkv = blockIdx.y, b = blockIdx.z;
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
  const int j = part * 64 + (tid >> 2);
  const int g = tid & 3;
  const bool valid = j < n;
  const int t = !valid ? 0 : (j < n_s ? j : lo + (j - n_s));
  const int tb = t & 63;
  const size_t bi = head * p.nblk_cap + (t >> 6);
  const uint8_t* cb = p.codes + bi * kCodesBytes;
  const uint32_t zw = *reinterpret_cast<const uint32_t*>(p.sz + bi * kSzBytes + sz_off(tb, g));
  const float s = lo_h(zw), z = hi_h(zw);
  const float s8 = h2f(*reinterpret_cast<const uint16_t*>(p.rsc + bi * kRscBytes + rsc_off(tb, g)));
  const int8_t* rb = p.res + bi * kResBytes;
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
  for (int h = 0; h < G; ++h) {
    float v = quad_sum(s * A[h] + z * qsum[h][g] + s8 * E[h]) * p.sm_scale;
    v = valid ? v : -INFINITY;
    v = wave_max(v);
    if (lane == 0) red[wave][h] = v;
  }
  __syncthreads();
  if (tid < G) {
    const float m = fmaxf(fmaxf(red[0][tid], red[1][tid]), fmaxf(red[2][tid], red[3][tid]));
    p.pmax[((size_t)b * p.npart + part) * p.Hq + qh0 + tid] = m;
  }
}

// ---------------------------------------------------------------------------
// pieces shared by the attend and dense kernels
// ---------------------------------------------------------------------------
constexpr int kWaves = 4;

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
// 8 int8 residuals -> MFMA A fragment of fp16 values 384 + e (exact)
__device__ inline uint32_t res_pair(uint32_t x, uint32_t sel) {
  return (__builtin_amdgcn_perm(x, x, sel) << 2) | 0x5C005C00u;
}
__device__ inline h8 unpack_res(uint2 r) {
  const uint32_t x = r.x ^ 0x80808080u, y = r.y ^ 0x80808080u;  // offset binary e + 128
  uint4 d;
  d.x = res_pair(x, 0x0C010C00u);
  d.y = res_pair(x, 0x0C030C02u);
  d.z = res_pair(y, 0x0C010C00u);
  d.w = res_pair(y, 0x0C030C02u);
  return __builtin_bit_cast(h8, d);
}

// Per-wave online-softmax state.  Scores arrive in MFMA C layout: lane
// (ks = lane>>4, column) holds rows 4ks..4ks+3 of a 16-token tile for the head
// of its column.  NS score sets per lane (FFD: one per 16-column tile).
template <int G, int NS>
struct WaveSoftmax {
  float m[NS];
  float l[NS];
  float acc[G][8];  // lane (co = lane&15, tp = lane>>4): channels 8co..8co+7, rows tp+4i
  __device__ void init() {
#pragma unroll
    for (int n = 0; n < NS; ++n) { m[n] = -INFINITY; l[n] = 0.f; }
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int k = 0; k < 8; ++k) acc[h][k] = 0.f;
  }
  // fold one score set: returns alpha = exp(m_old - m_new) of the lane's head
  __device__ float fold(int n, float (&s)[4], float* pw_rows /* [16][pg] */, int pg, int head, bool writer,
                        int ks) {
    float tm = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
    tm = fmaxf(tm, xor_lane(tm, 16));
    tm = fmaxf(tm, xor_lane(tm, 32));
    const float mn = fmaxf(m[n], tm);
    const bool live = mn > -INFINITY;
    const float alpha = live ? exp2f((m[n] - mn) * kLog2e) : 1.f;
    float ps = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float pi = live ? exp2f((s[i] - mn) * kLog2e) : 0.f;
      ps += pi;
      if (writer) pw_rows[(4 * ks + i) * pg + head] = pi;
    }
    ps += xor_lane(ps, 16);
    ps += xor_lane(ps, 32);
    l[n] = l[n] * alpha + ps;
    m[n] = mn;
    return alpha;
  }
  // acc = acc * alpha_h + sum_rows p[row][h] * V[row]
  template <int PG>
  __device__ void pv(const float (&alpha)[G], const uint4 (&Vr)[4], const float* pw_rows, int lane,
                     int n_rows_valid) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int k = 0; k < 8; ++k) acc[h][k] *= alpha[h];
    const int tp = lane >> 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = tp + 4 * i;
      if (r < n_rows_valid) {
        float pp[PG];
#pragma unroll
        for (int h4 = 0; h4 < PG; h4 += 4) {
          const float4 v4 = *reinterpret_cast<const float4*>(pw_rows + r * PG + h4);
          pp[h4] = v4.x; pp[h4 + 1] = v4.y; pp[h4 + 2] = v4.z; pp[h4 + 3] = v4.w;
        }
        const uint32_t vw[4] = {Vr[i].x, Vr[i].y, Vr[i].z, Vr[i].w};
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const float vk = (k & 1) ? hi_h(vw[k >> 1]) : lo_h(vw[k >> 1]);
#pragma unroll
          for (int h = 0; h < G; ++h) acc[h][k] = fmaf(pp[h], vk, acc[h][k]);
        }
      }
    }
  }
};

// LDS used by the end-of-chunk combine
template <int G>
struct CombineLds {
  float m[kWaves][G];
  float l[kWaves][G];
  float o[kWaves][G][kHeadDim];
};

// Combine the 4 waves' states into the chunk partial (o[128], m, l) per query
// head.  `head_m`/`head_l` are the lane's state for head `lane_head[n]`,
// stored when `state_writer[n]`.
template <int G, int NS>
__device__ void finish_chunk(const DecodeParams& p, CombineLds<G>& cl, float (&acc)[G][8], int wave, int lane,
                             int tid, int b, int hkv, int chunk, const float (&head_m)[NS],
                             const float (&head_l)[NS], const int (&lane_head)[NS], const bool (&state_writer)[NS]) {
  // reduce acc over the 4 row phases; lanes 0..15 then hold 8 channels each
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      float a = acc[h][k];
      a += xor_lane(a, 16);
      a += xor_lane(a, 32);
      acc[h][k] = a;
    }
  if (lane < 16) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      *reinterpret_cast<float4*>(&cl.o[wave][h][8 * lane]) = make_float4(acc[h][0], acc[h][1], acc[h][2], acc[h][3]);
      *reinterpret_cast<float4*>(&cl.o[wave][h][8 * lane + 4]) = make_float4(acc[h][4], acc[h][5], acc[h][6], acc[h][7]);
    }
  }
#pragma unroll
  for (int n = 0; n < NS; ++n)
    if (state_writer[n]) {
      cl.m[wave][lane_head[n]] = head_m[n];
      cl.l[wave][lane_head[n]] = head_l[n];
    }
  __syncthreads();
  const int qh0 = hkv * G;
  for (int i = tid; i < G * kHeadDim; i += 256) {
    const int h = i >> 7, ch = i & 127;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w)
      if (cl.l[w][h] > 0.f) M = fmaxf(M, cl.m[w][h]);
    float lsum = 0.f, o = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      if (cl.l[w][h] > 0.f) {
        const float f = exp2f((cl.m[w][h] - M) * kLog2e);
        lsum += cl.l[w][h] * f;
        o += cl.o[w][h][ch] * f;
      }
    }
    const size_t row = ((size_t)b * p.Hq + qh0 + h) * p.nchunk + chunk;
    if (lsum > 0.f) p.part_o[row * kHeadDim + ch] = o;
    if (ch == 0) p.part_ml[row] = make_float2(M, lsum);
  }
}

// ---------------------------------------------------------------------------
// Stages 2 + 3.
//
// Scan (phase A, MFMA 16x16x32 f16): per 16-token tile, A = codes as fp16
// (1 + c/4), tokens on rows; B = q with column n = 4*h + g holding head h
// restricted to group g (zero elsewhere), so one accumulator collects
// C[t][(h,g)] = sum_{k in g} (1 + c_k/4) q_hk; starting it at -sum_{k in g} q_hk
// leaves (q_g . c_g)/4.  The fp32 epilogue scales by the group's scale and adds
// zero*sum(q); a quad sum over g gives the estimate.  Block max per head against
// the head's threshold decides the block (union over the GQA group).
//
// Refine (phase B): the residual term uses the same MFMA shape with A = 384 + e
// (exact in fp16) and accumulator start -384*sum(q); exact score = estimate
// (kept in LDS from phase A) + rscale * (q . e); online softmax in the MFMA
// output layout; P.V on VALU with lanes over channels.
// ---------------------------------------------------------------------------
template <int G>
struct AttendCfg {
  static constexpr int NT = (G + 3) / 4;
  static constexpr int PG = (G + 3) & ~3;
  static constexpr int CBMAX = (G <= 4) ? 32 : 16;
};

template <int G>
__global__ __launch_bounds__(256) void attend_kernel(DecodeParams p) {
  constexpr int NT = AttendCfg<G>::NT, PG = AttendCfg<G>::PG, CBMAX = AttendCfg<G>::CBMAX;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int chunk = blockIdx.x, hkv = blockIdx.y, b = blockIdx.z;
  const int L = clamp_len(p, b);
  const int nblk = (L + 63) >> 6;
  const int blk0 = chunk * p.cb;
  if (blk0 >= nblk) return;
  const int nbl = min(p.cb, nblk - blk0);
  const size_t head = (size_t)b * p.Hkv + hkv;
  const int qh0 = hkv * G;

  __shared__ h2 q2[G][64];
  __shared__ float qg[G][kGroups];
  __shared__ float thr_s[G];
  __shared__ float tmax[CBMAX][kWaves][G];
  __shared__ int klist[CBMAX];
  __shared__ int nkeep;
  __shared__ float pw[kWaves][16 * PG];
  __shared__ union U {
    float est[CBMAX][kWaves][G][16];
    CombineLds<G> cl;
  } u;

  for (int i = tid; i < G * 64; i += 256)
    q2[i >> 6][i & 63] = __builtin_bit_cast(
        h2, *reinterpret_cast<const uint32_t*>(p.q + ((size_t)b * p.Hq + qh0 + (i >> 6)) * kHeadDim + 2 * (i & 63)));
  if (tid < G) {
    float m = -INFINITY;
    for (int pp = 0; pp < p.npart; ++pp) m = fmaxf(m, p.pmax[((size_t)b * p.npart + pp) * p.Hq + qh0 + tid]);
    thr_s[tid] = m - p.delta;
    if (chunk == 0 && p.dbg_mt) p.dbg_mt[(size_t)b * p.Hq + qh0 + tid] = m;
  }
  __syncthreads();
  if (tid < G * kGroups) {
    const int h = tid >> 2, g = tid & 3;
    float s = 0.f;
    for (int k = 0; k < 16; ++k) { const h2 v = q2[h][16 * g + k]; s += (float)v.x + (float)v.y; }
    qg[h][g] = s;
  }
  __syncthreads();

  // MFMA lane roles: A row / C column = lane & 15, k-slice / C row group = lane >> 4
  const int col = lane & 15, hc = col >> 2, gc = col & 3, ks = lane >> 4;
  h8 Bf[NT][kGroups];
  float c_est[NT], c_res[NT], qq[NT];
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
    const float Q = live ? qg[h][gc] : 0.f;
    c_est[nt] = -Q;
    c_res[nt] = -384.f * Q;
    qq[nt] = 0.25f * Q;
  }
  const float scale4 = 4.f * p.sm_scale;

  // ---- phase A: scan tile `wave` of every block of the chunk ----
  {
    const size_t bi0 = head * p.nblk_cap + blk0;
    const uint8_t* cbase = p.codes + bi0 * kCodesBytes + ((col * 4 + ks) * 4 + wave) * 8;
    const uint8_t* zbase = p.sz + bi0 * kSzBytes + ((gc * 4 + ks) * 4 + wave) * 16;
    for (int j0 = 0; j0 < nbl; j0 += 4) {
      uint2 cw[4];
      uint4 zw[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int jj = min(j0 + v, nbl - 1);
        cw[v] = *reinterpret_cast<const uint2*>(cbase + (size_t)jj * kCodesBytes);
        zw[v] = *reinterpret_cast<const uint4*>(zbase + (size_t)jj * kSzBytes);
      }
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int j = j0 + v;
        if (j < nbl) {
          const h8 a0 = unpack_even(cw[v].x), a1 = unpack_odd(cw[v].x);
          const h8 a2 = unpack_even(cw[v].y), a3 = unpack_odd(cw[v].y);
          const uint32_t zs[4] = {zw[v].x, zw[v].y, zw[v].z, zw[v].w};
          const int row0 = (blk0 + j) * 64 + 16 * wave + 4 * ks;
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            f4 c = {c_est[nt], c_est[nt], c_est[nt], c_est[nt]};
            c = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, Bf[nt][0], c, 0, 0, 0);
            c = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, Bf[nt][1], c, 0, 0, 0);
            c = __builtin_amdgcn_mfma_f32_16x16x32_f16(a2, Bf[nt][2], c, 0, 0, 0);
            c = __builtin_amdgcn_mfma_f32_16x16x32_f16(a3, Bf[nt][3], c, 0, 0, 0);
            float e4[4];
            float mx = -INFINITY;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              float v4 = quad_sum(fmaf(lo_h(zs[i]), c[i], hi_h(zs[i]) * qq[nt]));
              v4 = (row0 + i < L) ? v4 * scale4 : -INFINITY;
              e4[i] = v4;
              mx = fmaxf(mx, v4);
            }
            mx = fmaxf(mx, xor_lane(mx, 16));
            mx = fmaxf(mx, xor_lane(mx, 32));
            const int h = 4 * nt + hc;
            if (gc == 0 && h < G) {
              *reinterpret_cast<float4*>(&u.est[j][wave][h][4 * ks]) = make_float4(e4[0], e4[1], e4[2], e4[3]);
              if (ks == 0) tmax[j][wave][h] = mx;
            }
          }
        }
      }
    }
  }
  __syncthreads();

  // ---- block decisions: forced (sink/local) or some head reaches its threshold ----
  if (wave == 0) {
    bool kp = false;
    if (lane < nbl) {
      const int blk = blk0 + lane;
      const int sink_end = p.sink > 0 ? ((min(p.sink, L) + 63) >> 6) : 0;
      const int local_beg = p.local > 0 ? (max(0, L - p.local) >> 6) : nblk;
      kp = blk < sink_end || blk >= local_beg;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float bm = fmaxf(fmaxf(tmax[lane][0][h], tmax[lane][1][h]), fmaxf(tmax[lane][2][h], tmax[lane][3][h]));
        kp = kp || (bm >= thr_s[h]);
        if (p.dbg_bmax) p.dbg_bmax[((size_t)b * p.Hq + qh0 + h) * p.nblk_cap + blk] = bm;
      }
      if (p.dbg_keep) p.dbg_keep[head * p.nblk_cap + blk] = kp ? 1 : 0;
    }
    const uint64_t mask = __ballot(kp);
    if (kp) klist[__popcll(mask & ((1ull << lane) - 1ull))] = lane;
    if (lane == 0) nkeep = __popcll(mask);
  }
  __syncthreads();
  const int K = nkeep;

  // ---- phase B: refine tile `wave` of every kept block ----
  WaveSoftmax<G, NT> st;
  st.init();
  float* pwv = pw[wave];
  {
    const int co = lane & 15, tp = lane >> 4;
    const int t_a = 16 * wave + col;  // token of this lane's A-fragment row
    uint2 R[kGroups];
    uint2 S8;
    uint4 Vr[4];
    auto load_block = [&](int j) {
      const size_t bi = head * p.nblk_cap + blk0 + j;
      const int8_t* rb = p.res + bi * kResBytes;
#pragma unroll
      for (int g = 0; g < kGroups; ++g)
        R[g] = *reinterpret_cast<const uint2*>(rb + ((2 * g + (ks >> 1)) * 64 + t_a) * 16 + 8 * (ks & 1));
      S8 = *reinterpret_cast<const uint2*>(p.rsc + bi * kRscBytes + (gc * 64 + 16 * wave + 4 * ks) * 2);
      const uint16_t* vb = p.v + ((head * p.L_cap + (size_t)(blk0 + j) * 64 + 16 * wave + tp) * kHeadDim + 8 * co);
#pragma unroll
      for (int i = 0; i < 4; ++i) Vr[i] = *reinterpret_cast<const uint4*>(vb + (size_t)(4 * i) * kHeadDim);
    };
    if (K > 0) load_block(klist[0]);
    for (int kk = 0; kk < K; ++kk) {
      const int j = klist[kk];
      const int row_base = (blk0 + j) * 64 + 16 * wave;
      const int n_rows = min(16, L - row_base);
      // current block's registers; the next kept block is loaded meanwhile
      uint2 Rc[kGroups];
#pragma unroll
      for (int g = 0; g < kGroups; ++g) Rc[g] = R[g];
      const uint2 S8c = S8;
      uint4 Vc[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) Vc[i] = Vr[i];
      if (kk + 1 < K) load_block(klist[kk + 1]);
      if (n_rows <= 0) continue;  // this wave's tile lies past the sequence end

      const h8 r0 = unpack_res(Rc[0]), r1 = unpack_res(Rc[1]), r2 = unpack_res(Rc[2]), r3 = unpack_res(Rc[3]);
      const float s8r[4] = {lo_h(S8c.x), hi_h(S8c.x), lo_h(S8c.y), hi_h(S8c.y)};
      float alpha_l[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        f4 c = {c_res[nt], c_res[nt], c_res[nt], c_res[nt]};
        c = __builtin_amdgcn_mfma_f32_16x16x32_f16(r0, Bf[nt][0], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x32_f16(r1, Bf[nt][1], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x32_f16(r2, Bf[nt][2], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x32_f16(r3, Bf[nt][3], c, 0, 0, 0);
        const int h = 4 * nt + hc;
        const int hh = h < G ? h : 0;
        const float4 e4 = *reinterpret_cast<const float4*>(&u.est[j][wave][hh][4 * ks]);
        const float ev[4] = {e4.x, e4.y, e4.z, e4.w};
        float s[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float rterm = quad_sum(s8r[i] * c[i]);
          s[i] = (4 * ks + i < n_rows) ? fmaf(p.sm_scale, rterm, ev[i]) : -INFINITY;
        }
        alpha_l[nt] = st.fold(nt, s, pwv, PG, hh, gc == 0 && h < G, ks);
      }
      float alpha[G];
#pragma unroll
      for (int h = 0; h < G; ++h) alpha[h] = uniform_lane(alpha_l[h >> 2], 4 * (h & 3));
      st.template pv<PG>(alpha, Vc, pwv, lane, n_rows);
    }
  }
  __syncthreads();  // est is no longer read: its LDS is reused by the combine

  float hm[NT], hl[NT];
  int hidx[NT];
  bool hw[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    hm[nt] = st.m[nt];
    hl[nt] = st.l[nt];
    hidx[nt] = 4 * nt + hc;
    hw[nt] = (lane < 16) && (gc == 0) && (4 * nt + hc < G);
  }
  finish_chunk<G, NT>(p, u.cl, st.acc, wave, lane, tid, b, hkv, chunk, hm, hl, hidx, hw);
}

// ---------------------------------------------------------------------------
// Dense flash-decode over fp16 K/V (speed baseline) with the same chunking,
// softmax, P.V, combine and merge kernel.  QK on MFMA: A = K tile (16 tokens x 32
// channels per group), B = q with one column per head.
// ---------------------------------------------------------------------------
template <int G>
__global__ __launch_bounds__(256) void dense_kernel(DecodeParams p) {
  constexpr int PG = (G + 3) & ~3;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int chunk = blockIdx.x, hkv = blockIdx.y, b = blockIdx.z;
  const int L = clamp_len(p, b);
  const int nblk = (L + 63) >> 6;
  const int blk0 = chunk * p.cb;
  if (blk0 >= nblk) return;
  const int nbl = min(p.cb, nblk - blk0);
  const size_t head = (size_t)b * p.Hkv + hkv;
  const int qh0 = hkv * G;
  __shared__ h2 q2[G][64];
  __shared__ float pw[kWaves][16 * PG];
  __shared__ CombineLds<G> cl;
  for (int i = tid; i < G * 64; i += 256)
    q2[i >> 6][i & 63] = __builtin_bit_cast(
        h2, *reinterpret_cast<const uint32_t*>(p.q + ((size_t)b * p.Hq + qh0 + (i >> 6)) * kHeadDim + 2 * (i & 63)));
  __syncthreads();
  const int col = lane & 15, ks = lane >> 4;
  h8 Bd[kGroups];
#pragma unroll
  for (int g = 0; g < kGroups; ++g) {
    h8 f;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      h2 pr = {(_Float16)0.f, (_Float16)0.f};
      if (col < G) pr = q2[col][16 * g + 4 * ks + d];
      f[2 * d] = pr.x;
      f[2 * d + 1] = pr.y;
    }
    Bd[g] = f;
  }
  WaveSoftmax<G, 1> st;
  st.init();
  float* pwv = pw[wave];
  const int co = lane & 15, tp = lane >> 4;
  const int t_a = 16 * wave + col;
  uint4 Kr[kGroups], Vr[4];
  auto load_block = [&](int j) {
    const size_t row = head * p.L_cap + (size_t)(blk0 + j) * 64;
    const uint16_t* kb = p.k + (row + t_a) * kHeadDim + 8 * ks;
#pragma unroll
    for (int g = 0; g < kGroups; ++g) Kr[g] = *reinterpret_cast<const uint4*>(kb + 32 * g);
    const uint16_t* vb = p.v + (row + 16 * wave + tp) * kHeadDim + 8 * co;
#pragma unroll
    for (int i = 0; i < 4; ++i) Vr[i] = *reinterpret_cast<const uint4*>(vb + (size_t)(4 * i) * kHeadDim);
  };
  load_block(0);
  for (int j = 0; j < nbl; ++j) {
    const int row_base = (blk0 + j) * 64 + 16 * wave;
    const int n_rows = min(16, L - row_base);
    uint4 Kc[kGroups], Vc[4];
#pragma unroll
    for (int g = 0; g < kGroups; ++g) Kc[g] = Kr[g];
#pragma unroll
    for (int i = 0; i < 4; ++i) Vc[i] = Vr[i];
    if (j + 1 < nbl) load_block(j + 1);
    if (n_rows <= 0) continue;
    f4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int g = 0; g < kGroups; ++g)
      c = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, Kc[g]), Bd[g], c, 0, 0, 0);
    float s[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) s[i] = (4 * ks + i < n_rows) ? c[i] * p.sm_scale : -INFINITY;
    const int hh = col < G ? col : 0;
    const float al = st.fold(0, s, pwv, PG, hh, col < G, ks);
    float alpha[G];
#pragma unroll
    for (int h = 0; h < G; ++h) alpha[h] = uniform_lane(al, h);
    st.template pv<PG>(alpha, Vc, pwv, lane, n_rows);
  }
  const float hm[1] = {st.m[0]}, hl[1] = {st.l[0]};
  const int hidx[1] = {col < G ? col : 0};
  const bool hw[1] = {lane < G};
  finish_chunk<G, 1>(p, cl, st.acc, wave, lane, tid, b, hkv, chunk, hm, hl, hidx, hw);
}

// ---------------------------------------------------------------------------
// Log-sum-exp merge of the chunk partials -> fp16 out:
//   M = max_c m_c,  out = sum_c o_c e^{m_c - M} / sum_c l_c e^{m_c - M}.
// Grid (Hq, B, 4): work-group = one query head, 32 output channels; its 256
// threads are 8 chunk phases x 32 channels, chunk weights staged in LDS.
// ---------------------------------------------------------------------------
constexpr int kMergePiece = 1024;

__global__ __launch_bounds__(256) void merge_kernel(DecodeParams p) {
  __shared__ float wts[kMergePiece];
  __shared__ float red[8][33];
  __shared__ float Msh, Lsh;
  const int h = blockIdx.x, b = blockIdx.y, slice = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int L = clamp_len(p, b);
  const int nblk = (L + 63) >> 6;
  const int nch = (nblk + p.cb - 1) / p.cb;
  const size_t row = (size_t)b * p.Hq + h;
  const float2* ml = p.part_ml + row * p.nchunk;
  float m = -INFINITY;
  for (int c = tid; c < nch; c += 256) {
    const float2 v = ml[c];
    if (v.y > 0.f) m = fmaxf(m, v.x);
  }
  m = wave_max(m);
  if (lane == 0) red[0][wave] = m;
  __syncthreads();
  if (tid == 0) Msh = fmaxf(fmaxf(red[0][0], red[0][1]), fmaxf(red[0][2], red[0][3]));
  __syncthreads();
  const float M = Msh;
  const int cp = tid >> 5, ch = 32 * slice + (tid & 31);
  const float* po = p.part_o + row * p.nchunk * kHeadDim + ch;
  float o = 0.f, ls = 0.f;
  for (int c0 = 0; c0 < nch; c0 += kMergePiece) {
    const int n = min(kMergePiece, nch - c0);
    __syncthreads();
    for (int c = tid; c < n; c += 256) {
      const float2 v = ml[c0 + c];
      const float w = v.y > 0.f ? exp2f((v.x - M) * kLog2e) : 0.f;
      wts[c] = w;
      ls += w * (v.y > 0.f ? v.y : 0.f);
    }
    __syncthreads();
#pragma unroll 8
    for (int c = cp; c < n; c += 8) {
      const float w = wts[c];
      if (w > 0.f) o = fmaf(w, po[(size_t)(c0 + c) * kHeadDim], o);
    }
  }
  ls = wave_sum(ls);
  __syncthreads();
  red[cp][tid & 31] = o;
  __syncthreads();
  if (lane == 0) wts[wave] = ls;
  __syncthreads();
  if (tid < 32) {
    float acc = 0.f;
#pragma unroll
    for (int q = 0; q < 8; ++q) acc += red[q][tid];
    const float lsum = (wts[0] + wts[1]) + (wts[2] + wts[3]);
    p.out[row * kHeadDim + ch] = __builtin_bit_cast(uint16_t, (_Float16)(acc / lsum));
  }
}

// ---------------------------------------------------------------------------
// host-side launchers
// ---------------------------------------------------------------------------
template <int G>
static void launch_ffd_g(const DecodeParams& p, hipStream_t s) {
  const int stages = p.stages ? p.stages : 7;
  if (stages & 1)
    hipLaunchKernelGGL(pseudomax_kernel<G>, dim3(p.npart, p.Hkv, p.B), dim3(256), 0, s, p);
  if (stages & 2) {
    if (p.ev_start) (void)hipEventRecord(p.ev_start, s);
    hipLaunchKernelGGL(attend_kernel<G>, dim3(p.nchunk, p.Hkv, p.B), dim3(256), 0, s, p);
    if (p.ev_stop) (void)hipEventRecord(p.ev_stop, s);
  }
  if (stages & 4) hipLaunchKernelGGL(merge_kernel, dim3(p.Hq, p.B, 4), dim3(256), 0, s, p);
}
template <int G>
static void launch_dense_g(const DecodeParams& p, hipStream_t s) {
  hipLaunchKernelGGL(dense_kernel<G>, dim3(p.nchunk, p.Hkv, p.B), dim3(256), 0, s, p);
  hipLaunchKernelGGL(merge_kernel, dim3(p.Hq, p.B, 4), dim3(256), 0, s, p);
}

#define FFD_DISPATCH_G(FN, G_, P_, S_)    \
  switch (G_) {                           \
    case 1: FN<1>(P_, S_); break;         \
    case 2: FN<2>(P_, S_); break;         \
    case 3: FN<3>(P_, S_); break;         \
    case 4: FN<4>(P_, S_); break;         \
    case 5: FN<5>(P_, S_); break;         \
    case 6: FN<6>(P_, S_); break;         \
    case 7: FN<7>(P_, S_); break;         \
    case 8: FN<8>(P_, S_); break;         \
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
