// FFD decode on long caches as two kernels between the pseudo-max and the
// merge: a scan that decides which blocks are kept, and a refine over the kept
// blocks only, split evenly across the device.
//
// Page: "Faster Than Flash" (gist.science summary of arXiv 2609.00097),
// Method 3: stage 2 streams the 2-bit keys, computes provisional scores and
// filters blocks against the threshold; stage 3 loads the 8-bit residuals and
// the values of the selected blocks only and computes exact attention.
//
// scan_kernel   grid (chunks of 32 blocks, Hkv, B).  The thumbnail scan and
//               block decision of the fused kernel (same arithmetic, so the
//               same kept blocks) without any refine state, which lets more
//               waves share a SIMD.  Each work-group writes one 32-bit keep
//               bitmap word: bit j = block 32 * chunk + j is kept.
// refine_kernel a 1-D grid of work-groups that each rebuild the same
//               compaction from the bitmap words: per (sequence, KV head) its
//               kept blocks in increasing order, cut into units of
//               U = ceil(T / R) blocks (T = all kept blocks, R = the refine
//               work-groups resident at once), unit ids numbered head after
//               head.  There are at most R + B*Hkv units (a head's last unit
//               may be short) and as many work-groups: work-group u refines
//               unit u and writes its partial (o, m, l) per query head;
//               work-group 0 publishes the first unit of every head for the
//               merge.  The split of the blocks into units and
//               the partial of each unit depend only on the kept blocks, so
//               the result is deterministic.  The exact score of a kept token
//               is its estimate recomputed from the thumbnail (the scan's
//               estimates are not kept; the same arithmetic, so the same
//               bits) plus the residual term.
#include "ffd_tiles.h"

namespace ffd {

constexpr int kScanChunk = 32;  // blocks per scan work-group: one keep bitmap word

__device__ inline int wave_sum_i(int v) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v += __shfl_xor(v, m, 64);
  return v;
}

// inclusive prefix sum over the 64 lanes of a wave
__device__ inline int wave_prefix_i(int v, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int u = __shfl_up(v, d, 64);
    v += lane >= d ? u : 0;
  }
  return v;
}

// ---------------------------------------------------------------------------
// Stage 2 alone: scan 32 contiguous blocks of one (sequence, KV head), decide.
// Dynamic LDS: the block-max diagnostic's per-(block, wave row group) maxima
// [32][16][G] (only when the diagnostic is requested).
// ---------------------------------------------------------------------------
template <int G>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(G <= 4 ? 5 : 4))) void scan_kernel(
    DecodeParams p) {
  constexpr int NT = QFrags<G>::NT;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int col = lane & 15, ks = lane >> 4;
  const int chunk = blockIdx.x, hkv = blockIdx.y, b = blockIdx.z;
  __shared__ uint32_t qs[G * 64];
  __shared__ float pm_s[256];
  __shared__ int kflag[kWaves][kScanChunk];
  extern __shared__ __align__(16) float tmax[];
  const int L = clamp_len(p, b);
  const int nblk = (L + 63) >> 6;
  const int blk0 = chunk * kScanChunk;
  const int nbl = min(kScanChunk, nblk - blk0);
  if (nbl <= 0) return;
  const size_t head = (size_t)b * p.Hkv + hkv;
  const int qh0 = hkv * G;
  const TileOffsets to(wave, lane);
  const size_t hb = head * p.nblk_cap;
  const uint32_t nbc = (uint32_t)p.nblk_cap;
  const __amdgpu_buffer_rsrc_t r_codes = make_rsrc(p.codes + hb * kCodesBytes, nbc * kCodesBytes);
  const __amdgpu_buffer_rsrc_t r_sz = make_rsrc(p.sz + hb * kSzBytes, nbc * kSzBytes);

  // prologue: q, the first thumbnail batch and the partial pseudo-maxima together
  typename QFrags<G>::Stage qst;
  QFrags<G>::stage_load(p.q + ((size_t)b * p.Hq + qh0) * kHeadDim, tid, qst);
  uint2 cwA[4], cwB[4];
  uint32_t zwA[4], zwB[4];
  auto load_batch = [&](int j0, uint2 (&cw)[4], uint32_t (&zw)[4]) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const uint32_t blk = (uint32_t)(blk0 + min(j0 + v, nbl - 1));
      cw[v] = buf_load_b64<kNonTemporal>(r_codes, (uint32_t)to.codes, blk * kCodesBytes);
      zw[v] = buf_load_b32<kNonTemporal>(r_sz, (uint32_t)to.szt, blk * kSzBytes);
    }
  };
  load_batch(0, cwA, zwA);
  const int n_pm = p.npart * G;
  float pm_t = -INFINITY;
  {
    const float* pm = p.pmax + (size_t)b * p.npart * p.Hq + qh0;
    if (tid < n_pm) pm_t = pm[(size_t)(tid / G) * p.Hq + tid % G];
    for (int i = tid + (256 / G) * G; i < n_pm; i += (256 / G) * G) pm_t = fmaxf(pm_t, pm[(size_t)(i / G) * p.Hq + i % G]);
  }
  QFrags<G>::stage_store(qst, tid, qs);
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  pm_s[tid] = pm_t;
  __syncthreads();
  typename QFrags<G>::Load ql;
  QFrags<G>::load(qs, lane, ql);
  QFrags<G> qf;
  qf.build(ql, lane);
  int zsrc[kGroups];
#pragma unroll
  for (int g = 0; g < kGroups; ++g) zsrc[g] = (col | (g << 4)) << 2;
  // threshold of the lane's row-group head 4*nt + ks, in dot-product units
  const int n_pt = min(n_pm, (256 / G) * G) / G;
  float thr_t[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int h = min(4 * nt + ks, G - 1);
    float m = -INFINITY;
    for (int pp = 0; pp < n_pt; ++pp) m = fmaxf(m, pm_s[pp * G + h]);
    thr_t[nt] = 4 * nt + ks < G ? (m - p.delta) / p.sm_scale : INFINITY;
  }
  if (chunk == 0 && p.dbg_mt && tid < G) {
    float m = -INFINITY;
    for (int pp = 0; pp < n_pt; ++pp) m = fmaxf(m, pm_s[pp * G + tid]);
    p.dbg_mt[(size_t)b * p.Hq + qh0 + tid] = m;
  }
  const bool dbg_bmax = p.dbg_bmax != nullptr;
  // rows past the sequence end matter only without a local window (with one,
  // the block holding the last token is always kept) or for the diagnostic
  const bool tail_mask = p.local == 0 || dbg_bmax;

  auto scan_batch = [&](int j0, const uint2 (&cw)[4], const uint32_t (&zw)[4]) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int j = j0 + v;
      if (j < nbl) {
        const uint4 z4 = make_uint4((uint32_t)__builtin_amdgcn_ds_bpermute(zsrc[0], (int)zw[v]),
                                    (uint32_t)__builtin_amdgcn_ds_bpermute(zsrc[1], (int)zw[v]),
                                    (uint32_t)__builtin_amdgcn_ds_bpermute(zsrc[2], (int)zw[v]),
                                    (uint32_t)__builtin_amdgcn_ds_bpermute(zsrc[3], (int)zw[v]));
        float e[NT];
        qf.estimate_t(cw[v], z4, e);
        if (tail_mask && (blk0 + j + 1) * 64 > L) {
          const bool valid = (blk0 + j) * 64 + 16 * wave + col < L;
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) e[nt] = valid ? e[nt] : -INFINITY;
        }
        bool reach = false;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          reach = reach || (e[nt] >= thr_t[nt]);
          if (dbg_bmax) {
            float qm = fmaxf(e[nt], dpp<kQuadXor1>(e[nt]));
            qm = fmaxf(qm, dpp<kQuadXor2>(qm));
            const int h = 4 * nt + ks;
            if (h < G && (col & 3) == 0) tmax[(j * 4 * kWaves + 4 * wave + (col >> 2)) * G + h] = qm;
          }
        }
        const bool any = __builtin_amdgcn_ballot_w64(reach) != 0;
        if (lane == 0) kflag[wave][j] = any ? 1 : 0;
      }
    }
  };
  const int nbat = (nbl + 3) >> 2;
  int i0 = 0;
  for (; i0 + 2 < nbat; i0 += 2) {
    load_batch(4 * (i0 + 1), cwB, zwB);
    scan_batch(4 * i0, cwA, zwA);
    load_batch(4 * (i0 + 2), cwA, zwA);
    scan_batch(4 * (i0 + 1), cwB, zwB);
  }
  if (i0 + 1 < nbat) {
    load_batch(4 * (i0 + 1), cwB, zwB);
    scan_batch(4 * i0, cwA, zwA);
    scan_batch(4 * (i0 + 1), cwB, zwB);
  } else {
    scan_batch(4 * i0, cwA, zwA);
  }
  __syncthreads();

  // decision: forced blocks (sink, local window) or a head reaching its threshold
  if (wave == 0) {
    const int sink_end = p.sink > 0 ? ((min(p.sink, L) + 63) >> 6) : 0;
    const int local_beg = p.local > 0 ? (max(0, L - p.local) >> 6) : nblk;
    bool kp = false;
    if (lane < nbl) {
      const int blk = blk0 + lane;
      const int any = kflag[0][lane] | kflag[1][lane] | kflag[2][lane] | kflag[3][lane];
      kp = blk < sink_end || blk >= local_beg || any != 0;
      if (p.dbg_keep) p.dbg_keep[head * p.nblk_cap + blk] = kp ? 1 : 0;
      if (dbg_bmax) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float* tm = tmax + lane * 4 * kWaves * G + h;
          float bm = tm[0];
#pragma unroll
          for (int r = 1; r < 4 * kWaves; ++r) bm = fmaxf(bm, tm[r * G]);
          p.dbg_bmax[((size_t)b * p.Hq + qh0 + h) * p.nblk_cap + blk] = bm * p.sm_scale;
        }
      }
    }
    const uint64_t bal = __builtin_amdgcn_ballot_w64(kp);
    if (lane == 0) p.kmask[head * p.nword_cap + chunk] = (uint32_t)bal;
  }
}

// ---------------------------------------------------------------------------
// Stage 3 over the compacted kept blocks.
// ---------------------------------------------------------------------------
struct RefineTile {
  uint2 cw;     // codes of the lane's token row (transposed-scan layout)
  uint32_t zw;  // one (scale, zero) pair: token 16w + col, group ks
  uint2 R[kGroups], S8;
  uint4 V[4];
};

// kept blocks of one head in increasing order, from its bitmap words in LDS
// (wave-uniform state)
struct KeptIter {
  const uint32_t* words;
  int w;
  uint32_t m;
  __device__ int next() {
    while (m == 0) m = words[++w];
    const int blk = 32 * w + __builtin_ctz(m);
    m &= m - 1;
    return blk;
  }
};

// Dynamic LDS: bitmap words [B*Hkv][nword_cap], unit starts [B*Hkv + 1],
// kept counts [B*Hkv].
template <int G>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void refine_kernel(
    DecodeParams p) {
  constexpr int NT = QFrags<G>::NT;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int col = lane & 15, hc = col >> 2, gc = col & 3, ks = lane >> 4;
  __shared__ uint32_t qs[G * 64];
  __shared__ CombineLds<G> cl;
  __shared__ float estl[kWaves][G][16];  // a wave's estimates, scan layout -> refine layout
  __shared__ int s_u;
  extern __shared__ __align__(16) uint32_t words[];
  const int nheads = p.B * p.Hkv, nwc = p.nword_cap;
  int* const ustart = reinterpret_cast<int*>(words + (size_t)nheads * nwc);
  int* const kcount = ustart + nheads + 1;

  // 1. bitmap words (those past a sequence's last block read as 0)
  for (int i = tid; i < nheads * nwc; i += 256) {
    const int r = i / nwc, w = i - r * nwc;
    const int nb = (clamp_len(p, r / p.Hkv) + 63) >> 6;
    words[i] = 32 * w < nb ? p.kmask[i] : 0u;
  }
  __syncthreads();
  // 2. kept blocks per head
  for (int r = wave; r < nheads; r += kWaves) {
    int c = 0;
    for (int w = lane; w < nwc; w += 64) c += __popc(words[r * nwc + w]);
    c = wave_sum_i(c);
    if (lane == 0) kcount[r] = c;
  }
  __syncthreads();
  // 3. unit size U = ceil(T / grid) and the first unit of every head
  if (wave == 0) {
    int t = 0;
    for (int r = lane; r < nheads; r += 64) t += kcount[r];
    t = wave_sum_i(t);
    const int U = max(1, (t + p.refine_groups - 1) / p.refine_groups);
    int run = 0;
    for (int r0 = 0; r0 < nheads; r0 += 64) {
      const int r = r0 + lane;
      const int n = r < nheads ? (kcount[r] + U - 1) / U : 0;
      const int incl = wave_prefix_i(n, lane);
      if (r < nheads) ustart[r] = run + incl - n;
      run += __shfl(incl, 63, 64);
    }
    if (lane == 0) {
      ustart[nheads] = run;
      s_u = U;
    }
  }
  __syncthreads();
  const int U = s_u, nunits = ustart[nheads];
  if (blockIdx.x == 0)
    for (int r = tid; r <= nheads; r += 256) p.unit_start[r] = ustart[r];
  // one unit per work-group: there are at most refine_groups + B*Hkv units
  // (each head's last unit may be short), as many as work-groups
  const int ug = blockIdx.x;
  if (ug >= nunits) return;

  const float c2 = p.sm_scale * kLog2e, slack = 8.f / c2;
  const TileOffsets to(wave, lane);
  const uint32_t v_lane = (uint32_t)(((4 * wave + ks) * kHeadDim + 8 * col) * 4 * sizeof(uint16_t));
  const uint32_t nbc = (uint32_t)p.nblk_cap;
  {
    // the head holding unit ug: the last r with ustart[r] <= ug
    int lo = 0, hi = nheads - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (ustart[mid] <= ug) lo = mid;
      else hi = mid - 1;
    }
    const int r = lo;
    const int b = r / p.Hkv, hkv = r - b * p.Hkv;
    const int L = clamp_len(p, b);
    const int k0 = (ug - ustart[r]) * U, nk = min(U, kcount[r] - k0);
    const size_t hb = (size_t)r * p.nblk_cap;
    const __amdgpu_buffer_rsrc_t r_codes = make_rsrc(p.codes + hb * kCodesBytes, nbc * kCodesBytes);
    const __amdgpu_buffer_rsrc_t r_sz = make_rsrc(p.sz + hb * kSzBytes, nbc * kSzBytes);
    const __amdgpu_buffer_rsrc_t r_res = make_rsrc(p.res + hb * kResBytes, nbc * kResBytes);
    const __amdgpu_buffer_rsrc_t r_rsc = make_rsrc(p.rsc + hb * kRscBytes, nbc * kRscBytes);
    const __amdgpu_buffer_rsrc_t r_v = make_rsrc(p.v + (size_t)r * p.L_cap * kHeadDim, nbc * kVBytes);
    auto load_block = [&](int blk, RefineTile& x) {
      const uint32_t bo = (uint32_t)blk;
      x.cw = buf_load_b64<kNonTemporal>(r_codes, (uint32_t)to.codes, bo * kCodesBytes);
      x.zw = buf_load_b32<kNonTemporal>(r_sz, (uint32_t)to.szt, bo * kSzBytes);
#pragma unroll
      for (int g = 0; g < kGroups; ++g) x.R[g] = buf_load_b64<kNonTemporal>(r_res, (uint32_t)to.res + g * 2048, bo * kResBytes);
      x.S8 = buf_load_b64<kNonTemporal>(r_rsc, (uint32_t)to.rsc, bo * kRscBytes);
#pragma unroll
      for (int q = 0; q < 4; ++q) x.V[q] = buf_load_b128(r_v, v_lane + 16 * q, bo * kVBytes);
    };
    // the unit's first block: skip the head's first k0 kept blocks, a wave of
    // bitmap words at a time (every wave derives the same position)
    KeptIter it;
    it.words = words + (size_t)r * nwc;
    {
      int base = 0, w0 = 0;
      for (;; w0 += 64) {
        const int w = w0 + lane;
        const int c = w < nwc ? __popc(it.words[w]) : 0;
        const int incl = wave_prefix_i(c, lane);
        const uint64_t past = __builtin_amdgcn_ballot_w64(base + incl > k0);
        if (past) {
          const int lw = __builtin_ctzll(past);
          const int before = base + __shfl(incl - c, lw, 64);
          it.w = w0 + lw;
          uint32_t m = it.words[it.w];
          for (int s = before; s < k0; ++s) m &= m - 1;  // drop the kept blocks before the unit
          it.m = m;
          break;
        }
        base += __shfl(incl, 63, 64);
      }
    }
    RefineTile X, Y;
    int bx = it.next();
    // q of the head, staged through LDS, behind the first block's loads
    typename QFrags<G>::Stage qst;
    QFrags<G>::stage_load(p.q + ((size_t)b * p.Hq + hkv * G) * kHeadDim, tid, qst);
    load_block(bx, X);
    QFrags<G>::stage_store(qst, tid, qs);
    __syncthreads();
    typename QFrags<G>::Load ql;
    QFrags<G>::load(qs, lane, ql);
    QFrags<G> qf;
    qf.build(ql, lane);
    int zsrc[kGroups];  // lanes holding the (scale, zero) pairs of this lane's token, groups 0..3
#pragma unroll
    for (int g = 0; g < kGroups; ++g) zsrc[g] = (col | (g << 4)) << 2;
    MfmaSoftmax<NT> st;
    st.init();
    auto refine = [&](int blk, RefineTile& x) {
      const int tok0 = blk * 64 + 16 * wave;
      const int n_rows = min(16, L - tok0);
      if (n_rows <= 0) return;  // this wave's tile lies past the sequence end
      // the estimate as the scan computes it (transposed MFMA: lane = token
      // col, head row ks), moved to the refine's C layout through the wave's
      // own LDS tile (written and read by the same wave: no barrier)
      {
        const uint4 z4 = make_uint4((uint32_t)__builtin_amdgcn_ds_bpermute(zsrc[0], (int)x.zw),
                                    (uint32_t)__builtin_amdgcn_ds_bpermute(zsrc[1], (int)x.zw),
                                    (uint32_t)__builtin_amdgcn_ds_bpermute(zsrc[2], (int)x.zw),
                                    (uint32_t)__builtin_amdgcn_ds_bpermute(zsrc[3], (int)x.zw));
        float et[NT];
        qf.estimate_t(x.cw, z4, et);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          if (4 * nt + ks < G) estl[wave][4 * nt + ks][col] = et[nt];
      }
      float xs[NT][4];
      qf.residual(x.R, x.S8, xs);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int hh = min(4 * nt + hc, G - 1);
        const float4 e4 = *reinterpret_cast<const float4*>(&estl[wave][hh][4 * ks]);
        xs[nt][0] += e4.x;
        xs[nt][1] += e4.y;
        xs[nt][2] += e4.z;
        xs[nt][3] += e4.w;
      }
      if (n_rows < 16) {  // rows past the end: -inf scores, zero values (their bytes may be anything)
        const int r0 = 4 * ks;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int i = 0; i < 4; ++i) xs[nt][i] = r0 + i < n_rows ? xs[nt][i] : -INFINITY;
        const uint32_t m01 = (r0 < n_rows ? 0xffffu : 0u) | (r0 + 1 < n_rows ? 0xffff0000u : 0u);
        const uint32_t m23 = (r0 + 2 < n_rows ? 0xffffu : 0u) | (r0 + 3 < n_rows ? 0xffff0000u : 0u);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          x.V[q].x &= m01;
          x.V[q].y &= m23;
          x.V[q].z &= m01;
          x.V[q].w &= m23;
        }
      }
      if (p.dbg_tmask) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const int h = 4 * nt + hc;
          if (gc == 0 && h < G)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (4 * ks + i < n_rows) p.dbg_tmask[((size_t)b * p.Hq + hkv * G + h) * p.L_cap + tok0 + 4 * ks + i] = 1;
        }
      }
      h4 va[8];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        va[2 * q] = __builtin_bit_cast(h4, make_uint2(x.V[q].x, x.V[q].y));
        va[2 * q + 1] = __builtin_bit_cast(h4, make_uint2(x.V[q].z, x.V[q].w));
      }
      st.step(xs, c2, slack, va);
    };
    // the next kept block is loaded while the current one is computed
    for (int k = 0; k < nk; k += 2) {
      const int by = k + 1 < nk ? it.next() : bx;
      load_block(by, Y);
      refine(bx, X);
      if (k + 1 >= nk) break;
      const int bn = k + 2 < nk ? it.next() : by;
      load_block(bn, X);
      refine(by, Y);
      bx = bn;
    }
    st.template store<G>(cl, wave, lane, p.sm_scale);
    __syncthreads();
    // the unit's partial per query head of the group: slot ug
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
      const size_t slot = (size_t)ug * G + h;
      p.part_o[slot * kHeadDim + ch] = lsum > 0.f ? o : 0.f;
      if (ch == 0) p.part_ml[slot] = make_float2(M, lsum);
    }
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
template <int G>
static void launch_split_g(const DecodeParams& p, hipStream_t s, int which) {
  if (which & 1) {
    const size_t tmax_bytes = p.dbg_bmax ? (size_t)kScanChunk * 4 * kWaves * G * sizeof(float) : 0;
    hipLaunchKernelGGL(scan_kernel<G>, dim3(p.nword_cap, p.Hkv, p.B), dim3(256), tmax_bytes, s, p);
  }
  if (which & 2) {
    const size_t nheads = (size_t)p.B * p.Hkv;
    const size_t lds = (nheads * p.nword_cap + 2 * nheads + 1) * sizeof(uint32_t);
    hipLaunchKernelGGL(refine_kernel<G>, dim3(p.refine_groups + (unsigned)nheads), dim3(256), lds, s, p);
  }
}

hipError_t launch_split(const DecodeParams& p, hipStream_t s, int which) {
  switch (p.Hq / p.Hkv) {
    case 1: launch_split_g<1>(p, s, which); break;
    case 2: launch_split_g<2>(p, s, which); break;
    case 3: launch_split_g<3>(p, s, which); break;
    case 4: launch_split_g<4>(p, s, which); break;
    case 5: launch_split_g<5>(p, s, which); break;
    case 6: launch_split_g<6>(p, s, which); break;
    case 7: launch_split_g<7>(p, s, which); break;
    case 8: launch_split_g<8>(p, s, which); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace ffd
