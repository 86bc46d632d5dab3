// FFD decode attention, one step: pseudo-max, a fused kernel that scans the 2-bit
// thumbnail and refines the kept blocks, and a log-sum-exp merge; plus the dense
// flash-decode baseline built from the same pieces.
//
// Page: "Faster Than Flash" (gist.science summary of arXiv 2609.00097).
//   Method 2 (Top-delta): keep when s >= m~ - delta, m~ from sink + local tokens.
//   Method 3 stage 1, pseudo-max estimation               -> pm_group (leading
//                                                             work-groups of the
//                                                             attend grid), or
//                                                             pseudomax_kernel
//   Method 3 stage 2, stream the 2-bit keys, provisional
//            scores, filter blocks against the threshold   -> attend_kernel phase A
//   Method 3 stage 3, residuals + values of the selected
//            blocks, exact attention (reusing the stage-2
//            scores kept on chip)                          -> attend_kernel phase B
//   log-sum-exp merge of the per-chunk partials            -> merge64_kernel,
//                                                             merge_kernel
// Template parameters of attend_kernel: SEL chooses what each query head
// attends inside the kept blocks (the GQA union, its own kept blocks, or its
// own tokens by the per-token criterion of Method 2), ART the run-time
// termination of each chunk's refine stream (the ART page, "Attention Run-time
// Termination", Method 2.2-2.4).  DBG compiles in the optional diagnostic
// outputs (block maxima, keep flags, token masks, pseudo-maxima); the
// in-grid union kernel is also built without them for calls that request
// none, so that the common step carries none of their code.
//
// Scores are computed per 16-token tile with MFMA 16x16x32 f16, tokens on the
// rows.  The B operand holds q with column n = 4*h + g carrying head h
// restricted to 32-channel group g (zero elsewhere), so one accumulator
// collects per-(head, group) dot products whose fp32 epilogue applies that
// token-group's scale; a quad sum over g finishes the dot product.  Scores
// are kept as raw dot products x = q . k (s = sm_scale * x):
//   thumbnail: A = 4 + c (exact fp16), accumulator starts at -4*sum_g(q):
//              C = q_g . c_g;      est = scale*C + zero*sum_g(q)
//   residual:  A = 1152 + e (exact fp16), accumulator starts at -1152*sum_g(q):
//              C = q_g . e_g;      exact = est + rscale*C
//
// Work decomposition of attend/dense: one work-group (4 wave64) per chunk of
// `cb` 64-token blocks of one (sequence, KV head) -- contiguous blocks for
// dense, interleaved over the sequence (stride = number of chunks) for attend.
// Wave w owns token tile [16w, 16w+16) of every block of the chunk, so the
// four waves do identical work and each keeps its own online-softmax state;
// the states are combined in LDS into one partial per chunk, which
// merge_kernel combines.
#include "ffd_tiles.h"

namespace ffd {

template <int G>
__global__ __launch_bounds__(256) void pseudomax_kernel(DecodeParams p) {
  constexpr int NT = QFrags<G>::NT;
  __shared__ float red[kWaves][G];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int part = blockIdx.x, hkv = blockIdx.y, b = blockIdx.z;
  const size_t head = (size_t)b * p.Hkv + hkv;
  const int qh0 = hkv * G;
  __shared__ uint32_t qs[G * 64];
  typename QFrags<G>::Stage qst;
  QFrags<G>::stage_load(p.q + ((size_t)b * p.Hq + qh0) * kHeadDim, tid, qst);
  const int L = clamp_len_uniform(p, b);
  SupportTile st;
  support_tile_load(p, part, head, L, wave, lane, st);
  QFrags<G>::stage_store(qst, tid, qs);
  lds_barrier();  // q staged in LDS (the support tile loads stay in flight)
  typename QFrags<G>::Load ql;
  QFrags<G>::load(qs, lane, ql);
  QFrags<G> qf;
  qf.build(ql, lane);
  float mx[NT];
  support_tile_max<G>(p, qf, st, L, wave, lane, mx);
  const float m = support_wg_max<G>(mx, red, tid);
  if (tid < G) p.pmax[((size_t)b * p.npart + part) * p.Hq + qh0 + tid] = m;
}

// ---------------------------------------------------------------------------
// Stages 2 + 3 for one chunk of blocks.
//   prologue: first thumbnail batch, the lane's q share and the parts of its
//            head's pseudo-max are loaded at once; no barrier before the scan
//   phase A: every wave estimates its tile of every block of the chunk (loads
//            double-buffered in batches of 4 blocks); estimates stay in LDS
//            and the wave records whether some head of the tile reaches its
//            threshold m~ - delta
//   decide:  a block is kept if it holds a support token or some wave's tile
//            reached a threshold; every wave derives the same kept mask
//   phase B: every wave refines its tile of every kept block (residual, rscale
//            and V of the next kept block loaded while the current one is
//            computed), online softmax, P.V on MFMA
// Dynamic LDS: per-block estimates [cb][4 waves][G][16], the combine area, and
// (only when the block-max diagnostic is requested) per-(block, wave, row
// group) maxima [cb][16][G].
// ---------------------------------------------------------------------------
// One leading work-group of the attend grid: support part `part` of (b, hkv),
// published as the 64-bit word (epoch + 1) << 32 | fp32 bits per query head
// with agent-scope stores (the chunk work-groups read them with agent-scope
// loads, so no cache maintenance is needed).  `red` is LDS scratch.
template <int G>
__device__ void pm_group(const DecodeParams& p, int part, int hkv, int b, uint32_t* qs, float (&red)[kWaves][G]) {
  constexpr int NT = QFrags<G>::NT;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const size_t head = (size_t)b * p.Hkv + hkv;
  const int qh0 = hkv * G;
  typename QFrags<G>::Stage qst;
  QFrags<G>::stage_load(p.q + ((size_t)b * p.Hq + qh0) * kHeadDim, tid, qst);
  const unsigned long long ep = __hip_atomic_load(p.pm_sync + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const int L = clamp_len_uniform(p, b);
  SupportTile st;
  support_tile_load(p, part, head, L, wave, lane, st);
  QFrags<G>::stage_store(qst, tid, qs);
  lds_barrier();  // q staged in LDS (the support tile loads stay in flight)
  typename QFrags<G>::Load ql;
  QFrags<G>::load(qs, lane, ql);
  QFrags<G> qf;
  qf.build(ql, lane);
  float mx[NT];
  support_tile_max<G>(p, qf, st, L, wave, lane, mx);
  const float m = support_wg_max<G>(mx, red, tid);
  if (tid < G)
    __hip_atomic_store(p.pm_words + ((size_t)b * p.npart + part) * p.Hq + qh0 + tid,
                       ((unsigned long long)((uint32_t)ep + 1u) << 32) | __builtin_bit_cast(uint32_t, m),
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int G>
struct AttendCfg {
  static constexpr int NT = QFrags<G>::NT;
  static constexpr int CBMAX = (G <= 4) ? 32 : 24;
  // (room for whole batches of 4 blocks: a last batch past the chunk's end is computed and dropped)
  static constexpr size_t est_bytes(int cb) { return (size_t)((cb + 3) & ~3) * kWaves * G * 16 * sizeof(float); }
  static constexpr size_t tmax_bytes(int cb) { return (size_t)cb * 4 * kWaves * G * sizeof(float); }
  // the block-max diagnostic's area is allocated only when it is requested
  static constexpr size_t lds_bytes(int cb, bool bmax) {
    return est_bytes(cb) + sizeof(CombineLds<G>) + (bmax ? tmax_bytes(cb) : 0);
  }
};


// Register budget: 3 waves per SIMD for G <= 4 (<= 168 VGPRs, no spills); the
// G > 4 variant keeps twice the accumulators and runs at 2.
// PMG: the pseudo-max work-groups lead the grid; the chunks then scan before
// they know their thresholds and take the block decisions from the stored
// estimates after the scan (so that the wait for the published words overlaps
// the scan).  Without PMG the thresholds come from the separate launch's
// partial maxima before the scan, which takes the decisions as it goes.
template <int G, int SEL, bool ART, bool PMG, bool DBG>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(G <= 4 ? 3 : 2))) void attend_kernel(
    DecodeParams p) {
  if constexpr (!DBG) {  // (launched only when every diagnostic pointer is null)
    p.dbg_mt = nullptr;
    p.dbg_bmax = nullptr;
    p.dbg_keep = nullptr;
    p.dbg_tmask = nullptr;
  }
  constexpr int NT = AttendCfg<G>::NT, CBMAX = AttendCfg<G>::CBMAX;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int col = lane & 15, hc = col >> 2, gc = col & 3, ks = lane >> 4;
  __shared__ uint32_t qs[G * 64];
  __shared__ float pm_s[256];
  __shared__ float pm_red[kWaves][G];
  // Without PMG the grid is (nchunk, Hkv, B).  With it the grid is 1-D: the
  // npart * Hkv * B pseudo-max work-groups of every row first (dispatched
  // ahead of every chunk, so that they finish while the first chunks scan),
  // then the chunks in the same order as the 3-D grid.
  int chunk, hkv, b;
  if constexpr (PMG) {
    const int n_rows = p.Hkv * p.B;
    int w = blockIdx.x;
    if (w < p.npart * n_rows) {
      const int row = w / p.npart;
      pm_group<G>(p, w - row * p.npart, row % p.Hkv, row / p.Hkv, qs, pm_red);
      return;
    }
    w -= p.npart * n_rows;
    const int row = w / p.nchunk;
    chunk = w - row * p.nchunk;
    hkv = row % p.Hkv;
    b = row / p.Hkv;
  } else {
    chunk = blockIdx.x;
    hkv = blockIdx.y;
    b = blockIdx.z;
  }
  // The chunk's blocks are interleaved over the sequence: block j of chunk c
  // is c + j * nchunk, so the always-kept sink and local-window blocks (and
  // any cluster of kept blocks) spread over many work-groups.  Under run-time
  // termination a chunk is one stream of the call: the contiguous blocks
  // c * cb .. c * cb + cb - 1 (cb = the call's stream length).
  const int nck = p.nchunk;
  auto blk_of = [&](int j) { return ART ? chunk * p.cb + j : chunk + j * nck; };
  auto blocks_below = [&](int n) {  // blocks of the chunk below block index n
    return ART ? max(0, min(p.cb, n - chunk * p.cb)) : min(p.cb, (n - chunk + nck - 1) / nck);
  };
  const int nbl_cap = blocks_below(p.nblk_cap);
  const size_t head = (size_t)b * p.Hkv + hkv;
  const int qh0 = hkv * G;
  const int L = clamp_len_uniform(p, b);
  const TileOffsets to(wave, lane);
  // per-head buffer descriptors; lane offsets in VGPRs, block offsets in SGPRs
  const size_t hb = head * p.nblk_cap;  // first block of the head
  const uint32_t nbc = (uint32_t)p.nblk_cap;
  const __amdgpu_buffer_rsrc_t r_codes = make_rsrc(p.codes + hb * kCodesBytes, nbc * kCodesBytes);
  const __amdgpu_buffer_rsrc_t r_sz = make_rsrc(p.sz + hb * kSzBytes, nbc * kSzBytes);

  // ---- prologue: all loads issued together (q first: it is stored to LDS
  // and turned into MFMA fragments while the thumbnail batch is still in
  // flight) ----
  typename QFrags<G>::Stage qst;
  QFrags<G>::stage_load(p.q + ((size_t)b * p.Hq + qh0) * kHeadDim, tid, qst);
  // Thumbnail batches: per lane 8 bytes of codes (the token's row of the A
  // fragments) and one (scale, zero) pair -- token 16w + col, group ks; the
  // four pairs of a token reach its lanes through ds_bpermute in the scan.
  // Each load instruction of a wave covers whole cache lines of data read once:
  // non-temporal hint.
  uint2 cwA[4], cwB[4];
  uint32_t zwA[4], zwB[4];
  auto load_batch = [&](int j0, uint2 (&cw)[4], uint32_t (&zw)[4]) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int jj = min(j0 + v, nbl_cap - 1);
      cw[v] = buf_load_b64<kNonTemporal>(r_codes, (uint32_t)to.codes, (uint32_t)blk_of(jj) * kCodesBytes);
      zw[v] = buf_load_b32<kNonTemporal>(r_sz, (uint32_t)to.szt, (uint32_t)blk_of(jj) * kSzBytes);
    }
  };
  load_batch(0, cwA, zwA);
  // partial pseudo-maxima (part pp, head h) at thread pp*G + h, one load per
  // thread (maximum over several parts when there are more than 256/G)
  const int n_pm = p.npart * G;
  float pm_t = -INFINITY;
  unsigned long long pw = 0, pm_magic = 0, pm_epoch = 0;  // in-grid word of (part tid/G, head tid%G), sync
  // the word polled with agent-scope atomic loads after the scan, and read in
  // the prologue and during the scan as a device-coherent plain load (threads
  // past n_pm read the last one)
  unsigned long long* const pm_word = p.pm_words + ((size_t)b * p.npart + tid / G) * p.Hq + qh0 + tid % G;
  const __amdgpu_buffer_rsrc_t r_pw = make_rsrc(p.pm_words + (size_t)b * p.npart * p.Hq, (uint32_t)(p.npart * p.Hq * 8));
  const uint32_t pw_off = (uint32_t)(((min(tid, n_pm - 1) / G) * p.Hq + qh0 + min(tid, n_pm - 1) % G) * 8);
  if constexpr (PMG) {  // (the host keeps npart * G <= 256 here: one word per thread)
    // device-coherent plain loads: as atomic loads they would hold the q
    // barrier below until they land
    {  // every thread loads (threads past n_pm repeat the last word), so that the load counters are exact
      const uint2 w = buf_load_b64<kDeviceCoherent>(r_pw, pw_off, 0u);
      pw = (unsigned long long)w.y << 32 | w.x;
    }
    const uint4 sy = buf_load_b128<kDeviceCoherent>(make_rsrc(p.pm_sync, 16), 0u, 0u);  // magic, epoch
    pm_magic = (unsigned long long)sy.y << 32 | sy.x;
    pm_epoch = (unsigned long long)sy.w << 32 | sy.z;
  } else {
    const float* pm = p.pmax + (size_t)b * p.npart * p.Hq + qh0;
    if (tid < n_pm) pm_t = pm[(size_t)(tid / G) * p.Hq + tid % G];
    for (int i = tid + (256 / G) * G; i < n_pm; i += (256 / G) * G) pm_t = fmaxf(pm_t, pm[(size_t)(i / G) * p.Hq + i % G]);
  }

  QFrags<G>::stage_store(qst, tid, qs);
  // Blocks the wave's tile reached a threshold in: under the per-head block
  // selection the heads that did (bit h of kflag[wave][j]); otherwise bit j of
  // the wave's reach mask wk, published in wkf[wave] for the decision.
  __shared__ int kflag[kWaves][CBMAX];
  __shared__ uint64_t wkf[kWaves];
  uint64_t wk = 0;  // (wave-uniform)
  __shared__ __align__(16) int vote[2][kWaves];  // per-wave votes of wg_all (two sets, used in turn)
  __shared__ float art_lds[ART ? 2 : 1][ART ? kWaves * (2 + kArtProbe) : 1];
  extern __shared__ __align__(16) float dyn[];
  const int cb = p.cb;
  float* est = dyn;  // [cb rounded up to whole batches of 4][kWaves][G][16]
  CombineLds<G>& cl = *reinterpret_cast<CombineLds<G>*>(dyn + AttendCfg<G>::est_bytes(cb) / sizeof(float));
  float* tmax = dyn + (AttendCfg<G>::est_bytes(cb) + sizeof(CombineLds<G>)) / sizeof(float);  // [cb][4*kWaves][G]

  const int nblk = (L + 63) >> 6;
  const int nbl = blocks_below(nblk);
  if (nbl <= 0) {  // a chunk past the sequence end: empty partial (weight 0 in the merge)
    if (tid < G) p.part_ml[((size_t)b * p.Hq + qh0 + tid) * p.nchunk + chunk] = make_float2(-INFINITY, 0.f);
    return;
  }
  lds_barrier();  // q staged in LDS (the thumbnail batch stays in flight)
  typename QFrags<G>::Load ql;
  QFrags<G>::load(qs, lane, ql);
  QFrags<G> qf;
  qf.build(ql, lane);
  const bool dbg_bmax = p.dbg_bmax != nullptr;
  // Rows past the sequence end get estimate -inf only where it can matter:
  // with a local window the block holding the last token is always kept (and
  // the refine masks its rows past the end), so its estimates there decide
  // nothing; without one, or for the block-max diagnostic, they are masked.
  const bool tail_mask = p.local == 0 || dbg_bmax;
  // Drain every load issued so far (first batch, q, the pseudo-max parts) so
  // that the pipelined scan below starts from an exact count of loads in flight.
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  // In-grid pseudo-max: every word must carry this step's tag (epoch + 1).
  // When every word was already there in the prologue (work-groups that start
  // after the pseudo-max work-groups have published), the thresholds are
  // known before the scan and the blocks are decided as they are scanned.
  // Otherwise (usually at the start of the grid) the words still missing are
  // loaded again during the scan and checked after it, where the thresholds
  // are first needed; words still missing then are polled a bounded number
  // of times, after which (or before the merge has initialised the sync
  // words, or under pm_local) the work-group computes the pseudo-max itself.
  // All conditions are work-group uniform.
  const uint32_t pm_want = (uint32_t)pm_epoch + 1u;
  const bool pm_trusted = PMG && pm_magic == p.pm_magic && !p.pm_local;
  bool pm_mine = tid >= n_pm || (uint32_t)(pw >> 32) == pm_want;
  bool pm_early = false;
  if constexpr (PMG) {
    // the thread's part goes to LDS with its vote (a part whose word is stale
    // is never read)
    pm_s[tid] = tid < n_pm ? __builtin_bit_cast(float, (uint32_t)pw) : -INFINITY;
    pm_early = wg_all(pm_trusted && pm_mine, vote[0], wave, lane);
  } else {
    pm_s[tid] = pm_t;
    __syncthreads();  // the partial maxima
  }
  // Refine loads of a block: residual, its scales, V.
  // lane's V^T span: channels 8*col..8*col+7 of token quad 4*wave+ks (64 bytes).
  // The residual and its scales load with the non-temporal hint (a wave's
  // instruction covers whole lines); V keeps the default policy, since a
  // lane's span is split over four loads and every line is read by four
  // instructions in turn (with the hint, 25% slower).
  const uint32_t v_lane = (uint32_t)(((4 * wave + ks) * kHeadDim + 8 * col) * 4 * sizeof(uint16_t));
  const __amdgpu_buffer_rsrc_t r_res = make_rsrc(p.res + hb * kResBytes, nbc * kResBytes);
  const __amdgpu_buffer_rsrc_t r_rsc = make_rsrc(p.rsc + hb * kRscBytes, nbc * kRscBytes);
  const __amdgpu_buffer_rsrc_t r_v = make_rsrc(p.v + head * p.L_cap * kHeadDim, nbc * kVBytes);
  // j < 0: the same instructions through descriptors of size 0, which return
  // zeros without a memory access (a refine loop's load past the last block:
  // the load counters stay exact, and nothing is left to wait for)
  const __amdgpu_buffer_rsrc_t r_none = make_rsrc(p.res, 0);
  auto load_block = [&](int j, RefineRegs& x) {
    const bool live = j >= 0;
    const uint32_t blk = live ? (uint32_t)blk_of(j) : 0u;
    const __amdgpu_buffer_rsrc_t rr = live ? r_res : r_none, rs = live ? r_rsc : r_none, rv = live ? r_v : r_none;
#pragma unroll
    for (int g = 0; g < kGroups; ++g) x.R[g] = buf_load_b64<kNonTemporal>(rr, (uint32_t)to.res + g * 2048, blk * kResBytes);
    x.S8 = buf_load_b64<kNonTemporal>(rs, (uint32_t)to.rsc, blk * kRscBytes);
#pragma unroll
    for (int q = 0; q < 4; ++q) x.V[q] = buf_load_b128(rv, v_lane + 16 * q, blk * kVBytes);
  };
  // Blocks always kept (sink and local window) are known before any threshold:
  // the refine takes them first (the union selection without run-time
  // termination, whose streams keep their order), and the first one's loads go
  // out here, before the scan, so that its latency overlaps the scan and the
  // decisions.
  const int sink_end = p.sink > 0 ? ((min(p.sink, L) + 63) >> 6) : 0;
  const int local_beg = p.local > 0 ? (max(0, L - p.local) >> 6) : nblk;
  const uint64_t fmask = __builtin_amdgcn_ballot_w64(lane < nbl && (blk_of(lane) < sink_end || blk_of(lane) >= local_beg));
  constexpr bool kForcedFirst = !ART;
  RefineRegs X, Y;
  if (kForcedFirst && fmask) load_block(__builtin_ctzll(fmask), X);
  int zsrc[kGroups];  // lanes holding the (scale, zero) pairs of this lane's token, groups 0..3
#pragma unroll
  for (int g = 0; g < kGroups; ++g) zsrc[g] = (col | (g << 4)) << 2;
  // pseudo-max of head h: maximum over the parts of the per-thread values
  int n_pt = min(n_pm, (256 / G) * G) / G;  // parts held in pm_s
  float thr[NT];    // threshold of the lane column's head, in dot-product units
  float thr_t[NT];  // threshold of the lane's head in the transposed scan (row group ks)
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) thr[nt] = thr_t[nt] = INFINITY;  // (until known)
  auto pseudo_max = [&](int h) {
    float m = -INFINITY;
    for (int pp = 0; pp < n_pt; ++pp) m = fmaxf(m, pm_s[pp * G + h]);
    return m;
  };
  auto compute_thresholds = [&]() {
    // Pseudo-maxima of the lane's two heads (column head 4*nt + hc for the
    // refine, row-group head 4*nt + ks for the transposed scan), parts read 8 at
    // a time so that the LDS reads go out together; part indices are clamped to
    // the last part (a repeated part leaves a maximum unchanged) and padding
    // heads h >= G read head G-1 (their thresholds are +inf).
    float pm_c[NT], pm_k[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) pm_c[nt] = pm_k[nt] = -INFINITY;
    for (int pp0 = 0; pp0 < n_pt; pp0 += 8) {
      float vc[NT][8], vk[NT][8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int r = min(pp0 + i, n_pt - 1) * G;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          vc[nt][i] = pm_s[r + min(4 * nt + hc, G - 1)];
          vk[nt][i] = pm_s[r + min(4 * nt + ks, G - 1)];
        }
      }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          pm_c[nt] = fmaxf(pm_c[nt], vc[nt][i]);
          pm_k[nt] = fmaxf(pm_k[nt], vk[nt][i]);
        }
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      thr[nt] = 4 * nt + hc < G ? (pm_c[nt] - p.delta) / p.sm_scale : INFINITY;
      thr_t[nt] = 4 * nt + ks < G ? (pm_k[nt] - p.delta) / p.sm_scale : INFINITY;
    }
    if (chunk == 0 && p.dbg_mt && tid < G) p.dbg_mt[(size_t)b * p.Hq + qh0 + tid] = pseudo_max(tid);
  };
  if (!PMG || pm_early) compute_thresholds();
  // A word still missing is loaded again inside the last scan batch: late
  // enough that the pseudo-max work-groups have usually published it by then,
  // early enough that it is back when the scan ends.
  const bool pm_reload = pm_trusted && !pm_mine;

  // ---- phase A: estimate tile `wave` of every block of the chunk ----
  // estimates are kept as dot products (logit / sm_scale); rows past the
  // sequence end (only in the last block) are set to -inf under tail_mask
  // A batch is straight-line code: blocks past the chunk's end (only in its
  // last batch) are estimated from the clamped loads and dropped (the
  // estimate array has room for them, and their reach bits are masked), so
  // that the compiler interleaves the four blocks' LDS, MFMA and FMA
  // latencies instead of running them one after another.
  const bool decide_now = !PMG || pm_early;  // (work-group uniform)
  const int row_lim = tail_mask ? L : INT_MAX;  // rows at or past it get estimate -inf
  auto scan_batch = [&](int j0, const uint2 (&cw)[4], const uint32_t (&zw)[4], bool last) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      if (PMG && last && v == 1) {  // every thread loads; the threads with a stale word take it
        const uint2 w2 = buf_load_b64<kDeviceCoherent>(r_pw, pw_off, 0u);
        pw = pm_reload ? ((unsigned long long)w2.y << 32 | w2.x) : pw;
      }
      const int j = j0 + v;
      const bool live = j < nbl;
      const uint4 z4 = make_uint4((uint32_t)__builtin_amdgcn_ds_bpermute(zsrc[0], (int)zw[v]),
                                  (uint32_t)__builtin_amdgcn_ds_bpermute(zsrc[1], (int)zw[v]),
                                  (uint32_t)__builtin_amdgcn_ds_bpermute(zsrc[2], (int)zw[v]),
                                  (uint32_t)__builtin_amdgcn_ds_bpermute(zsrc[3], (int)zw[v]));
      float e[NT];
      qf.estimate_t(cw[v], z4, e);
      const bool valid = blk_of(j) * 64 + 16 * wave + col < row_lim;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) e[nt] = valid ? e[nt] : -INFINITY;
      // per-head block selection: bit h = head h reaches its threshold in
      // this tile (lanes 16*ks .. 16*ks + 15 hold head 4*nt + ks); otherwise
      // bit j of the wave's reach mask: some head of the group reaches it
      // (without PMG; with it after the scan)
      uint32_t hreach = 0;
      bool reach = false;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        if constexpr (SEL == kSelectHeadBlock) {
          const uint64_t bal = __builtin_amdgcn_ballot_w64(e[nt] >= thr_t[nt]);
          hreach |= (((bal & 0xffffull) != 0) | (((bal >> 16) & 0xffffull) != 0) << 1 |
                     (((bal >> 32) & 0xffffull) != 0) << 2 | (((bal >> 48) & 0xffffull) != 0) << 3)
                    << (4 * nt);
        } else {
          reach |= e[nt] >= thr_t[nt];
        }
        const int h = 4 * nt + ks;
        if (h < G) est[((j * kWaves + wave) * G + h) * 16 + col] = e[nt];
        if (dbg_bmax && live) {
          // block-max diagnostic: maximum over each 4-token quad of lanes
          float qm = fmaxf(e[nt], dpp<kQuadXor1>(e[nt]));
          qm = fmaxf(qm, dpp<kQuadXor2>(qm));
          if (h < G && (col & 3) == 0) tmax[(j * 4 * kWaves + 4 * wave + (col >> 2)) * G + h] = qm;
        }
      }
      // (bitwise, not short-circuit, so that no branch splits the batch)
      if constexpr (SEL == kSelectHeadBlock) {
        if (decide_now & live & (lane == 0)) kflag[wave][j] = (int)hreach;
      } else {
        const bool any = __builtin_amdgcn_ballot_w64(reach) != 0;
        wk |= (decide_now & live & any) ? 1ull << j : 0ull;
      }
    }
  };
  // Two batches alternate: one is in flight while the other is scanned.  Inside
  // the loop every load is unconditional, so the compiler's load counters wait
  // for the batch being scanned only, not for the one in flight; the last one
  // or two batches are peeled off, so no load is issued past the chunk (a
  // load nobody reads would still be waited for when its registers are
  // reused).  Batch i is in A for even i, in B for odd i.
  const int nbat = (nbl + 3) >> 2;
  int i0 = 0;
  for (; i0 + 2 < nbat; i0 += 2) {
    load_batch(4 * (i0 + 1), cwB, zwB);
    scan_batch(4 * i0, cwA, zwA, false);
    load_batch(4 * (i0 + 2), cwA, zwA);
    scan_batch(4 * (i0 + 1), cwB, zwB, false);
  }
  if (i0 + 1 < nbat) {
    load_batch(4 * (i0 + 1), cwB, zwB);
    scan_batch(4 * i0, cwA, zwA, false);
    scan_batch(4 * (i0 + 1), cwB, zwB, true);
  } else {
    scan_batch(4 * i0, cwA, zwA, true);
  }

  // ---- PMG: pseudo-maxima, thresholds and the reach flags after the scan ----
  if (PMG && !pm_early) {
    bool pm_fb = false;
    {
      pm_mine = tid >= n_pm || (uint32_t)(pw >> 32) == pm_want;
      // The thread's part goes to LDS before the vote, so that one barrier
      // publishes both; a value whose word is stale is never read (the
      // work-group then takes the fallback below, which rewrites what it reads).
      pm_s[tid] = tid < n_pm ? __builtin_bit_cast(float, (uint32_t)pw) : -INFINITY;
      bool all = wg_all(pm_trusted && pm_mine, vote[1], wave, lane);
      // words still missing: polled, the first time at once
      for (int s = 0; !all && pm_trusted && s < kPmSpin; ++s) {
        if (s > 0) __builtin_amdgcn_s_sleep(8);
        if (!pm_mine) {
          pw = __hip_atomic_load(pm_word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          pm_mine = (uint32_t)(pw >> 32) == pm_want;
        }
        pm_s[tid] = tid < n_pm ? __builtin_bit_cast(float, (uint32_t)pw) : -INFINITY;
        all = wg_all(pm_mine, vote[s & 1], wave, lane);
      }
      pm_fb = !all;
    }
    if (pm_fb) {
      float m = -INFINITY;  // (threads tid < G) head tid
      for (int part = 0; part < p.npart; ++part) {
        SupportTile st;
        support_tile_load(p, part, head, L, wave, lane, st);
        float mx[NT];
        support_tile_max<G>(p, qf, st, L, wave, lane, mx);
        m = fmaxf(m, support_wg_max<G>(mx, pm_red, tid));
        __syncthreads();  // pm_red is written again by the next part
      }
      if (tid < G) pm_s[tid] = m;
      __syncthreads();
      n_pt = 1;
    }
    compute_thresholds();

    // ---- reach flags from the stored estimates, now that the thresholds are
    // known: per head, or one bit per block for the group (lanes 16*ks .. 16*ks + 15
    // hold head 4*nt + ks; each lane reads back the estimates it stored).  The
    // reads go out 8 blocks at a time (indices clamped to the chunk).
    for (int j0 = 0; j0 < nbl; j0 += 8) {
      float e8[8][NT];
#pragma unroll
      for (int v = 0; v < 8; ++v) {
        const int j = min(j0 + v, nbl - 1);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const int h = 4 * nt + ks;
          e8[v][nt] = h < G ? est[((j * kWaves + wave) * G + h) * 16 + col] : -INFINITY;
        }
      }
#pragma unroll
      for (int v = 0; v < 8; ++v) {
        if (j0 + v < nbl) {
          uint32_t hreach = 0;
          bool reach = false;
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            if constexpr (SEL == kSelectHeadBlock) {
              const uint64_t bal = __builtin_amdgcn_ballot_w64(e8[v][nt] >= thr_t[nt]);
              hreach |= (((bal & 0xffffull) != 0) | (((bal >> 16) & 0xffffull) != 0) << 1 |
                         (((bal >> 32) & 0xffffull) != 0) << 2 | (((bal >> 48) & 0xffffull) != 0) << 3)
                        << (4 * nt);
            } else {
              reach = reach || (e8[v][nt] >= thr_t[nt]);
            }
          }
          if constexpr (SEL == kSelectHeadBlock) {
            if (lane == 0) kflag[wave][j0 + v] = (int)hreach;
          } else {
            wk |= __builtin_amdgcn_ballot_w64(reach) != 0 ? 1ull << (j0 + v) : 0ull;
          }
        }
      }
    }
  }
  if constexpr (SEL != kSelectHeadBlock)
    if (lane == 0) wkf[wave] = wk;
  lds_barrier();

  // ---- block decisions (every wave derives the same mask) ----
  // forced blocks: [0, sink_end) and [local_beg, nblk)
  uint64_t kmask;
  {
    bool kp = false;
    if (lane < nbl) {
      const int blk = blk_of(lane);
      // the four waves' flags are read unconditionally (one LDS round trip,
      // not a chain of short-circuit reads)
      int any;
      if constexpr (SEL == kSelectHeadBlock)
        any = kflag[0][lane] | kflag[1][lane] | kflag[2][lane] | kflag[3][lane];
      else
        any = (int)(((wkf[0] | wkf[1]) | (wkf[2] | wkf[3])) >> lane) & 1;
      kp = blk < sink_end || blk >= local_beg || any != 0;
      if (wave == 0) {
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
    }
    kmask = __builtin_amdgcn_ballot_w64(kp);
  }
  if (PMG && kmask == 0) {
    // Nothing kept (so no forced block and no refine load in flight): the
    // chunk's partial is empty; write it as the combine would (weight 0 in
    // the merge, o never read) and free the slot.  Only in the in-grid launch:
    // in the other variants this exit made the run-time termination kernels
    // spill registers.
    if (tid < G) p.part_ml[((size_t)b * p.Hq + qh0 + tid) * p.nchunk + chunk] = make_float2(-INFINITY, 0.f);
    return;
  }

  // ---- phase B: refine tile `wave` of every kept block ----
  MfmaSoftmax<NT> st;
  st.init();
  {
    const float c2 = p.sm_scale * kLog2e, slack = 8.f / c2;
    // support tokens [0, sup_lo) and [sup_hi, L) (always attended per token)
    const int sup_lo = min(p.sink, L), sup_hi = max(0, L - p.local);
    auto refine = [&](int j, RefineRegs& x) {
      const int tok0 = blk_of(j) * 64 + 16 * wave;  // first row of the wave's tile
      const int n_rows = min(16, L - tok0);
      if (n_rows <= 0) return;  // this wave's tile lies past the sequence end
      float xs[NT][4];
      qf.residual(x.R, x.S8, xs);
      // heads that attend this block under the per-head block selection
      uint32_t hb = ~0u;
      if constexpr (SEL == kSelectHeadBlock) {
        const int blk = blk_of(j);
        if (blk >= sink_end && blk < local_beg) hb = kflag[0][j] | kflag[1][j] | kflag[2][j] | kflag[3][j];
      }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int h = 4 * nt + hc;
        const int hh = h < G ? h : 0;
        const float4 e4 = *reinterpret_cast<const float4*>(&est[((j * kWaves + wave) * G + hh) * 16 + 4 * ks]);
        const float ev[4] = {e4.x, e4.y, e4.z, e4.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          bool att = true;
          if constexpr (SEL == kSelectHeadBlock) att = (hb >> hh) & 1u;
          if constexpr (SEL == kSelectHeadToken) {
            const int t = tok0 + 4 * ks + i;
            att = t < sup_lo || t >= sup_hi || ev[i] >= thr[nt];
          }
          xs[nt][i] = att ? xs[nt][i] + ev[i] : -INFINITY;
        }
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
              if (4 * ks + i < n_rows)
                p.dbg_tmask[((size_t)b * p.Hq + qh0 + h) * p.L_cap + tok0 + 4 * ks + i] =
                    xs[nt][i] != -INFINITY ? 1 : 0;
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
    // Run-time termination of the chunk's stream (the ART page, Method 2.2-2.4):
    // after every refined block lane 0 of each wave publishes its running
    // (max, sum, first kArtProbe output channels) of the group's first head;
    // after a barrier every thread combines the four wave states into the
    // chunk's probe x and compares it with the previous one.  All threads
    // compute the same values from the same LDS words, so the decision is
    // uniform.  Slots alternate by step parity so that one barrier per step
    // suffices.
    int art_step_no = 0, art_stable = 0;
    float art_prev[kArtProbe];
    auto art_stop = [&]() -> bool {
      float* slot = art_lds[art_step_no & 1];
      if (lane == 0) {
        slot[wave * (2 + kArtProbe)] = st.m[0];
        slot[wave * (2 + kArtProbe) + 1] = st.l[0];
#pragma unroll
        for (int k = 0; k < kArtProbe; ++k) slot[wave * (2 + kArtProbe) + 2 + k] = st.o[0][k][0];
      }
      __syncthreads();
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < kWaves; ++w)
        if (slot[w * (2 + kArtProbe) + 1] > 0.f) M = fmaxf(M, slot[w * (2 + kArtProbe)]);
      float lt = 0.f, x[kArtProbe];
#pragma unroll
      for (int k = 0; k < kArtProbe; ++k) x[k] = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float* e = slot + w * (2 + kArtProbe);
        if (e[1] > 0.f) {
          const float f = __builtin_amdgcn_exp2f((e[0] - M) * c2);
          lt = fmaf(e[1], f, lt);
#pragma unroll
          for (int k = 0; k < kArtProbe; ++k) x[k] = fmaf(e[2 + k], f, x[k]);
        }
      }
      const float inv = 1.f / lt;
      float n1 = 0.f, n0 = 0.f, dot = 0.f;
#pragma unroll
      for (int k = 0; k < kArtProbe; ++k) {
        x[k] *= inv;
        n1 = fmaf(x[k], x[k], n1);
        n0 = fmaf(art_prev[k], art_prev[k], n0);
        dot = fmaf(x[k], art_prev[k], dot);
      }
      bool stop = false;
      if (art_step_no > 0) {
        n1 = sqrtf(n1);
        n0 = sqrtf(n0);
        const float d_scale = fabsf(n1 - n0);
        const float d_dir = (n1 > 0.f && n0 > 0.f) ? 1.f - dot / (n1 * n0) : 1.f;
        art_stable = (d_scale < p.art_tau && d_dir < p.art_phi) ? art_stable + 1 : 0;
        stop = art_stable >= p.art_patience;
      }
#pragma unroll
      for (int k = 0; k < kArtProbe; ++k) art_prev[k] = x[k];
      ++art_step_no;
      return stop;
    };
    // kept blocks from the (wave-uniform) masks: the forced ones first, then
    // the others, each in increasing order (under run-time termination all in
    // increasing order).  The next block is loaded while the current one is
    // computed, unconditionally as in the scan (past the end of the list
    // through the empty descriptors, so no memory is read and the last
    // block's wait is not held up).
    uint64_t rem_f = kForcedFirst ? (kmask & fmask) : 0ull, rem_o = kForcedFirst ? (kmask & ~fmask) : kmask;
    auto pop = [&]() -> int {
      if (rem_f) {
        const int j = __builtin_ctzll(rem_f);
        rem_f &= rem_f - 1;
        return j;
      }
      if (rem_o) {
        const int j = __builtin_ctzll(rem_o);
        rem_o &= rem_o - 1;
        return j;
      }
      return -1;
    };
    int jx = pop();
    if (jx >= 0) {
      if (!(kForcedFirst && fmask)) load_block(jx, X);  // (else loaded before the scan)
      while (true) {
        const int jy = pop();
        load_block(jy, Y);
        refine(jx, X);
        if constexpr (ART)
          if (art_stop()) break;
        if (jy < 0) break;
        const int jn = pop();
        load_block(jn, X);
        refine(jy, Y);
        if constexpr (ART)
          if (art_stop()) break;
        if (jn < 0) break;
        jx = jn;
      }
    }
  }
  st.template store<G>(cl, wave, lane, p.sm_scale);
  __syncthreads();
  combine_chunk<G>(p, cl, tid, b, hkv, chunk);
}

// ---------------------------------------------------------------------------
// Dense flash-decode over fp16 K/V (speed baseline) with the same chunking,
// softmax, P.V, combine and merge kernel.  QK on MFMA: A = K tile (16 tokens x
// 32 channels per group), B = q with one column per head.
// ---------------------------------------------------------------------------
template <int G>
__global__ __launch_bounds__(256) void dense_kernel(DecodeParams p) {
  constexpr int PG = (G + 3) & ~3;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int chunk = blockIdx.x, hkv = blockIdx.y, b = blockIdx.z;
  const int blk0 = chunk * p.cb;
  const int nbl_cap = min(p.cb, p.nblk_cap - blk0);
  const size_t head = (size_t)b * p.Hkv + hkv;
  const int qh0 = hkv * G;
  const int col = lane & 15, ks = lane >> 4;
  const int co = lane & 15, tp = lane >> 4;
  const int t_a = 16 * wave + col;
  uint4 Kr[kGroups], Vr[4];
  auto load_block = [&](int j) {
    const size_t row = head * p.L_cap + (size_t)(blk0 + min(j, nbl_cap - 1)) * 64;
    const uint16_t* kb = p.k + (row + t_a) * kHeadDim + 8 * ks;
#pragma unroll
    for (int g = 0; g < kGroups; ++g) Kr[g] = *reinterpret_cast<const uint4*>(kb + 32 * g);
    // V rows: each instruction reads 4 whole 256-byte rows (non-temporal hint);
    // a K row's lines are read by two instructions in turn (default policy)
    const uint16_t* vb = p.v + (row + 16 * wave + tp) * kHeadDim + 8 * co;
#pragma unroll
    for (int i = 0; i < 4; ++i) Vr[i] = load_b128_nt(vb + (size_t)(4 * i) * kHeadDim);
  };
  load_block(0);
  // B fragments: column col = head, k-slice ks of each group (zero past G)
  h8 Bd[kGroups];
  {
    const uint16_t* qh = p.q + ((size_t)b * p.Hq + qh0 + (col < G ? col : 0)) * kHeadDim + 8 * ks;
#pragma unroll
    for (int g = 0; g < kGroups; ++g) {
      uint4 f = make_uint4(0, 0, 0, 0);
      if (col < G) f = *reinterpret_cast<const uint4*>(qh + 32 * g);
      Bd[g] = __builtin_bit_cast(h8, f);
    }
  }
  __shared__ float pw[kWaves][16 * PG];
  __shared__ CombineLds<G> cl;
  const int L = clamp_len_uniform(p, b);
  const int nblk = (L + 63) >> 6;
  if (blk0 >= nblk) {  // a chunk past the sequence end: empty partial (weight 0 in the merge)
    if (tid < G) p.part_ml[((size_t)b * p.Hq + qh0 + tid) * p.nchunk + chunk] = make_float2(-INFINITY, 0.f);
    return;
  }
  const int nbl = min(p.cb, nblk - blk0);
  WaveSoftmax<G, 1> st;
  st.init();
  float* pwv = pw[wave];
  for (int j = 0; j < nbl; ++j) {
    const int n_rows = min(16, L - ((blk0 + j) * 64 + 16 * wave));
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
// Grid (Hq, B, 4): work-group = one query head, 32 output channels; thread =
// (chunk phase cp = tid/32, channel).  Partials are read in pieces of 256
// chunks, all loads of a piece issued together, with an online rescale across
// pieces.  Chunks that kept nothing have weight 0 (selected, never
// multiplied, so their unwritten o is never used).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void merge_kernel(DecodeParams p) {
  constexpr int kPiece = 256;
  constexpr int kPer = kPiece / 8;
  __shared__ float wts[kPiece];
  __shared__ float red[8][32];
  __shared__ float wmax[kWaves];
  __shared__ float wsum[kWaves];
  const int h = blockIdx.x, b = blockIdx.y, slice = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int cp = tid >> 5, ch = 32 * slice + (tid & 31);
  // the step's in-grid pseudo-max words are consumed: advance the epoch (the
  // next attend launch sees it) and mark the sync words initialised
  if (p.pm_in_grid && h == 0 && b == 0 && slice == 0 && tid == 0) {
    const unsigned long long e = __hip_atomic_load(p.pm_sync + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(p.pm_sync + 1, (unsigned long long)((uint32_t)e + 1u), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(p.pm_sync, p.pm_magic, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  const size_t row = (size_t)b * p.Hq + h;
  const float2* ml;
  const float* po;
  size_t ml_stride, o_stride;
  int nch;
  if (p.split) {
    // the refine units of the head's (sequence, KV head), slots [s0, s0 + nch)
    const int G = p.Hq / p.Hkv, r = b * p.Hkv + h / G, g = h - (h / G) * G;
    const int s0 = p.unit_start[r];
    nch = p.unit_start[r + 1] - s0;
    ml = p.part_ml + (size_t)s0 * G + g;
    po = p.part_o + ((size_t)s0 * G + g) * kHeadDim + ch;
    ml_stride = G;
    o_stride = (size_t)G * kHeadDim;
  } else {
    // every chunk of the launch: each writes its (m, l), l = 0 when empty
    // (no block of the sequence, or nothing kept), so the partials are read
    // without waiting for the sequence length
    nch = p.nchunk;
    ml = p.part_ml + row * p.nchunk;
    po = p.part_o + row * p.nchunk * kHeadDim + ch;
    ml_stride = 1;
    o_stride = kHeadDim;
  }
  float M = -INFINITY, o = 0.f, ls = 0.f;
  for (int c0 = 0; c0 < nch; c0 += kPiece) {
    const int n = min(kPiece, nch - c0);
    const float2 v = tid < n ? ml[(size_t)(c0 + tid) * ml_stride] : make_float2(-INFINITY, 0.f);
    float x[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int c = cp + 8 * i;
      x[i] = c < n ? po[(size_t)(c0 + c) * o_stride] : 0.f;
    }
    const bool live = v.y > 0.f;
    float mp = wave_max(live ? v.x : -INFINITY);
    if (lane == 0) wmax[wave] = mp;
    __syncthreads();
    mp = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
    const float Mn = fmaxf(M, mp);
    const float w = live ? exp2f((v.x - Mn) * kLog2e) : 0.f;
    wts[tid] = w;
    const float sc = M > -INFINITY ? exp2f((M - Mn) * kLog2e) : 0.f;
    ls = ls * sc + (live ? w * v.y : 0.f);
    o *= sc;
    M = Mn;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const float wi = wts[cp + 8 * i];
      o = wi > 0.f ? fmaf(wi, x[i], o) : o;
    }
    __syncthreads();
  }
  ls = wave_sum(ls);
  red[cp][tid & 31] = o;
  if (lane == 0) wsum[wave] = ls;
  __syncthreads();
  if (tid < 32) {
    float acc = 0.f;
#pragma unroll
    for (int q = 0; q < 8; ++q) acc += red[q][tid];
    const float lsum = (wsum[0] + wsum[1]) + (wsum[2] + wsum[3]);
    p.out[row * kHeadDim + ch] = __builtin_bit_cast(uint16_t, (_Float16)(acc / lsum));
  }
}

// ---------------------------------------------------------------------------
// The same merge for heads with at most 64 chunk partials (fused and dense
// paths with nchunk <= 64): one wave per 32 output channels of a head, no
// barriers, no LDS.  Lane c holds chunk c's (m, l) and computes its weight;
// lane (channel j, half t) accumulates the chunk phases 4t .. 4t+3 (chunk
// phase = c mod 8) of channel j, reading each chunk's weight with a lane read.
// The association is merge_kernel's exactly (each phase in increasing chunk
// order, the eight phases summed in order, the weight sum over the 64 lanes
// by the same reduction), so both kernels give the same bits and the choice
// between them never changes an output.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void merge64_kernel(DecodeParams p) {
  const int lane = threadIdx.x;
  if (p.pm_in_grid && blockIdx.x == 0 && lane == 0) {  // as in merge_kernel
    const unsigned long long e = __hip_atomic_load(p.pm_sync + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(p.pm_sync + 1, (unsigned long long)((uint32_t)e + 1u), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(p.pm_sync, p.pm_magic, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  const size_t row = blockIdx.x >> 2;  // query head row; blockIdx.x & 3 = channel quarter
  const int ch = 32 * (blockIdx.x & 3) + (lane & 31), half = lane >> 5;
  // Every chunk of the launch writes its (m, l), an empty chunk (no block of
  // the sequence, or nothing kept) l = 0, so the partials are read without
  // waiting for the sequence length; partial o of chunk c at byte
  // c * 512 + 4 * channel, read as zero past the last chunk (bounds of the
  // descriptor); a chunk of weight 0 contributes nothing.
  const int nch = p.nchunk;
  const __amdgpu_buffer_rsrc_t r_o = make_rsrc(p.part_o + row * p.nchunk * kHeadDim, (uint32_t)nch * 512u);
  const float2 v = lane < nch ? p.part_ml[row * p.nchunk + lane] : make_float2(-INFINITY, 0.f);
  const uint32_t v_off = (uint32_t)ch * 4u + (uint32_t)half * 4u * 512u;  // + chunk (phase 4 * half)
  float x[4][8];  // phase 4 * half + q, chunk 4 * half + q + 8 * i
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) x[q][i] = __builtin_bit_cast(float, buf_load_b32(r_o, v_off, (uint32_t)(q + 8 * i) * 512u));
  const bool live = v.y > 0.f;
  const float M = wave_max(live ? v.x : -INFINITY);
  const float w = live ? exp2f((v.x - M) * kLog2e) : 0.f;
  const float ls = wave_sum(live ? w * v.y : 0.f);
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float w0 = uniform_lane(w, q + 8 * i), w1 = uniform_lane(w, 4 + q + 8 * i);
      const float wc = half ? w1 : w0;
      acc[q] = wc > 0.f ? fmaf(wc, x[q][i], acc[q]) : acc[q];
    }
  // phases 0..3 (half 0), then 4..7 from the lane 32 places up
  float o = 0.f;
#pragma unroll
  for (int q = 0; q < 4; ++q) o += acc[q];
#pragma unroll
  for (int q = 0; q < 4; ++q) o += __shfl_down(acc[q], 32, 64);
  const float lsum = (ls + 0.f) + (0.f + 0.f);
  if (half == 0) p.out[row * kHeadDim + ch] = __builtin_bit_cast(uint16_t, (_Float16)(o / lsum));
}

static void launch_merge(const DecodeParams& p, hipStream_t s) {
  if (!p.split && p.nchunk <= 64 && 4ll * p.B * p.Hq < (1ll << 31))
    hipLaunchKernelGGL(merge64_kernel, dim3((unsigned)(4ll * p.B * p.Hq)), dim3(64), 0, s, p);
  else
    hipLaunchKernelGGL(merge_kernel, dim3(p.Hq, p.B, 4), dim3(256), 0, s, p);
}

// ---------------------------------------------------------------------------
// host-side launchers
// ---------------------------------------------------------------------------
template <int G, int SEL, bool ART, bool PMG, bool DBG = true>
static void launch_attend(const DecodeParams& p, hipStream_t s) {
  const dim3 grid = PMG ? dim3((unsigned)((p.npart + p.nchunk) * p.Hkv * p.B)) : dim3(p.nchunk, p.Hkv, p.B);
  hipLaunchKernelGGL((attend_kernel<G, SEL, ART, PMG, DBG>), grid, dim3(256), AttendCfg<G>::lds_bytes(p.cb, p.dbg_bmax != nullptr), s,
                     p);
}
template <int G>
static void launch_ffd_g(const DecodeParams& p, hipStream_t s) {
  const int stages = p.stages ? p.stages : 7;
  if ((stages & 1) && !p.pm_in_grid)
    hipLaunchKernelGGL(pseudomax_kernel<G>, dim3(p.npart, p.Hkv, p.B), dim3(256), 0, s, p);
  if (p.split) {
    const int which = ((stages & 2) ? 3 : 0) | ((stages & 8) ? 1 : 0) | ((stages & 16) ? 2 : 0);
    if (which) {
      if (p.ev_start) (void)hipEventRecord(p.ev_start, s);
      (void)launch_split(p, s, which);
      if (p.ev_stop) (void)hipEventRecord(p.ev_stop, s);
    }
  } else if (stages & 2) {
    if (p.ev_start) (void)hipEventRecord(p.ev_start, s);
    const bool dbg = p.dbg_mt || p.dbg_bmax || p.dbg_keep || p.dbg_tmask;
    if (p.pm_in_grid && !dbg)  // (union selection without run-time termination only)
      launch_attend<G, kSelectUnion, false, true, false>(p, s);
    else if (p.pm_in_grid)
      launch_attend<G, kSelectUnion, false, true>(p, s);
    else if (p.art_patience > 0)  // run-time termination (union selection only)
      launch_attend<G, kSelectUnion, true, false>(p, s);
    else if (p.select == kSelectHeadBlock)
      launch_attend<G, kSelectHeadBlock, false, false>(p, s);
    else if (p.select == kSelectHeadToken)
      launch_attend<G, kSelectHeadToken, false, false>(p, s);
    else
      launch_attend<G, kSelectUnion, false, false>(p, s);
    if (p.ev_stop) (void)hipEventRecord(p.ev_stop, s);
  }
  if (stages & 4) launch_merge(p, s);
}
template <int G>
static void launch_dense_g(const DecodeParams& p, hipStream_t s) {
  hipLaunchKernelGGL(dense_kernel<G>, dim3(p.nchunk, p.Hkv, p.B), dim3(256), 0, s, p);
  launch_merge(p, s);
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
