// Device-side building blocks shared by the decode kernels (fused attend,
// split scan / refine, pseudo-max, dense baseline): MFMA operand builders for
// the 2-bit thumbnail and the int8 residual, per-lane tile offsets, support
// (pseudo-max) tiles, online-softmax states and the end-of-chunk combine.
#pragma once

#include "ffd_device.h"
#include "ffd_launch.h"

namespace ffd {

constexpr int kWaves = 4;
constexpr int kArtProbe = 8;  // run-time termination probe: first 8 output channels of the group's first head
// s_waitcnt immediate (gfx9 encoding): vmcnt 0, expcnt and lgkmcnt not waited on
constexpr int kWaitVmcnt0 = 0x0F70;

__device__ inline int clamp_len(const DecodeParams& p, int b) {
  const int L = p.seq_lens[b];
  return L < 1 ? 1 : (L > p.L_cap ? p.L_cap : L);
}
// The same for a work-group-uniform b, read through the scalar cache (the
// lengths are never written by a launch that reads them), so that the load
// does not queue behind the vector loads issued with it.
__device__ inline int clamp_len_uniform(const DecodeParams& p, int b) {
  const int L = ((const __attribute__((address_space(4))) int*)p.seq_lens)[b];
  return L < 1 ? 1 : (L > p.L_cap ? p.L_cap : L);
}

// quad (4 adjacent lanes) sum, result in every lane of the quad
__device__ inline float quad_sum(float v) {
  v += dpp<kQuadXor1>(v);
  v += dpp<kQuadXor2>(v);
  return v;
}

// ballot over a tile's lanes -> bit hc set when some lane of head column hc
// (lanes with (lane & 15) >> 2 == hc, any row group) voted
__device__ inline uint32_t head_bits(uint64_t bal) {
  uint32_t x = (uint32_t)bal | (uint32_t)(bal >> 32);
  x = (x | (x >> 16)) & 0xffffu;
  x |= x >> 1;
  x |= x >> 2;
  return (x & 1u) | ((x >> 3) & 2u) | ((x >> 6) & 4u) | ((x >> 9) & 8u);
}

// 2-bit code word -> MFMA A fragment of 8 fp16 values 4 + c (channels j = 0..7):
// the code lands in mantissa bits 8-9 of an fp16 with exponent 2 (ulp 1/4)
constexpr uint32_t kCodeMask = 0x03000300u, kOneHalf2 = 0x44004400u;
// (`mask` = kCodeMask in an SGPR, `one` = kOneHalf2 in a VGPR)
__device__ inline h8 unpack_even(uint32_t w, uint32_t mask, uint32_t one) {
  uint4 d;
  d.x = and_or(w, mask, one);
  d.y = and_or(w >> 2, mask, one);
  d.z = and_or(w >> 4, mask, one);
  d.w = and_or(w >> 6, mask, one);
  return __builtin_bit_cast(h8, d);
}
__device__ inline h8 unpack_odd(uint32_t w, uint32_t mask, uint32_t one) {
  uint4 d;
  d.x = and_or(w << 8, mask, one);
  d.y = and_or(w << 6, mask, one);
  d.z = and_or(w << 4, mask, one);
  d.w = and_or(w << 2, mask, one);
  return __builtin_bit_cast(h8, d);
}
// 8 int8 residuals -> MFMA A fragment of fp16 values 1152 + e (exact): after
// the XOR each byte is e + 128, and one byte permute places two of them as the
// low mantissa bytes of fp16 values with high byte 0x64 (1024 + byte)
constexpr uint32_t kResHigh = 0x64646464u;
__device__ inline h8 unpack_res(uint2 r) {
  const uint32_t x = r.x ^ 0x80808080u, y = r.y ^ 0x80808080u;
  uint4 d;
  d.x = __builtin_amdgcn_perm(kResHigh, x, 0x04010400u);
  d.y = __builtin_amdgcn_perm(kResHigh, x, 0x04030402u);
  d.z = __builtin_amdgcn_perm(kResHigh, y, 0x04010400u);
  d.w = __builtin_amdgcn_perm(kResHigh, y, 0x04030402u);
  return __builtin_bit_cast(h8, d);
}

// ---------------------------------------------------------------------------
// q operands of the tile MFMAs.  Lane roles: col = lane & 15 (C column,
// head hc = col >> 2 of the 4-head column tile, group gc = col & 3),
// ks = lane >> 4 (A/B k-slice, C row group).
// ---------------------------------------------------------------------------
template <int G>
struct QFrags {
  static constexpr int NT = (G + 3) / 4;  // 16-column tiles (4 heads x 4 groups each)
  h8 B[NT][kGroups];
  float c_est[NT], c_res[NT], qq[NT];  // accumulator starts; qq = sum_g(q) of the lane's column
  // transposed scan (estimate_t): Q of head 4*nt + ks for the four groups and
  // the accumulator start -4*Q of the lane's four C rows
  float Qt[NT][kGroups];
  f4 cinit_t[NT];
  uint32_t code_mask, code_one;        // kCodeMask (SGPR), kOneHalf2 (VGPR)

  // q of the group's G heads ([G][128] fp16 at `qh`) is read once per
  // work-group, one dword per thread, into `lds` ([G*64] dwords): every wave
  // reading its own copy would send four times the requests to the few L2
  // lines that all work-groups of a head share.  stage_load issues the
  // global loads, stage_store writes them to LDS once they have landed.
  static constexpr int kQPer = (G * 64 + 255) / 256;
  struct Stage {
    uint32_t w[kQPer];
  };
  __device__ static void stage_load(const uint16_t* qh, int tid, Stage& st) {
#pragma unroll
    for (int k = 0; k < kQPer; ++k) {
      const int i = tid + 256 * k;
      st.w[k] = i < G * 64 ? reinterpret_cast<const uint32_t*>(qh)[i] : 0u;
    }
  }
  __device__ static void stage_store(const Stage& st, int tid, uint32_t* lds) {
#pragma unroll
    for (int k = 0; k < kQPer; ++k)
      if (tid + 256 * k < G * 64) lds[tid + 256 * k] = st.w[k];
  }
  // The lane's share of q (after a barrier): channels 32*gc + 8*ks .. +7 of
  // head 4*nt + hc, the only nonzero part of its B fragments (zero for the
  // padding heads of the last column tile)
  struct Load {
    uint4 v[NT];
  };
  __device__ static void load(const uint32_t* lds, int lane, Load& ql) {
    const int col = lane & 15, hc = col >> 2, gc = col & 3, ks = lane >> 4;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int h = 4 * nt + hc;
      ql.v[nt] = make_uint4(0, 0, 0, 0);
      if (h < G) ql.v[nt] = *reinterpret_cast<const uint4*>(lds + h * 64 + 16 * gc + 4 * ks);
    }
  }
  // B fragments and per-(head, group) sums Q of q (sum over the four k-slice
  // lanes of the column), once the loads have landed
  __device__ void build(const Load& ql, int lane) {
    const int gc = lane & 3;
    code_one = opaque_vgpr(kOneHalf2);
    code_mask = __builtin_amdgcn_readfirstlane(opaque_vgpr(kCodeMask));
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const uint4 z = make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int g = 0; g < kGroups; ++g) B[nt][g] = __builtin_bit_cast(h8, g == gc ? ql.v[nt] : z);
      const uint32_t w[4] = {ql.v[nt].x, ql.v[nt].y, ql.v[nt].z, ql.v[nt].w};
      float part = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) part += lo_h(w[i]) + hi_h(w[i]);
      const float Q = rows_sum(part);
      c_est[nt] = -4.f * Q;
      c_res[nt] = -1152.f * Q;
      qq[nt] = Q;
      // Q of (head 4*nt + ks, group g) sits in the lanes of column 4*ks + g
      const int ks = lane >> 4;
#pragma unroll
      for (int g = 0; g < kGroups; ++g) Qt[nt][g] = __shfl(Q, 4 * ks + g, 64);
      cinit_t[nt] = f4{-4.f * Qt[nt][0], -4.f * Qt[nt][1], -4.f * Qt[nt][2], -4.f * Qt[nt][3]};
    }
  }

  // Transposed estimate of the scan: the same registers with the operands
  // swapped, so the C rows are (head, group) = (4*nt + ks, g) and the columns
  // are the 16 tokens of the tile; the lane (token col, head row ks) then holds
  // all four group terms of its (token, head) and sums them without lane
  // exchanges.  zs = (scale, zero) of the lane's token for groups 0..3.
  __device__ void estimate_t(uint2 cw, uint4 zs, float (&e)[NT]) const {
    const h8 a0 = unpack_even(cw.x, code_mask, code_one), a1 = unpack_odd(cw.x, code_mask, code_one);
    const h8 a2 = unpack_even(cw.y, code_mask, code_one), a3 = unpack_odd(cw.y, code_mask, code_one);
    const uint32_t z[4] = {zs.x, zs.y, zs.z, zs.w};
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      // MFMA g adds to the rows of group g only (exact zeros elsewhere), so the
      // four run on their own accumulators, back to back, and row g is taken
      // from the g-th: the same bits as one accumulator chained through all four
      const f4 c0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(B[nt][0], a0, cinit_t[nt], 0, 0, 0);
      const f4 c1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(B[nt][1], a1, cinit_t[nt], 0, 0, 0);
      const f4 c2 = __builtin_amdgcn_mfma_f32_16x16x32_f16(B[nt][2], a2, cinit_t[nt], 0, 0, 0);
      const f4 c3 = __builtin_amdgcn_mfma_f32_16x16x32_f16(B[nt][3], a3, cinit_t[nt], 0, 0, 0);
      const f4 c = {c0[0], c1[1], c2[2], c3[3]};
      // zero-point terms first (they do not wait for the MFMA), then the
      // scale terms
      float acc = 0.f;
#pragma unroll
      for (int g = 0; g < kGroups; ++g) acc = fmaf(hi_h(z[g]), Qt[nt][g], acc);
#pragma unroll
      for (int g = 0; g < kGroups; ++g) acc = fmaf(lo_h(z[g]), c[g], acc);
      e[nt] = acc;
    }
  }

  // estimated dot products q . (zero + c*scale) of the lane's 4 C rows; cw =
  // codes words (groups 0,1 | 2,3) of the lane's A row, zw = (scale, zero) of
  // the lane's 4 C rows for group gc
  __device__ void estimate(uint2 cw, uint4 zw, float (&e)[NT][4]) const {
    const h8 a0 = unpack_even(cw.x, code_mask, code_one), a1 = unpack_odd(cw.x, code_mask, code_one);
    const h8 a2 = unpack_even(cw.y, code_mask, code_one), a3 = unpack_odd(cw.y, code_mask, code_one);
    const uint32_t zs[4] = {zw.x, zw.y, zw.z, zw.w};
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      f4 c = {c_est[nt], c_est[nt], c_est[nt], c_est[nt]};
      c = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, B[nt][0], c, 0, 0, 0);
      c = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, B[nt][1], c, 0, 0, 0);
      c = __builtin_amdgcn_mfma_f32_16x16x32_f16(a2, B[nt][2], c, 0, 0, 0);
      c = __builtin_amdgcn_mfma_f32_16x16x32_f16(a3, B[nt][3], c, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) e[nt][i] = quad_sum(fmaf(lo_h(zs[i]), c[i], fmaf(hi_h(zs[i]), qq[nt], 0.f)));
    }
  }

  // residual dot products sum_g rscale_g * (q_g . e_g) of the lane's 4 C rows;
  // R[g] = residual bytes of the lane's A row for group g, S8 = rscale of the
  // lane's 4 C rows for group gc
  __device__ void residual(const uint2 (&R)[kGroups], uint2 S8, float (&r)[NT][4]) const {
    const h8 a0 = unpack_res(R[0]), a1 = unpack_res(R[1]), a2 = unpack_res(R[2]), a3 = unpack_res(R[3]);
    const uint32_t s8[4] = {S8.x, S8.x >> 16, S8.y, S8.y >> 16};
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      f4 c = {c_res[nt], c_res[nt], c_res[nt], c_res[nt]};
      c = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, B[nt][0], c, 0, 0, 0);
      c = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, B[nt][1], c, 0, 0, 0);
      c = __builtin_amdgcn_mfma_f32_16x16x32_f16(a2, B[nt][2], c, 0, 0, 0);
      c = __builtin_amdgcn_mfma_f32_16x16x32_f16(a3, B[nt][3], c, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) r[nt][i] = quad_sum(fmaf(lo_h(s8[i]), c[i], 0.f));
    }
  }
};

// per-lane byte offsets of one tile's packed data inside a block
struct TileOffsets {
  int codes, sz, szt, res, rsc;
  __device__ TileOffsets(int wave, int lane) {
    const int col = lane & 15, gc = col & 3, ks = lane >> 4;
    szt = sz_off(16 * wave + col, ks);                                      // token 16w+col, group ks
    codes = codes_word_off(16 * wave + col, ks, 0);                         // A row token 16w+col, slice ks
    sz = sz_off(16 * wave + 4 * ks, gc);                                    // C rows 16w+4ks.., group gc
    res = (((ks >> 1) * 64) + 16 * wave + col) * 16 + 8 * (ks & 1);         // + group * 2048
    rsc = rsc_off(16 * wave + 4 * ks, gc);                                  // C rows 16w+4ks.., group gc
  }
};

__device__ inline void load_residual(const int8_t* rb, const uint8_t* sb, const TileOffsets& to,
                                     uint2 (&R)[kGroups], uint2& S8) {
#pragma unroll
  for (int g = 0; g < kGroups; ++g) R[g] = *reinterpret_cast<const uint2*>(rb + to.res + g * 2048);
  S8 = *reinterpret_cast<const uint2*>(sb + to.rsc);
}

// ---------------------------------------------------------------------------
// Stage 1: pseudo-max over support tokens [0, min(S,L)) U [max(0,L-W), L),
// exact scores with K-hat.  The support parts of a head are the blocks that
// can hold support tokens: the sink blocks first, then the local-window blocks
// not already covered.  Wave w of a work-group takes its 16-token tile of a
// part; the part's maximum per query head goes to the attend kernel either
// through a separate launch (pseudomax_kernel) or through 64-bit words written
// by the leading work-groups of the attend launch itself.
// ---------------------------------------------------------------------------
struct SupportTile {
  uint2 cw;
  uint4 zw;
  uint2 R[kGroups], S8;
  int blk;    // block index (0 when the part is past the sequence)
  bool live;  // the part is a block of the sequence
};

// issue the loads of the wave's tile of support part `part` (head = b*Hkv + kv head)
__device__ inline void support_tile_load(const DecodeParams& p, int part, size_t head, int L, int wave, int lane,
                                         SupportTile& st) {
  const int nblk = (L + 63) >> 6;
  const int s_end = min(p.sink, L);
  const int l_beg = p.local > 0 ? max(0, L - p.local) : L;
  const int n_sink_blk = (s_end + 63) >> 6;
  const int first_local = max(l_beg >> 6, n_sink_blk);
  const int blk = part < n_sink_blk ? part : first_local + (part - n_sink_blk);
  st.live = blk < nblk && (part < n_sink_blk || l_beg < L);
  st.blk = st.live ? blk : 0;
  const size_t bi = head * p.nblk_cap + st.blk;
  const TileOffsets to(wave, lane);
  st.cw = *reinterpret_cast<const uint2*>(p.codes + bi * kCodesBytes + to.codes);
  st.zw = *reinterpret_cast<const uint4*>(p.sz + bi * kSzBytes + to.sz);
  load_residual(p.res + bi * kResBytes, p.rsc + bi * kRscBytes, to, st.R, st.S8);
}

// largest exact score (softmax logit) over the support tokens of the tile, per
// lane for head 4*nt + hc (reduced over the tile's rows; -inf without support)
template <int G>
__device__ void support_tile_max(const DecodeParams& p, const QFrags<G>& qf, const SupportTile& st, int L,
                                 int wave, int lane, float (&mx)[QFrags<G>::NT]) {
  constexpr int NT = QFrags<G>::NT;
  const int s_end = min(p.sink, L);
  const int l_beg = p.local > 0 ? max(0, L - p.local) : L;
  float e[NT][4], r[NT][4];
  qf.estimate(st.cw, st.zw, e);
  qf.residual(st.R, st.S8, r);
  const int ks = lane >> 4;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = st.blk * 64 + 16 * wave + 4 * ks + i;
      const bool sup = st.live && t < L && (t < s_end || t >= l_beg);
      m = fmaxf(m, sup ? (e[nt][i] + r[nt][i]) * p.sm_scale : -INFINITY);
    }
    mx[nt] = rows_max(m);
  }
}

// the work-group's maximum per query head h < G (valid in threads tid < G)
// from the per-lane tile maxima; `red` is [kWaves][G] in LDS (a caller that
// reuses it needs a barrier before the next call)
template <int G>
__device__ float support_wg_max(const float (&mx)[QFrags<G>::NT], float (&red)[kWaves][G], int tid) {
  constexpr int NT = QFrags<G>::NT;
  const int wave = tid >> 6, lane = tid & 63;
  const int col = lane & 15, hc = col >> 2, gc = col & 3, ks = lane >> 4;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int h = 4 * nt + hc;
    if (ks == 0 && gc == 0 && h < G) red[wave][h] = mx[nt];
  }
  __syncthreads();
  float m = -INFINITY;
  if (tid < G) m = fmaxf(fmaxf(red[0][tid], red[1][tid]), fmaxf(red[2][tid], red[3][tid]));
  return m;
}

// Separate launch: grid (npart, Hkv, B), work-group `part` writes its part's
// maximum per query head (-inf for parts without a block); the attend kernel
// takes the maximum over parts.

// ---------------------------------------------------------------------------
// Per-wave online-softmax state.  Scores arrive in MFMA C layout: lane
// (ks = lane>>4, column) holds rows 4ks..4ks+3 of a 16-token tile for the head
// of its column.  NS score sets per lane (FFD: one per 16-column tile).
// ---------------------------------------------------------------------------
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
  __device__ float fold(int n, const float (&s)[4], float* pw_rows /* [16][pg] */, int pg, int head,
                        bool writer, int ks) {
    const float tm = rows_max(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])));
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
    ps = rows_sum(ps);
    l[n] = l[n] * alpha + ps;
    m[n] = mn;
    return alpha;
  }
  // acc = acc * alpha_h + sum_rows p[row][h] * V[row]
  template <int PG>
  __device__ void pv(const float (&alpha)[G], const uint4 (&Vr)[4], const float* pw_rows, int lane,
                     int n_rows_valid) {
    bool rescale = false;  // alpha is wave-uniform: skip the rescale when no head's max moved
#pragma unroll
    for (int h = 0; h < G; ++h) rescale = rescale || (alpha[h] != 1.f);
    if (rescale) {
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int k = 0; k < 8; ++k) acc[h][k] *= alpha[h];
    }
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

// Combine the 4 waves' states (stored in `cl`) into the chunk partial
// (o[128], m, l) of every query head of the group.
// Every LDS word is read up front and the waves' terms are selected, not
// branched on, so the reads go out together (a chain of dependent reads under
// per-wave branches cost about a microsecond per work-group).
template <int G>
__device__ void combine_chunk(const DecodeParams& p, const CombineLds<G>& cl, int tid, int b, int hkv, int chunk) {
  const int qh0 = hkv * G;
  // all LDS reads first (they go out together), then the arithmetic
  constexpr int kIt = (G * kHeadDim + 255) / 256;
  float lwk[kIt][kWaves], mwk[kIt][kWaves], owk[kIt][kWaves];
#pragma unroll
  for (int k = 0; k < kIt; ++k) {
    const int i = min(tid + 256 * k, G * kHeadDim - 1);
    const int h = i >> 7, ch = i & 127;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      lwk[k][w] = cl.l[w][h];
      mwk[k][w] = cl.m[w][h];
      owk[k][w] = cl.o[w][h][ch];
    }
  }
#pragma unroll
  for (int k = 0; k < kIt; ++k) {
    const int i = tid + 256 * k;
    if (i >= G * kHeadDim) break;
    const int h = i >> 7, ch = i & 127;
    const float(&lw)[kWaves] = lwk[k];
    const float(&mw)[kWaves] = mwk[k];
    const float(&ow)[kWaves] = owk[k];
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = lw[w] > 0.f ? fmaxf(M, mw[w]) : M;
    float lsum = 0.f, o = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      // a wave with l = 0 never weighted a token: its o is +0 and it adds +0,
      // which leaves the sums unchanged (they are never -0)
      const bool live = lw[w] > 0.f;
      const float f = live ? exp2f((mw[w] - M) * kLog2e) : 0.f;
      lsum = fmaf(lw[w], f, lsum);
      o = fmaf(ow[w], f, o);
    }
    const size_t row = ((size_t)b * p.Hq + qh0 + h) * p.nchunk + chunk;
    if (lsum > 0.f) p.part_o[row * kHeadDim + ch] = o;
    if (ch == 0) p.part_ml[row] = make_float2(M, lsum);
  }
}

// Dense kernel's end of chunk: reduce acc over the 4 row phases (lanes 0..15
// then hold 8 channels each), store the wave states, combine.  `head_m`/`head_l`
// are the lane's state for head `lane_head[n]`, stored when `state_writer[n]`.
template <int G, int NS>
__device__ void finish_chunk(const DecodeParams& p, CombineLds<G>& cl, float (&acc)[G][8], int wave, int lane,
                             int tid, int b, int hkv, int chunk, const float (&head_m)[NS],
                             const float (&head_l)[NS], const int (&lane_head)[NS], const bool (&state_writer)[NS]) {
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      acc[h][k] = rows_sum(acc[h][k]);
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
  combine_chunk<G>(p, cl, tid, b, hkv, chunk);
}

// ---------------------------------------------------------------------------
// Refinement state of one wave, P.V on MFMA 16x16x16 f16 as O^T = V^T P^T:
//   A = V^T: lane (m = lane&15, ks = lane>>4) holds channel 8m + jm of tile
//       tokens 4ks..4ks+3 for MFMA jm = 0..7 (8 contiguous bytes of the
//       token-quad tiled V);
//   B = P^T: tile tokens 4ks..4ks+3 of column col = lane&15, i.e. exactly the
//       lane's own softmax weights in the score MFMA's C layout;
//   C: lane holds O[channel 32ks + 8i + jm][col] for i = 0..3.
// The four group columns 4h..4h+3 of a head carry identical copies.  P is
// split into fp16 hi + lo parts (two MFMAs each), so the product keeps about
// 21 bits of the fp32 weights.
// ---------------------------------------------------------------------------
typedef _Float16 h4 __attribute__((ext_vector_type(4)));

template <int NT>
struct MfmaSoftmax {
  float m[NT], l[NT];  // running max and sum of the lane column's head
  // P.V accumulators.  One column tile (G <= 4): column 4h + g carries head h
  // (four identical copies).  Two tiles (G > 4): one dense tile whose column c
  // is head c, so each head is accumulated once (half the MFMAs and
  // registers); its column equals the first copy of the one-tile layout bit
  // for bit, since an MFMA computes every output column independently.
  f4 o[1][8];
  __device__ void init() {
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      m[n] = -INFINITY;
      l[n] = 0.f;
    }
#pragma unroll
    for (int jm = 0; jm < 8; ++jm) o[0][jm] = f4{0.f, 0.f, 0.f, 0.f};
  }
  // fold one tile.  x = raw dot products q.k of the lane's 4 rows per column
  // tile (rows past the sequence end -inf), c2 = sm_scale * log2(e), va = V^T
  // fragments (rows past the end zeroed).  The reference max m moves only when
  // a tile's max exceeds it by more than `slack` (8 / c2: weights stay below
  // 2^8), so most tiles skip the rescale of the accumulators.
  __device__ void step(const float (&x)[NT][4], float c2, float slack, const h4 (&va)[8]) {
    float alpha[NT];
    h4 bhi[NT], blo[NT];
    bool moved = false;
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const float tm = rows_max(fmaxf(fmaxf(x[n][0], x[n][1]), fmaxf(x[n][2], x[n][3])));
      const bool mv = tm > m[n] + slack;
      const float mn = mv ? tm : m[n];
      alpha[n] = mv ? __builtin_amdgcn_exp2f((m[n] - mn) * c2) : 1.f;
      moved = moved || mv;
      const float off = mn == -INFINITY ? 0.f : -mn * c2;
      float pr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) pr[i] = __builtin_amdgcn_exp2f(fmaf(x[n][i], c2, off));
      l[n] = fmaf(l[n], alpha[n], rows_sum((pr[0] + pr[1]) + (pr[2] + pr[3])));
      m[n] = mn;
      const h2 h01 = __builtin_bit_cast(h2, __builtin_amdgcn_cvt_pkrtz(pr[0], pr[1]));
      const h2 h23 = __builtin_bit_cast(h2, __builtin_amdgcn_cvt_pkrtz(pr[2], pr[3]));
      const h2 l01 = __builtin_bit_cast(
          h2, __builtin_amdgcn_cvt_pkrtz(fmaf(-(float)h01.x, 1.f, pr[0]), fmaf(-(float)h01.y, 1.f, pr[1])));
      const h2 l23 = __builtin_bit_cast(
          h2, __builtin_amdgcn_cvt_pkrtz(fmaf(-(float)h23.x, 1.f, pr[2]), fmaf(-(float)h23.y, 1.f, pr[3])));
      bhi[n] = h4{h01.x, h01.y, h23.x, h23.y};
      blo[n] = h4{l01.x, l01.y, l23.x, l23.y};
    }
    h4 ph, pl;  // the B operand (weights) of the accumulator tile
    float al;   // the rescale of the lane's accumulator column
    if constexpr (NT == 1) {
      ph = bhi[0];
      pl = blo[0];
      al = alpha[0];
    } else {
      // lane (column c, k-slice ks) takes head c's weights from lane
      // (4 * (c mod 4), ks) of column tile c / 4; columns of no tile are zero
      const int lane = __lane_id();
      const int src = (((lane & 48) | ((lane & 3) << 2))) << 2, tile = (lane & 15) >> 2;
      auto pick = [&](const h4 (&t)[NT], int k) {
        const int v0 = __builtin_amdgcn_ds_bpermute(src, __builtin_bit_cast(int2, t[0])[k]);
        const int v1 = __builtin_amdgcn_ds_bpermute(src, __builtin_bit_cast(int2, t[1])[k]);
        return tile == 0 ? v0 : (tile == 1 ? v1 : 0);
      };
      ph = __builtin_bit_cast(h4, make_int2(pick(bhi, 0), pick(bhi, 1)));
      pl = __builtin_bit_cast(h4, make_int2(pick(blo, 0), pick(blo, 1)));
      const float a0 = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src, __builtin_bit_cast(int, alpha[0])));
      const float a1 = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src, __builtin_bit_cast(int, alpha[1])));
      al = tile == 0 ? a0 : (tile == 1 ? a1 : 1.f);
    }
    if (__builtin_amdgcn_ballot_w64(moved) != 0) {
#pragma unroll
      for (int jm = 0; jm < 8; ++jm) o[0][jm] *= al;
    }
#pragma unroll
    for (int jm = 0; jm < 8; ++jm) {
      o[0][jm] = __builtin_amdgcn_mfma_f32_16x16x16f16(va[jm], ph, o[0][jm], 0, 0, 0);
      o[0][jm] = __builtin_amdgcn_mfma_f32_16x16x16f16(va[jm], pl, o[0][jm], 0, 0, 0);
    }
  }
  // store the wave's state for the combine (m converted to a softmax logit):
  // lanes of group column 0 of each live head write its 128 channels (32 per
  // row group ks) and m, l
  template <int G>
  __device__ void store(CombineLds<G>& cl, int wave, int lane, float sm_scale) const {
    const int col = lane & 15, hc = col >> 2, gc = col & 3, ks = lane >> 4;
    // accumulator column col holds head hc (one tile, copy gc == 0) or head col
    const int h_o = NT == 1 ? hc : col;
    if ((NT == 1 ? gc == 0 : true) && h_o < G) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float* dst = &cl.o[wave][h_o][32 * ks + 8 * i];
        *reinterpret_cast<float4*>(dst) = make_float4(o[0][0][i], o[0][1][i], o[0][2][i], o[0][3][i]);
        *reinterpret_cast<float4*>(dst + 4) = make_float4(o[0][4][i], o[0][5][i], o[0][6][i], o[0][7][i]);
      }
    }
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const int h = 4 * n + hc;
      if (gc == 0 && h < G && ks == 0) {
        cl.m[wave][h] = m[n] * sm_scale;
        cl.l[wave][h] = l[n];
      }
    }
  }
};


struct RefineRegs {
  uint2 R[kGroups];
  uint2 S8;
  uint4 V[4];
};

}  // namespace ffd
