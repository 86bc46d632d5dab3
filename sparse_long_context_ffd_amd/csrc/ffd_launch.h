// Kernel parameter block and host-side launchers (internal to libffd).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ffd {

// what each query head attends inside the kept blocks
constexpr int kSelectUnion = 0;      // every valid token
constexpr int kSelectHeadBlock = 1;  // forced blocks and blocks reaching the head's own threshold
constexpr int kSelectHeadToken = 2;  // support tokens and tokens reaching the head's own threshold

// in-grid pseudo-max: the workspace's sync words are trusted once the merge
// has written this value; polls of a part's word before a chunk computes the
// pseudo-max itself (each poll sleeps ~512 clocks plus a memory round trip)
constexpr unsigned long long kPmMagic = 0x4646442d706d6178ull;
constexpr int kPmSpin = 4096;

// Field order: the scalars and the pointers every attend work-group reads come
// first, so that they share the first 64-byte lines of the kernel-argument
// segment that a work-group's first scalar loads bring in (a field on a later
// line costs one more scalar-cache round trip, on the critical path of a
// short step); rarely used pointers and host-only fields come last.
struct DecodeParams {
  int B, Hq, Hkv, L_cap, nblk_cap, nchunk, cb, npart, sink, local;
  float delta, sm_scale;
  int stages;              // bit 0: pseudo-max, bit 1: scan + refine, bit 2: merge (split path:
                           // bit 3 the scan kernel alone, bit 4 the refine kernel alone)
  int select;              // kSelectUnion / kSelectHeadBlock / kSelectHeadToken
  int art_patience;        // run-time termination: stable steps before a chunk stops (0 = off)
  float art_tau, art_phi;  // ... thresholds on the probe's norm change and 1 - cosine
  int pm_in_grid;          // 1: pseudo-max work-groups lead the attend grid (no separate launch)
  int pm_local;            // 1: every chunk computes the pseudo-max itself (tests the fallback)
  // split path (long caches): scan kernel -> keep bitmap words, refine kernel
  // over the compacted kept blocks -> per-unit partials [slot][G] (o, m, l)
  int split;               // 1: scan + refine kernels instead of the fused attend kernel
  int nword_cap;           // ceil(nblk_cap / 32)
  int refine_groups;       // refine work-groups
  unsigned long long pm_magic;  // kPmMagic keyed to the word layout (written by the merge, checked by chunks)
  const uint16_t* q;       // [B][Hq][128] fp16
  const uint8_t* codes;    // packed cache fields (layouts in include/ffd.h)
  const uint8_t* sz;
  const int8_t* res;
  const uint8_t* rsc;
  const uint16_t* v;       // fp16 V [B][Hkv][L_cap][128]: token-quad tiled (FFD), natural (dense)
  const int32_t* seq_lens; // [B]
  // Pseudo-max inside the attend launch: the first npart work-groups of each
  // (batch, KV head) row publish their part's maxima as 64-bit words
  // (epoch + 1) << 32 | fp32 bits; the merge advances the epoch once per step.
  unsigned long long* pm_words;  // [B][npart][Hq]
  unsigned long long* pm_sync;   // [0] kPmMagic once initialised, [1] epoch (low 32 bits)
  float* part_o;           // [B][Hq][nchunk][128]
  float2* part_ml;         // [B][Hq][nchunk] (m, l)
  uint16_t* out;           // [B][Hq][128] fp16
  const uint16_t* k;       // dense baseline: fp16 K [B][Hkv][L_cap][128]
  float* pmax;             // [B][npart][Hq] partial pseudo-maxima (separate pseudo-max launch)
  uint32_t* kmask;         // [B * Hkv][nword_cap] keep bitmap words (bit j: block 32 * word + j)
  int* unit_start;         // [B * Hkv + 1] first refine unit of each (sequence, KV head)
  float* dbg_mt;           // optional [B][Hq]
  float* dbg_bmax;         // optional [B][Hq][nblk_cap]
  uint8_t* dbg_keep;       // optional [B][Hkv][nblk_cap]
  uint8_t* dbg_tmask;      // optional [B][Hq][L_cap]: token attended by the head (kept blocks only)
  hipEvent_t ev_start;     // optional, recorded around the attend kernel (host only)
  hipEvent_t ev_stop;
};

hipError_t launch_pack(const void* k, int B, int Hkv, int L_cap, int t_begin, int t_end, void* codes,
                       void* sz, void* res, void* rsc, hipStream_t stream);
hipError_t launch_pack_v(const void* v, int B, int Hkv, int L_cap, int t_begin, int t_end, void* vt,
                         hipStream_t stream);
hipError_t launch_append(const void* k_new, const void* v_new, const int32_t* pos, int B, int Hkv, int L_cap,
                         void* codes, void* sz, void* res, void* rsc, void* vt, hipStream_t stream);
hipError_t launch_ffd_decode(const DecodeParams& p, hipStream_t s);
// split path: which = 1 scan, 2 refine, 3 both
hipError_t launch_split(const DecodeParams& p, hipStream_t s, int which);
hipError_t launch_dense_decode(const DecodeParams& p, hipStream_t s);
// streaming-read probe over kStreamReadGroups work-groups; sink holds one
// 32-bit XOR per work-group
constexpr int kStreamReadGroups = 2048;
hipError_t launch_stream_read(const void* src, size_t bytes, void* sink, hipStream_t s);

}  // namespace ffd
