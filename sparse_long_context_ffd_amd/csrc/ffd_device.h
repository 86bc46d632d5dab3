// Device-side helpers shared by the FFD kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ffd {

constexpr int kHeadDim = 128;
constexpr int kBlock = 64;
constexpr int kGroup = 32;
constexpr int kGroups = 4;
constexpr int kMaxG = 8;                // query heads per KV head supported
constexpr int kCodesBytes = 2048;       // per 64-token block and head
constexpr int kSzBytes = 1024;
constexpr int kResBytes = 8192;
constexpr int kRscBytes = 512;
constexpr int kVBytes = 16384;          // fp16 V of one 64-token block, token-quad tiled
constexpr float kLog2e = 1.4426950408889634f;

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// packed-cache layout (byte offsets inside one 64-token block of one head).
// Codes, (scale, zero) and residual scales are tile-major: the 16 tokens
// 16w..16w+15 that wave w handles occupy one contiguous 512-byte (codes),
// 256-byte (scale, zero) and 128-byte (residual scale) run, so a wave's loads
// cover whole cache lines.
// ---------------------------------------------------------------------------
__host__ __device__ inline int codes_word_off(int t, int kq, int p) { return (t * 4 + kq) * 8 + p * 4; }
__host__ __device__ inline int sz_off(int t, int g) {
  return (((t >> 4) * 4 + g) * 4 + ((t >> 2) & 3)) * 16 + (t & 3) * 4;
}
__host__ __device__ inline int res_off(int t, int ch) { return ((ch >> 4) * 64 + t) * 16 + (ch & 15); }
__host__ __device__ inline int rsc_off(int t, int g) { return (((t >> 4) * 4 + g) * 16 + (t & 15)) * 2; }
// bit of channel (32g + 8kq + j) inside its word
__host__ __device__ inline int code_bit(int g, int j) {
  const int d = j >> 1;
  return (g & 1) ? ((j & 1) ? 16 + 2 * d : 2 * d) : ((j & 1) ? 24 + 2 * d : 8 + 2 * d);
}

// ---------------------------------------------------------------------------
// small conversions
// ---------------------------------------------------------------------------
__device__ inline float h2f(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }
__device__ inline float lo_h(uint32_t w) { return h2f((uint16_t)(w & 0xffffu)); }
__device__ inline float hi_h(uint32_t w) { return h2f((uint16_t)(w >> 16)); }

// ---------------------------------------------------------------------------
// cross-lane reductions (wave64)
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ inline float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}
constexpr int kQuadXor1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;
constexpr int kRowMirror = 0x140;

__device__ inline float xor_lane(float v, int mask) { return __shfl_xor(v, mask, 64); }

// Reductions over the four 16-lane rows of a wave (lanes l, l^16, l^32, l^48)
// with the gfx950 row-swap permutes; every lane receives the result.  The swap
// is written as inline asm (with the wait states it needs around it): the
// compiler's builtin form folds the two swapped halves of a float into one.
__device__ inline void swap_rows32(uint32_t& x, uint32_t& y) {  // x.hi32 <-> y.lo32
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(x), "+v"(y));
}
__device__ inline void swap_rows16(uint32_t& x, uint32_t& y) {  // x.odd rows <-> y.even rows
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 1" : "+v"(x), "+v"(y));
}
__device__ inline float rows_max(float v) {
  uint32_t x = __builtin_bit_cast(uint32_t, v), y = x;
  swap_rows32(x, y);
  v = fmaxf(__builtin_bit_cast(float, x), __builtin_bit_cast(float, y));
  x = __builtin_bit_cast(uint32_t, v);
  y = x;
  swap_rows16(x, y);
  return fmaxf(__builtin_bit_cast(float, x), __builtin_bit_cast(float, y));
}
__device__ inline float rows_sum(float v) {
  uint32_t x = __builtin_bit_cast(uint32_t, v), y = x;
  swap_rows32(x, y);
  v = __builtin_bit_cast(float, x) + __builtin_bit_cast(float, y);
  x = __builtin_bit_cast(uint32_t, v);
  y = x;
  swap_rows16(x, y);
  return __builtin_bit_cast(float, x) + __builtin_bit_cast(float, y);
}

// Buffer loads: a wave-uniform descriptor (base, size in bytes) plus a 32-bit
// lane offset (VGPR) and a wave-uniform offset (SGPR).  Streaming loads in this
// form need no per-load 64-bit address registers, so the compiler never has to
// wait for a load in flight just to reuse an address register.  Offsets at or
// past `bytes` read as zero.  (Descriptor word 3 value for gfx9 raw buffers.)
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
//
// CPOL is the load's cache-policy field: 0, or kNonTemporal (the `nt` bit) for
// data read exactly once whose cache lines are each covered by one load
// instruction (a wave's loads of 64 lanes span whole lines).  On MI355X a
// streaming read with the hint runs about 11% faster (7.0 vs 6.3 TB/s over
// 1 GiB).  Lines that several instructions read in turn must keep the default
// policy: with the hint each of them fetches the line again.
constexpr int kNonTemporal = 2;
// kDeviceCoherent (the `sc1` bit) reads at device scope, past stale copies in
// another XCD's L2: the policy an agent-scope atomic load is issued with, as a
// plain load, so that a barrier ordering LDS only need not wait for it.
constexpr int kDeviceCoherent = 16;
// 16-byte global load with the non-temporal hint (same rule as above)
__device__ inline uint4 load_b128_nt(const void* ptr) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_nontemporal_load(static_cast<const u32x4*>(ptr));
  return make_uint4(v.x, v.y, v.z, v.w);
}
template <int CPOL = 0>
__device__ inline uint2 buf_load_b64(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)voff, (int)soff, CPOL);
  return make_uint2(v[0], v[1]);
}
template <int CPOL = 0>
__device__ inline uint32_t buf_load_b32(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, (int)soff, CPOL);
}
template <int CPOL = 0>
__device__ inline uint4 buf_load_b128(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, CPOL);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// A 32-bit constant in a VGPR whose value the compiler cannot see.  With the
// mask in an SGPR and the constant in a VGPR, (x & mask) | bits is selected as
// one v_and_or_b32 (with both as visible literals the compiler emits two
// instructions); keeping the op itself in compiled code, not inline asm, lets
// the compiler account for its wait states before an MFMA reads the result.
__device__ inline uint32_t opaque_vgpr(uint32_t k) {
  uint32_t r;
  asm volatile("v_mov_b32 %0, %1\n\ts_nop 1" : "=v"(r) : "s"(k));  // wait states cover any reader
  return r;
}
__device__ inline uint32_t and_or(uint32_t x, uint32_t mask, uint32_t bits) { return (x & mask) | bits; }

// Work-group barrier that orders LDS accesses only: global loads still in
// flight stay in flight (__syncthreads also waits for every outstanding
// vector memory access of the wave).  For hand-overs through LDS.
__device__ inline void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// True in every thread iff `pred` holds in every thread of a work-group of
// four waves: one vote per wave in `vote` (4 ints in LDS, 16-byte aligned) and
// one barrier.  Consecutive calls must alternate between two vote arrays (a
// wave past the barrier may write its next vote while another still reads).
__device__ inline bool wg_all(bool pred, int* vote, int wave, int lane) {
  const bool w = __builtin_amdgcn_ballot_w64(!pred) == 0;
  if (lane == 0) vote[wave] = w ? 1 : 0;
  lds_barrier();
  const int4 v = *reinterpret_cast<const int4*>(vote);
  return (v.x & v.y & v.z & v.w) != 0;
}

// maximum over all 64 lanes, returned in every lane
__device__ inline float wave_max(float v) {
  v = fmaxf(v, dpp<kQuadXor1>(v));
  v = fmaxf(v, dpp<kQuadXor2>(v));
  v = fmaxf(v, dpp<kRowHalfMirror>(v));
  v = fmaxf(v, dpp<kRowMirror>(v));
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

// sum over all 64 lanes, returned in every lane
__device__ inline float wave_sum(float v) {
  v += dpp<kQuadXor1>(v);
  v += dpp<kQuadXor2>(v);
  v += dpp<kRowHalfMirror>(v);
  v += dpp<kRowMirror>(v);
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
  return (r0 + r1) + (r2 + r3);
}

__device__ inline float uniform_lane(float v, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

}  // namespace ffd
