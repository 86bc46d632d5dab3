// C ABI of libffd: argument validation, work split, workspace carving and
// launches on the caller's stream.  The entry points and their contract are
// declared and documented in include/ffd.h.
#include <math.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

#include <hip/hip_runtime.h>

#include "../../include/ffd.h"
#include "ffd_device.h"
#include "ffd_launch.h"

static_assert(ffd::kSelectUnion == FFD_SELECT_UNION && ffd::kSelectHeadBlock == FFD_SELECT_HEAD_BLOCK &&
                  ffd::kSelectHeadToken == FFD_SELECT_HEAD_TOKEN,
              "selection codes of the ABI and the kernels differ");

namespace {

constexpr size_t kAlign = 256;
// Work-groups per launch the automatic split aims for: about 1.8 rounds of the
// 768 resident ones (256 CUs x 3), so that fewer, longer work-groups amortise
// each one's prologue and first memory round trip (at 256K context, 24 blocks
// per chunk instead of 16: scan alone -9%, the whole kernel -2.5%).
constexpr int kTargetGroups = 1380;
// The dense baseline streams every block with no scan, and its best split is
// about 2048 work-groups (at 256K: 171 us with 16 blocks per chunk, 179 us
// with 24).
constexpr int kDenseTargetGroups = 2048;
constexpr int kSmallGroups = 256;    // ... and at least this many blocks per 4-block group on short caches

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_shape(const ffd_shape_t* s) {
  if (!s) return FFD_ERR_NULL;
  if (s->head_dim != 128 || s->block != 64) return FFD_ERR_SHAPE;
  if (s->batch < 1 || s->num_kv_heads < 1 || s->num_q_heads < 1) return FFD_ERR_SHAPE;
  if (s->num_q_heads % s->num_kv_heads != 0) return FFD_ERR_SHAPE;
  const int G = s->num_q_heads / s->num_kv_heads;
  if (G < 1 || G > ffd::kMaxG) return FFD_ERR_SHAPE;
  if (s->sink < 0 || s->local < 0 || s->chunk_blocks < 0) return FFD_ERR_SHAPE;
  if (s->sink == 0 && s->local == 0) return FFD_ERR_SHAPE;  // the pseudo-max needs a support set
  if (s->max_seq_len < 64 || s->max_seq_len % 64 != 0) return FFD_ERR_SHAPE;
  // the kernels address one head's blocks with 32-bit byte offsets (its
  // values take max_seq_len * 256 bytes)
  if ((long long)s->max_seq_len * ffd::kHeadDim * 2 > 0xFFFFFFFFll) return FFD_ERR_SHAPE;
  // batch and KV heads are launch-grid dimensions (at most 65535 each)
  if (s->batch > 65535 || s->num_kv_heads > 65535) return FFD_ERR_SHAPE;
  return FFD_OK;
}

// Split path (long caches): refine work-groups at most (the workspace holds a
// partial slot per refine unit: at most this many plus one per (sequence, KV
// head)), and bitmap words the refine keeps in LDS at most.
constexpr int kRefineGroupsMax = 2048;
constexpr long long kSplitMaxWords = 8192;
constexpr long long kSplitMaxHeads = 1024;  // (sequence, KV head) pairs: unit starts and counts in LDS

struct Plan {
  int nblk_cap, cb, nchunk, npart, nword_cap;
  size_t sync_off, pmw_off, pmax_off, ml_off, o_off;
  size_t km_off, us_off, sml_off, so_off;  // split path: bitmap words, unit starts, unit partials
  size_t total;
};

// Work split: one work-group per chunk of cb blocks (4 waves, one 16-token tile
// of every block each).  cb is sized for about kTargetGroups work-groups per
// launch and bounded by the LDS the per-block estimates of a chunk need.
// `fixed_cb` > 0 sets the blocks per work-group (run-time termination: the
// call's stream length) in place of the shape's choice.
Plan make_plan(const ffd_shape_t* s, long long target = kTargetGroups, int fixed_cb = 0) {
  Plan p;
  const int G = s->num_q_heads / s->num_kv_heads;
  const int cb_max = G <= 4 ? 32 : 24;
  p.nblk_cap = s->max_seq_len / 64;
  long long cb;
  if (fixed_cb > 0) {
    cb = fixed_cb;
  } else if (s->chunk_blocks > 0) {
    cb = s->chunk_blocks;
  } else {
    // about kTargetGroups work-groups on long caches; short caches take up to
    // 4 blocks per work-group so that one wave of work-groups covers them
    const long long total = (long long)s->batch * s->num_kv_heads * p.nblk_cap;
    cb = (total + target - 1) / target;
    if (cb < 4) {
      const long long small = (total + kSmallGroups - 1) / kSmallGroups;
      cb = small < 4 ? small : 4;
    }
  }
  if (cb > cb_max) cb = cb_max;
  if (cb > p.nblk_cap) cb = p.nblk_cap;
  if (cb < 1) cb = 1;
  p.cb = (int)cb;
  p.nchunk = (p.nblk_cap + p.cb - 1) / p.cb;
  // pseudo-max work-groups: one per block that can hold support tokens (sink
  // blocks, then the blocks spanned by the local window, at most one extra)
  const long long sink_blocks = ((long long)(s->sink < s->max_seq_len ? s->sink : s->max_seq_len) + 63) / 64;
  const long long local_blocks = s->local > 0 ? ((long long)s->local + 63) / 64 + 1 : 0;
  const long long np = sink_blocks + local_blocks;
  p.npart = (int)(np < p.nblk_cap ? np : p.nblk_cap);
  const size_t rows = (size_t)s->batch * s->num_q_heads;
  // the in-grid pseudo-max's sync words sit at the start for every shape, so
  // the epoch they hold carries over when a workspace changes shape
  p.sync_off = 0;
  p.pmw_off = kAlign;
  p.pmax_off = p.pmw_off + round_up((size_t)s->batch * p.npart * s->num_q_heads * sizeof(uint64_t), kAlign);
  p.ml_off = p.pmax_off + round_up((size_t)s->batch * p.npart * s->num_q_heads * sizeof(float), kAlign);
  p.o_off = p.ml_off + round_up(rows * p.nchunk * 2 * sizeof(float), kAlign);
  const size_t fused_end = p.o_off + round_up(rows * p.nchunk * 128 * sizeof(float), kAlign);
  // the split path's arrays reuse the space of the fused path's partials
  const size_t heads = (size_t)s->batch * s->num_kv_heads;
  const size_t slots = ((size_t)kRefineGroupsMax + heads) * (s->num_q_heads / s->num_kv_heads);
  p.nword_cap = (p.nblk_cap + 31) / 32;
  p.km_off = p.ml_off;
  p.us_off = p.km_off + round_up(heads * p.nword_cap * sizeof(uint32_t), kAlign);
  p.sml_off = p.us_off + round_up((heads + 1) * sizeof(int32_t), kAlign);
  p.so_off = p.sml_off + round_up(slots * 2 * sizeof(float), kAlign);
  const size_t split_end = p.so_off + round_up(slots * 128 * sizeof(float), kAlign);
  p.total = fused_end > split_end ? fused_end : split_end;
  return p;
}

int from_hip(hipError_t e) { return e == hipSuccess ? FFD_OK : FFD_ERR_HIP; }

// default placement of the pseudo-max for a whole union step: inside the
// attend launch whenever its words fit one per thread of a work-group and the
// grid fits one dimension.  Measured on MI355X the in-grid placement is the
// faster one at every benchmark shape (16K step 18.6 -> 17.4 us, 256K 65.7 ->
// 64.7, batched Qwen-like 139.9 -> 136.7, stress 295.2 -> 292.6): a long
// cache's chunks scan before they need the maxima, so they never wait.
bool pm_default_in_grid(const ffd_shape_t* s, const Plan& pl) {
  const bool fits = (long long)pl.npart * (s->num_q_heads / s->num_kv_heads) <= 256;
  return fits && (long long)(pl.npart + pl.nchunk) * s->num_kv_heads * s->batch < (1ll << 31);
}

// run-time termination: the call's stream length (0 = the default), or -1
// when it is out of range for the shape
int art_stream_blocks(const ffd_shape_t* s, const ffd_decode_opts_t& o) {
  const int G = s->num_q_heads / s->num_kv_heads;
  const int sb = o.art_stream_blocks == 0 ? FFD_ART_STREAM_BLOCKS_DEFAULT : o.art_stream_blocks;
  return (sb < 1 || sb > (G <= 4 ? 32 : 16)) ? -1 : sb;
}

// the plan a decode call with options `o` runs
Plan decode_plan(const ffd_shape_t* s, const ffd_decode_opts_t& o) {
  return o.art_patience > 0 ? make_plan(s, kTargetGroups, art_stream_blocks(s, o)) : make_plan(s);
}

// The split scan + refine kernels run a union step whose pseudo-max has its
// own launch when the refine's bitmap words fit its LDS.  They are not the
// default anywhere: measured on MI355X they are slower than the fused kernel
// at every benchmark shape (256K: scan 21.4 us + refine 42.9 us against 57.9
// us fused; the batched Qwen-like and stress shapes keep nearly every block,
// where re-reading their thumbnail costs more), so a whole step chooses them
// only when debug->split_mode asks.
bool split_possible(const ffd_shape_t* s, const Plan& pl) {
  const long long heads = (long long)s->batch * s->num_kv_heads;
  return heads <= kSplitMaxHeads && heads * pl.nword_cap <= kSplitMaxWords;
}
bool split_default(const ffd_shape_t*, const Plan&) { return false; }

// Work-groups of the refine kernel: as many as are resident at once on the
// current device (compute units x 2: the kernel runs at 2 waves per SIMD), at
// most kRefineGroupsMax.  The compute-unit count is queried once per device.
constexpr int kMaxDevicesCu = 64;
std::atomic<int> g_cu_count[kMaxDevicesCu];

int refine_groups(int G, int* groups) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevicesCu) return FFD_ERR_HIP;
  int cus = g_cu_count[dev].load(std::memory_order_relaxed);
  if (cus <= 0) {
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      return FFD_ERR_HIP;
    g_cu_count[dev].store(cus, std::memory_order_relaxed);
  }
  (void)G;
  const int n = cus * 2;
  *groups = n < kRefineGroupsMax ? n : kRefineGroupsMax;
  return FFD_OK;
}

}  // namespace

extern "C" {

int ffd_version(void) { return 800; }

const char* ffd_strerror(int code) {
  switch (code) {
    case FFD_OK: return "ok";
    case FFD_ERR_NULL: return "required pointer is NULL";
    case FFD_ERR_SHAPE: return "unsupported shape (head_dim 128, block 64, Hq = G*Hkv with G <= 8, max_seq_len multiple of 64)";
    case FFD_ERR_ALIGN: return "tensor pointer is not 16-byte aligned";
    case FFD_ERR_DELTA: return "delta is NaN or -infinity";
    case FFD_ERR_WORKSPACE: return "workspace missing or too small";
    case FFD_ERR_ARG: return "bad scalar argument (token range or sm_scale)";
    case FFD_ERR_HIP: return "HIP kernel launch failed";
    case FFD_ERR_TOO_LARGE: return "shape needs more than the static scratch of ffd_decode_attn_noalloc (FFD_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown ffd status code";
  }
}

int ffd_cache_bytes(const ffd_shape_t* shape, size_t* codes_bytes, size_t* sz_bytes, size_t* res_bytes,
                    size_t* rscale_bytes, size_t* v_bytes) {
  const int st = check_shape(shape);
  if (st) return st;
  if (!codes_bytes || !sz_bytes || !res_bytes || !rscale_bytes || !v_bytes) return FFD_ERR_NULL;
  const size_t blocks = (size_t)shape->batch * shape->num_kv_heads * (shape->max_seq_len / 64);
  *codes_bytes = blocks * ffd::kCodesBytes;
  *sz_bytes = blocks * ffd::kSzBytes;
  *res_bytes = blocks * ffd::kResBytes;
  *rscale_bytes = blocks * ffd::kRscBytes;
  *v_bytes = blocks * ffd::kVBytes;
  return FFD_OK;
}

int ffd_workspace_bytes(const ffd_shape_t* shape, size_t* bytes) {
  const int st = check_shape(shape);
  if (st) return st;
  if (!bytes) return FFD_ERR_NULL;
  // one workspace serves the FFD decode, the dense baseline and run-time
  // termination with the default stream length
  const size_t a = make_plan(shape).total, d = make_plan(shape, kDenseTargetGroups).total;
  const size_t r = make_plan(shape, kTargetGroups, FFD_ART_STREAM_BLOCKS_DEFAULT).total;
  *bytes = a > d ? a : d;
  if (r > *bytes) *bytes = r;
  return FFD_OK;
}

int ffd_workspace_bytes_ex(const ffd_shape_t* shape, const ffd_decode_opts_t* opts, size_t* bytes) {
  const int st = check_shape(shape);
  if (st) return st;
  if (!bytes) return FFD_ERR_NULL;
  ffd_decode_opts_t o = {};
  if (opts) o = *opts;
  if (o.art_patience > 0 && art_stream_blocks(shape, o) < 0) return FFD_ERR_ARG;
  *bytes = decode_plan(shape, o).total;
  return FFD_OK;
}

int ffd_plan(const ffd_shape_t* shape, int32_t* chunk_blocks, int32_t* n_chunks) {
  const int st = check_shape(shape);
  if (st) return st;
  if (!chunk_blocks || !n_chunks) return FFD_ERR_NULL;
  const Plan p = make_plan(shape);
  *chunk_blocks = p.cb;
  *n_chunks = p.nchunk;
  return FFD_OK;
}

int ffd_plan_split(const ffd_shape_t* shape, int32_t* split) {
  const int st = check_shape(shape);
  if (st) return st;
  if (!split) return FFD_ERR_NULL;
  *split = split_default(shape, make_plan(shape)) ? 1 : 0;
  return FFD_OK;
}

int ffd_plan_pseudomax(const ffd_shape_t* shape, int32_t* n_parts, int32_t* in_grid) {
  const int st = check_shape(shape);
  if (st) return st;
  if (!n_parts || !in_grid) return FFD_ERR_NULL;
  const Plan p = make_plan(shape);
  *n_parts = p.npart;
  *in_grid = pm_default_in_grid(shape, p) ? 1 : 0;
  return FFD_OK;
}

int ffd_quantize_k(const ffd_shape_t* shape, const void* k, int32_t t_begin, int32_t t_end,
                   const ffd_cache_t* cache, void* stream) {
  const int st = check_shape(shape);
  if (st) return st;
  if (!k || !cache || !cache->codes || !cache->sz || !cache->res || !cache->rscale) return FFD_ERR_NULL;
  if (!aligned16(k) || !aligned16(cache->codes) || !aligned16(cache->sz) || !aligned16(cache->res) ||
      !aligned16(cache->rscale))
    return FFD_ERR_ALIGN;
  if (t_begin < 0 || t_end < t_begin || t_end > shape->max_seq_len) return FFD_ERR_ARG;
  if (t_end == t_begin) return FFD_OK;
  return from_hip(ffd::launch_pack(k, shape->batch, shape->num_kv_heads, shape->max_seq_len, t_begin, t_end,
                                   cache->codes, cache->sz, cache->res, cache->rscale,
                                   static_cast<hipStream_t>(stream)));
}

int ffd_pack_v(const ffd_shape_t* shape, const void* v, int32_t t_begin, int32_t t_end, const ffd_cache_t* cache,
               void* stream) {
  const int st = check_shape(shape);
  if (st) return st;
  if (!v || !cache || !cache->v) return FFD_ERR_NULL;
  if (!aligned16(v) || !aligned16(cache->v)) return FFD_ERR_ALIGN;
  if (t_begin < 0 || t_end < t_begin || t_end > shape->max_seq_len) return FFD_ERR_ARG;
  if (t_end == t_begin) return FFD_OK;
  return from_hip(ffd::launch_pack_v(v, shape->batch, shape->num_kv_heads, shape->max_seq_len, t_begin, t_end,
                                     cache->v, static_cast<hipStream_t>(stream)));
}

int ffd_append_kv(const ffd_shape_t* shape, const void* k_new, const void* v_new, const int32_t* pos,
                  const ffd_cache_t* cache, void* stream) {
  const int st = check_shape(shape);
  if (st) return st;
  if (!k_new || !v_new || !pos || !cache || !cache->codes || !cache->sz || !cache->res || !cache->rscale ||
      !cache->v)
    return FFD_ERR_NULL;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(cache->codes) || !aligned16(cache->sz) ||
      !aligned16(cache->res) || !aligned16(cache->rscale) || !aligned16(cache->v) ||
      (reinterpret_cast<uintptr_t>(pos) & 3u))
    return FFD_ERR_ALIGN;
  return from_hip(ffd::launch_append(k_new, v_new, pos, shape->batch, shape->num_kv_heads, shape->max_seq_len,
                                     cache->codes, cache->sz, cache->res, cache->rscale, cache->v,
                                     static_cast<hipStream_t>(stream)));
}

int ffd_decode_attn(const ffd_shape_t* shape, const void* q, const ffd_cache_t* cache, const int32_t* seq_lens,
                    float delta, float sm_scale, void* out, void* workspace, size_t workspace_bytes,
                    const ffd_debug_t* debug, void* stream) {
  return ffd_decode_attn_select(shape, q, cache, seq_lens, delta, sm_scale, FFD_SELECT_UNION, out, workspace,
                                workspace_bytes, debug, stream);
}

int ffd_decode_attn_select(const ffd_shape_t* shape, const void* q, const ffd_cache_t* cache,
                           const int32_t* seq_lens, float delta, float sm_scale, int32_t selection, void* out,
                           void* workspace, size_t workspace_bytes, const ffd_debug_t* debug, void* stream) {
  ffd_decode_opts_t o = {};
  o.selection = selection;
  return ffd_decode_attn_ex(shape, q, cache, seq_lens, delta, sm_scale, &o, out, workspace, workspace_bytes, debug,
                            stream);
}

}  // extern "C"

namespace {

// Allocation-free decode: its workspace is this static device array (one copy
// per GPU, held until the process ends).  Host code never passes the array's
// name to a kernel: its device address is looked up once per device.
__device__ __align__(256) unsigned char scratch[FFD_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// device address of `scratch` on the device `stream` runs on (which must be
// the current device); looked up with hipGetSymbolAddress on the first call
// per device, with that device current
int scratch_address(hipStream_t stream, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FFD_ERR_HIP;
  if (stream) {
    hipDevice_t sdev = -1;
    if (hipStreamGetDevice(stream, &sdev) != hipSuccess) return FFD_ERR_HIP;
    if ((int)sdev != dev) return FFD_ERR_ARG;
  }
  void* ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!ptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    ptr = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!ptr) {
      if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return FFD_ERR_HIP;
      g_scratch_ptr[dev].store(ptr, std::memory_order_release);
    }
  }
  *out = ptr;
  return FFD_OK;
}

// Shared body of the decode entry points.  With `noalloc` the workspace
// arguments are ignored and the step runs on the static scratch array.
int decode_impl(const ffd_shape_t* shape, const void* q, const ffd_cache_t* cache, const int32_t* seq_lens,
                float delta, float sm_scale, const ffd_decode_opts_t* opts, void* out, void* workspace,
                size_t workspace_bytes, const ffd_debug_t* debug, void* stream, bool noalloc) {
  ffd_decode_opts_t o = {};
  if (opts) o = *opts;
  const int32_t selection = o.selection;
  const int st = check_shape(shape);
  if (st) return st;
  if (!q || !cache || !seq_lens || !out || !cache->codes || !cache->sz || !cache->res || !cache->rscale ||
      !cache->v)
    return FFD_ERR_NULL;
  if (!aligned16(q) || !aligned16(out) || !aligned16(cache->codes) || !aligned16(cache->sz) ||
      !aligned16(cache->res) || !aligned16(cache->rscale) || !aligned16(cache->v) ||
      (reinterpret_cast<uintptr_t>(seq_lens) & 3u))
    return FFD_ERR_ALIGN;
  if (isnan(delta) || (isinf(delta) && delta < 0)) return FFD_ERR_DELTA;
  if (!(sm_scale > 0.f) || isinf(sm_scale)) return FFD_ERR_ARG;
  if (selection != FFD_SELECT_UNION && selection != FFD_SELECT_HEAD_BLOCK && selection != FFD_SELECT_HEAD_TOKEN)
    return FFD_ERR_ARG;
  if (o.art_patience < 0) return FFD_ERR_ARG;
  if (o.art_patience > 0 && (selection != FFD_SELECT_UNION || !(o.art_tau >= 0.f) || isinf(o.art_tau) ||
                             !(o.art_phi >= 0.f) || isinf(o.art_phi) || art_stream_blocks(shape, o) < 0))
    return FFD_ERR_ARG;
  const Plan pl = decode_plan(shape, o);
  if (noalloc) {
    if (pl.total > (size_t)FFD_NOALLOC_SCRATCH_BYTES) return FFD_ERR_TOO_LARGE;
    const int sa = scratch_address(static_cast<hipStream_t>(stream), &workspace);
    if (sa) return sa;
    workspace_bytes = FFD_NOALLOC_SCRATCH_BYTES;
  }
  if (!workspace || workspace_bytes < pl.total) return FFD_ERR_WORKSPACE;
  if (!aligned16(workspace)) return FFD_ERR_ALIGN;

  ffd::DecodeParams p = {};
  p.select = selection;
  p.art_patience = o.art_patience;
  p.art_tau = o.art_tau;
  p.art_phi = o.art_phi;
  char* ws = static_cast<char*>(workspace);
  p.q = static_cast<const uint16_t*>(q);
  p.codes = static_cast<const uint8_t*>(cache->codes);
  p.sz = static_cast<const uint8_t*>(cache->sz);
  p.res = static_cast<const int8_t*>(cache->res);
  p.rsc = static_cast<const uint8_t*>(cache->rscale);
  p.v = static_cast<const uint16_t*>(cache->v);
  p.seq_lens = seq_lens;
  p.pmax = reinterpret_cast<float*>(ws + pl.pmax_off);
  p.part_ml = reinterpret_cast<float2*>(ws + pl.ml_off);
  p.part_o = reinterpret_cast<float*>(ws + pl.o_off);
  p.pm_words = reinterpret_cast<unsigned long long*>(ws + pl.pmw_off);
  p.pm_sync = reinterpret_cast<unsigned long long*>(ws + pl.sync_off);
  int pm_mode = 0;
  int split_mode = 0;
  if (debug) {
    if (debug->stages < 0 || debug->stages > 31) return FFD_ERR_ARG;
    if (debug->pm_mode < 0 || debug->pm_mode > 3) return FFD_ERR_ARG;
    if (debug->split_mode < 0 || debug->split_mode > 2) return FFD_ERR_ARG;
    split_mode = debug->split_mode;
    pm_mode = debug->pm_mode;
    p.stages = debug->stages;
    p.dbg_mt = debug->m_tilde;
    p.dbg_bmax = debug->bmax;
    p.dbg_keep = debug->keep;
    p.dbg_tmask = debug->tmask;
    p.ev_start = static_cast<hipEvent_t>(debug->attend_start);
    p.ev_stop = static_cast<hipEvent_t>(debug->attend_stop);
  }
  p.out = static_cast<uint16_t*>(out);
  p.B = shape->batch;
  p.Hq = shape->num_q_heads;
  p.Hkv = shape->num_kv_heads;
  p.L_cap = shape->max_seq_len;
  p.nblk_cap = pl.nblk_cap;
  p.nchunk = pl.nchunk;
  p.cb = pl.cb;
  p.npart = pl.npart;
  p.sink = shape->sink;
  p.local = shape->local;
  p.delta = delta;
  p.sm_scale = sm_scale;
  // Pseudo-max inside the attend launch: possible for the union selection
  // without run-time termination, when the call also enqueues the merge (which
  // advances the epoch of the published words) and the words fit one per
  // thread of a work-group; the default then (pm_default_in_grid).  The
  // magic the merge writes is keyed to the word layout, so words left by
  // another shape are never trusted.
  const bool whole = p.stages == 0 || (p.stages & 6) == 6;
  const bool fits = (long long)pl.npart * (shape->num_q_heads / shape->num_kv_heads) <= 256;
  const bool grid1d = (long long)(pl.npart + pl.nchunk) * shape->num_kv_heads * shape->batch < (1ll << 31);
  const bool can = selection == FFD_SELECT_UNION && o.art_patience == 0 && whole && fits && grid1d;
  if (pm_mode >= 2 && !can) return FFD_ERR_ARG;
  p.pm_in_grid = pm_mode >= 2 || (pm_mode == 0 && can && pm_default_in_grid(shape, pl));
  p.pm_local = pm_mode == 3;
  p.pm_magic = ffd::kPmMagic ^ ((unsigned long long)shape->batch << 40) ^ ((unsigned long long)shape->num_q_heads << 24) ^
               ((unsigned long long)pl.npart << 4);
  // Split path: the union selection without run-time termination, with the
  // pseudo-max in its own launch (debug->pm_mode 1); never the default
  // (split_default), forced on or off by debug->split_mode 2 / 1.
  const bool split_ok = selection == FFD_SELECT_UNION && o.art_patience == 0 && !p.pm_in_grid &&
                        split_possible(shape, pl);
  if (split_mode == 2 && !split_ok) return FFD_ERR_ARG;
  if ((p.stages & 24) && !(split_mode == 2 || (split_mode == 0 && split_ok && split_default(shape, pl))))
    return FFD_ERR_ARG;  // the scan / refine stage bits exist on the split path only
  p.split = split_mode == 2 || (split_mode == 0 && split_ok && split_default(shape, pl));
  p.nword_cap = pl.nword_cap;
  if (p.split) {
    const int rg = refine_groups(shape->num_q_heads / shape->num_kv_heads, &p.refine_groups);
    if (rg) return rg;
    p.kmask = reinterpret_cast<uint32_t*>(ws + pl.km_off);
    p.unit_start = reinterpret_cast<int*>(ws + pl.us_off);
    p.part_ml = reinterpret_cast<float2*>(ws + pl.sml_off);
    p.part_o = reinterpret_cast<float*>(ws + pl.so_off);
  }
  return from_hip(ffd::launch_ffd_decode(p, static_cast<hipStream_t>(stream)));
}


}  // namespace

extern "C" {

int ffd_decode_attn_ex(const ffd_shape_t* shape, const void* q, const ffd_cache_t* cache, const int32_t* seq_lens,
                       float delta, float sm_scale, const ffd_decode_opts_t* opts, void* out, void* workspace,
                       size_t workspace_bytes, const ffd_debug_t* debug, void* stream) {
  return decode_impl(shape, q, cache, seq_lens, delta, sm_scale, opts, out, workspace, workspace_bytes, debug,
                     stream, false);
}

int ffd_decode_attn_noalloc(const ffd_shape_t* shape, const void* q, const ffd_cache_t* cache,
                            const int32_t* seq_lens, float delta, float sm_scale, void* out, void* stream) {
  return decode_impl(shape, q, cache, seq_lens, delta, sm_scale, nullptr, out, nullptr, 0, nullptr, stream, true);
}

int ffd_dense_decode_attn(const ffd_shape_t* shape, const void* q, const void* k, const void* v,
                          const int32_t* seq_lens, float sm_scale, void* out, void* workspace,
                          size_t workspace_bytes, void* stream) {
  const int st = check_shape(shape);
  if (st) return st;
  if (!q || !k || !v || !seq_lens || !out) return FFD_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) ||
      (reinterpret_cast<uintptr_t>(seq_lens) & 3u))
    return FFD_ERR_ALIGN;
  if (!(sm_scale > 0.f) || isinf(sm_scale)) return FFD_ERR_ARG;
  const Plan pl = make_plan(shape, kDenseTargetGroups);
  if (!workspace || workspace_bytes < pl.total) return FFD_ERR_WORKSPACE;
  if (!aligned16(workspace)) return FFD_ERR_ALIGN;
  ffd::DecodeParams p = {};
  char* ws = static_cast<char*>(workspace);
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.seq_lens = seq_lens;
  p.pmax = reinterpret_cast<float*>(ws + pl.pmax_off);
  p.part_ml = reinterpret_cast<float2*>(ws + pl.ml_off);
  p.part_o = reinterpret_cast<float*>(ws + pl.o_off);
  p.out = static_cast<uint16_t*>(out);
  p.B = shape->batch;
  p.Hq = shape->num_q_heads;
  p.Hkv = shape->num_kv_heads;
  p.L_cap = shape->max_seq_len;
  p.nblk_cap = pl.nblk_cap;
  p.nchunk = pl.nchunk;
  p.cb = pl.cb;
  p.npart = pl.npart;
  p.sm_scale = sm_scale;
  return from_hip(ffd::launch_dense_decode(p, static_cast<hipStream_t>(stream)));
}

int ffd_stream_read(const void* src, size_t bytes, void* sink, void* stream) {
  if (!src || !sink) return FFD_ERR_NULL;
  if (!aligned16(src) || (bytes & 15u) || (reinterpret_cast<uintptr_t>(sink) & 3u)) return FFD_ERR_ALIGN;
  static_assert(ffd::kStreamReadGroups * sizeof(uint32_t) == FFD_STREAM_READ_SINK_BYTES, "probe sink size");
  return from_hip(ffd::launch_stream_read(src, bytes, sink, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
