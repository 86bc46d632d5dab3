/*
 * ffd.h -- C ABI of libffd, FFD sparse decode attention for MI355X (gfx950).
 *
 * The method is the one summarised in "Faster Than Flash: Exploiting Attention
 * Sparsity for Efficient Long-Context Decoding" (gist.science technical
 * summary of arXiv 2609.00097):
 *   Method 1  K is stored as a 2-bit quantized thumbnail (for score estimates)
 *             plus 8-bit residuals that rebuild K near fp16;
 *   Method 2  Top-delta: a token is kept when its score s >= m~ - delta, with the
 *             pseudo-max m~ taken over the sink and local tokens only;
 *   Method 3  three stages: pseudo-max estimation, a scan of the 2-bit keys that
 *             filters blocks against the threshold, and exact attention with the
 *             residuals and the values on the kept blocks.
 *
 * Conventions fixed by this library where the page is silent:
 *   - head_dim 128, blocks of 64 tokens, 32-channel quantization groups;
 *   - per token and group: zero = min, scale = fp16 RNE((max-min)/3),
 *     code c = #{k in 1..3 : x - zero >= (k - 1/2) scale} (0 if scale == 0),
 *     residual r = x - (zero + c*scale), rscale = fp16 RNE(max|r| / 127),
 *     res = sign(r) * min(127, #{k >= 1 : |r| >= (k - 1/2) rscale}) (0 if rscale == 0),
 *     K-hat = zero + c*scale + res*rscale; signed zeros stored as +0;
 *   - scores are softmax logits s = (q . k) * sm_scale (natural-log units);
 *     estimated scores use zero + c*scale, exact scores use K-hat;
 *   - support (pseudo-max) tokens [0, min(sink, L)) U [max(0, L-local), L);
 *     a block is kept if it holds a support token, or if for some query head h
 *     of its GQA group  max_{t in block} s_est[h][t] >= m~[h] - delta;
 *     every query head of the group attends to every valid token of every
 *     kept block; dropped tokens contribute nothing (softmax renormalised);
 *   - query head h uses KV head h / (Hq / Hkv).
 *
 * Memory: every pointer is a device pointer (hipMalloc / PyTorch CUDA tensor)
 * unless said otherwise; the caller allocates and frees everything.  Calls
 * enqueue work on `stream` (a hipStream_t, or NULL for the null stream) and
 * return without synchronising the host.  The library keeps no state between
 * calls apart from two documented exceptions: the step counter a workspace
 * carries from one ffd_decode_attn call to the next (ffd_workspace_bytes), and
 * the static scratch array of ffd_decode_attn_noalloc.  Errors are returned
 * as negative codes; argument checks happen
 * before any HIP call, so a non-zero return means nothing was enqueued
 * (except FFD_ERR_HIP, which reports a failed launch).
 */
#ifndef FFD_H_
#define FFD_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum ffd_status {
  FFD_OK = 0,
  FFD_ERR_NULL = -1,      /* a required pointer is NULL                          */
  FFD_ERR_SHAPE = -2,     /* unsupported shape (see ffd_shape_t)                 */
  FFD_ERR_ALIGN = -3,     /* a tensor pointer is not 16-byte aligned             */
  FFD_ERR_DELTA = -4,     /* delta is NaN or -infinity                           */
  FFD_ERR_WORKSPACE = -5, /* workspace NULL or smaller than ffd_workspace_bytes  */
  FFD_ERR_ARG = -6,       /* bad scalar argument (token range, sm_scale)         */
  FFD_ERR_HIP = -7,       /* a kernel launch failed                              */
  FFD_ERR_TOO_LARGE = -8  /* the shape needs more scratch than the static buffer  */
                          /* of ffd_decode_attn_noalloc                          */
};

/* Problem shape.  Requirements: batch >= 1, num_kv_heads >= 1,
 * num_q_heads = G * num_kv_heads with 1 <= G <= 8, head_dim == 128,
 * block == 64, sink >= 0, local >= 0, sink + local > 0 (the pseudo-max needs
 * at least one support token), max_seq_len a positive multiple of 64 below
 * 2^24 (the kernels address one head's 256 bytes of values per token with
 * 32-bit offsets),
 * chunk_blocks >= 0 (0 = library choice; otherwise the number of 64-token
 * blocks one work-group scans and refines, capped at 32 for G <= 4 and 24
 * above; it changes only the summation order of the result, and run-time
 * termination ignores it), batch and
 * num_kv_heads at most 65535 (launch-grid dimensions). */
typedef struct ffd_shape {
  int32_t batch;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t block;
  int32_t sink;
  int32_t local;
  int32_t max_seq_len;
  int32_t chunk_blocks;
} ffd_shape_t;

/* Packed FFD cache of one layer.  nblk = max_seq_len / 64; "head" = (b, kv_head),
 * head index b * num_kv_heads + kv_head.  Every field is 16-byte aligned.
 *
 *  codes   uint8  [B][Hkv][nblk][2048]  2-bit codes.  Token t of a block
 *          (t = 0..63), channel slice kq = 0..3, group pair p = 0..1 own the
 *          32-bit little-endian word at byte
 *              (t*4 + kq)*8 + p*4
 *          holding channels 32g + 8kq + j (j = 0..7) of groups g = 2p and 2p+1:
 *          even g: j = 2d at bit 8+2d,  j = 2d+1 at bit 24+2d   (d = 0..3)
 *          odd g:  j = 2d at bit 2d,    j = 2d+1 at bit 16+2d.
 *  sz      fp16   [B][Hkv][nblk][512]   (scale, zero) pairs.  Token t
 *          (tt = t/16, kq = (t/4)%4, i = t%4), group g: scale at byte
 *              ((tt*4 + g)*4 + kq)*16 + i*4, zero 2 bytes after it
 *          (codes and pairs of the 16-token tile tt are one contiguous run).
 *  res     int8   [B][Hkv][nblk][8192]  residual of token t, channel ch at byte
 *              ((ch/16)*64 + t)*16 + ch%16   (two's complement).
 *  rscale  fp16   [B][Hkv][nblk][256]   residual scale of token t (tt = t/16),
 *              group g at element (tt*4 + g)*16 + t%16.
 *  v       fp16   [B][Hkv][max_seq_len*128]  values, token-quad tiled: token
 *          t, channel ch at element ((t/4)*128 + ch)*4 + t%4 (so the four
 *          tokens 4j..4j+3 of one channel are 8 contiguous bytes; one 64-token
 *          block is 16384 contiguous bytes).  Written by ffd_pack_v.
 *
 * Positions the pack never wrote (beyond the sequence) may hold any bytes:
 * decode masks them before any arithmetic that could propagate them. */
typedef struct ffd_cache {
  void* codes;
  void* sz;
  void* res;
  void* rscale;
  void* v;
} ffd_cache_t;

/* Optional diagnostics of ffd_decode_attn (each pointer may be NULL).
 *  m_tilde       f32 [B][Hq]        pseudo-max per query head
 *  bmax          f32 [B][Hq][nblk]  largest estimated score per block (valid blocks only)
 *  keep          u8  [B][Hkv][nblk] 1 = block kept (valid blocks only)
 *  tmask         u8  [B][Hq][max_seq_len]  1 = the query head attends the token,
 *                0 = masked by the selection; written for the valid tokens of
 *                kept blocks only (the rest of the array is left as it was)
 *  attend_start  hipEvent_t recorded on the stream right before the fused
 *  attend_stop   scan + refine kernel, and right after it
 *  stages        0 = the whole step; otherwise a bitmask of the launches to
 *                enqueue (1 = pseudo-max, 2 = scan + refine, 4 = merge; see
 *                split_mode for 8 and 16).  A
 *                partial call reuses what the previous call left in the same
 *                workspace (for timing one kernel alone).  When the
 *                pseudo-max runs inside the scan + refine launch (pm_mode),
 *                bit 1 is ignored.
 *  pm_mode       where the pseudo-max runs.  0 = the library's choice: inside
 *                the scan + refine launch for the union selection without
 *                run-time termination when the call enqueues 2 and 4 (and the
 *                support words fit, see ffd_plan_pseudomax), else its own
 *                launch;
 *                1 = its own launch; 2 = inside the scan + refine launch;
 *                3 = inside it, but every chunk computes the pseudo-max itself
 *                (the path of a workspace's first call).  2 and 3 need the
 *                union selection, no run-time termination and stages 0 or both
 *                2 and 4, else FFD_ERR_ARG.
 *  split_mode    how stages 2 and 3 run for the union selection without
 *                run-time termination: as the one fused scan + refine kernel,
 *                or split into two kernels -- a scan that writes one keep
 *                bitmap word per 32 blocks, and a refine over the compacted
 *                kept blocks only, cut into equal units spread over the
 *                device.  0 = the library's choice (ffd_plan_split: at
 *                present the fused kernel everywhere, the faster one on the
 *                shapes measured); 1 = the fused kernel; 2 = the two kernels
 *                (needs the pseudo-max in its own launch, at most 1024
 *                (sequence, KV head) pairs and 8192 bitmap words, else
 *                FFD_ERR_ARG).  On the
 *                split path stages bit 8 enqueues the scan alone and bit 16
 *                the refine alone (bit 2 both); elsewhere bits 8 and 16 are
 *                FFD_ERR_ARG.  The kept blocks are the same on both paths; the
 *                outputs differ only in summation order.                      */
typedef struct ffd_debug {
  float* m_tilde;
  float* bmax;
  uint8_t* keep;
  void* attend_start;
  void* attend_stop;
  int32_t stages;
  uint8_t* tmask;
  int32_t pm_mode;
  int32_t split_mode;
} ffd_debug_t;

/* What each query head attends inside the blocks kept for its KV head (the
 * blocks loaded and refined are the same in every case).
 *  FFD_SELECT_UNION       every valid token of every kept block (the block
 *                         filter of Method 3 stage 2, shared by the GQA group)
 *  FFD_SELECT_HEAD_BLOCK  the kept blocks that hold a support token or whose
 *                         largest estimated score reaches this head's own
 *                         threshold m~[h] - delta
 *  FFD_SELECT_HEAD_TOKEN  Method 2's criterion per token and head: the support
 *                         tokens plus every token whose estimated score
 *                         reaches this head's threshold */
enum ffd_selection { FFD_SELECT_UNION = 0, FFD_SELECT_HEAD_BLOCK = 1, FFD_SELECT_HEAD_TOKEN = 2 };

/* Bytes of each packed-cache field for `shape` (host call, no GPU work). */
int ffd_cache_bytes(const ffd_shape_t* shape, size_t* codes_bytes, size_t* sz_bytes,
                    size_t* res_bytes, size_t* rscale_bytes, size_t* v_bytes);

/* Workspace bytes ffd_decode_attn, ffd_decode_attn_select, ffd_decode_attn_ex
 * with run-time termination at the default stream length, and
 * ffd_dense_decode_attn need for `shape` (host call; the largest of their
 * work splits).  The workspace holds partial pseudo-maxima and per-chunk
 * attention partials; its contents need no initialisation.  It also carries a
 * step counter from one ffd_decode_attn call to the next: when the pseudo-max
 * runs inside the scan + refine launch (the default for a union step, see
 * ffd_debug_t.pm_mode) its results are tagged with that counter.  The first
 * such call on a workspace (or the first after a change of batch, query heads
 * or support size) computes the pseudo-max in every chunk, which is slower;
 * later calls use the published values.  Calls that share a workspace must be
 * ordered (same stream). */
int ffd_workspace_bytes(const ffd_shape_t* shape, size_t* bytes);

/* Work split ffd_decode_attn chooses for `shape`: blocks per work-group and
 * chunks per sequence (host call).  shape->chunk_blocks > 0 forces the blocks
 * per work-group (capped at 32, or 24 when a KV head serves more than 4 query
 * heads); otherwise about 1380 work-groups per launch, at most 4 blocks each
 * on short caches.  ffd_dense_decode_attn aims at about 2048 instead. */
int ffd_plan(const ffd_shape_t* shape, int32_t* chunk_blocks, int32_t* n_chunks);

/* Whether a whole ffd_decode_attn step (union selection, no debug) for
 * `shape` runs stages 2 and 3 as the split scan + refine kernels (split = 1)
 * or as the fused kernel (0); see ffd_debug_t.split_mode (host call). */
int ffd_plan_split(const ffd_shape_t* shape, int32_t* split);

/* Where the pseudo-max of a whole ffd_decode_attn step (union selection, no
 * debug) runs for `shape` (host call): n_parts = support blocks per sequence
 * (work-groups per KV head), in_grid = 1 when they lead the scan + refine
 * launch, 0 when they have their own launch (see ffd_debug_t.pm_mode): in
 * the grid unless the support parts times query heads per KV head exceed 256
 * words or the one-dimensional grid would exceed 2^31 - 1 work-groups. */
int ffd_plan_pseudomax(const ffd_shape_t* shape, int32_t* n_parts, int32_t* in_grid);

/* K-cache pack (Method 1): quantize tokens [t_begin, t_end) of every (b, kv
 * head) of `k` (fp16 [B][Hkv][max_seq_len][128]) into `cache` (codes, sz,
 * res, rscale; cache->v is not used).  0 <= t_begin <= t_end <= max_seq_len;
 * an empty range is a no-op.  Other positions of the cache are untouched, so
 * a decode loop appends one token with t_end = t_begin + 1.  K must be finite.
 * Byte-exact with the conventions above. */
int ffd_quantize_k(const ffd_shape_t* shape, const void* k, int32_t t_begin, int32_t t_end,
                   const ffd_cache_t* cache, void* stream);

/* Value store for the refinement (Method 3, stage 3 loads the values of the
 * selected blocks): copy tokens [t_begin, t_end) of every (b, kv head) of `v`
 * (fp16 [B][Hkv][max_seq_len][128], natural row-major, 16-byte aligned) into
 * cache->v in the tiled layout above.  The fp16 values are unchanged; only
 * their order differs.  Same range rules as ffd_quantize_k (other positions
 * untouched; t_end = t_begin + 1 appends one token); only cache->v is used. */
int ffd_pack_v(const ffd_shape_t* shape, const void* v, int32_t t_begin, int32_t t_end,
               const ffd_cache_t* cache, void* stream);

/* Decode-loop append (the decode step writes the new token's key and value
 * before attending; the page's Method section captures the step in graphs to
 * remove launch overhead): quantize one new key per (b, kv head) exactly as
 * ffd_quantize_k does and store its value as ffd_pack_v does, at token index
 * pos[b], a position read on the device so that the call can be captured in a
 * graph with ffd_decode_attn.
 *   k_new, v_new  fp16 [B][Hkv][128], natural order, 16-byte aligned
 *   pos           int32 [B] device array; a position outside
 *                 [0, max_seq_len) skips that sequence (nothing is written)
 *   cache         every field is written at the token; other tokens untouched
 * The usual loop appends at pos = L then decodes with seq_lens = L + 1. */
int ffd_append_kv(const ffd_shape_t* shape, const void* k_new, const void* v_new, const int32_t* pos,
                  const ffd_cache_t* cache, void* stream);

/* One FFD decode-attention step (Method 3 stages 1-3 plus the log-sum-exp
 * merge of per-chunk partials).
 *   q         fp16 [B][Hq][128]
 *   seq_lens  int32 [B] device array, 1 <= L <= max_seq_len (values outside
 *             are clamped into that range)
 *   delta     Top-delta margin in natural-log units; +INFINITY keeps every
 *             block; NaN and -INFINITY are rejected
 *   sm_scale  softmax scale, finite and > 0 (usually 1/sqrt(128))
 *   out       fp16 [B][Hq][128]
 *   workspace >= ffd_workspace_bytes(shape) bytes, 16-byte aligned
 *   debug     NULL or diagnostic outputs */
int ffd_decode_attn(const ffd_shape_t* shape, const void* q, const ffd_cache_t* cache,
                    const int32_t* seq_lens, float delta, float sm_scale, void* out,
                    void* workspace, size_t workspace_bytes, const ffd_debug_t* debug,
                    void* stream);

/* Options of ffd_decode_attn_ex.
 *  selection          enum ffd_selection
 *  art_patience       run-time termination of the refine streams (the ART
 *                     page, "Attention Run-time Termination", Method 2.1-2.4:
 *                     a streaming attention unit stops folding in KV blocks
 *                     once its running output is stable).  Stream s of each
 *                     (sequence, KV head) is the contiguous run of blocks
 *                     [s * S, (s + 1) * S), S = art_stream_blocks, cut at the
 *                     sequence end; it visits its kept blocks in increasing
 *                     order (block 0, forced kept, opens stream 0).  After
 *                     each block it takes the probe x = the first 8 channels
 *                     of the running normalised output of the group's first
 *                     query head; from the second block on, a step is stable
 *                     when | ||x|| - ||x_prev|| | < art_tau and
 *                     1 - cos(x, x_prev) < art_phi, and after art_patience
 *                     consecutive stable steps the stream skips its
 *                     remaining blocks (all query heads of the group follow
 *                     it).  The visited blocks depend only on the sequence,
 *                     the query and these options (not on the batch, the
 *                     cache capacity or shape->chunk_blocks).  0 turns it off;
 *                     > 0 requires FFD_SELECT_UNION, finite art_tau,
 *                     art_phi >= 0, and 1 <= S <= 32 (16 when a KV head
 *                     serves more than 4 query heads).
 *  art_stream_blocks  S, the stream length in 64-token blocks
 *                     (0 = FFD_ART_STREAM_BLOCKS_DEFAULT); also the blocks per
 *                     work-group of such a call.
 * The debug tmask marks the tokens of the blocks actually refined. */
#define FFD_ART_STREAM_BLOCKS_DEFAULT 16
typedef struct ffd_decode_opts {
  int32_t selection;
  int32_t art_patience;
  float art_tau;
  float art_phi;
  int32_t art_stream_blocks;
} ffd_decode_opts_t;

/* Workspace bytes one ffd_decode_attn_ex call with options `opts` (NULL =
 * defaults) needs (host call): the figure for another art_stream_blocks than
 * the default.  FFD_ERR_ARG for an out-of-range stream length. */
int ffd_workspace_bytes_ex(const ffd_shape_t* shape, const ffd_decode_opts_t* opts, size_t* bytes);

/* ffd_decode_attn with options (NULL = defaults: union selection, no
 * run-time termination); invalid options return FFD_ERR_ARG. */
int ffd_decode_attn_ex(const ffd_shape_t* shape, const void* q, const ffd_cache_t* cache, const int32_t* seq_lens,
                       float delta, float sm_scale, const ffd_decode_opts_t* opts, void* out, void* workspace,
                       size_t workspace_bytes, const ffd_debug_t* debug, void* stream);

/* ffd_decode_attn with a selection variant (enum ffd_selection; any other
 * value returns FFD_ERR_ARG).  ffd_decode_attn is this call with
 * FFD_SELECT_UNION. */
int ffd_decode_attn_select(const ffd_shape_t* shape, const void* q, const ffd_cache_t* cache,
                           const int32_t* seq_lens, float delta, float sm_scale, int32_t selection, void* out,
                           void* workspace, size_t workspace_bytes, const ffd_debug_t* debug, void* stream);

/* Allocation-free ffd_decode_attn, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same step with the union selection, no run-time
 * termination and no diagnostics, whose workspace is a static device array of
 * FFD_NOALLOC_SCRATCH_BYTES bytes inside the library (one per GPU, held until
 * the process ends).  The call allocates and frees nothing; the caller still
 * owns q, the cache, seq_lens and out (same rules as ffd_decode_attn).
 *  - A shape whose workspace (ffd_workspace_bytes' FFD part) exceeds
 *    FFD_NOALLOC_SCRATCH_BYTES returns FFD_ERR_TOO_LARGE.
 *  - `stream` must belong to the current device (else FFD_ERR_ARG).  The
 *    first call on a device looks the array's address up on that device
 *    (a host query, no allocation); make it once outside any graph capture.
 *  - Every call on one GPU shares that GPU's array and leaves its contents
 *    for the next: calls that overlap on one GPU (other streams, other host
 *    threads without ordering) race and must not be issued.  Calls ordered
 *    on one stream are safe in any sequence of shapes. */
#define FFD_NOALLOC_SCRATCH_BYTES (32u << 20)
int ffd_decode_attn_noalloc(const ffd_shape_t* shape, const void* q, const ffd_cache_t* cache,
                            const int32_t* seq_lens, float delta, float sm_scale, void* out, void* stream);

/* Dense flash-decode attention over fp16 K and V ([B][Hkv][max_seq_len][128]),
 * the speed baseline.  The page's main results measure FFD's kernel and
 * end-to-end speed against dense FlashAttention-2 decoding, which loads the
 * whole fp16 KV cache every step (its problem statement: decode is bound by
 * reloading the cache); this is that dense computation, as a split-KV
 * flash-decode kernel of this library: out = softmax(q k^T * sm_scale) v over
 * tokens [0, L), per query head h with KV head h / (Hq / Hkv).  K and V are in
 * natural row-major order, 16-byte aligned, caller-owned; q, seq_lens, out,
 * workspace and the error codes follow ffd_decode_attn (the workspace of
 * ffd_workspace_bytes covers this call). */
int ffd_dense_decode_attn(const ffd_shape_t* shape, const void* q, const void* k, const void* v,
                          const int32_t* seq_lens, float sm_scale, void* out, void* workspace,
                          size_t workspace_bytes, void* stream);

/* Measurement aid, not part of the decode path: reads the `bytes` bytes at
 * device address `src` once, with 16-byte loads over a fixed grid of 2048
 * work-groups, and writes to `sink` (device, FFD_STREAM_READ_SINK_BYTES bytes,
 * 4-byte aligned) one 32-bit word per work-group: the XOR of the 32-bit words
 * that work-group read, so the XOR over all of sink equals that of the whole
 * buffer (0 for bytes == 0).  The time of one call gives the achievable HBM
 * read rate beside the nominal peak.  Errors: FFD_ERR_NULL (src or sink NULL),
 * FFD_ERR_ALIGN (src not 16-byte aligned, bytes not a multiple of 16, sink not
 * 4-byte aligned), FFD_ERR_HIP.  Asynchronous on `stream`. */
#define FFD_STREAM_READ_SINK_BYTES 8192
int ffd_stream_read(const void* src, size_t bytes, void* sink, void* stream);

/* Static description of an error code. */
const char* ffd_strerror(int code);

/* Library version, major*10000 + minor*100 + patch. */
int ffd_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FFD_H_ */
