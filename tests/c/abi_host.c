/* A plain C99 user of the libffd C ABI (include/ffd.h): host queries and the
 * argument checks that run before any HIP call, so it needs no GPU.  Built and
 * run by tests/test_abi_c.py; prints "ok" and exits 0 when every check holds. */
#include <math.h>
#include <stdio.h>
#include <string.h>

#include "ffd.h"

static int failures = 0;
#define CHECK(cond)                                                   \
  do {                                                                \
    if (!(cond)) {                                                    \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      ++failures;                                                     \
    }                                                                 \
  } while (0)

static ffd_shape_t shape16k(void) {
  ffd_shape_t s;
  memset(&s, 0, sizeof s);
  s.batch = 1;
  s.num_q_heads = 32;
  s.num_kv_heads = 8;
  s.head_dim = 128;
  s.block = 64;
  s.sink = 64;
  s.local = 256;
  s.max_seq_len = 16384;
  s.chunk_blocks = 0;
  return s;
}

int main(void) {
  ffd_shape_t s = shape16k();
  size_t ws = 0, codes = 0, sz = 0, res = 0, rsc = 0, v = 0;
  int32_t cb = 0, nchunk = 0, nparts = 0, in_grid = 0;

  CHECK(ffd_version() > 0);
  CHECK(strcmp(ffd_strerror(FFD_OK), "ok") == 0);
  CHECK(strlen(ffd_strerror(FFD_ERR_SHAPE)) > 0);

  /* packed-cache sizes: 440 bytes per token-head in five fields */
  CHECK(ffd_cache_bytes(&s, &codes, &sz, &res, &rsc, &v) == FFD_OK);
  CHECK(codes + sz + res + rsc + v == (size_t)440 * 8 * 16384);
  CHECK(codes == (size_t)32 * 8 * 16384 && v == (size_t)256 * 8 * 16384);

  /* plan and workspace of the 16K decode layer */
  CHECK(ffd_plan(&s, &cb, &nchunk) == FFD_OK);
  CHECK(cb >= 1 && (long)cb * nchunk >= 16384 / 64);
  CHECK(ffd_plan_pseudomax(&s, &nparts, &in_grid) == FFD_OK);
  CHECK(nparts == 6 && in_grid == 1);
  CHECK(ffd_workspace_bytes(&s, &ws) == FFD_OK && ws > 0);

  /* shape checks */
  {
    ffd_shape_t bad = s;
    bad.head_dim = 64;
    CHECK(ffd_workspace_bytes(&bad, &ws) == FFD_ERR_SHAPE);
    bad = s;
    bad.num_q_heads = 36; /* not a multiple of the KV heads */
    CHECK(ffd_workspace_bytes(&bad, &ws) == FFD_ERR_SHAPE);
    bad = s;
    bad.max_seq_len = 1000; /* not a multiple of 64 */
    CHECK(ffd_plan(&bad, &cb, &nchunk) == FFD_ERR_SHAPE);
  }
  CHECK(ffd_workspace_bytes(NULL, &ws) == FFD_ERR_NULL);

  /* decode-call argument checks, all before any device work: a NULL query,
   * a NaN delta, a missing workspace */
  {
    static uint16_t q[32 * 128], out[32 * 128];
    static int32_t lens[1] = {16384};
    ffd_cache_t c;
    memset(&c, 0, sizeof c);
    CHECK(ffd_decode_attn(&s, NULL, &c, lens, 5.0f, 0.088f, out, NULL, 0, NULL, NULL) == FFD_ERR_NULL);
    c.codes = c.sz = c.res = c.rscale = c.v = (void*)q; /* aligned, never dereferenced here */
    CHECK(ffd_decode_attn(&s, q, &c, lens, NAN, 0.088f, out, (void*)q, ws, NULL, NULL) == FFD_ERR_DELTA);
    CHECK(ffd_decode_attn(&s, q, &c, lens, 5.0f, 0.088f, out, NULL, ws, NULL, NULL) == FFD_ERR_WORKSPACE);
  }

  if (failures) return 1;
  printf("ok\n");
  return 0;
}
