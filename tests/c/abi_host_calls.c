/* A plain C99 consumer of include/beamattn.h: the header compiles without C++ or HIP
 * headers, the library links, and the host-only functions and argument checks behave.
 * Nothing here launches GPU work: every attention call below fails its checks first.
 * Exit status 0 on success; each failed check prints a line and sets status 1. */
#include <stdio.h>
#include <string.h>

#include "beamattn.h"

static int failures = 0;
#define CHECK(cond)                                                   \
  do {                                                                \
    if (!(cond)) {                                                    \
      printf("FAILED: %s (line %d)\n", #cond, __LINE__);              \
      failures = 1;                                                   \
    }                                                                 \
  } while (0)

static beam_layer_desc layer(int32_t kind) {
  beam_layer_desc d;
  memset(&d, 0, sizeof d);
  d.num_q_heads = 48;
  d.num_kv_heads = 8;
  d.head_dim = 128;
  d.page_size = 64;
  d.kind = kind;
  d.window = kind == BEAM_LAYER_SWA ? 512 : 0;
  d.rope_theta = 1e4f;
  d.rms_eps = 1e-6f;
  d.ssmax_base = 2048.f;
  d.ssmax_exponent = 0.1f;
  d.sm_scale = 0.08838834764831845f;
  return d;
}

int main(void) {
  /* version and the KV-size closed form: 9 full layers x 2 (K, V) x 8 heads x 128 */
  CHECK(beam_abi_version() == BEAM_ABI_VERSION);
  CHECK(beam_kv_bytes_per_token(9, 8, 128, BEAM_KV_BF16) == 36864u);
  CHECK(beam_kv_bytes_per_token(9, 8, 128, BEAM_KV_FP8_E4M3) == 18432u);
  CHECK(beam_kv_bytes_per_token(52, 8, 128, BEAM_KV_BF16) == 212992u);
  CHECK(strcmp(beam_status_string(BEAM_OK), beam_status_string(BEAM_ERR_WORKSPACE)) != 0);

  /* workspace sizing: none for one split, some for a long context */
  beam_layer_desc full = layer(BEAM_LAYER_FULL), swa = layer(BEAM_LAYER_SWA);
  CHECK(beam_attn_decode_workspace_bytes(&full, 1, 1, 512) == 0);
  CHECK(beam_attn_decode_workspace_bytes(&full, 1, 1, 100000) > 0);
  CHECK(beam_attn_decode_workspace_bytes(&swa, 1, 1, 1000000) == 0);
  CHECK(beam_attn_decode_workspace_bytes(&full, 1, 17, 100000) == 0); /* q_len above 16 */

  /* argument checks fail before any launch and leave a message */
  beam_layer_desc bad = full;
  bad.head_dim = 64;
  CHECK(beam_attn_prefill(&bad, NULL, NULL, NULL, 0, NULL, 0, NULL, NULL, 0, NULL) ==
        BEAM_ERR_INVALID_ARG);
  CHECK(strlen(beam_last_error()) > 0);
  CHECK(beam_attn_decode(&full, NULL, NULL, NULL, 0, NULL, 0, NULL, NULL, 0, NULL, 0, NULL) ==
        BEAM_ERR_INVALID_ARG);
  CHECK(beam_head_gate(&full, 4, NULL, 6144, NULL, 6144, NULL, NULL, 6144, NULL) ==
        BEAM_ERR_INVALID_ARG);

  /* an empty batch (every sequence finished) sizes no workspace and launches nothing;
   * the cache and tensor pointers are never dereferenced on this path */
  CHECK(beam_attn_decode_workspace_bytes(&full, 0, 1, 100000) == 0);
  CHECK(beam_attn_decode_workspace_bytes(&swa, 0, 16, 1048584) == 0);
  {
    static uint64_t fake[64]; /* 16-byte aligned host storage standing in for device buffers */
    beam_kv_cache cache;
    beam_batch empty;
    memset(&cache, 0, sizeof cache);
    memset(&empty, 0, sizeof empty);
    cache.k = fake;
    cache.v = fake + 32;
    cache.num_pages = 1;
    cache.dtype = BEAM_KV_BF16;
    empty.num_seqs = 0;
    empty.max_pages = 1563;
    empty.max_q_len = 1;
    empty.max_kv_len = 100000;
    empty.num_tokens = 0;
    CHECK(beam_attn_decode(&full, &empty, &cache, NULL, 6144, NULL, 6144, NULL, NULL, 6144, NULL, 0,
                           NULL) == BEAM_OK);
    CHECK(beam_attn_decode(&swa, &empty, &cache, NULL, 6144, NULL, 6144, NULL, NULL, 6144, NULL, 0,
                           NULL) == BEAM_OK);
  }

  /* the projection GEMM: k must be a multiple of 64, and a 256-row tile of x or w must
   * span fewer than 2^31 bytes (row strides up to 4,194,303 elements); the checks fail
   * before any launch, so host pointers stand in for device buffers */
  {
    static uint64_t fake[64];
    CHECK(beam_linear_bf16(16, 64, 100, fake, 128, fake, 128, fake + 32, 64, NULL) ==
          BEAM_ERR_INVALID_ARG);
    CHECK(beam_linear_bf16(16, 64, 64, fake, 4194304, fake, 64, fake + 32, 64, NULL) ==
          BEAM_ERR_INVALID_ARG);
    CHECK(strstr(beam_last_error(), "stride") != NULL);
    CHECK(beam_linear_bf16(16, 64, 64, fake, 64, fake, 4194304, fake + 32, 64, NULL) ==
          BEAM_ERR_INVALID_ARG);
  }

  /* prefill moves a row tile's q, gate and out rows through 32-bit offsets: token
   * strides above 4,194,303 elements are refused before any launch, for both kinds */
  {
    static uint64_t fake[64];
    static int32_t meta[4];
    beam_kv_cache cache;
    beam_batch one;
    memset(&cache, 0, sizeof cache);
    memset(&one, 0, sizeof one);
    cache.k = fake;
    cache.v = fake + 32;
    cache.num_pages = 1;
    cache.dtype = BEAM_KV_BF16;
    one.num_seqs = 1;
    one.q_start = meta;
    one.kv_len = meta + 2;
    one.block_table = meta + 3;
    one.max_pages = 1;
    one.max_q_len = 1;
    one.max_kv_len = 1;
    one.num_tokens = 1;
    CHECK(beam_attn_prefill(&swa, &one, &cache, fake, 4194304, NULL, 0, NULL, fake + 32, 6144,
                            NULL) == BEAM_ERR_INVALID_ARG);
    CHECK(strstr(beam_last_error(), "stride") != NULL);
    CHECK(beam_attn_prefill(&swa, &one, &cache, fake, 6144, fake, 4194304, fake, fake + 32, 6144,
                            NULL) == BEAM_ERR_INVALID_ARG);
    CHECK(beam_attn_prefill(&swa, &one, &cache, fake, 6144, NULL, 0, NULL, fake + 32, 4194304,
                            NULL) == BEAM_ERR_INVALID_ARG);
    CHECK(beam_attn_prefill(&full, &one, &cache, fake, 4194304, NULL, 0, NULL, fake + 32, 6144,
                            NULL) == BEAM_ERR_INVALID_ARG);
  }

  if (!failures) printf("ok\n");
  return failures;
}
