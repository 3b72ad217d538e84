/*
 * libbeamattn: the attention core of one decoder layer of the hybrid sliding-window /
 * NoPE GQA model (48 query heads, 8 KV heads, head dim 128), as hand-written HIP for
 * one AMD Instinct MI355X (gfx950).
 *
 * What it computes comes from the model descriptions in "Reflection Beam 1.0 on vLLM:
 * Day 0 Serving, Agent-Optimized Kernels, and DFlash2 Speculative Decoding" (section
 * "Attention: sliding-window layers plus NoPE full-attention layers") and "SGLang
 * natively supports Reflection's Beam" (sections "Hybrid attention and output gating",
 * "SSMax", "Unified memory for target and draft KV", "Fusion optimizations").
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Plain C ABI. Pointers marked "device" are device memory of the current HIP device;
 *    pointers marked "host" are host memory read before the call returns. The caller
 *    owns every buffer; the library keeps no pointer after a call returns, allocates
 *    nothing, and is safe to call from several threads. Its only mutable global state is
 *    the per-device address of the scratch array of beam_attn_decode_noalloc.
 *  - `stream` is a hipStream_t passed as void*; NULL means the null stream. Every call
 *    only enqueues work on it and returns; nothing synchronises.
 *  - Element types: bf16 tensors are 16-bit bfloat16 values; fp8 caches hold OCP E4M3FN
 *    codes. Strides are in elements, not bytes. Within a token, heads are contiguous and
 *    each head's 128 values are contiguous (head stride = head_dim).
 *  - Errors: every host-visible argument is checked before anything is launched. On a
 *    failed check the call returns a non-zero beam_status, records a message readable
 *    with beam_last_error() (thread-local), and launches nothing. A failed launch returns
 *    BEAM_ERR_HIP. Device-resident metadata (q_start, kv_len, block_table) is a
 *    precondition and is not read by the host: it must satisfy the beam_batch rules
 *    below. No C++ exception crosses this interface, and the library never prints or
 *    aborts.
 *  - Debug builds (compiled with BEAMATTN_DEBUG, built as libbeamattn_debug.so): the
 *    K/V-write, prefill and decode entry points first check the device metadata against
 *    the beam_batch rules on the GPU and return BEAM_ERR_INVALID_ARG naming the first
 *    broken rule and sequence, before any other kernel runs. That check allocates 4
 *    bytes and synchronises the stream, so debug builds are not for graph capture.
 */
#ifndef BEAMATTN_H
#define BEAMATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BEAM_ABI_VERSION 2

typedef enum beam_status {
  BEAM_OK = 0,
  BEAM_ERR_INVALID_ARG = 1,  /* a pointer, size, stride, alignment or constant is invalid */
  BEAM_ERR_UNSUPPORTED = 2,  /* valid but not implemented by this library version       */
  BEAM_ERR_WORKSPACE = 3,    /* decode workspace missing or smaller than required        */
  BEAM_ERR_HIP = 4           /* the HIP runtime reported an error while launching        */
} beam_status;

/* The two layer types ("Attention: sliding-window layers plus NoPE full-attention
 * layers"): sliding layers attend to the most recent `window` keys and rotate Q/K with
 * RoPE; full layers attend to every earlier key, use no positional encoding, and scale
 * each query by SSMax. */
typedef enum beam_layer_kind { BEAM_LAYER_SWA = 0, BEAM_LAYER_FULL = 1 } beam_layer_kind;

/* KV cache element type. FP8 uses OCP E4M3FN codes with one fp32 scale per tensor
 * (stored code * scale = value). */
typedef enum beam_kv_dtype { BEAM_KV_BF16 = 0, BEAM_KV_FP8_E4M3 = 1 } beam_kv_dtype;

/* Every constant of a layer, explicit. Supported: head_dim == 128, page_size == 64,
 * num_q_heads % num_kv_heads == 0 with a group of at most 16 query heads per KV head. */
typedef struct beam_layer_desc {
  int32_t num_q_heads;    /* 48 */
  int32_t num_kv_heads;   /* 8  */
  int32_t head_dim;       /* 128 */
  int32_t page_size;      /* 64 tokens per KV page */
  int32_t kind;           /* beam_layer_kind */
  int32_t window;         /* keys visible to a sliding-layer query, its own included: 512; ignored for FULL */
  float rope_theta;       /* 1e4: pair i of a head turns by pos * theta^(-2i/head_dim) (rotate-half) */
  float rms_eps;          /* 1e-6: y = w * x / sqrt(mean(x^2) + eps) per head */
  float ssmax_base;       /* 2048: full-layer query scale (1 + p/base)^exponent, p = pos + 1 */
  float ssmax_exponent;   /* 0.1 */
  float sm_scale;         /* softmax scale on q.k: 1/sqrt(128) */
} beam_layer_desc;

/* One layer's paged KV cache. K and V are separate device arrays shaped
 * [num_pages][num_kv_heads][page_size][head_dim] of bf16 values or fp8 codes, so one
 * KV head's page is a contiguous 16 KiB (bf16) or 8 KiB (fp8) block. */
typedef struct beam_kv_cache {
  void* k;                /* device */
  void* v;                /* device */
  int64_t num_pages;      /* pages in the pool; every block_table entry read must be below it */
  int32_t dtype;          /* beam_kv_dtype */
  float k_scale;          /* fp8 only: value = code * k_scale (> 0); ignored for bf16 */
  float v_scale;          /* fp8 only */
} beam_kv_cache;

/* A batch of sequences, each adding n_b >= 0 new tokens in this call.
 * Token order: the new tokens of sequence b are rows q_start[b] .. q_start[b+1]-1 of the
 * token-indexed tensors. kv_len[b] counts the keys of sequence b after the call, new
 * ones included, so new token i of sequence b sits at 0-based position
 * pos = kv_len[b] - n_b + i; the SSMax position is p = pos + 1.
 * Virtual -> physical translation ("Unified memory for target and draft KV": reads and
 * writes use one contract): token pos of sequence b lives in physical page
 * block_table[b * max_pages + pos / page_size] at slot pos % page_size.
 * Preconditions on the device arrays: q_start is non-decreasing with q_start[0] = 0 and
 * q_start[num_seqs] <= num_tokens; n_b <= max_q_len; n_b <= kv_len[b] <= max_kv_len; and
 * every block_table entry for a page that holds a visible key (and, for the K/V write,
 * a new token) is in [0, num_pages). Entries for pages with no visible key are never
 * read.
 * Rows q_start[num_seqs] .. num_tokens-1 are padding: no K/V is stored for them and no
 * attention output is written for them (beam_head_gate, which has no batch, gates them
 * like any row). With padding and host bounds that cover every step (max_q_len,
 * max_kv_len, max_pages), one recorded HIP graph of a decode step replays for any
 * lengths within the bounds: only the device arrays and tensor contents change.
 * Window-only pools for sliding layers ("Reflection Beam 1.0 on vLLM": sliding layers
 * keep only the window's KV): several logical pages of a sequence may share one
 * physical page, e.g. a ring of R pages with logical page p at ring page p mod R. The
 * K/V write of a call lands before its attention reads, so a call may add at most
 * R * page_size - window + 1 new tokens to such a sequence (65 for R = 9, page 64,
 * window 512); then no key a new token sees has been overwritten. */
typedef struct beam_batch {
  int32_t num_seqs;
  const int32_t* q_start;      /* device [num_seqs + 1] */
  const int32_t* kv_len;       /* device [num_seqs] */
  const int32_t* block_table;  /* device [num_seqs][max_pages] */
  int32_t max_pages;           /* row stride of block_table; >= ceil(max_kv_len / page_size) */
  int32_t max_q_len;           /* host bound on n_b */
  int64_t max_kv_len;          /* host bound on kv_len[b] */
  int64_t num_tokens;          /* rows of the token-indexed tensors, >= q_start[num_seqs] */
} beam_batch;

/* Fused per-head Q/K RMSNorm + RoPE (sliding layer) or SSMax query scaling (full layer)
 * + bf16 rounding + paged K/V store ("Agent-driven optimization", changes 2 and 6, of
 * the vLLM page: one kernel normalises Q/K, applies RoPE or SSMax, and writes K and V
 * into the cache; "Fusion optimizations" of the SGLang page).
 *  q        device bf16 [num_tokens][num_q_heads][head_dim], token stride q_stride
 *  k, v     device bf16 [num_tokens][num_kv_heads][head_dim], token strides k_stride, v_stride
 *  q_norm_w, k_norm_w  device bf16 [head_dim] shared by all heads (norm_w_head_stride = 0)
 *           or [heads][head_dim] with head stride norm_w_head_stride
 *  q_out    device bf16 [num_tokens][num_q_heads][head_dim], token stride q_out_stride:
 *           q' = bf16(norm(q) rotated, or scaled by SSMax). May equal q (in place) when
 *           q_out_stride == q_stride; must not otherwise overlap q.
 * K is normalised (and rotated on sliding layers; never scaled) and stored with V
 * (unchanged) at each new token's slot: bf16 as is, fp8 as e4m3(value / scale) with
 * round-to-nearest-even and saturation at +-448. Math is fp32; angles are formed in
 * fp64. Only the new tokens' slots are written. */
beam_status beam_qknorm_rope_ssmax_kvwrite(const beam_layer_desc* layer, const beam_batch* batch,
                                           const beam_kv_cache* cache,
                                           const void* q, int64_t q_stride,
                                           const void* k, int64_t k_stride,
                                           const void* v, int64_t v_stride,
                                           const void* q_norm_w, const void* k_norm_w,
                                           int64_t norm_w_head_stride,
                                           void* q_out, int64_t q_out_stride, void* stream);

/* Causal prefill attention over the paged cache ("Reflection Beam 1.0 on vLLM", section
 * "Attention: sliding-window layers plus NoPE full-attention layers"), bf16 or fp8-e4m3
 * cache, MFMA bf16 with fp32 softmax, GQA (query head h reads KV head
 * h / (num_q_heads/num_kv_heads)), optional fused output gate.
 *  q     device bf16 q' from beam_qknorm_rope_ssmax_kvwrite, [num_tokens][Hq][D], stride q_stride
 *  gate  device bf16 [num_tokens][Hq*D], token stride gate_stride, or NULL for no gate
 *  gate_bias device bf16 [Hq] (ignored when gate is NULL)
 *  out   device bf16 [num_tokens][Hq][D], token stride out_stride:
 *        out[t,h,d] = sum_j softmax_j(sm_scale * q'[t,h].k[j,g]) v[j,g,d], times
 *        sigmoid(gate[t, h*D + d] + gate_bias[h]) when gated, rounded to bf16.
 * New token t at position pos sees keys [0, pos] (full) or [max(0, pos-window+1), pos]
 * (sliding), which include earlier new tokens of the same call: their K/V must already
 * be in the cache (beam_qknorm_rope_ssmax_kvwrite writes them). A query with no new
 * tokens in its sequence produces nothing. Over an fp8 cache the codes are widened
 * exactly to bf16 on their way into the kernel's tiles; scores use sm_scale * k_scale
 * and the output is scaled by v_scale (chunked prefill with an fp8 KV cache, "SGLang
 * natively supports Reflection's Beam": the serving setup runs FP8 KV).
 * On full layers with at least 1,024 keys the library may split a row tile's keys
 * between two halves of its workgroup, which merge their partial softmaxes; results
 * agree with the unsplit path within rounding. The environment variable
 * BEAMATTN_PREFILL_KEY_SPLIT=0 turns this off and =1 splits every row tile (read on each
 * call). Returns BEAM_ERR_INVALID_ARG when the launch would exceed 2^30 row tiles, or
 * when q_stride, out_stride or (gated) gate_stride exceeds 4,194,303 elements. */
beam_status beam_attn_prefill(const beam_layer_desc* layer, const beam_batch* batch,
                              const beam_kv_cache* cache, const void* q, int64_t q_stride,
                              const void* gate, int64_t gate_stride, const void* gate_bias,
                              void* out, int64_t out_stride, void* stream);

/* Decode / speculative-verify attention: the same result as beam_attn_prefill for
 * 1..16 new tokens per sequence (causal within the block), over a bf16 or fp8 cache.
 * Defined by "Reflection Beam 1.0 on vLLM", section "Attention: sliding-window layers
 * plus NoPE full-attention layers" (what each layer kind attends to), and by "SGLang
 * natively supports Reflection's Beam", DFlash2 section (a drafted block of tokens is
 * checked by one forward of the target model, so its tokens attend causally among
 * themselves on top of the cached prefix). An empty batch (num_seqs == 0) launches
 * nothing and returns BEAM_OK.
 * The keys are split into chunks processed in parallel; partial (max, sum, output)
 * triples go to `workspace` (device, at least beam_attn_decode_workspace_bytes(...)
 * bytes, 256-byte aligned; its contents need no initialisation and are scratch after
 * the call) and are merged by log-sum-exp, then gated and stored as bf16.
 * Returns BEAM_ERR_WORKSPACE if workspace_bytes is too small, BEAM_ERR_INVALID_ARG if
 * max_q_len is not in 1..16. Calls that share a workspace must not overlap in time. */
beam_status beam_attn_decode(const beam_layer_desc* layer, const beam_batch* batch,
                             const beam_kv_cache* cache, const void* q, int64_t q_stride,
                             const void* gate, int64_t gate_stride, const void* gate_bias,
                             void* out, int64_t out_stride,
                             void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes beam_attn_decode needs for these host bounds (0 on invalid input and
 * for an empty batch). */
size_t beam_attn_decode_workspace_bytes(const beam_layer_desc* layer, int32_t num_seqs,
                                        int32_t max_q_len, int64_t max_kv_len);

/* Bytes of the device scratch array behind beam_attn_decode_noalloc (32 MiB per device). */
#define BEAM_DECODE_NOALLOC_SCRATCH_BYTES (32u * 1024u * 1024u)

/* beam_attn_decode without a workspace argument, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc. Same arguments, checks, kernels and results as beam_attn_decode (bit for
 * bit); the split partials go to a file-scope device array of
 * BEAM_DECODE_NOALLOC_SCRATCH_BYTES that each device the library runs on holds until the
 * process ends. The call allocates nothing (no hipMalloc, no allocating library call).
 * Returns BEAM_ERR_WORKSPACE, launching nothing, when the host bounds need more scratch
 * than that (beam_attn_decode_workspace_bytes tells the need; e.g. 32 sequences of up to
 * 131,072 keys, or one 16-token block over 1,048,584 keys, fit). The scratch needs no
 * initialisation. Every call on one device shares that device's scratch and leaves its
 * partials there: calls that may overlap in time on one device (several streams, several
 * threads) race and must be serialised by the caller. Debug builds do not run their
 * batch-metadata check in this entry point (that check allocates). */
beam_status beam_attn_decode_noalloc(const beam_layer_desc* layer, const beam_batch* batch,
                                     const beam_kv_cache* cache, const void* q, int64_t q_stride,
                                     const void* gate, int64_t gate_stride, const void* gate_bias,
                                     void* out, int64_t out_stride, void* stream);

/* Standalone output gate ("Attention: sliding-window layers plus NoPE full-attention
 * layers" of the vLLM page: a sigmoid of the gate projection plus a per-head bias scales
 * each head's output ahead of o_proj; "Fusion optimizations" of the SGLang page: one
 * kernel for the bias add, sigmoid and product):
 *  out[t,h,d] = bf16(attn[t,h,d] * sigmoid(gate[t,h*D+d] + gate_bias[h])), fp32 math.
 *  attn, out device bf16 [num_tokens][Hq][D] (token strides attn_stride, out_stride; out may
 *  equal attn); gate device bf16 [num_tokens][Hq*D]; gate_bias device bf16 [Hq]. */
beam_status beam_head_gate(const beam_layer_desc* layer, int64_t num_tokens,
                           const void* attn, int64_t attn_stride,
                           const void* gate, int64_t gate_stride, const void* gate_bias,
                           void* out, int64_t out_stride, void* stream);

/* bf16 linear layer y = x W^T for the projections on either side of the attention core:
 * the packed Q/K/V/gate projection (hidden 5120 -> 14336 = 6144 q + 1024 k + 1024 v + 6144
 * gate columns; "Agent-driven optimization" of the vLLM page: one packed GEMM feeds the
 * fused norm kernel, whose strided inputs are column ranges of its output) and o_proj
 * (6144 -> 5120). y[i][j] = bf16(sum_c x[i][c] * w[j][c]) with fp32 accumulation.
 *  m, n, k  rows of x (tokens), output features, input features; k % 64 == 0, n % 4 == 0
 *  x        device bf16 [m][k], row stride x_stride (>= k, a multiple of 8, at most
 *           4,194,303)
 *  w        device bf16 [n][k] (the weight in its [out][in] layout), row stride w_stride
 *           (>= k, a multiple of 8, at most 4,194,303)
 *  y        device bf16 [m][n], row stride y_stride (>= n, a multiple of 8); must not
 *           overlap x or w
 * m == 0 launches nothing. Sized for prefill token counts (tiles of 256 tokens x 256
 * features); it is correct for any m. */
beam_status beam_linear_bf16(int64_t m, int64_t n, int64_t k, const void* x, int64_t x_stride,
                             const void* w, int64_t w_stride, void* y, int64_t y_stride,
                             void* stream);

/* KV-cache bytes that grow with each token (the "Attention" section of the vLLM pages):
 * num_full_layers * 2 (K and V) * num_kv_heads * head_dim * bytes per value; only the
 * full layers keep the whole history. 36 KiB bf16 / 18 KiB fp8 for 9 layers, 8 KV
 * heads, head dim 128. 0 on invalid input. */
uint64_t beam_kv_bytes_per_token(int32_t num_full_layers, int32_t num_kv_heads, int32_t head_dim,
                                 int32_t dtype);

/* Static description of a status code. */
const char* beam_status_string(beam_status status);
/* Message of the last failed call on this thread ("" if none). */
const char* beam_last_error(void);
/* BEAM_ABI_VERSION of the loaded library. */
int32_t beam_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* BEAMATTN_H */
