// C ABI of libbeamattn: validates every host-visible argument, then launches the HIP
// kernels on the caller's stream. No allocation, no synchronisation, no global mutable
// state except the thread-local last-error message and the per-device address table of
// the allocation-free decode's scratch array (debug builds add a synchronous check of
// the device-resident batch metadata, see debug_check_batch).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "beam_common.h"
#include "beamattn.h"

namespace {

thread_local char g_last_error[512] = "";

beam_status fail(beam_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return s;
}

beam_status ok() {
  g_last_error[0] = '\0';
  return BEAM_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Decode work split: a workgroup (4 waves, one page per wave per step) covers
// keys_per_split keys of one (sequence, KV head, row chunk). A split is at least as
// long as keeps its partial results (rows x 130 fp32 written, then read by the merge)
// near 1.5% of the fp8 K/V bytes it reads (256 bytes per key). The count of splits is
// set against the workgroups the device holds at once (CUs x resident workgroups per
// CU, "slots"):
//  * one sequence: every split has the same length, so pick the length that minimizes
//    (rounds of slots) x (keys per split + a fixed cost of about 128 keys per
//    workgroup) -- a few more workgroups than slots would otherwise run a second, almost
//    empty round;
//  * several sequences: their lengths are only known on the device, so aim at about 32
//    workgroups per CU sized for the longest (measured best on a 32-sequence batch of
//    8K..128K keys); workgroups past a shorter sequence's end exit at once and the
//    dispatcher balances the rest.
int device_cu_count() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    cus = 256;
  return cus;
}

// Prefill key split (full layers): one prefill workgroup runs per CU at a time (its
// registers and LDS), so an XCD's share of the row tiles runs in rounds of one tile per
// CU. Halving a row tile and giving each half of its key tiles to one of two 4-wave
// streams gives two workgroups of about 0.58 of the time each (the second stream's own
// tile copies and the merge cost the rest). Mode 2 splits as many tiles of an XCD's last
// round as that round leaves CUs idle: 384 row tiles on 256 CUs (2 rounds, the second
// half empty) run 256 whole tiles, then 256 split halves; the 192 tiles of a 1,024-token
// prefill (one round, 64 CUs idle) split their 64 longest (the last 8 of each XCD's 24,
// causal tiles that see the most keys); a grid of a few dozen tiles runs all split.
// Contexts under 1,024 keys keep whole ranges: a workgroup's fixed costs would dominate
// its half.
// BEAMATTN_PREFILL_KEY_SPLIT=0 (never) or 1 (every row tile) in the environment overrides
// the choice.
int choose_prefill_split_mode(const beam::LayerParams& L, const beam::BatchParams& B) {
  if (L.kind != BEAM_LAYER_FULL) return 0;
  if (const char* e = getenv("BEAMATTN_PREFILL_KEY_SPLIT")) {
    if (e[0] == '0') return 0;
    if (e[0] == '1') return 1;
  }
  return B.max_kv_len < 1024 ? 0 : 2;
}

beam::DecodeSplit choose_decode_split(int32_t G, int32_t kind, int32_t window, int32_t num_seqs,
                                      int32_t max_q_len, int64_t max_kv_len, int32_t Hkv,
                                      int32_t kv_dtype) {
  beam::DecodeSplit s{};
  s.num_splits = 1;
  s.row_chunks = 1;
  s.rows_per_chunk = 16;
  s.keys_per_split = beam::kDecodeKeysPerBlockStep;
  s.waves = beam::kDecodeWaves;
  // an empty batch launches nothing: any geometry will do, and the one above needs no
  // workspace (the sizing below would otherwise divide by zero workgroups per split)
  if (num_seqs <= 0 || max_q_len <= 0) return s;
  const int64_t rows = (int64_t)G * max_q_len;
  s.row_chunks = (int32_t)((rows + beam::kDecodeMaxRowsPerChunk - 1) / beam::kDecodeMaxRowsPerChunk);
  if (s.row_chunks < 1) s.row_chunks = 1;
  s.rows_per_chunk = s.row_chunks == 1 ? (int32_t)(((rows + 15) / 16) * 16) : beam::kDecodeMaxRowsPerChunk;
  if (s.rows_per_chunk < 16) s.rows_per_chunk = 16;
  // keys a sequence visits, from its first visited page to its last key
  int64_t range = max_kv_len;
  if (kind == BEAM_LAYER_SWA) {
    const int64_t w = (int64_t)window + max_q_len - 1 + (beam::kPage - 1);
    if (w < range) range = w;
  }
  if (range < 1) range = 1;
  const int64_t unit = (int64_t)num_seqs * Hkv * s.row_chunks;   // workgroups per split index
  const int64_t slots = (int64_t)device_cu_count() * beam::decode_wgs_per_cu(s.rows_per_chunk / 16, kv_dtype);
  const int64_t step = beam::kDecodeKeysPerBlockStep;
  const int64_t rows_in_chunk = rows < s.rows_per_chunk ? rows : s.rows_per_chunk;
  int64_t min_keys = rows_in_chunk * (beam::kHeadDim + 2) * 4 * 64 / 256;
  min_keys = ((min_keys + step - 1) / step) * step;
  // One sequence whose splits at that length would leave CUs idle (few KV heads, e.g. the
  // share of one GPU when the heads are split over 8) takes splits of 512 keys and up:
  // there parallelism matters more than the partials' traffic (measured on 1 KV head:
  // batch-1 decode 24.3 -> 19.2 us, the 8-token 1M verify 110 -> 72 us).
  // (a range that fits one split at that length stays one split: no merge launch)
  if (num_seqs == 1 && range > min_keys &&
      unit * ((range + min_keys - 1) / min_keys) < device_cu_count() && min_keys > 2 * step)
    min_keys = 2 * step;
  const int64_t max_keys = ((range + step - 1) / step) * step;
  if (min_keys > max_keys) min_keys = max_keys;
  int64_t kps = min_keys;
  if (num_seqs == 1) {
    double best = -1.0;
    for (int64_t k = min_keys; k <= max_keys; k += step) {
      const int64_t wgs = unit * ((range + k - 1) / k);
      const double cost = (double)((wgs + slots - 1) / slots) * (double)(k + 128);
      if (best < 0.0 || cost < best) { best = cost; kps = k; }
    }
  } else {
    const int64_t target = 32 * (int64_t)device_cu_count();
    const int64_t want = (target + unit - 1) / unit;                 // splits per sequence
    kps = (range + want - 1) / want;
    kps = ((kps + step - 1) / step) * step;
    if (kps < min_keys) kps = min_keys;
  }
  // the merge kernel holds one weight per split in LDS
  const int64_t kps_cap = (range + beam::kDecodeMaxSplits - 1) / beam::kDecodeMaxSplits;
  if (kps < kps_cap) kps = ((kps_cap + step - 1) / step) * step;
  s.keys_per_split = (int32_t)kps;
  s.num_splits = (int32_t)((range + kps - 1) / kps);
  if (s.num_splits < 1) s.num_splits = 1;
  // A launch of one split that leaves most CUs idle is latency-bound: there, 16-row
  // chunks (each reading the same keys) finish sooner than one workgroup that carries
  // two or three 16-row blocks through every step. Re-read bytes are what this trades,
  // so it applies only while the workgroups are fewer than the CUs.
  if (s.num_splits == 1 && s.rows_per_chunk > 16 &&
      (int64_t)num_seqs * Hkv * s.row_chunks < device_cu_count()) {
    s.row_chunks = (int32_t)((rows + 15) / 16);
    s.rows_per_chunk = 16;
  }
  // Such a launch with one 16-row block and at least 16 workgroups runs wide ones: one
  // per CU, each wave streaming about one page instead of two or three (measured: -14%
  // on 32 sequences' sliding-window decode, -9% on an 8-token sliding verify). With
  // fewer workgroups (batch-1) the fixed costs dominate and 4 waves were slightly faster.
  const int64_t wgs = (int64_t)num_seqs * Hkv * s.row_chunks;
  s.waves = beam::kDecodeWaves;
  if (s.num_splits == 1 && s.rows_per_chunk == 16 && wgs >= 16 && wgs <= device_cu_count())
    s.waves = beam::kDecodeWideWaves;
  return s;
}

size_t decode_workspace_bytes(const beam::DecodeSplit& s, int32_t num_seqs, int32_t max_q_len,
                              int32_t Hq) {
  if (s.num_splits <= 1) return 0;
  return (size_t)s.num_splits * (size_t)num_seqs * (size_t)max_q_len * (size_t)Hq *
         (size_t)(beam::kHeadDim + 2) * sizeof(float);
}

beam_status check_layer(const beam_layer_desc* L, beam::LayerParams* out) {
  if (!L) return fail(BEAM_ERR_INVALID_ARG, "layer descriptor is NULL");
  if (L->head_dim != beam::kHeadDim)
    return fail(BEAM_ERR_INVALID_ARG, "head_dim must be 128 (got %d)", L->head_dim);
  if (L->page_size != beam::kPage)
    return fail(BEAM_ERR_INVALID_ARG, "page_size must be 64 (got %d)", L->page_size);
  if (L->num_q_heads <= 0 || L->num_kv_heads <= 0 || L->num_q_heads % L->num_kv_heads != 0)
    return fail(BEAM_ERR_INVALID_ARG, "num_q_heads (%d) must be a positive multiple of num_kv_heads (%d)",
                L->num_q_heads, L->num_kv_heads);
  const int32_t G = L->num_q_heads / L->num_kv_heads;
  if (G > 16) return fail(BEAM_ERR_INVALID_ARG, "at most 16 query heads per KV head (got %d)", G);
  if (L->kind != BEAM_LAYER_SWA && L->kind != BEAM_LAYER_FULL)
    return fail(BEAM_ERR_INVALID_ARG, "unknown layer kind %d", L->kind);
  if (L->kind == BEAM_LAYER_SWA && L->window < 1)
    return fail(BEAM_ERR_INVALID_ARG, "sliding window must be >= 1 (got %d)", L->window);
  if (!(std::isfinite(L->sm_scale) && L->sm_scale > 0.f))
    return fail(BEAM_ERR_INVALID_ARG, "sm_scale must be finite and > 0");
  if (!(std::isfinite(L->rms_eps) && L->rms_eps >= 0.f))
    return fail(BEAM_ERR_INVALID_ARG, "rms_eps must be finite and >= 0");
  if (L->kind == BEAM_LAYER_SWA && !(std::isfinite(L->rope_theta) && L->rope_theta > 1.f))
    return fail(BEAM_ERR_INVALID_ARG, "rope_theta must be finite and > 1");
  if (L->kind == BEAM_LAYER_FULL &&
      !(std::isfinite(L->ssmax_base) && L->ssmax_base > 0.f && std::isfinite(L->ssmax_exponent)))
    return fail(BEAM_ERR_INVALID_ARG, "ssmax_base must be finite and > 0, ssmax_exponent finite");
  *out = beam::LayerParams{L->num_q_heads, L->num_kv_heads, G, L->kind,
                           L->kind == BEAM_LAYER_SWA ? L->window : 0, L->rope_theta, L->rms_eps,
                           L->ssmax_base, L->ssmax_exponent, L->sm_scale};
  return BEAM_OK;
}

beam_status check_batch(const beam_batch* B, beam::BatchParams* out) {
  if (!B) return fail(BEAM_ERR_INVALID_ARG, "batch is NULL");
  if (B->num_seqs < 0 || B->num_seqs > 65535)
    return fail(BEAM_ERR_INVALID_ARG, "num_seqs must be in [0, 65535] (got %d)", B->num_seqs);
  if (B->num_tokens < 0 || B->max_q_len < 0 || B->max_kv_len < 0 || B->max_pages < 0)
    return fail(BEAM_ERR_INVALID_ARG, "negative batch bound");
  if (B->num_tokens > (int64_t)B->num_seqs * B->max_q_len)
    return fail(BEAM_ERR_INVALID_ARG, "num_tokens (%lld) exceeds num_seqs * max_q_len",
                (long long)B->num_tokens);
  if (B->num_tokens > 0x7FFFFFFF) return fail(BEAM_ERR_INVALID_ARG, "num_tokens too large");
  if (B->max_q_len > B->max_kv_len)
    return fail(BEAM_ERR_INVALID_ARG, "max_q_len exceeds max_kv_len");
  if (B->max_kv_len > 0x7FFFFFFF)
    return fail(BEAM_ERR_INVALID_ARG, "max_kv_len must fit in int32 (kv_len entries are int32)");
  if ((int64_t)B->max_pages * beam::kPage < B->max_kv_len)
    return fail(BEAM_ERR_INVALID_ARG, "max_pages (%d) * 64 < max_kv_len (%lld)", B->max_pages,
                (long long)B->max_kv_len);
  if (B->num_seqs > 0 && (!B->q_start || !B->kv_len || !B->block_table))
    return fail(BEAM_ERR_INVALID_ARG, "q_start, kv_len and block_table must be non-NULL");
  *out = beam::BatchParams{B->num_seqs, B->q_start, B->kv_len, B->block_table,
                           B->max_pages, B->max_q_len, B->max_kv_len, B->num_tokens};
  return BEAM_OK;
}

beam_status check_cache(const beam_kv_cache* C, beam::CacheParams* out) {
  if (!C) return fail(BEAM_ERR_INVALID_ARG, "cache is NULL");
  if (!C->k || !C->v) return fail(BEAM_ERR_INVALID_ARG, "cache k/v pointers must be non-NULL");
  if (!aligned16(C->k) || !aligned16(C->v))
    return fail(BEAM_ERR_INVALID_ARG, "cache k/v must be 16-byte aligned");
  if (C->num_pages <= 0) return fail(BEAM_ERR_INVALID_ARG, "cache num_pages must be > 0");
  if (C->dtype != BEAM_KV_BF16 && C->dtype != BEAM_KV_FP8_E4M3)
    return fail(BEAM_ERR_INVALID_ARG, "unknown cache dtype %d", C->dtype);
  if (C->dtype == BEAM_KV_FP8_E4M3 &&
      !(std::isfinite(C->k_scale) && C->k_scale > 0.f && std::isfinite(C->v_scale) && C->v_scale > 0.f))
    return fail(BEAM_ERR_INVALID_ARG, "fp8 cache scales must be finite and > 0");
  *out = beam::CacheParams{C->k, C->v, C->num_pages, C->dtype, C->k_scale, C->v_scale};
  return BEAM_OK;
}

// Largest token stride (elements) of q, gate and out for prefill.
constexpr int64_t kMaxRowStride = 4194303;

beam_status check_tensor(const char* name, const void* p, int64_t stride, int64_t min_stride,
                         int64_t num_tokens) {
  if (num_tokens == 0) return BEAM_OK;
  if (!p) return fail(BEAM_ERR_INVALID_ARG, "%s is NULL", name);
  if (!aligned16(p)) return fail(BEAM_ERR_INVALID_ARG, "%s must be 16-byte aligned", name);
  if (stride < min_stride || stride % 8 != 0)
    return fail(BEAM_ERR_INVALID_ARG, "%s token stride %lld must be >= %lld and a multiple of 8",
                name, (long long)stride, (long long)min_stride);
  return BEAM_OK;
}

beam_status check_gate(const void* gate, int64_t gate_stride, const void* bias, int32_t Hq,
                       int64_t num_tokens) {
  if (!gate) return BEAM_OK;
  beam_status s = check_tensor("gate", gate, gate_stride, (int64_t)Hq * beam::kHeadDim, num_tokens);
  if (s != BEAM_OK) return s;
  if (!bias) return fail(BEAM_ERR_INVALID_ARG, "gate_bias is NULL while gate is given");
  return BEAM_OK;
}

beam_status launched(hipError_t e) {
  if (e != hipSuccess) return fail(BEAM_ERR_HIP, "HIP launch failed: %s", hipGetErrorString(e));
  return ok();
}

#ifdef BEAMATTN_DEBUG
// Debug builds only: check the device-resident batch metadata against the beam_batch
// rules before any kernel reads it. Allocates a 4-byte result, synchronises the stream
// and frees it, so it is neither allocation-free nor usable under graph capture.
beam_status debug_check_batch(const beam::LayerParams& L, const beam::BatchParams& B,
                              int64_t num_pages, hipStream_t stream) {
  if (B.num_seqs == 0) return BEAM_OK;
  int* err = nullptr;
  if (hipMalloc(&err, sizeof(int)) != hipSuccess)
    return fail(BEAM_ERR_HIP, "batch check: hipMalloc failed");
  int h = 0;
  hipError_t e = hipMemsetAsync(err, 0, sizeof(int), stream);
  if (e == hipSuccess) e = beam::launch_validate_batch(L, B, num_pages, err, stream);
  if (e == hipSuccess) e = hipMemcpyAsync(&h, err, sizeof(int), hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  hipFree(err);
  if (e != hipSuccess) return fail(BEAM_ERR_HIP, "batch check: %s", hipGetErrorString(e));
  if (h == 0) return BEAM_OK;
  static const char* const what[] = {
      "", "q_start[0] is not 0", "q_start decreases", "q_start[num_seqs] exceeds num_tokens",
      "new tokens exceed max_q_len", "kv_len is below the sequence's new tokens",
      "kv_len exceeds max_kv_len", "a block_table entry the call reads is outside [0, num_pages)"};
  const int code = h / 65536, seq = h % 65536;
  return fail(BEAM_ERR_INVALID_ARG, "batch metadata: %s (sequence %d)",
              code >= 1 && code <= 7 ? what[code] : "unknown rule", seq);
}
#define BEAM_DEBUG_CHECK_BATCH(L, B, C, stream)                                                  \
  do {                                                                                          \
    beam_status ds_ = debug_check_batch(L, B, (C).num_pages, static_cast<hipStream_t>(stream)); \
    if (ds_ != BEAM_OK) return ds_;                                                             \
  } while (0)
#else
#define BEAM_DEBUG_CHECK_BATCH(L, B, C, stream) \
  do {                                          \
  } while (0)
#endif

// ---- scratch of the allocation-free decode entry point. The split partials go into this
// file-scope device array instead of a caller workspace; every device the library runs on
// holds its own copy for the life of the process. In host code `scratch` names only a
// host-side stand-in symbol: its device address on the current device comes from
// hipGetSymbolAddress, taken once per device and kept in g_scratch_addr.
constexpr size_t kNoAllocScratchBytes = BEAM_DECODE_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices] = {};

beam_status scratch_on_current_device(void** addr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(BEAM_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(BEAM_ERR_UNSUPPORTED, "device index %d is beyond the %d this library tracks", dev,
                kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(BEAM_ERR_HIP, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev,
                  hipGetErrorString(e));
    g_scratch_addr[dev] = p;
  }
  *addr = g_scratch_addr[dev];
  return BEAM_OK;
}

bool ranges_overlap(const void* a, int64_t a_bytes, const void* b, int64_t b_bytes) {
  const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
  return pa < pb + (uintptr_t)b_bytes && pb < pa + (uintptr_t)a_bytes;
}

}  // namespace

extern "C" {

beam_status beam_qknorm_rope_ssmax_kvwrite(const beam_layer_desc* layer, const beam_batch* batch,
                                           const beam_kv_cache* cache, const void* q,
                                           int64_t q_stride, const void* k, int64_t k_stride,
                                           const void* v, int64_t v_stride, const void* q_norm_w,
                                           const void* k_norm_w, int64_t norm_w_head_stride,
                                           void* q_out, int64_t q_out_stride, void* stream) {
  beam::LayerParams L;
  beam::BatchParams B;
  beam::CacheParams C;
  beam_status s;
  if ((s = check_layer(layer, &L)) != BEAM_OK) return s;
  if ((s = check_batch(batch, &B)) != BEAM_OK) return s;
  if ((s = check_cache(cache, &C)) != BEAM_OK) return s;
  const int64_t N = B.num_tokens;
  if ((s = check_tensor("q", q, q_stride, (int64_t)L.Hq * beam::kHeadDim, N)) != BEAM_OK) return s;
  if ((s = check_tensor("k", k, k_stride, (int64_t)L.Hkv * beam::kHeadDim, N)) != BEAM_OK) return s;
  if ((s = check_tensor("v", v, v_stride, (int64_t)L.Hkv * beam::kHeadDim, N)) != BEAM_OK) return s;
  if ((s = check_tensor("q_out", q_out, q_out_stride, (int64_t)L.Hq * beam::kHeadDim, N)) != BEAM_OK) return s;
  if (N > 0) {
    if (!q_norm_w || !k_norm_w || !aligned16(q_norm_w) || !aligned16(k_norm_w))
      return fail(BEAM_ERR_INVALID_ARG, "norm weights must be non-NULL and 16-byte aligned");
    if (norm_w_head_stride != 0 && (norm_w_head_stride < beam::kHeadDim || norm_w_head_stride % 8 != 0))
      return fail(BEAM_ERR_INVALID_ARG, "norm_w_head_stride must be 0 or >= 128 and a multiple of 8");
    if (q_out != q) {
      const int64_t qb = ((N - 1) * q_stride + (int64_t)L.Hq * beam::kHeadDim) * 2;
      const int64_t ob = ((N - 1) * q_out_stride + (int64_t)L.Hq * beam::kHeadDim) * 2;
      if (ranges_overlap(q, qb, q_out, ob))
        return fail(BEAM_ERR_INVALID_ARG, "q_out overlaps q without being the same buffer");
    } else if (q_out_stride != q_stride) {
      return fail(BEAM_ERR_INVALID_ARG, "in-place q_out needs q_out_stride == q_stride");
    }
  }
  BEAM_DEBUG_CHECK_BATCH(L, B, C, stream);
  return launched(beam::launch_qknorm_kvwrite(L, B, C, q, q_stride, k, k_stride, v, v_stride,
                                              q_norm_w, k_norm_w, norm_w_head_stride, q_out,
                                              q_out_stride, static_cast<hipStream_t>(stream)));
}

beam_status beam_attn_prefill(const beam_layer_desc* layer, const beam_batch* batch,
                              const beam_kv_cache* cache, const void* q, int64_t q_stride,
                              const void* gate, int64_t gate_stride, const void* gate_bias,
                              void* out, int64_t out_stride, void* stream) {
  beam::LayerParams L;
  beam::BatchParams B;
  beam::CacheParams C;
  beam_status s;
  if ((s = check_layer(layer, &L)) != BEAM_OK) return s;
  if ((s = check_batch(batch, &B)) != BEAM_OK) return s;
  if ((s = check_cache(cache, &C)) != BEAM_OK) return s;
  const int64_t N = B.num_tokens;
  const int64_t row = (int64_t)L.Hq * beam::kHeadDim;
  if ((s = check_tensor("q", q, q_stride, row, N)) != BEAM_OK) return s;
  if ((s = check_tensor("out", out, out_stride, row, N)) != BEAM_OK) return s;
  if ((s = check_gate(gate, gate_stride, gate_bias, L.Hq, N)) != BEAM_OK) return s;
  if ((int64_t)B.max_q_len * L.G > 0x7FFFFFFF)
    return fail(BEAM_ERR_INVALID_ARG, "max_q_len * query heads per KV head must fit in int32");
  // a row tile's q, gate and out rows move through 32-bit offsets from the tile's first
  // token (at most 255 tokens on)
  if (q_stride > kMaxRowStride || out_stride > kMaxRowStride || (gate != nullptr && gate_stride > kMaxRowStride))
    return fail(BEAM_ERR_INVALID_ARG, "prefill token strides must be at most %lld elements",
                (long long)kMaxRowStride);
  {
    const int64_t rpb = beam::prefill_rows_per_block(L.kind, false);
    const int64_t tiles = ((int64_t)B.max_q_len * L.G + rpb - 1) / rpb;
    if (tiles * L.Hkv * B.num_seqs > 0x3FFFFFFF)
      return fail(BEAM_ERR_INVALID_ARG, "prefill row tiles x KV heads x sequences must be at most 2^30");
  }
  BEAM_DEBUG_CHECK_BATCH(L, B, C, stream);
  return launched(beam::launch_attn_prefill(L, B, C, choose_prefill_split_mode(L, B),
                                            device_cu_count(), q, q_stride, gate, gate_stride,
                                            gate_bias, out, out_stride,
                                            static_cast<hipStream_t>(stream)));
}

size_t beam_attn_decode_workspace_bytes(const beam_layer_desc* layer, int32_t num_seqs,
                                        int32_t max_q_len, int64_t max_kv_len) {
  beam::LayerParams L;
  if (check_layer(layer, &L) != BEAM_OK) return 0;
  if (num_seqs < 0 || max_q_len < 1 || max_q_len > 16 || max_kv_len < max_q_len) return 0;
  if (num_seqs == 0) return 0;   // an empty batch launches nothing
  // the split depends on the cache dtype (resident workgroups per CU): size for either
  size_t need = 0;
  for (int32_t dt : {(int32_t)BEAM_KV_BF16, (int32_t)BEAM_KV_FP8_E4M3}) {
    const beam::DecodeSplit s =
        choose_decode_split(L.G, L.kind, L.window, num_seqs, max_q_len, max_kv_len, L.Hkv, dt);
    const size_t b = decode_workspace_bytes(s, num_seqs, max_q_len, L.Hq);
    if (b > need) need = b;
  }
  return need;
}

}  // extern "C"

namespace {

// Shared body of the two decode entry points. scratch_mode: the partials go to the
// file-scope scratch array (no caller workspace, no allocation, no batch-metadata check
// even in debug builds, since that check allocates).
beam_status attn_decode(const beam_layer_desc* layer, const beam_batch* batch,
                        const beam_kv_cache* cache, const void* q, int64_t q_stride,
                        const void* gate, int64_t gate_stride, const void* gate_bias, void* out,
                        int64_t out_stride, void* workspace, size_t workspace_bytes,
                        bool scratch_mode, void* stream) {
  beam::LayerParams L;
  beam::BatchParams B;
  beam::CacheParams C;
  beam_status s;
  if ((s = check_layer(layer, &L)) != BEAM_OK) return s;
  if ((s = check_batch(batch, &B)) != BEAM_OK) return s;
  if ((s = check_cache(cache, &C)) != BEAM_OK) return s;
  if (B.max_q_len < 1 || B.max_q_len > 16)
    return fail(BEAM_ERR_INVALID_ARG, "decode needs max_q_len in 1..16 (got %d)", B.max_q_len);
  if (B.num_seqs == 0) return ok();   // an empty batch (e.g. every sequence finished)
  const int64_t N = B.num_tokens;
  const int64_t row = (int64_t)L.Hq * beam::kHeadDim;
  if ((s = check_tensor("q", q, q_stride, row, N)) != BEAM_OK) return s;
  if ((s = check_tensor("out", out, out_stride, row, N)) != BEAM_OK) return s;
  if ((s = check_gate(gate, gate_stride, gate_bias, L.Hq, N)) != BEAM_OK) return s;
  const beam::DecodeSplit S = choose_decode_split(L.G, L.kind, L.window, B.num_seqs, B.max_q_len,
                                                  B.max_kv_len, L.Hkv, C.dtype);
  const size_t need = decode_workspace_bytes(S, B.num_seqs, B.max_q_len, L.Hq);
  if (scratch_mode) {
    workspace = nullptr;
    if (need > kNoAllocScratchBytes)
      return fail(BEAM_ERR_WORKSPACE,
                  "allocation-free decode needs %zu bytes of scratch for these bounds; its "
                  "scratch holds %zu (use beam_attn_decode with a workspace)",
                  need, kNoAllocScratchBytes);
    if (need > 0 && (s = scratch_on_current_device(&workspace)) != BEAM_OK) return s;
  } else {
    if (need > 0) {
      if (!workspace || workspace_bytes < need)
        return fail(BEAM_ERR_WORKSPACE, "decode workspace needs %zu bytes (got %zu%s)", need,
                    workspace_bytes, workspace ? "" : ", NULL pointer");
      if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
        return fail(BEAM_ERR_INVALID_ARG, "decode workspace must be 256-byte aligned");
    }
    BEAM_DEBUG_CHECK_BATCH(L, B, C, stream);
  }
  return launched(beam::launch_attn_decode(L, B, C, S, q, q_stride, gate, gate_stride, gate_bias,
                                           out, out_stride, workspace,
                                           static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

beam_status beam_attn_decode(const beam_layer_desc* layer, const beam_batch* batch,
                             const beam_kv_cache* cache, const void* q, int64_t q_stride,
                             const void* gate, int64_t gate_stride, const void* gate_bias,
                             void* out, int64_t out_stride, void* workspace,
                             size_t workspace_bytes, void* stream) {
  return attn_decode(layer, batch, cache, q, q_stride, gate, gate_stride, gate_bias, out,
                     out_stride, workspace, workspace_bytes, false, stream);
}

beam_status beam_attn_decode_noalloc(const beam_layer_desc* layer, const beam_batch* batch,
                                     const beam_kv_cache* cache, const void* q, int64_t q_stride,
                                     const void* gate, int64_t gate_stride, const void* gate_bias,
                                     void* out, int64_t out_stride, void* stream) {
  return attn_decode(layer, batch, cache, q, q_stride, gate, gate_stride, gate_bias, out,
                     out_stride, nullptr, 0, true, stream);
}

beam_status beam_head_gate(const beam_layer_desc* layer, int64_t num_tokens, const void* attn,
                           int64_t attn_stride, const void* gate, int64_t gate_stride,
                           const void* gate_bias, void* out, int64_t out_stride, void* stream) {
  beam::LayerParams L;
  beam_status s;
  if ((s = check_layer(layer, &L)) != BEAM_OK) return s;
  if (num_tokens < 0) return fail(BEAM_ERR_INVALID_ARG, "num_tokens must be >= 0");
  const int64_t row = (int64_t)L.Hq * beam::kHeadDim;
  if ((s = check_tensor("attn", attn, attn_stride, row, num_tokens)) != BEAM_OK) return s;
  if ((s = check_tensor("out", out, out_stride, row, num_tokens)) != BEAM_OK) return s;
  if (num_tokens > 0 && !gate) return fail(BEAM_ERR_INVALID_ARG, "gate is NULL");
  if ((s = check_gate(gate, gate_stride, gate_bias, L.Hq, num_tokens)) != BEAM_OK) return s;
  if (out != attn && num_tokens > 0) {
    const int64_t ab = ((num_tokens - 1) * attn_stride + row) * 2;
    const int64_t ob = ((num_tokens - 1) * out_stride + row) * 2;
    if (ranges_overlap(attn, ab, out, ob))
      return fail(BEAM_ERR_INVALID_ARG, "out overlaps attn without being the same buffer");
  } else if (out == attn && attn_stride != out_stride) {
    return fail(BEAM_ERR_INVALID_ARG, "in-place gate needs out_stride == attn_stride");
  }
  return launched(beam::launch_head_gate(L, num_tokens, attn, attn_stride, gate, gate_stride,
                                         gate_bias, out, out_stride,
                                         static_cast<hipStream_t>(stream)));
}

beam_status beam_linear_bf16(int64_t m, int64_t n, int64_t k, const void* x, int64_t x_stride,
                             const void* w, int64_t w_stride, void* y, int64_t y_stride,
                             void* stream) {
  if (m < 0 || n <= 0 || k <= 0) return fail(BEAM_ERR_INVALID_ARG, "linear needs m >= 0, n > 0, k > 0");
  if (k % 64 != 0) return fail(BEAM_ERR_INVALID_ARG, "linear k (%lld) must be a multiple of 64", (long long)k);
  if (n % 4 != 0) return fail(BEAM_ERR_INVALID_ARG, "linear n (%lld) must be a multiple of 4", (long long)n);
  if (m > 0x7FFFFFFFLL || n > 0x7FFFFFFFLL || k > 0x7FFFFFFFLL)
    return fail(BEAM_ERR_INVALID_ARG, "linear dimensions must fit in 31 bits");
  beam_status s;
  if ((s = check_tensor("x", x, x_stride, k, m)) != BEAM_OK) return s;
  if ((s = check_tensor("w", w, w_stride, k, n)) != BEAM_OK) return s;
  // the kernel reads a 256-row tile of x or w through 32-bit byte offsets
  if (x_stride > (int64_t)0x7FFFFFFF / 512 || w_stride > (int64_t)0x7FFFFFFF / 512)
    return fail(BEAM_ERR_INVALID_ARG, "linear x and w row strides must be at most %lld elements",
                (long long)((int64_t)0x7FFFFFFF / 512));
  if ((s = check_tensor("y", y, y_stride, n, m)) != BEAM_OK) return s;
  if (m > 0) {
    const int64_t xb = ((m - 1) * x_stride + k) * 2, wb = ((n - 1) * w_stride + k) * 2,
                  yb = ((m - 1) * y_stride + n) * 2;
    if (ranges_overlap(y, yb, x, xb) || ranges_overlap(y, yb, w, wb))
      return fail(BEAM_ERR_INVALID_ARG, "linear y must not overlap x or w");
  }
  return launched(beam::launch_linear_bf16(m, n, k, x, x_stride, w, w_stride, y, y_stride,
                                           static_cast<hipStream_t>(stream)));
}

uint64_t beam_kv_bytes_per_token(int32_t num_full_layers, int32_t num_kv_heads, int32_t head_dim,
                                 int32_t dtype) {
  if (num_full_layers < 0 || num_kv_heads < 0 || head_dim < 0) return 0;
  uint64_t bytes;
  if (dtype == BEAM_KV_BF16) bytes = 2;
  else if (dtype == BEAM_KV_FP8_E4M3) bytes = 1;
  else return 0;
  return (uint64_t)num_full_layers * 2u * (uint64_t)num_kv_heads * (uint64_t)head_dim * bytes;
}

const char* beam_status_string(beam_status status) {
  switch (status) {
    case BEAM_OK: return "ok";
    case BEAM_ERR_INVALID_ARG: return "invalid argument";
    case BEAM_ERR_UNSUPPORTED: return "unsupported";
    case BEAM_ERR_WORKSPACE: return "workspace too small";
    case BEAM_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

const char* beam_last_error(void) { return g_last_error; }

int32_t beam_abi_version(void) { return BEAM_ABI_VERSION; }

}  // extern "C"
