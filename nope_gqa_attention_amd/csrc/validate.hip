// Device-side check of a batch's metadata (q_start, kv_len, block_table) against the
// beam_batch rules: the entry points run it first in BEAMATTN_DEBUG builds, where a
// malformed batch then returns an error instead of reading or writing out of bounds.
//
// One thread per sequence checks its token range, its key count and every block-table
// entry the call can touch: the pages from the first visible key of its first new token
// (sliding layers: the window start; full layers: key 0) through its last key.
#include "beam_common.h"

namespace beam {
namespace {

__device__ __forceinline__ void report(int* err, int code, int b) {
  atomicCAS(err, 0, code * 65536 + b);           // first error wins
}

__global__ __launch_bounds__(256) void validate_batch_kernel(LayerParams L, BatchParams B,
                                                             int64_t num_pages, int* err) {
  const int b = blockIdx.x * 256 + threadIdx.x;
  if (b >= B.num_seqs) return;
  const int32_t q0 = B.q_start[b], q1 = B.q_start[b + 1];
  if (b == 0 && q0 != 0) { report(err, kBadQStart0, b); return; }
  if (q1 < q0) { report(err, kBadQOrder, b); return; }
  if (b == B.num_seqs - 1 && (int64_t)q1 > B.num_tokens) { report(err, kBadTokens, b); return; }
  const int32_t n = q1 - q0;
  if (n > B.max_q_len) { report(err, kBadQLen, b); return; }
  const int32_t kv = B.kv_len[b];
  if (kv < n) { report(err, kBadKvShort, b); return; }
  if ((int64_t)kv > B.max_kv_len) { report(err, kBadKvLong, b); return; }
  if (kv == 0) return;
  const int32_t first_pos = kv - n;
  int32_t lo = 0;
  if (L.kind == BEAM_LAYER_SWA) lo = first_pos - L.window + 1 > 0 ? first_pos - L.window + 1 : 0;
  const int32_t p_end = (kv + kPage - 1) / kPage;
  const int32_t* row = B.block_table + (int64_t)b * B.max_pages;
  for (int32_t p = lo / kPage; p < p_end; ++p) {
    const int32_t page = row[p];
    if (page < 0 || (int64_t)page >= num_pages) { report(err, kBadPage, b); return; }
  }
}

}  // namespace

hipError_t launch_validate_batch(const LayerParams& L, const BatchParams& B, int64_t num_pages,
                                 int* err, hipStream_t stream) {
  if (B.num_seqs == 0) return hipSuccess;
  hipLaunchKernelGGL(validate_batch_kernel, dim3((unsigned)((B.num_seqs + 255) / 256)), dim3(256), 0,
                     stream, L, B, num_pages, err);
  return hipGetLastError();
}

}  // namespace beam
