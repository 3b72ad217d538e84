// Standalone sigmoid output gate: out[t,h,d] = attn[t,h,d] * sigmoid(gate[t,h*D+d] + bias[h]).
//
// What it computes: "Reflection Beam 1.0 on vLLM", section "Attention: sliding-window
// layers plus NoPE full-attention layers" (a per-element sigmoid gate with a bias per
// head, fed by a projection of its own, scales every head's output, which lets a token
// silence a head), and "SGLang natively supports Reflection's Beam", section "Fusion
// optimizations" (the three elementwise steps in one kernel).
// The attention kernels apply the same gate in their epilogues; this entry point serves
// callers that keep attention and gate apart.
//
// HBM-bound elementwise pass: 8 bf16 values (16 bytes) per lane, 6 bytes moved per value.
#include "beam_common.h"

namespace beam {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void head_gate_kernel(
    int32_t Hq, int64_t num_tokens, const uint16_t* __restrict__ attn, int64_t attn_stride,
    const uint16_t* __restrict__ gate, int64_t gate_stride, const uint16_t* __restrict__ bias,
    uint16_t* out, int64_t out_stride) {
  const int64_t vec_per_token = (int64_t)Hq * kHeadDim / 8;
  const int64_t total = num_tokens * vec_per_token;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * kThreads) {
    const int64_t t = i / vec_per_token;
    const int64_t e = (i - t * vec_per_token) * 8;      // element within the token
    const int h = (int)(e / kHeadDim);
    const u32x4_t a = *reinterpret_cast<const u32x4_t*>(attn + t * attn_stride + e);
    const u32x4_t g = *reinterpret_cast<const u32x4_t*>(gate + t * gate_stride + e);
    const float bh = bf16_to_f32(bias[h]);
    u32x4_t o;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float a0 = bf16_to_f32(a[j] & 0xFFFFu), a1 = bf16_to_f32(a[j] >> 16);
      const float g0 = bf16_to_f32(g[j] & 0xFFFFu) + bh, g1 = bf16_to_f32(g[j] >> 16) + bh;
      const float s0 = gate_sigmoid(g0);
      const float s1 = gate_sigmoid(g1);
      o[j] = pack_bf16x2(a0 * s0, a1 * s1);
    }
    *reinterpret_cast<u32x4_t*>(out + t * out_stride + e) = o;
  }
}

}  // namespace

hipError_t launch_head_gate(const LayerParams& L, int64_t num_tokens, const void* attn,
                            int64_t attn_stride, const void* gate, int64_t gate_stride,
                            const void* gate_bias, void* out, int64_t out_stride,
                            hipStream_t stream) {
  if (num_tokens == 0) return hipSuccess;
  const int64_t total = num_tokens * (int64_t)L.Hq * kHeadDim / 8;
  int64_t blocks = (total + kThreads - 1) / kThreads;
  if (blocks > 256 * 64) blocks = 256 * 64;   // grid-stride beyond 64 workgroups per CU
  hipLaunchKernelGGL(head_gate_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, L.Hq,
                     num_tokens, static_cast<const uint16_t*>(attn), attn_stride,
                     static_cast<const uint16_t*>(gate), gate_stride,
                     static_cast<const uint16_t*>(gate_bias), static_cast<uint16_t*>(out),
                     out_stride);
  return hipGetLastError();
}

}  // namespace beam
