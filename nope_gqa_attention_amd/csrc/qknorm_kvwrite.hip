// Fused per-head Q/K RMSNorm + RoPE (sliding layers) or SSMax query scaling (full NoPE
// layers) + bf16 rounding + paged K/V store.
//
// What it computes: "Reflection Beam 1.0 on vLLM", section "Attention: sliding-window
// layers plus NoPE full-attention layers" (per-head Q/K RMS normalisation before RoPE or
// SSMax; SSMax multiplies each query by (1 + p/2048)^0.1, p 1-based), and the same
// page's "Agent-driven optimization" list, changes 2 and 6 (norm + RoPE/SSMax in one
// kernel that also writes K and V into the cache). Slot translation follows "SGLang
// natively supports Reflection's Beam", section "Unified memory for target and draft
// KV": writes go through the same virtual -> physical page contract as reads.
//
// Work decomposition: one 256-thread workgroup per new token. The token's
// Hq + 2*Hkv head vectors (q heads, k heads, v heads) are handled 16 at a time: 16
// lanes per head, 8 consecutive values (one 16-byte load) per lane. The RMS reduction
// is a 16-lane butterfly; rotate-half pairs value i with value i+64, i.e. lane j with
// lane j^8 of the same head. Angles are formed in fp64 (positions reach 2^20, where an
// fp32 angle would be off by up to 0.06 rad), reduced mod 2*pi, and their cos/sin
// shared through LDS; norm, rotation and scaling are fp32; one bf16 rounding at the end.
#include "beam_common.h"

namespace beam {
namespace {

constexpr int kThreads = 256;
constexpr int kLanesPerHead = 16;
constexpr int kHeadsPerPass = kThreads / kLanesPerHead;   // 16

template <int KV_DTYPE>
__global__ __launch_bounds__(kThreads) void qknorm_kvwrite_kernel(
    LayerParams L, BatchParams B, CacheParams C, const uint16_t* __restrict__ q, int64_t q_stride,
    const uint16_t* __restrict__ k, int64_t k_stride, const uint16_t* __restrict__ v,
    int64_t v_stride, const uint16_t* __restrict__ q_norm_w, const uint16_t* __restrict__ k_norm_w,
    int64_t norm_w_head_stride, uint16_t* q_out, int64_t q_out_stride) {
  __shared__ float s_cos[kHeadDim / 2];
  __shared__ float s_sin[kHeadDim / 2];
  __shared__ float s_qscale;

  const int64_t t = blockIdx.x;                 // token index in call order
  const int tid = threadIdx.x;
  if (t >= B.q_start[B.num_seqs]) return;       // padding row past the last sequence

  // sequence of token t: last b with q_start[b] <= t (q_start non-decreasing)
  int lo = 0, hi = B.num_seqs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if ((int64_t)B.q_start[mid] <= t) lo = mid; else hi = mid - 1;
  }
  const int b = lo;
  const int64_t n_b = (int64_t)B.q_start[b + 1] - B.q_start[b];
  const int64_t pos = (int64_t)B.kv_len[b] - n_b + (t - B.q_start[b]);
  const int64_t page = B.block_table[(int64_t)b * B.max_pages + pos / kPage];
  const int slot = (int)(pos % kPage);

  const bool swa = (L.kind == BEAM_LAYER_SWA);
  if (swa && tid < kHeadDim / 2) {
    // angle of pair i at this position, exactly as far as fp64 allows
    const double inv_freq = exp2(-(2.0 * tid / kHeadDim) * log2((double)L.rope_theta));
    const double ang = (double)pos * inv_freq;
    const double two_pi = 6.283185307179586476925286766559;
    const double r = ang - two_pi * rint(ang / two_pi);
    double sd, cd;
    sincos(r, &sd, &cd);
    s_cos[tid] = (float)cd;
    s_sin[tid] = (float)sd;
  }
  // SSMax scale (1 + p/base)^exponent, p = pos + 1, formed once per token in fp64 and
  // used in fp32
  if (!swa && tid == 0)
    s_qscale = (float)pow(1.0 + (double)(pos + 1) / (double)L.ssmax_base, (double)L.ssmax_exponent);
  __syncthreads();
  const float q_scale = swa ? 1.0f : s_qscale;

  const int lane16 = tid % kLanesPerHead;       // which 8 values of the head
  const int head_slot = tid / kLanesPerHead;    // 0..15
  const int total_heads = L.Hq + 2 * L.Hkv;
  const int64_t kv_elem_base = (page * L.Hkv) * (int64_t)kPage * kHeadDim + (int64_t)slot * kHeadDim;

  for (int hh = head_slot; hh < total_heads; hh += kHeadsPerPass) {
    const bool is_q = hh < L.Hq;
    const bool is_k = !is_q && hh < L.Hq + L.Hkv;
    const int head = is_q ? hh : (is_k ? hh - L.Hq : hh - L.Hq - L.Hkv);
    const uint16_t* src = is_q ? q + t * q_stride + (int64_t)head * kHeadDim
                        : is_k ? k + t * k_stride + (int64_t)head * kHeadDim
                               : v + t * v_stride + (int64_t)head * kHeadDim;
    const u32x4_t raw = *reinterpret_cast<const u32x4_t*>(src + lane16 * 8);
    float x[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[2 * j] = bf16_to_f32(raw[j] & 0xFFFFu);
      x[2 * j + 1] = bf16_to_f32(raw[j] >> 16);
    }
    uint32_t out_bits[4];
    if (is_q || is_k) {
      float ss = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) ss = fmaf(x[j], x[j], ss);
      ss += __shfl_xor(ss, 1, 64);
      ss += __shfl_xor(ss, 2, 64);
      ss += __shfl_xor(ss, 4, 64);
      ss += __shfl_xor(ss, 8, 64);
      const float rs = 1.0f / sqrtf(ss * (1.0f / kHeadDim) + L.rms_eps);
      const uint16_t* w = (is_q ? q_norm_w : k_norm_w) + (int64_t)head * norm_w_head_stride;
      const u32x4_t wraw = *reinterpret_cast<const u32x4_t*>(w + lane16 * 8);
      float y[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        y[2 * j] = bf16_to_f32(wraw[j] & 0xFFFFu) * (x[2 * j] * rs);
        y[2 * j + 1] = bf16_to_f32(wraw[j] >> 16) * (x[2 * j + 1] * rs);
      }
      if (swa) {
        // partner lane holds the other half of each rotation pair
        float p[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) p[j] = __shfl_xor(y[j], 8, 64);
        const bool first_half = lane16 < 8;
        const int i0 = (lane16 & 7) * 8;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float c = s_cos[i0 + j], s = s_sin[i0 + j];
          // first half: y_i c - y_{i+64} s ; second half: y_{i+64} c + y_i s
          y[j] = first_half ? fmaf(y[j], c, -p[j] * s) : fmaf(y[j], c, p[j] * s);
        }
      } else if (is_q) {
#pragma unroll
        for (int j = 0; j < 8; ++j) y[j] *= q_scale;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) out_bits[j] = pack_bf16x2(y[2 * j], y[2 * j + 1]);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) out_bits[j] = raw[j];
    }

    if (is_q) {
      u32x4_t o = {out_bits[0], out_bits[1], out_bits[2], out_bits[3]};
      *reinterpret_cast<u32x4_t*>(q_out + t * q_out_stride + (int64_t)head * kHeadDim + lane16 * 8) = o;
    } else {
      const int64_t off = kv_elem_base + (int64_t)head * kPage * kHeadDim + lane16 * 8;
      if (KV_DTYPE == BEAM_KV_BF16) {
        uint16_t* dst = static_cast<uint16_t*>(is_k ? C.k : C.v);
        u32x4_t o = {out_bits[0], out_bits[1], out_bits[2], out_bits[3]};
        *reinterpret_cast<u32x4_t*>(dst + off) = o;
      } else {
        // the stored value is the bf16-rounded one over the tensor scale: the code of the
        // exact quotient
        const float scale = is_k ? C.k_scale : C.v_scale;
        uint32_t codes[2] = {0u, 0u};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint32_t h16 = (out_bits[j / 2] >> (16 * (j % 2))) & 0xFFFFu;
          const uint32_t c = e4m3_of_quotient(bf16_to_f32(h16), scale);
          codes[j / 4] |= c << (8 * (j % 4));
        }
        uint8_t* dst = static_cast<uint8_t*>(is_k ? C.k : C.v);
        u32x2_t o = {codes[0], codes[1]};
        *reinterpret_cast<u32x2_t*>(dst + off) = o;
      }
    }
  }
}

}  // namespace

hipError_t launch_qknorm_kvwrite(const LayerParams& L, const BatchParams& B, const CacheParams& C,
                                 const void* q, int64_t q_stride, const void* k, int64_t k_stride,
                                 const void* v, int64_t v_stride, const void* q_norm_w,
                                 const void* k_norm_w, int64_t norm_w_head_stride, void* q_out,
                                 int64_t q_out_stride, hipStream_t stream) {
  if (B.num_tokens == 0) return hipSuccess;
  const dim3 grid((unsigned)B.num_tokens), block(kThreads);
  auto args = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, grid, block, 0, stream, L, B, C, static_cast<const uint16_t*>(q),
                       q_stride, static_cast<const uint16_t*>(k), k_stride,
                       static_cast<const uint16_t*>(v), v_stride,
                       static_cast<const uint16_t*>(q_norm_w),
                       static_cast<const uint16_t*>(k_norm_w), norm_w_head_stride,
                       static_cast<uint16_t*>(q_out), q_out_stride);
  };
  if (C.dtype == BEAM_KV_BF16) args(qknorm_kvwrite_kernel<BEAM_KV_BF16>);
  else args(qknorm_kvwrite_kernel<BEAM_KV_FP8_E4M3>);
  return hipGetLastError();
}

}  // namespace beam
