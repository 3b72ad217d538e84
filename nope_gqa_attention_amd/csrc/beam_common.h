// Internal header of libbeamattn: launch parameter blocks passed from the validating C
// ABI layer (api.cpp) to the kernel launchers, plus small device helpers shared by the
// kernels. Everything here targets gfx950 (CDNA4, wave64) only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "beamattn.h"

namespace beam {

constexpr int kHeadDim = 128;
constexpr int kPage = 64;

// ---------------------------------------------------------------- launch parameters

struct LayerParams {
  int32_t Hq, Hkv, G;          // query heads, KV heads, query heads per KV head
  int32_t kind;                // beam_layer_kind
  int32_t window;              // sliding-window length in keys (own key included)
  float rope_theta, rms_eps, ssmax_base, ssmax_exponent, sm_scale;
};

struct BatchParams {
  int32_t num_seqs;
  const int32_t* q_start;
  const int32_t* kv_len;
  const int32_t* block_table;
  int32_t max_pages;
  int32_t max_q_len;
  int64_t max_kv_len;
  int64_t num_tokens;
};

struct CacheParams {
  void* k;
  void* v;
  int64_t num_pages;
  int32_t dtype;               // beam_kv_dtype
  float k_scale, v_scale;
};

// Decode split geometry, chosen on the host from the batch bounds (the same function
// sizes the workspace).
struct DecodeSplit {
  int32_t num_splits;          // splits per (sequence, KV head, row chunk)
  int32_t keys_per_split;      // multiple of kDecodeKeysPerBlockStep
  int32_t row_chunks;          // ceil(G * max_q_len / kDecodeRowsPerChunk)
  int32_t rows_per_chunk;      // 16, 32 or 48 (a multiple of 16)
  int32_t waves;               // waves per workgroup: kDecodeWaves, or kDecodeWideWaves
};

constexpr int kDecodeWaves = 4;                       // waves per decode workgroup
// Waves per workgroup of a latency-bound single-split launch (one 16-row block): one
// workgroup per CU, 3 waves per SIMD, each wave streaming about one page.
constexpr int kDecodeWideWaves = 12;
constexpr int kDecodeKeysPerBlockStep = kDecodeWaves * kPage;  // one page per wave per step
constexpr int kDecodeMaxRowsPerChunk = 48;
constexpr int kDecodeMaxSplits = 2048;                // bound of the merge kernel's weight table
// Decode split-kernel workgroups (of 4 waves) resident per CU that its register and LDS
// budgets are built for, i.e. waves per SIMD: 2. Each wave streams with its next
// half-step's loads in flight, and stages K and V rows in 17 KiB of LDS (70 KiB per
// workgroup), which admits 2 workgroups per CU.
constexpr int decode_wgs_per_cu(int row_blocks, int kv_dtype) {
  return (void)row_blocks, (void)kv_dtype, 2;
}

hipError_t launch_qknorm_kvwrite(const LayerParams& L, const BatchParams& B, const CacheParams& C,
                                 const void* q, int64_t q_stride, const void* k, int64_t k_stride,
                                 const void* v, int64_t v_stride, const void* q_norm_w,
                                 const void* k_norm_w, int64_t norm_w_head_stride, void* q_out,
                                 int64_t q_out_stride, hipStream_t stream);

hipError_t launch_linear_bf16(int64_t M, int64_t N, int64_t K, const void* x, int64_t x_stride,
                              const void* w, int64_t w_stride, void* y, int64_t y_stride,
                              hipStream_t stream);

// Batch-metadata check (BEAMATTN_DEBUG builds): *err (device, zeroed by the caller) gets
// code * 65536 + sequence of the first rule found broken, or stays 0.
enum BatchError {
  kBadQStart0 = 1,    // q_start[0] != 0
  kBadQOrder = 2,     // q_start decreases
  kBadTokens = 3,     // q_start[num_seqs] > num_tokens
  kBadQLen = 4,       // n_b > max_q_len
  kBadKvShort = 5,    // kv_len[b] < n_b
  kBadKvLong = 6,     // kv_len[b] > max_kv_len
  kBadPage = 7,       // a block-table entry the call touches is outside [0, num_pages)
};
hipError_t launch_validate_batch(const LayerParams& L, const BatchParams& B, int64_t num_pages,
                                 int* err, hipStream_t stream);

hipError_t launch_head_gate(const LayerParams& L, int64_t num_tokens, const void* attn,
                            int64_t attn_stride, const void* gate, int64_t gate_stride,
                            const void* gate_bias, void* out, int64_t out_stride,
                            hipStream_t stream);

hipError_t launch_attn_decode(const LayerParams& L, const BatchParams& B, const CacheParams& C,
                              const DecodeSplit& S, const void* q, int64_t q_stride,
                              const void* gate, int64_t gate_stride, const void* gate_bias,
                              void* out, int64_t out_stride, void* workspace, hipStream_t stream);

// Prefill workgroups: 8 waves for full layers, 4 for sliding ones, one 32-row block per
// wave; with the key split (full layers only) the 8 waves form two 4-wave streams over
// the same 128 rows, each walking half of the key tiles.
constexpr int prefill_waves(int kind) { return kind == BEAM_LAYER_SWA ? 4 : 8; }
constexpr int prefill_rows_per_block(int kind, bool key_split) {
  return 32 * (kind == BEAM_LAYER_SWA ? 4 : (key_split ? 4 : 8));
}

// split_mode: 0 no key split, 1 every row tile split, 2 as many row tiles of an XCD's last
// round as it leaves CUs idle (full layers; sliding ones never split); cus: the device's
// compute units.
hipError_t launch_attn_prefill(const LayerParams& L, const BatchParams& B, const CacheParams& C,
                               int split_mode, int cus, const void* q, int64_t q_stride,
                               const void* gate, int64_t gate_stride, const void* gate_bias,
                               void* out, int64_t out_stride, hipStream_t stream);

// ---------------------------------------------------------------- device helpers

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4_t;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2_t;

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Two floats -> two bf16 (round to nearest even, NaN stays NaN), packed low/high.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t r;
  r[0] = (__bf16)lo;
  r[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ uint32_t bf16_bits_rne(float f) {
  return pack_bf16x2(f, 0.0f) & 0xFFFFu;
}

// OCP E4M3FN encode with saturation: |x| >= 448 -> +-448, NaN -> 0x7F, otherwise the
// nearest representable value. Written from the format: 4 exponent bits with bias 7
// (normals 2^-6 .. 2^8), 3 mantissa bits, subnormals M * 2^-9. x is a rounded stand-in
// for an exact value; `dir` says where that exact value lies when x sits exactly on a
// midpoint between two codes: > 0 beyond |x| (round the magnitude up), < 0 short of it
// (round down), 0 on it (ties to the even mantissa).
__device__ __forceinline__ uint32_t f32_to_e4m3_sat(float x, int dir = 0) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return 0x7Fu;                  // NaN
  if (a >= 0x43E00000u) return sign | 0x7Eu;          // >= 448 (incl. inf) saturates
  const int e = (int)(a >> 23) - 127;
  if (e >= -6) {                                       // normal range of e4m3
    uint32_t q = (a >> 20) & 7u;                       // top 3 mantissa bits
    const uint32_t rem = a & 0xFFFFFu;
    const uint32_t up = (rem > 0x80000u) ||
                        (rem == 0x80000u && (dir > 0 || (dir == 0 && (q & 1u))));
    uint32_t code = ((uint32_t)(e + 7) << 3) + q + up;   // carry into exponent is exact
    return sign | code;
  }
  // subnormal: value / 2^-9 rounded to an integer; 8 becomes 2^-6 (0x08)
  const float t = __uint_as_float(a) * 512.0f;         // exact power-of-two scaling
  const float fl = __builtin_floorf(t);
  uint32_t m;
  if (t - fl == 0.5f && dir != 0) m = (uint32_t)fl + (dir > 0 ? 1u : 0u);
  else m = (uint32_t)__builtin_rintf(t);                // ties to even
  return sign | m;
}

// e4m3 code of the exact quotient x / scale (scale finite and > 0), i.e. the nearest
// code to the real number x / scale, not to its binary32 rounding. The binary32
// quotient q keeps the exact quotient's side of every e4m3 midpoint (midpoints are
// binary32 numbers, and rounding is monotone), but it can land on one. The remainder
// x - q * scale is exact in binary32 (one fma, q correctly rounded) and its sign says
// on which side of q the exact quotient lies, which settles such a landing.
__device__ __forceinline__ uint32_t e4m3_of_quotient(float x, float scale) {
  const float q = x / scale;                 // correctly rounded (IEEE division)
  const float r = __builtin_fmaf(-q, scale, x);
  const int dir = (r == 0.0f || q == 0.0f) ? 0 : (((r > 0.0f) == (q > 0.0f)) ? 1 : -1);
  return f32_to_e4m3_sat(q, dir);
}

// Output gate sigmoid(x) = 1 / (1 + 2^(-x log2(e))) through the hardware exp2 and
// reciprocal, each within about one binary32 ulp: a relative error of a few 1e-7, far
// below the bf16 rounding of the gated output. x -> -inf: 2^+big = inf and 1/inf = 0, so
// a closed gate gives exactly 0; x -> +inf: exactly 1.
__device__ __forceinline__ float gate_sigmoid(float x) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(x * -1.4426950408889634f));
}

// Wave-wide helpers (wave64).
// 8 OCP e4m3 codes (two little-endian words) -> 8 bf16 values; exact (every e4m3 value
// is a bf16 value), scale 1.
__device__ __forceinline__ bf16x8_t fp8x8_to_bf16x8(uint32_t w0, uint32_t w1) {
  const bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false);
  const bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true);
  const bf16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false);
  const bf16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true);
  bf16x8_t r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}

__device__ __forceinline__ float wave_xor_max(float v, int mask) {
  return fmaxf(v, __shfl_xor(v, mask, 64));
}

}  // namespace beam
