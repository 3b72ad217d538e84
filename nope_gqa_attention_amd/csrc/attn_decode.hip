// Decode / speculative-verify attention over a paged bf16 or fp8 KV cache.
//
// What it computes: attention of 1..16 new tokens per sequence over every visible key
// (full NoPE layers: all earlier keys; sliding layers: the most recent `window` keys,
// own key included), GQA with query head h reading KV head h / G, then the sigmoid
// head gate -- "Reflection Beam 1.0 on vLLM", section "Attention: sliding-window layers
// plus NoPE full-attention layers". New tokens of one call form a causal block (the
// target model verifies a drafted block in one forward: "SGLang natively supports
// Reflection's Beam", section on DFlash2 with data-parallel attention). FP8 KV is the
// serving configuration of both pages (kv-cache dtype fp8).
//
// Design (HBM-bound, MI355X):
//  * Grid (split, KV head x row chunk, sequence). A row is one (new token, query head)
//    pair of the KV head's group: G*n_b rows, up to 48 per chunk, all sharing every K/V
//    byte that is read, so each byte of the cache crosses HBM once per layer call.
//  * A workgroup is 4 waves; wave w streams pages w, w+4, ... of its split: a 64-key
//    page of one KV head is one contiguous 16 KiB (bf16) / 8 KiB (fp8) block.
//  * Scores use MFMA 16x16x32 bf16 as S^T = K Q^T: K comes straight from global memory
//    as the A operand (fp8 codes decoded to bf16 exactly in registers; the scale folds
//    into the softmax scale), Q^T stays in registers. Each lane then owns one row's
//    scores for 8 keys, so the online softmax needs only two cross-lane steps.
//  * P V uses O^T = V^T P^T: P^T is the score accumulator re-packed to bf16 in place;
//    V^T comes from a row-major LDS copy of the V rows through the gfx950 transposing
//    LDS read (ds_read_b64_tr_b16), so no register transpose is needed.
//  * The running max is raised only when a row's maximum grows by more than 2^8 (log2
//    domain), so the output rescale is skipped on almost every step.
//  * The 4 waves merge their (max, sum, output) in LDS; splits are merged by
//    log-sum-exp in a second kernel, which also applies the gate; with one split the
//    first kernel writes the gated output itself.
#include "beam_common.h"

namespace beam {
namespace {

constexpr int kThreads = kDecodeWaves * 64;
constexpr int kVRowBytes = kHeadDim * 2 + 16;     // bf16 V row in LDS, padded
constexpr int kVRowsPerWave = 32;                 // keys staged per half-page step
constexpr int kLdsBytes = kDecodeWaves * kVRowsPerWave * kVRowBytes;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescaleSlack = 8.0f;                // log2 headroom before rescaling

// Start of the 8-value slice of head dimension used by MFMA i (0..3) in lane group g
// (lane / 16). bf16: one 16-byte load per MFMA; fp8: one 16-byte load feeds 2 MFMAs.
template <int KV>
__device__ __forceinline__ int dslice(int i, int g) {
  return KV == BEAM_KV_BF16 ? 32 * i + 8 * g : 64 * (i / 2) + 16 * g + 8 * (i % 2);
}


__device__ __forceinline__ int seq_of_token(const int32_t* q_start, int num_seqs, int64_t t) {
  int lo = 0, hi = num_seqs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if ((int64_t)q_start[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// First key of the sequence's visited range, rounded down to a page.
__device__ __forceinline__ int64_t range_base(const LayerParams& L, int64_t kv, int64_t n) {
  const int64_t first_pos = kv - n;
  int64_t lo = 0;
  if (L.kind == BEAM_LAYER_SWA) lo = first_pos - L.window + 1 > 0 ? first_pos - L.window + 1 : 0;
  return (lo / kPage) * kPage;
}

template <int KV, int RB>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(decode_wgs_per_cu(RB)))) void decode_split_kernel(
    LayerParams L, BatchParams B, CacheParams C, DecodeSplit S,
    const uint16_t* __restrict__ q, int64_t q_stride, const uint16_t* __restrict__ gate,
    int64_t gate_stride, const uint16_t* __restrict__ gate_bias, uint16_t* out,
    int64_t out_stride, float* __restrict__ ws_o, float* __restrict__ ws_ml, int64_t ws_rows) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[kLdsBytes];
  __shared__ float s_m[kDecodeWaves][kDecodeMaxRowsPerChunk];
  __shared__ float s_l[kDecodeWaves][kDecodeMaxRowsPerChunk];

  const int split = blockIdx.x;
  const int g = blockIdx.y / S.row_chunks;
  const int chunk = blockIdx.y % S.row_chunks;
  const int b = blockIdx.z;
  const int wave = threadIdx.x / 64;
  const int lane = threadIdx.x % 64;
  const int lg = lane / 16;          // lane group: 4 keys of each 16-key score block
  const int lc = lane % 16;          // lane column: the row this lane owns

  const int64_t q0 = B.q_start[b];
  const int64_t n = (int64_t)B.q_start[b + 1] - q0;
  if (n <= 0) return;
  const int64_t kv = B.kv_len[b];
  const int64_t rows_b = n * L.G;
  const int64_t row0 = (int64_t)chunk * S.rows_per_chunk;
  if (row0 >= rows_b) return;
  const int64_t base = range_base(L, kv, n);
  const int64_t k_begin = base + (int64_t)split * S.keys_per_split;
  if (k_begin >= kv) return;
  const int64_t k_end = k_begin + S.keys_per_split < kv ? k_begin + S.keys_per_split : kv;
  const int64_t first_pos = kv - n;

  // ---- this lane's rows: Q^T operand, position and window start
  bf16x8_t qop[RB][4];
  int row_pos[RB], row_lo[RB];        // positions fit in 32 bits (kv_len is int32)
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int64_t r = row0 + 16 * rb + lc;
    const bool valid = r < rows_b && (r - row0) < S.rows_per_chunk;
    const int64_t t = valid ? r / L.G : 0;
    const int h = g * L.G + (int)(valid ? r % L.G : 0);
    row_pos[rb] = valid ? (int)(first_pos + t) : -1;
    row_lo[rb] = (L.kind == BEAM_LAYER_SWA && valid)
                     ? (row_pos[rb] - L.window + 1 > 0 ? row_pos[rb] - L.window + 1 : 0) : 0;
    const uint16_t* qrow = q + (q0 + t) * q_stride + (int64_t)h * kHeadDim;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      u32x4_t v = {0u, 0u, 0u, 0u};
      if (valid) v = *reinterpret_cast<const u32x4_t*>(qrow + dslice<KV>(i, lg));
      qop[rb][i] = __builtin_bit_cast(bf16x8_t, v);
    }
  }
  // keys needing no mask: visible to every row of the sequence
  const int64_t all_lo = (L.kind == BEAM_LAYER_SWA)
                             ? (kv - 1 - L.window + 1 > 0 ? kv - L.window : 0) : 0;
  const int64_t all_hi = first_pos;   // inclusive

  const float c = L.sm_scale * kLog2e * (KV == BEAM_KV_FP8_E4M3 ? C.k_scale : 1.0f);
  float m_run[RB], l_run[RB];
  f32x4_t acc[RB][8];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    m_run[rb] = -INFINITY;
    l_run[rb] = 0.f;
#pragma unroll
    for (int d = 0; d < 8; ++d) acc[rb][d] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  unsigned char* vlds = lds + wave * kVRowsPerWave * kVRowBytes;

  // This wave's pages: keys pk = k_begin + 64*(wave + 4*pi), pi = 0, 1, ...; each page is
  // two half-steps of 32 keys, each loaded into one register set and then computed. The
  // kernel is built for 2-3 resident waves per SIMD, whose loads hide each other's
  // latency; a second register set per wave would halve that residency.
  const int64_t first_pk = k_begin + (int64_t)kPage * wave;
  int n_half = 0;
  if (first_pk < k_end) {
    const int64_t n_pages = (k_end - first_pk + kDecodeKeysPerBlockStep - 1) / kDecodeKeysPerBlockStep;
    const int64_t last_pk = first_pk + (n_pages - 1) * kDecodeKeysPerBlockStep;
    n_half = (int)(2 * (n_pages - 1) + (last_pk + 32 < k_end ? 2 : 1));
  }
  // block-table entries of the wave's pages, 64 at a time: lane i holds page i of the chunk
  const int32_t* bt_row = B.block_table + (int64_t)b * B.max_pages;
  int bt_chunk = -1;
  int32_t bt_lane = 0;
  auto page_of = [&](int pi) -> int64_t {
    if (pi / 64 != bt_chunk) {
      bt_chunk = pi / 64;
      const int64_t my_pk = first_pk + (int64_t)kDecodeKeysPerBlockStep * (64 * bt_chunk + lane);
      bt_lane = my_pk < k_end ? bt_row[my_pk / kPage] : 0;
    }
    return (int64_t)__builtin_amdgcn_readlane(bt_lane, pi % 64);
  };

  constexpr int kKRegs = KV == BEAM_KV_BF16 ? 8 : 4;   // 16-byte K loads per lane per half-step
  constexpr int kVRegs = KV == BEAM_KV_BF16 ? 8 : 4;   // 16-byte V loads per lane per half-step
  u32x4_t kreg[kKRegs], vreg[kVRegs];

  // Per-lane byte offsets inside one KV head's page (loop constants, 32-bit), so every
  // load is a uniform 64-bit page base in scalar registers plus a lane offset.
  constexpr int kElem = KV == BEAM_KV_BF16 ? 2 : 1;
  constexpr int kRow = kHeadDim * kElem;                  // bytes per key row
  uint32_t koff[kKRegs], voff[kVRegs];
  if (KV == BEAM_KV_BF16) {
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int i = 0; i < 4; ++i) koff[4 * sb + i] = (16 * sb + lc) * kRow + dslice<KV>(i, lg) * 2;
#pragma unroll
    for (int it = 0; it < 8; ++it) voff[it] = (lane / 16 + 4 * it) * kRow + lc * 16;
  } else {
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) koff[2 * sb + jj] = (16 * sb + lc) * kRow + 64 * jj + 16 * lg;
#pragma unroll
    for (int it = 0; it < 4; ++it) voff[it] = (lane / 8 + 8 * it) * kRow + (lane % 8) * 16;
  }
  const int64_t head_bytes = (int64_t)kPage * kRow;       // one KV head's page
  auto fetch = [&](int j, u32x4_t* kr, u32x4_t* vr) {
    const int pi = j >> 1, hs = j & 1;
    const int64_t page = page_of(pi);
    const int64_t base = (page * L.Hkv + g) * head_bytes + (int64_t)(32 * hs) * kRow;
    const char* kb = static_cast<const char*>(C.k) + base;
    const char* vb = static_cast<const char*>(C.v) + base;
#pragma unroll
    for (int i = 0; i < kKRegs; ++i) kr[i] = *reinterpret_cast<const u32x4_t*>(kb + koff[i]);
#pragma unroll
    for (int i = 0; i < kVRegs; ++i) vr[i] = *reinterpret_cast<const u32x4_t*>(vb + voff[i]);
  };


  auto compute = [&](const u32x4_t* kreg, const u32x4_t* vreg, int j) {
    const int kk0 = (int)(first_pk + (int64_t)kDecodeKeysPerBlockStep * (j >> 1) + 32 * (j & 1));
    // ---- S^T = K Q^T (32 keys = 2 score blocks of 16)
    f32x4_t sc[RB][2];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      bf16x8_t kop[4];
      if (KV == BEAM_KV_BF16) {
#pragma unroll
        for (int i = 0; i < 4; ++i) kop[i] = __builtin_bit_cast(bf16x8_t, kreg[4 * sb + i]);
      } else {
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          const u32x4_t w = kreg[2 * sb + jj];
          kop[2 * jj] = fp8x8_to_bf16x8(w[0], w[1]);
          kop[2 * jj + 1] = fp8x8_to_bf16x8(w[2], w[3]);
        }
      }
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        f32x4_t sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 4; ++i) sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[i], qop[rb][i], sacc, 0, 0, 0);
        sc[rb][sb] = sacc;
      }
    }
    // ---- stage V rows (row-major bf16) in this wave's LDS region; keys >= kv are
    // zeroed so that their (zero) probabilities never meet NaN payloads
    if (KV == BEAM_KV_BF16) {
#pragma unroll
      for (int it = 0; it < 8; ++it) {
        const int r = lane / 16 + 4 * it;
        u32x4_t w = vreg[it];
        if (kk0 + r >= kv) w = u32x4_t{0u, 0u, 0u, 0u};
        *reinterpret_cast<u32x4_t*>(vlds + r * kVRowBytes + lc * 16) = w;
      }
    } else {
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const int r = lane / 8 + 8 * it;
        const int cc = lane % 8;
        u32x4_t w = vreg[it];
        if (kk0 + r >= kv) w = u32x4_t{0u, 0u, 0u, 0u};
        *reinterpret_cast<bf16x8_t*>(vlds + r * kVRowBytes + cc * 32) = fp8x8_to_bf16x8(w[0], w[1]);
        *reinterpret_cast<bf16x8_t*>(vlds + r * kVRowBytes + cc * 32 + 16) = fp8x8_to_bf16x8(w[2], w[3]);
      }
    }
    // ---- mask, online softmax, P^T as bf16 (k-slot order: block 0 keys 4lg..4lg+3,
    // then block 1 keys 16+4lg..)
    const bool need_mask = (kk0 + 31 > all_hi) || (kk0 < all_lo);
    bf16x8_t pop[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      float sv[8];
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int v = 0; v < 4; ++v) sv[4 * sb + v] = sc[rb][sb][v];
      if (need_mask) {
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int jk = kk0 + 16 * sb + 4 * lg + v;
            if (jk > row_pos[rb] || jk < row_lo[rb]) sv[4 * sb + v] = -INFINITY;
          }
      }
      float mx = sv[0];
#pragma unroll
      for (int e = 1; e < 8; ++e) mx = fmaxf(mx, sv[e]);
      mx = wave_xor_max(mx, 16);
      mx = wave_xor_max(mx, 32);
      mx *= c;
      // raise the running max only when some row's maximum grew by more than 2^8 (log2
      // domain): the rescale of the output is then skipped on almost every step, and the
      // final division by the running sum (accumulated against the same max) is exact
      if (__builtin_amdgcn_ballot_w64(mx > m_run[rb] + kRescaleSlack) != 0) {
        const float m_new = fmaxf(m_run[rb], mx);
        const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run[rb] - m_new);
        l_run[rb] *= alpha;
#pragma unroll
        for (int d = 0; d < 8; ++d) acc[rb][d] *= alpha;
        m_run[rb] = m_new;
      }
      const float m_use = m_run[rb] == -INFINITY ? 0.f : m_run[rb];
      float psum = 0.f;
      bf16x8_t pb;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float pe = __builtin_amdgcn_exp2f(fmaf(sv[e], c, -m_use));
        psum += pe;
        pb[e] = (__bf16)pe;
      }
      l_run[rb] += psum;
      pop[rb] = pb;
    }
    // ---- O^T += V^T P^T, V^T via transposing LDS reads
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const int col = 16 * db + 4 * (lc % 4);
      const unsigned char* a0 = vlds + (4 * lg + lc / 4) * kVRowBytes + col * 2;
      const unsigned char* a1 = vlds + (16 + 4 * lg + lc / 4) * kVRowBytes + col * 2;
      const i16x4_t t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4_t*)(a0));
      const i16x4_t t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4_t*)(a1));
      const u32x2_t u0 = __builtin_bit_cast(u32x2_t, t0), u1 = __builtin_bit_cast(u32x2_t, t1);
      const u32x4_t uv = {u0[0], u0[1], u1[0], u1[1]};
      const bf16x8_t vop = __builtin_bit_cast(bf16x8_t, uv);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
        acc[rb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pop[rb], acc[rb][db], 0, 0, 0);
    }
  };

  // one register set: fetch a half-step, compute it; other waves hide the latency
#pragma unroll 1
  for (int j = 0; j < n_half; ++j) {
    fetch(j, kreg, vreg);
    compute(kreg, vreg, j);
  }

  // ---- merge the 4 waves of this workgroup (LDS), then write
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    l_run[rb] += __shfl_xor(l_run[rb], 16, 64);
    l_run[rb] += __shfl_xor(l_run[rb], 32, 64);
    if (lg == 0) {
      s_m[wave][16 * rb + lc] = m_run[rb];
      s_l[wave][16 * rb + lc] = l_run[rb];
    }
  }
  __syncthreads();                     // every wave is done with its V region
  // Sum the waves' outputs in a fixed order (wave 0 writes, waves 1..3 add in turn) so
  // results are bitwise reproducible; [48 rows][128] fp32 fits in the V regions.
  float* o_sum = reinterpret_cast<float*>(lds);
  for (int w = 0; w < kDecodeWaves; ++w) {
    if (wave == w) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const int row = 16 * rb + lc;
        float mw = -INFINITY;
#pragma unroll
        for (int u = 0; u < kDecodeWaves; ++u) mw = fmaxf(mw, s_m[u][row]);
        const float wgt = (m_run[rb] == -INFINITY) ? 0.f : exp2f(m_run[rb] - mw);
#pragma unroll
        for (int db = 0; db < 8; ++db)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            float* dst = &o_sum[row * kHeadDim + 16 * db + 4 * lg + v];
            const float val = acc[rb][db][v] * wgt;
            *dst = (w == 0) ? val : *dst + val;
          }
      }
    }
    __syncthreads();
  }

  // one thread per (row, 2 dims) writes the workgroup's result
  const float vsc = (KV == BEAM_KV_FP8_E4M3) ? C.v_scale : 1.0f;
  for (int i = threadIdx.x; i < S.rows_per_chunk * (kHeadDim / 2); i += kThreads) {
    const int row = i / (kHeadDim / 2);
    const int d = 2 * (i % (kHeadDim / 2));
    const int64_t r = row0 + row;
    if (r >= rows_b) continue;
    float mw = -INFINITY;
#pragma unroll
    for (int w = 0; w < kDecodeWaves; ++w) mw = fmaxf(mw, s_m[w][row]);
    float lw = 0.f;
#pragma unroll
    for (int w = 0; w < kDecodeWaves; ++w)
      lw += (s_m[w][row] == -INFINITY) ? 0.f : s_l[w][row] * exp2f(s_m[w][row] - mw);
    const int64_t t = r / L.G;
    const int h = g * L.G + (int)(r % L.G);
    const int64_t tok = q0 + t;
    const float o0 = o_sum[row * kHeadDim + d] * vsc, o1 = o_sum[row * kHeadDim + d + 1] * vsc;
    if (S.num_splits == 1) {
      const float inv = lw > 0.f ? 1.0f / lw : 0.f;
      float y0 = o0 * inv, y1 = o1 * inv;
      if (gate != nullptr) {
        const uint32_t gw = *reinterpret_cast<const uint32_t*>(gate + tok * gate_stride + (int64_t)h * kHeadDim + d);
        const float bh = bf16_to_f32(gate_bias[h]);
        y0 *= 1.0f / (1.0f + expf(-(bf16_to_f32(gw & 0xFFFFu) + bh)));
        y1 *= 1.0f / (1.0f + expf(-(bf16_to_f32(gw >> 16) + bh)));
      }
      *reinterpret_cast<uint32_t*>(out + tok * out_stride + (int64_t)h * kHeadDim + d) = pack_bf16x2(y0, y1);
    } else {
      const int64_t wrow = (int64_t)split * ws_rows + tok * L.Hq + h;
      *reinterpret_cast<float2*>(ws_o + wrow * kHeadDim + d) = make_float2(o0, o1);
      if (d == 0) *reinterpret_cast<float2*>(ws_ml + wrow * 2) = make_float2(mw, lw);
    }
  }
}

// Log-sum-exp merge of the split partials of each (token, head) row, then the gate.
// One 256-thread workgroup per row: the 4 waves take splits w, w+4, ... with independent
// loads in flight, each lane owning 2 of the 128 output dims; the waves then combine in
// a fixed order through LDS.
__global__ __launch_bounds__(256) void decode_merge_kernel(
    LayerParams L, BatchParams B, DecodeSplit S, const float* __restrict__ ws_o,
    const float* __restrict__ ws_ml, int64_t ws_rows, const uint16_t* __restrict__ gate,
    int64_t gate_stride, const uint16_t* __restrict__ gate_bias, uint16_t* out,
    int64_t out_stride) {
  __shared__ float s_red[4];
  __shared__ float s_o[4][kHeadDim];
  __shared__ float s_l[4];
  const int64_t row = blockIdx.x;                 // tok * Hq + h
  const int64_t tok = row / L.Hq;
  const int h = (int)(row % L.Hq);
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  if (tok >= B.q_start[B.num_seqs]) return;      // padding row past the last sequence
  const int b = seq_of_token(B.q_start, B.num_seqs, tok);
  const int64_t n = (int64_t)B.q_start[b + 1] - B.q_start[b];
  const int64_t kv = B.kv_len[b];
  const int64_t base = range_base(L, kv, n);
  const int used = (int)((kv - base + S.keys_per_split - 1) / S.keys_per_split);

  float M = -INFINITY;
  for (int s = threadIdx.x; s < used; s += 256) M = fmaxf(M, ws_ml[((int64_t)s * ws_rows + row) * 2]);
  for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, 64));
  if (lane == 0) s_red[wave] = M;
  __syncthreads();
  M = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));

  float lsum = 0.f, o0 = 0.f, o1 = 0.f;
#pragma unroll 4
  for (int s = wave; s < used; s += 4) {
    const int64_t wrow = (int64_t)s * ws_rows + row;
    const float2 ml = *reinterpret_cast<const float2*>(ws_ml + wrow * 2);
    const float2 o = *reinterpret_cast<const float2*>(ws_o + wrow * kHeadDim + 2 * lane);
    const float w = ml.x == -INFINITY ? 0.f : exp2f(ml.x - M);
    lsum += w * ml.y;
    o0 += w * o.x;
    o1 += w * o.y;
  }
  s_o[wave][2 * lane] = o0;
  s_o[wave][2 * lane + 1] = o1;
  if (lane == 0) s_l[wave] = lsum;
  __syncthreads();
  if (wave != 0) return;
  const float ltot = ((s_l[0] + s_l[1]) + s_l[2]) + s_l[3];
  const int d = 2 * lane;
  float y0 = ((s_o[0][d] + s_o[1][d]) + s_o[2][d]) + s_o[3][d];
  float y1 = ((s_o[0][d + 1] + s_o[1][d + 1]) + s_o[2][d + 1]) + s_o[3][d + 1];
  const float inv = ltot > 0.f ? 1.0f / ltot : 0.f;
  y0 *= inv;
  y1 *= inv;
  if (gate != nullptr) {
    const uint32_t gw = *reinterpret_cast<const uint32_t*>(gate + tok * gate_stride + (int64_t)h * kHeadDim + d);
    const float bh = bf16_to_f32(gate_bias[h]);
    y0 *= 1.0f / (1.0f + expf(-(bf16_to_f32(gw & 0xFFFFu) + bh)));
    y1 *= 1.0f / (1.0f + expf(-(bf16_to_f32(gw >> 16) + bh)));
  }
  *reinterpret_cast<uint32_t*>(out + tok * out_stride + (int64_t)h * kHeadDim + d) = pack_bf16x2(y0, y1);
}

template <int KV>
hipError_t launch_kv(const LayerParams& L, const BatchParams& B, const CacheParams& C,
                     const DecodeSplit& S, const void* q, int64_t q_stride, const void* gate,
                     int64_t gate_stride, const void* gate_bias, void* out, int64_t out_stride,
                     void* workspace, hipStream_t stream) {
  const int64_t ws_rows = (int64_t)B.num_seqs * B.max_q_len * L.Hq;
  float* ws_o = static_cast<float*>(workspace);
  float* ws_ml = ws_o + (S.num_splits > 1 ? (int64_t)S.num_splits * ws_rows * kHeadDim : 0);
  const dim3 grid(S.num_splits, L.Hkv * S.row_chunks, B.num_seqs), block(kThreads);
  const int rb = S.rows_per_chunk / 16;
#define BEAM_DECODE_LAUNCH(RBV)                                                               \
  hipLaunchKernelGGL((decode_split_kernel<KV, RBV>), grid, block, 0, stream, L, B, C, S,      \
                     static_cast<const uint16_t*>(q), q_stride,                               \
                     static_cast<const uint16_t*>(gate), gate_stride,                         \
                     static_cast<const uint16_t*>(gate_bias), static_cast<uint16_t*>(out),    \
                     out_stride, ws_o, ws_ml, ws_rows)
  if (rb == 1) BEAM_DECODE_LAUNCH(1);
  else if (rb == 2) BEAM_DECODE_LAUNCH(2);
  else BEAM_DECODE_LAUNCH(3);
#undef BEAM_DECODE_LAUNCH
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || S.num_splits == 1) return e;
  hipLaunchKernelGGL(decode_merge_kernel, dim3((unsigned)(B.num_tokens * L.Hq)), dim3(256), 0, stream, L,
                     B, S, ws_o, ws_ml, ws_rows, static_cast<const uint16_t*>(gate), gate_stride,
                     static_cast<const uint16_t*>(gate_bias), static_cast<uint16_t*>(out),
                     out_stride);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_decode(const LayerParams& L, const BatchParams& B, const CacheParams& C,
                              const DecodeSplit& S, const void* q, int64_t q_stride,
                              const void* gate, int64_t gate_stride, const void* gate_bias,
                              void* out, int64_t out_stride, void* workspace, hipStream_t stream) {
  if (B.num_tokens == 0 || B.num_seqs == 0) return hipSuccess;
  if (C.dtype == BEAM_KV_BF16)
    return launch_kv<BEAM_KV_BF16>(L, B, C, S, q, q_stride, gate, gate_stride, gate_bias, out,
                                   out_stride, workspace, stream);
  return launch_kv<BEAM_KV_FP8_E4M3>(L, B, C, S, q, q_stride, gate, gate_stride, gate_bias, out,
                                     out_stride, workspace, stream);
}

}  // namespace beam
