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
//  * A workgroup is W waves (4; 12 for latency-bound single-split launches); wave w
//    streams pages w, w+W, ... of its split: a 64-key page of one KV head is one
//    contiguous 16 KiB (bf16) / 8 KiB (fp8) block, read in 32-key halves through
//    non-temporal buffer loads.
//  * Scores use MFMA 16x16x32 bf16 as S^T = K Q^T: K rows are loaded whole and staged in
//    LDS (bf16 rows, or fp8 codes as they are), then read in operand layout (fp8 codes
//    decoded to bf16 exactly in registers; the scale folds into the softmax scale); Q^T
//    stays in registers. The 12-wave kernel loads K straight into operand layout. Each
//    lane then owns one row's scores for 8 keys, so the online softmax needs only two
//    cross-lane steps.
//  * P V uses O^T = V^T P^T: P^T is the score accumulator re-packed to bf16 in place;
//    V^T comes from a row-major LDS copy of the V rows through the gfx950 transposing
//    LDS reads (ds_read_b64_tr_b16 on bf16 rows; ds_read_b64_tr_b8 on raw fp8 rows,
//    widened after the read), so no register transpose is needed.
//  * Weights are formed against the running max first; the row max is only formed, and
//    the running max raised, when some weight of a step exceeds 2^8 (or a row has no
//    reference yet), so the max and the output rescale are skipped on almost every step.
//  * The waves merge their (max, sum, output) in LDS; splits are merged by log-sum-exp
//    in a second kernel, which also applies the gate; with one split the first kernel
//    writes the gated output itself.
#include "beam_common.h"

namespace beam {
namespace {

constexpr int kVRowBytes = kHeadDim * 2 + 16;     // bf16 K or V row in LDS, padded
                                                  // (fp8 rows use kK8RowBytes within it)
constexpr int kVRowsPerWave = 32;                 // keys staged per half-page step
// K goes through LDS as well in the 4-wave kernel (see fetch_k); the 12-wave kernel of
// latency-bound launches keeps the V staging only, to fit its 12 waves in LDS.
constexpr bool k_staged(int waves) { return waves == kDecodeWaves; }
constexpr int lds_bytes(int waves) {
  return waves * kVRowsPerWave * kVRowBytes * (k_staged(waves) ? 2 : 1);
}
// Output regions of the in-workgroup merge: the largest divisor of the wave count whose
// regions (fp32 [rows][128], padded) fit the V staging space.
constexpr int merge_regions(int waves, int region_bytes) {
  int r = waves;
  while (r > 1 && (waves % r != 0 || r * region_bytes > lds_bytes(waves))) --r;
  return r;
}
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kWeightCeiling = 256.0f;             // 2^8: a larger step sum raises the max
constexpr int kBufferRsrcWord3 = 0x00020000;         // raw buffer, 32-bit data format (CDNA)
constexpr int kLoadNonTemporal = 2;                  // cache-policy bit: nt

// Start of the 8-value slice of head dimension used by MFMA i (0..3) in lane group g
// (lane / 16). bf16 K (from LDS or straight from the cache): one 16-byte piece per MFMA;
// fp8 K (raw codes, from LDS or straight from the cache): one 16-byte piece feeds 2 MFMAs.
template <int KV, bool KST>
__device__ __forceinline__ int dslice(int i, int g) {
  return KV == BEAM_KV_BF16 ? 32 * i + 8 * g : 64 * (i / 2) + 16 * g + 8 * (i % 2);
}
// fp8 K staged in LDS as its raw codes: 128-byte rows padded to 144, so that the 16 rows
// of one operand read (16 bytes each) fall in distinct bank groups
constexpr int kK8RowBytes = kHeadDim + 16;
typedef int v2i32_t __attribute__((ext_vector_type(2)));


// Max / sum over lanes l, l^16, l^32, l^48 (the four lane groups that hold one row's
// scores) with the gfx950 lane-row swaps: plain VALU instructions, where a shuffle
// through LDS (ds_bpermute) would put an LDS round trip on the softmax's critical path.
// Each swap returns two values whose elementwise max (or sum) combines lane l with
// lane l^16 (resp. l^32), whichever rows the instruction exchanged.
__device__ __forceinline__ float max_over_lane_groups(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const float m = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const uint32_t v = __float_as_uint(m);
  const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum_over_lane_groups(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const float m = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const uint32_t v = __float_as_uint(m);
  const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// First key of the sequence's visited range, rounded down to a page.
__device__ __forceinline__ int64_t range_base(const LayerParams& L, int64_t kv, int64_t n) {
  const int64_t first_pos = kv - n;
  int64_t lo = 0;
  if (L.kind == BEAM_LAYER_SWA) lo = first_pos - L.window + 1 > 0 ? first_pos - L.window + 1 : 0;
  return (lo / kPage) * kPage;
}

template <int KV, int RB, int W>
__global__ __launch_bounds__(W * 64) __attribute__((amdgpu_waves_per_eu(W == kDecodeWideWaves ? 3 : decode_wgs_per_cu(RB, KV)))) void decode_split_kernel(
    LayerParams L, BatchParams B, CacheParams C, DecodeSplit S,
    const uint16_t* __restrict__ q, int64_t q_stride, const uint16_t* __restrict__ gate,
    int64_t gate_stride, const uint16_t* __restrict__ gate_bias, uint16_t* out,
    int64_t out_stride, float* __restrict__ ws_o, float* __restrict__ ws_ml, int64_t ws_rows) {
  constexpr int kThreads = W * 64;
  constexpr int kLdsBytes = lds_bytes(W);
  constexpr bool KST = k_staged(W);
  constexpr int kStep = W * kPage;                    // keys of one page per wave
  __shared__ __attribute__((aligned(16))) unsigned char lds[kLdsBytes];
  __shared__ float s_m[W][kDecodeMaxRowsPerChunk];
  __shared__ float s_l[W][kDecodeMaxRowsPerChunk];

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
  if (k_begin >= kv) {
    // a split past this sequence's keys: its rows get an empty partial (max -inf, sum
    // 0), so that the merge can weigh every split of the launch without reading the
    // batch metadata
    if (S.num_splits > 1) {
      for (int i = threadIdx.x; i < S.rows_per_chunk; i += kThreads) {
        const int64_t r = row0 + i;
        if (r >= rows_b) break;
        const int64_t wrow = (int64_t)split * ws_rows + (q0 + r / L.G) * L.Hq + g * L.G + r % L.G;
        *reinterpret_cast<float2*>(ws_ml + wrow * 2) = make_float2(-INFINITY, 0.f);
      }
    }
    return;
  }
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
      if (valid) v = *reinterpret_cast<const u32x4_t*>(qrow + dslice<KV, KST>(i, lg));
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

  unsigned char* vlds = lds + wave * kVRowsPerWave * kVRowBytes * (KST ? 2 : 1);
  unsigned char* klds = vlds + kVRowsPerWave * kVRowBytes;     // (K staging, KST only)

  // This wave's pages: keys pk = k_begin + 64*(wave + W*pi), pi = 0, 1, ...; each page is
  // two half-steps of 32 keys, each loaded into one register set and then computed. The
  // kernel is built for 2-3 resident waves per SIMD, whose loads hide each other's
  // latency; a second register set per wave would halve that residency. (The wave index
  // is read into a scalar register: a per-lane 64-bit first page made the three-block
  // fp8 kernel spill.)
  const int64_t first_pk = k_begin + (int64_t)kPage * __builtin_amdgcn_readfirstlane(wave);
  int n_half = 0;
  if (first_pk < k_end) {
    const int64_t n_pages = (k_end - first_pk + kStep - 1) / kStep;
    const int64_t last_pk = first_pk + (n_pages - 1) * kStep;
    n_half = (int)(2 * (n_pages - 1) + (last_pk + 32 < k_end ? 2 : 1));
  }
  // block-table entries of the wave's pages, 64 at a time: lane i holds page i of the chunk
  const int32_t* bt_row = B.block_table + (int64_t)b * B.max_pages;
  int bt_chunk = -1;
  int32_t bt_lane = 0;
  auto page_of = [&](int pi) -> int64_t {
    if (pi / 64 != bt_chunk) {
      bt_chunk = pi / 64;
      const int64_t my_pk = first_pk + (int64_t)kStep * (64 * bt_chunk + lane);
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
  // V (and staged K): every load instruction reads whole rows, 1 KiB of consecutive
  // bytes (4 bf16 or 8 fp8 rows). K read straight into MFMA operands instead takes 16
  // rows x 64 bytes per instruction (half cache lines), which streams about 20% slower.
  if (KV == BEAM_KV_BF16) {
#pragma unroll
    for (int it = 0; it < 8; ++it) voff[it] = (lane / 16 + 4 * it) * kRow + lc * 16;
    if (KST) {
#pragma unroll
      for (int it = 0; it < 8; ++it) koff[it] = voff[it];
    } else {
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int i = 0; i < 4; ++i) koff[4 * sb + i] = (16 * sb + lc) * kRow + dslice<KV, KST>(i, lg) * 2;
    }
  } else {
#pragma unroll
    for (int it = 0; it < 4; ++it) voff[it] = (lane / 8 + 8 * it) * kRow + (lane % 8) * 16;
    if (KST) {
#pragma unroll
      for (int it = 0; it < 4; ++it) koff[it] = voff[it];
    } else {
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) koff[2 * sb + jj] = (16 * sb + lc) * kRow + 64 * jj + 16 * lg;
    }
  }
  const int64_t head_bytes = (int64_t)kPage * kRow;       // one KV head's page
  // One buffer resource per half-page: the uniform base sits in scalar registers and
  // each lane adds a 32-bit offset, so no per-lane 64-bit addresses are formed. The
  // loads carry the non-temporal hint: every cache byte is read once per call, and
  // streaming it past the caches raised the achieved HBM rate by about 10%.
  auto page_base = [&](int j) -> int64_t {
    const int64_t page = page_of(j >> 1);
    return (page * L.Hkv + g) * head_bytes + (int64_t)(32 * (j & 1)) * kRow;
  };
  auto half_rsrc = [&](const void* p, int j) {
    return __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(static_cast<const char*>(p) + page_base(j)), 0, 32 * kRow, kBufferRsrcWord3);
  };
  auto fetch_k = [&](int j) {
    const __amdgpu_buffer_rsrc_t r = half_rsrc(C.k, j);
#pragma unroll
    for (int i = 0; i < kKRegs; ++i) kreg[i] = __builtin_amdgcn_raw_buffer_load_b128(r, koff[i], 0, kLoadNonTemporal);
  };
  auto fetch_v = [&](int j) {
    const __amdgpu_buffer_rsrc_t r = half_rsrc(C.v, j);
#pragma unroll
    for (int i = 0; i < kVRegs; ++i) vreg[i] = __builtin_amdgcn_raw_buffer_load_b128(r, voff[i], 0, kLoadNonTemporal);
  };
  // With 2 waves per SIMD the loop is software-pipelined inside the one register set: the
  // next half-step's K and V loads are issued once this step's K and V are staged in LDS,
  // so they fly during this step's scores, softmax and P V (-11% time on the 8-token
  // 1M-key verify, -7% on batch-1 bf16 decode against the unpipelined loop at 3 waves per
  // SIMD). bf16 with three blocks has no registers to spare and fetches, then computes;
  // so do the wide single-split workgroups (3 waves per SIMD, K loaded straight into
  // operand layout).
  constexpr bool kPipe = W == kDecodeWaves && decode_wgs_per_cu(RB, KV) == 2 &&
                         !(KV == BEAM_KV_BF16 && RB == 3);

  // stage 32 K or V rows (row-major bf16) in this wave's LDS region: `reg` holds whole
  // rows as loaded (see voff); fp8 codes are widened exactly to bf16 on the way
  auto stage_rows = [&](unsigned char* dst, const u32x4_t (&reg)[kVRegs], int kk0, bool zero_tail) {
    if (KV == BEAM_KV_BF16) {
#pragma unroll
      for (int it = 0; it < 8; ++it) {
        const int r = lane / 16 + 4 * it;
        u32x4_t w = reg[it];
        if (zero_tail && kk0 + r >= kv) w = u32x4_t{0u, 0u, 0u, 0u};
        *reinterpret_cast<u32x4_t*>(dst + r * kVRowBytes + lc * 16) = w;
      }
    } else {
      // fp8 V rows as their raw codes, key r = 16 b + 4 g + e at LDS row 8 g + 4 b + e:
      // the 8 keys one transposing read gathers (see the P V step) are then 8 consecutive
      // rows, whose 144-byte pitch puts them in distinct banks
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const int r = lane / 8 + 8 * it;
        const int row = 8 * ((r % 16) / 4) + 4 * (r / 16) + r % 4;
        u32x4_t w = reg[it];
        if (zero_tail && kk0 + r >= kv) w = u32x4_t{0u, 0u, 0u, 0u};
        *reinterpret_cast<u32x4_t*>(dst + row * kK8RowBytes + (lane % 8) * 16) = w;
      }
    }
  };

  auto compute = [&](int j) {
    const int kk0 = (int)(first_pk + (int64_t)kStep * (j >> 1) + 32 * (j & 1));
    if constexpr (KST) {
      // K and V rows of this half-step into LDS; the registers are then free for the
      // next half-step's loads, which fly during this step's compute. (Rows past the
      // sequence end: V is zeroed, K may hold anything -- those scores are masked.)
      if constexpr (KV == BEAM_KV_BF16) {
        stage_rows(klds, kreg, kk0, false);
      } else {
#pragma unroll
        for (int it = 0; it < 4; ++it)
          *reinterpret_cast<u32x4_t*>(klds + (lane / 8 + 8 * it) * kK8RowBytes + (lane % 8) * 16) = kreg[it];
      }
      if (kk0 + 32 > kv) stage_rows(vlds, vreg, kk0, true);   // (the sequence's last keys)
      else stage_rows(vlds, vreg, kk0, false);
      if (kPipe && j + 1 < n_half) { fetch_k(j + 1); fetch_v(j + 1); }
    }
    // ---- S^T = K Q^T (32 keys = 2 score blocks of 16)
    f32x4_t sc[RB][2];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      bf16x8_t kop[4];
      if (KST && KV == BEAM_KV_BF16) {
        // MFMA layout from the staged rows: lane (lc, lg) reads row 16 sb + lc, dims
        // 32 i + 8 lg; the 16-byte row padding puts the 16 rows of one read in distinct
        // banks
#pragma unroll
        for (int i = 0; i < 4; ++i)
          kop[i] = *reinterpret_cast<const bf16x8_t*>(klds + (16 * sb + lc) * kVRowBytes + (32 * i + 8 * lg) * 2);
      } else if (KST) {
        // raw fp8 rows: one 16-byte read of row 16 sb + lc (codes 64 jj + 16 lg ..) feeds
        // MFMAs 2 jj and 2 jj + 1, widened exactly to bf16 here
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          const u32x4_t w = *reinterpret_cast<const u32x4_t*>(klds + (16 * sb + lc) * kK8RowBytes + 64 * jj + 16 * lg);
          kop[2 * jj] = fp8x8_to_bf16x8(w[0], w[1]);
          kop[2 * jj + 1] = fp8x8_to_bf16x8(w[2], w[3]);
        }
      } else if (KV == BEAM_KV_BF16) {
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
    if constexpr (!KST) {
      if (kPipe && j + 1 < n_half) fetch_k(j + 1);
      // ---- stage V rows (row-major bf16) in this wave's LDS region; keys >= kv are
      // zeroed so that their (zero) probabilities never meet NaN payloads
      if (kk0 + 32 > kv) stage_rows(vlds, vreg, kk0, true);
      else stage_rows(vlds, vreg, kk0, false);
      if (kPipe && j + 1 < n_half) fetch_v(j + 1);
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
      // Weights against the running max first, summed in bf16 pairs by v_dot2 (the
      // values P V multiplies). Only when a lane's partial sum exceeds 2^8 (some weight
      // grew past the slack, or overflowed) or a row has no reference yet does the wave
      // form the row maximum, raise the running max and redo the weights.
      bf16x8_t pb;
      float part;
      auto weights = [&](float mu) {
#pragma unroll
        for (int e = 0; e < 8; ++e) pb[e] = (__bf16)__builtin_amdgcn_exp2f(fmaf(sv[e], c, -mu));
        const bf16x2_t one = {(__bf16)1.0f, (__bf16)1.0f};
        float ps = 0.f;
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const bf16x2_t pair = {pb[e], pb[e + 1]};
          ps = __builtin_amdgcn_fdot2_f32_bf16(pair, one, ps, false);
        }
        part = ps;
      };
      weights(m_run[rb] == -INFINITY ? 0.f : m_run[rb]);
      if (__builtin_amdgcn_ballot_w64(!(part <= kWeightCeiling) || (row_pos[rb] >= 0 && m_run[rb] == -INFINITY)) != 0) {
        float mx = sv[0];
#pragma unroll
        for (int e = 1; e < 8; ++e) mx = fmaxf(mx, sv[e]);
        mx = max_over_lane_groups(mx);
        mx *= c;
        const float m_new = fmaxf(m_run[rb], mx);
        const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run[rb] - m_new);
        l_run[rb] *= alpha;
#pragma unroll
        for (int d = 0; d < 8; ++d) acc[rb][d] *= alpha;
        m_run[rb] = m_new;
        weights(m_new == -INFINITY ? 0.f : m_new);
      }
      l_run[rb] += part;
      pop[rb] = pb;
    }
    // ---- O^T += V^T P^T, V^T via transposing LDS reads
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      bf16x8_t vop;
      if constexpr (KV == BEAM_KV_BF16) {
        const int col = 16 * db + 4 * (lc % 4);
        const unsigned char* a0 = vlds + (4 * lg + lc / 4) * kVRowBytes + col * 2;
        const unsigned char* a1 = vlds + (16 + 4 * lg + lc / 4) * kVRowBytes + col * 2;
        const i16x4_t t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4_t*)(a0));
        const i16x4_t t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4_t*)(a1));
        const u32x2_t u0 = __builtin_bit_cast(u32x2_t, t0), u1 = __builtin_bit_cast(u32x2_t, t1);
        const u32x4_t uv = {u0[0], u0[1], u1[0], u1[1]};
        vop = __builtin_bit_cast(bf16x8_t, uv);
      } else {
        // ds_read_b64_tr_b8: in each 16-lane group, lane i receives byte i % 8 of the
        // 8-byte pieces addressed by lanes 2 j + i / 8, j = 0..7. Lane 2 j + h addresses
        // LDS row 8 lg + j (key slot j of this lane group) at codes 16 db + 8 h, so lane
        // lc gets dimension 16 db + lc of its 8 keys, in the k-slot order of P^T
        const unsigned char* a = vlds + (8 * lg + (lc >> 1)) * kK8RowBytes + 16 * db + 8 * (lc & 1);
        const v2i32_t t = __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) v2i32_t*)(a));
        vop = fp8x8_to_bf16x8((uint32_t)t[0], (uint32_t)t[1]);
      }
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
        acc[rb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pop[rb], acc[rb][db], 0, 0, 0);
    }
  };

  if (kPipe) {
    if (n_half > 0) { fetch_k(0); fetch_v(0); }
#pragma unroll 1
    for (int j = 0; j < n_half; ++j) compute(j);
  } else {
    // one register set: fetch a half-step, compute it; other waves hide the latency
#pragma unroll 1
    for (int j = 0; j < n_half; ++j) { fetch_k(j); fetch_v(j); compute(j); }
  }

  // ---- merge the waves of this workgroup (LDS), then write
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    l_run[rb] = sum_over_lane_groups(l_run[rb]);
    if (lg == 0) {
      s_m[wave][16 * rb + lc] = m_run[rb];
      s_l[wave][16 * rb + lc] = l_run[rb];
    }
  }
  __syncthreads();                     // every wave is done with its V region
  // The waves' outputs, each scaled to the workgroup's row maximum, go into kRegions
  // fp32 [rows][128] regions of the V staging space (padded rows; one 16-byte write per
  // accumulator). Waves w and w + kRegions share region w: the first writes, the later
  // ones add in turn, so sums run in a fixed order (bitwise reproducible).
  constexpr int kORow = kHeadDim * 4 + 16;                        // padded fp32 row
  constexpr int kRegions = merge_regions(W, RB * 16 * kORow);
  static_assert(kLdsBytes >= RB * 16 * kORow, "one output region must fit the staging space");
  float wgt[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int row = 16 * rb + lc;
    float mw = -INFINITY;
#pragma unroll
    for (int u = 0; u < W; ++u) mw = fmaxf(mw, s_m[u][row]);
    wgt[rb] = (m_run[rb] == -INFINITY) ? 0.f : exp2f(m_run[rb] - mw);
  }
#pragma unroll
  for (int round = 0; round < W / kRegions; ++round) {
    if (wave / kRegions == round) {
      unsigned char* reg = lds + (wave % kRegions) * (RB * 16 * kORow);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int db = 0; db < 8; ++db) {
          f32x4_t* dst = reinterpret_cast<f32x4_t*>(reg + (16 * rb + lc) * kORow + (16 * db + 4 * lg) * 4);
          const f32x4_t val = acc[rb][db] * wgt[rb];
          *dst = round == 0 ? val : *dst + val;
        }
    }
    __syncthreads();
  }

  // one thread per (row, 4 dims) writes the workgroup's result
  const float vsc = (KV == BEAM_KV_FP8_E4M3) ? C.v_scale : 1.0f;
  for (int i = threadIdx.x; i < S.rows_per_chunk * (kHeadDim / 4); i += kThreads) {
    const int row = i / (kHeadDim / 4);
    const int d = 4 * (i % (kHeadDim / 4));
    const int64_t r = row0 + row;
    if (r >= rows_b) continue;
    float mw = -INFINITY;
#pragma unroll
    for (int w = 0; w < W; ++w) mw = fmaxf(mw, s_m[w][row]);
    float lw = 0.f;
#pragma unroll
    for (int w = 0; w < W; ++w)
      lw += (s_m[w][row] == -INFINITY) ? 0.f : s_l[w][row] * exp2f(s_m[w][row] - mw);
    const int64_t t = r / L.G;
    const int h = g * L.G + (int)(r % L.G);
    const int64_t tok = q0 + t;
    f32x4_t o = *reinterpret_cast<const f32x4_t*>(lds + row * kORow + d * 4);
#pragma unroll
    for (int rg = 1; rg < kRegions; ++rg)
      o += *reinterpret_cast<const f32x4_t*>(lds + rg * (RB * 16 * kORow) + row * kORow + d * 4);
    o *= vsc;
    if (S.num_splits == 1) {
      const float inv = lw > 0.f ? 1.0f / lw : 0.f;
      f32x4_t y = o * inv;
      if (gate != nullptr) {
        const u32x2_t gw = *reinterpret_cast<const u32x2_t*>(gate + tok * gate_stride + (int64_t)h * kHeadDim + d);
        const float bh = bf16_to_f32(gate_bias[h]);
        y[0] *= gate_sigmoid(bf16_to_f32(gw[0] & 0xFFFFu) + bh);
        y[1] *= gate_sigmoid(bf16_to_f32(gw[0] >> 16) + bh);
        y[2] *= gate_sigmoid(bf16_to_f32(gw[1] & 0xFFFFu) + bh);
        y[3] *= gate_sigmoid(bf16_to_f32(gw[1] >> 16) + bh);
      }
      const u32x2_t packed = {pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
      *reinterpret_cast<u32x2_t*>(out + tok * out_stride + (int64_t)h * kHeadDim + d) = packed;
    } else {
      const int64_t wrow = (int64_t)split * ws_rows + tok * L.Hq + h;
      *reinterpret_cast<f32x4_t*>(ws_o + wrow * kHeadDim + d) = o;
      if (d == 0) *reinterpret_cast<float2*>(ws_ml + wrow * 2) = make_float2(mw, lw);
    }
  }
}

// Log-sum-exp merge of the split partials of each (token, head) row, then the gate.
// One 256-thread workgroup per row. Lane group (t % 32) owns 4 of the 128 output dims
// and split group t / 32 the splits t/32, t/32 + 8, ...; the (m, l) pairs and the first
// 128 splits' partial outputs are all requested before anything waits, so the merge
// costs one memory round trip. Sums run in a fixed order (bitwise reproducible).
constexpr int kMergeThreads = 256;
constexpr int kMergeGroups = kMergeThreads / 32;       // split groups
constexpr int kMergeUnroll = 16;                        // partials in flight per thread
constexpr int kMergeChunk = kMergeGroups * kMergeUnroll;

__global__ __launch_bounds__(kMergeThreads) void decode_merge_kernel(
    LayerParams L, BatchParams B, DecodeSplit S, const float* __restrict__ ws_o,
    const float* __restrict__ ws_ml, int64_t ws_rows, const uint16_t* __restrict__ gate,
    int64_t gate_stride, const uint16_t* __restrict__ gate_bias, uint16_t* out,
    int64_t out_stride) {
  __shared__ float s_w[kDecodeMaxSplits];
  __shared__ float s_red[kMergeThreads / 64];
  __shared__ f32x4_t s_acc[kMergeGroups][32];
  const int64_t row = blockIdx.x;                 // tok * Hq + h
  const int64_t tok = row / L.Hq;
  const int h = (int)(row % L.Hq);
  const int t = threadIdx.x, wave = t / 64, lane = t % 64;
  const int q4 = t % 32, grp = t / 32;
  // ---- issue everything first: this row's gate values, this thread's first (m, l)
  // pair and its first chunk of partial outputs, for every split the launch has (splits
  // past this row's sequence hold an empty pair, weight 0)
  u32x2_t gw = {0u, 0u};
  if (gate != nullptr && t < 32) gw = *reinterpret_cast<const u32x2_t*>(gate + tok * gate_stride + (int64_t)h * kHeadDim + 4 * q4);
  // (rows past the workspace's are padding rows: they read nothing and return below)
  const int nsp = row < ws_rows ? S.num_splits : 0;
  float2 ml0 = make_float2(-INFINITY, 0.f);
  if (t < nsp) ml0 = *reinterpret_cast<const float2*>(ws_ml + ((int64_t)t * ws_rows + row) * 2);
  f32x4_t ov[kMergeUnroll];
#pragma unroll
  for (int u = 0; u < kMergeUnroll; ++u) {
    const int sp = grp + kMergeGroups * u;
    ov[u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if (sp < nsp) ov[u] = *reinterpret_cast<const f32x4_t*>(ws_o + ((int64_t)sp * ws_rows + row) * kHeadDim + 4 * q4);
  }
  // padding rows past the last sequence get no output (the test sits before the output
  // write only, so its load overlaps the others)
  const bool padding = tok >= B.q_start[B.num_seqs];
  // ---- global max of the split maxima. Every split of the launch has a pair for this
  // row: splits past the sequence's keys wrote (-inf, 0).
  float M = ml0.x;
  for (int sp = t + kMergeThreads; sp < nsp; sp += kMergeThreads)
    M = fmaxf(M, ws_ml[((int64_t)sp * ws_rows + row) * 2]);
  float lsum = 0.f;
  if (nsp <= 64) {
    // one wave holds every pair: reduce without the workgroup
    if (wave == 0) {
      M = wave_xor_max(M, 1); M = wave_xor_max(M, 2); M = wave_xor_max(M, 4);
      M = wave_xor_max(M, 8); M = wave_xor_max(M, 16); M = wave_xor_max(M, 32);
      const float w = ml0.x == -INFINITY ? 0.f : exp2f(ml0.x - M);
      if (t < nsp) s_w[t] = w;
      lsum = w * ml0.y;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) lsum += __shfl_xor(lsum, o, 64);
      if (lane == 0) s_red[0] = lsum;
    }
    __syncthreads();
    lsum = s_red[0];
  } else {
    M = wave_xor_max(M, 1); M = wave_xor_max(M, 2); M = wave_xor_max(M, 4);
    M = wave_xor_max(M, 8); M = wave_xor_max(M, 16); M = wave_xor_max(M, 32);
    if (lane == 0) s_red[wave] = M;
    __syncthreads();
    M = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
    __syncthreads();                                 // s_red is reused for the sum below
    // ---- split weights (LDS) and the weighted sum of the l's
    for (int sp = t; sp < nsp; sp += kMergeThreads) {
      const float2 ml = sp == t ? ml0 : *reinterpret_cast<const float2*>(ws_ml + ((int64_t)sp * ws_rows + row) * 2);
      const float w = ml.x == -INFINITY ? 0.f : exp2f(ml.x - M);
      s_w[sp] = w;
      lsum += w * ml.y;
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) lsum += __shfl_xor(lsum, o, 64);
    if (lane == 0) s_red[wave] = lsum;
    __syncthreads();
    lsum = ((s_red[0] + s_red[1]) + s_red[2]) + s_red[3];
  }
  const float ltot = lsum;
  // ---- weighted partial outputs, chunk by chunk (a split of weight 0 -- empty, or no
  // visible key for this row -- is skipped: its partial output may hold anything)
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  for (int c0 = 0; c0 < nsp; c0 += kMergeChunk) {
    if (c0 > 0) {
#pragma unroll
      for (int u = 0; u < kMergeUnroll; ++u) {
        const int sp = c0 + grp + kMergeGroups * u;
        ov[u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        if (sp < nsp) ov[u] = *reinterpret_cast<const f32x4_t*>(ws_o + ((int64_t)sp * ws_rows + row) * kHeadDim + 4 * q4);
      }
    }
#pragma unroll
    for (int u = 0; u < kMergeUnroll; ++u) {
      const int sp = c0 + grp + kMergeGroups * u;
      if (sp < nsp && s_w[sp] != 0.f) acc += s_w[sp] * ov[u];
    }
  }
  s_acc[grp][q4] = acc;
  __syncthreads();
  if (t >= 32 || padding) return;
  f32x4_t y = s_acc[0][q4];
#pragma unroll
  for (int gi = 1; gi < kMergeGroups; ++gi) y += s_acc[gi][q4];
  const float inv = ltot > 0.f ? 1.0f / ltot : 0.f;
  y *= inv;
  const int d = 4 * q4;
  if (gate != nullptr) {
    const float bh = bf16_to_f32(gate_bias[h]);
    y[0] *= gate_sigmoid(bf16_to_f32(gw[0] & 0xFFFFu) + bh);
    y[1] *= gate_sigmoid(bf16_to_f32(gw[0] >> 16) + bh);
    y[2] *= gate_sigmoid(bf16_to_f32(gw[1] & 0xFFFFu) + bh);
    y[3] *= gate_sigmoid(bf16_to_f32(gw[1] >> 16) + bh);
  }
  const u32x2_t packed = {pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
  *reinterpret_cast<u32x2_t*>(out + tok * out_stride + (int64_t)h * kHeadDim + d) = packed;
}

template <int KV>
hipError_t launch_kv(const LayerParams& L, const BatchParams& B, const CacheParams& C,
                     const DecodeSplit& S, const void* q, int64_t q_stride, const void* gate,
                     int64_t gate_stride, const void* gate_bias, void* out, int64_t out_stride,
                     void* workspace, hipStream_t stream) {
  const int64_t ws_rows = (int64_t)B.num_seqs * B.max_q_len * L.Hq;
  float* ws_o = static_cast<float*>(workspace);
  float* ws_ml = ws_o + (S.num_splits > 1 ? (int64_t)S.num_splits * ws_rows * kHeadDim : 0);
  const dim3 grid(S.num_splits, L.Hkv * S.row_chunks, B.num_seqs);
  const int rb = S.rows_per_chunk / 16;
#define BEAM_DECODE_LAUNCH(RBV, WV)                                                            \
  hipLaunchKernelGGL((decode_split_kernel<KV, RBV, WV>), grid, dim3(WV * 64), 0, stream, L, B, \
                     C, S, static_cast<const uint16_t*>(q), q_stride,                          \
                     static_cast<const uint16_t*>(gate), gate_stride,                          \
                     static_cast<const uint16_t*>(gate_bias), static_cast<uint16_t*>(out),     \
                     out_stride, ws_o, ws_ml, ws_rows)
  if (rb == 1 && S.waves == kDecodeWideWaves) BEAM_DECODE_LAUNCH(1, kDecodeWideWaves);
  else if (rb == 1) BEAM_DECODE_LAUNCH(1, kDecodeWaves);
  else if (rb == 2) BEAM_DECODE_LAUNCH(2, kDecodeWaves);
  else BEAM_DECODE_LAUNCH(3, kDecodeWaves);
#undef BEAM_DECODE_LAUNCH
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || S.num_splits == 1) return e;
  hipLaunchKernelGGL(decode_merge_kernel, dim3((unsigned)(B.num_tokens * L.Hq)), dim3(kMergeThreads), 0, stream, L,
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
