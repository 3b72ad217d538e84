// Causal prefill attention over the paged bf16 KV cache (sliding window or full).
//
// What it computes: for new token t at position pos and query head h,
//   o[t,h] = sum_{j visible} softmax_j(sm_scale * q'[t,h] . k[j, h/G]) v[j, h/G],
// visible = [0, pos] on full NoPE layers, the most recent `window` keys (own key
// included) on sliding layers ("Reflection Beam 1.0 on vLLM", section "Attention:
// sliding-window layers plus NoPE full-attention layers"), optionally times the sigmoid
// head gate of the same section. Earlier new tokens of the call are visible (causal).
//
// Design (MFMA-bound, MI355X):
//  * Rows are (token, query head) pairs of one KV head's group, flattened token-major:
//    a workgroup owns 256 consecutive rows (about 43 tokens x 6 heads), so every K/V
//    tile it stages in LDS serves all 6 query heads of the group (GQA reuse) and all of
//    its tokens. Grid: (row tile, KV head, sequence).
//  * K/V tiles are one 64-token page of one KV head (16 KiB each), copied straight from
//    global memory into LDS with gfx950's global_load_lds_dwordx4 (no staging registers)
//    and double-buffered: the next page is in flight while the current one is consumed.
//    Each 256-byte row is stored with its 16-byte chunks XOR-swizzled by the row index so
//    that the operand reads below hit distinct LDS banks.
//  * 4 waves x 64 rows. Per 32-key half of a tile a wave computes S^T = K Q^T with MFMA
//    32x32x16 bf16 for two 32-row blocks sharing each K operand; a lane then holds 16
//    scores of one row, so row max/sum take one cross-half swap (permlane32).
//  * O^T += V^T P^T: P^T is the score accumulator packed to bf16 in place (its key order
//    is the MFMA's k-slot order); V^T comes from the row-major V tile through the
//    transposing LDS read ds_read_b64_tr_b16.
//  * The running maximum is only raised when a row's maximum grows by more than 2^8
//    (log2 domain), so the 128-value output rescale is skipped on almost every tile;
//    the final division by the same running sum keeps the result exact.
//  * Fully visible tiles skip the mask; tiles wholly outside a wave's rows skip compute.
#include <type_traits>

#include "beam_common.h"

namespace beam {
namespace {

// Workgroup shape: RB 32-row MFMA blocks per wave, WAVES waves, 256 rows in all.
constexpr int kRowsPerBlock = 256;
constexpr int kRB = 1;                                   // 32 rows per wave ...
constexpr int kWaves = kRowsPerBlock / (32 * kRB);       // ... 8 waves, 2 per SIMD
constexpr int kThreads = kWaves * 64;
constexpr int kRowsPerWave = 32 * kRB;
constexpr int kRowBytes = kHeadDim * 2;                  // 256-byte bf16 row, swizzled chunks
constexpr int kTileBytes = kPage * kRowBytes;            // one K or V page tile: 16 KiB
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescaleSlack = 8.0f;                    // log2 headroom before rescaling

typedef __attribute__((address_space(3))) void lds_void_t;

// byte offset of 16-byte chunk `c` (0..15) of row `r` inside a swizzled tile
__device__ __forceinline__ int swz(int r, int c) { return r * kRowBytes + ((c ^ (r & 15)) << 4); }

__device__ __forceinline__ float swap_halves_max(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float swap_halves_sum(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int KIND>
__global__ __launch_bounds__(kThreads) void prefill_kernel(
    LayerParams L, BatchParams B, CacheParams C, const uint16_t* __restrict__ q, int64_t q_stride,
    const uint16_t* __restrict__ gate, int64_t gate_stride, const uint16_t* __restrict__ gate_bias,
    uint16_t* out, int64_t out_stride) {
  __shared__ __attribute__((aligned(1024))) unsigned char lds[2 * 2 * kTileBytes];

  const int tile = blockIdx.x;
  const int g = blockIdx.y;
  const int b = blockIdx.z;
  const int tid = threadIdx.x;
  const int wave = tid / 64;
  const int lane = tid % 64;
  const int half = lane / 32;      // which 8-slice of each 16-wide k step this lane feeds
  const int lr = lane % 32;        // the row (within a 32-row block) this lane owns
  constexpr bool swa = KIND == BEAM_LAYER_SWA;

  const int q0 = B.q_start[b];
  const int n = B.q_start[b + 1] - q0;
  const int rows_b = n * L.G;
  const int tile_row0 = tile * kRowsPerBlock;
  if (n <= 0 || tile_row0 >= rows_b) return;
  const int kv = B.kv_len[b];
  const int first_pos = kv - n;
  const int tile_rows = rows_b - tile_row0 < kRowsPerBlock ? rows_b - tile_row0 : kRowsPerBlock;

  // key range of the workgroup, in 64-key tiles
  const int pos_first = first_pos + tile_row0 / L.G;
  const int pos_last = first_pos + (tile_row0 + tile_rows - 1) / L.G;
  const int key_lo = swa ? max(pos_first - L.window + 1, 0) : 0;
  const int kt_begin = key_lo / kPage;
  const int kt_end = pos_last / kPage + 1;               // exclusive

  // rows of this wave
  const int wrow0 = tile_row0 + wave * kRowsPerWave;
  const int wrows = min(tile_row0 + tile_rows - wrow0, kRowsPerWave);   // may be <= 0
  const bool wave_active = wrows > 0;
  const int w_min_pos = wave_active ? first_pos + wrow0 / L.G : 0;
  const int w_max_pos = wave_active ? first_pos + (wrow0 + wrows - 1) / L.G : -1;
  const int w_max_lo = swa ? max(w_max_pos - L.window + 1, 0) : 0;
  const int w_min_lo = swa ? max(w_min_pos - L.window + 1, 0) : 0;

  // per-lane rows: Q^T operand, position, window start
  bf16x8_t qop[kRB][8];
  int row_pos[kRB], row_lo[kRB];
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) {
    const int r = wrow0 + 32 * rb + lr;
    const bool valid = wave_active && (r - wrow0) < wrows;
    const int t = valid ? r / L.G : 0;
    const int h = g * L.G + (valid ? r % L.G : 0);
    row_pos[rb] = valid ? first_pos + t : -1;
    row_lo[rb] = (swa && valid) ? max(row_pos[rb] - L.window + 1, 0) : 0;
    const uint16_t* qrow = q + (int64_t)(q0 + t) * q_stride + (int64_t)h * kHeadDim;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      u32x4_t v = {0u, 0u, 0u, 0u};
      if (valid) v = *reinterpret_cast<const u32x4_t*>(qrow + 16 * i + 8 * half);
      qop[rb][i] = __builtin_bit_cast(bf16x8_t, v);
    }
  }

  const float c = L.sm_scale * kLog2e;
  float m_run[kRB], l_run[kRB];
  f32x16_t acc[kRB][4];
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) {
    m_run[rb] = -INFINITY;
    l_run[rb] = 0.f;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[rb][db][e] = 0.f;
  }

  // ---- direct global -> LDS copy of one K and one V page tile. Wave w copies rows
  // [w*R, w*R + R) of each (R = 64 / waves): R/4 instructions per tensor, each 64 lanes
  // x 16 bytes = 4 rows.
  // Lane l writes LDS bytes [16 l, 16 l + 16) of its 1 KiB block, i.e. row 4i + l/16,
  // chunk slot l%16, which holds the row's chunk (l%16) ^ (row & 15).
  const char* kcache = static_cast<const char*>(C.k);
  const char* vcache = static_cast<const char*>(C.v);
  const int32_t* bt_row = B.block_table + (int64_t)b * B.max_pages;
  auto issue_tile = [&](int kt, int buf) {
    const int64_t page = bt_row[kt];
    const int64_t base = (page * L.Hkv + g) * (int64_t)kTileBytes;
    unsigned char* kl = lds + buf * 2 * kTileBytes;
    unsigned char* vl = kl + kTileBytes;
    constexpr int kRowsCopied = kPage / kWaves;
#pragma unroll
    for (int i = 0; i < kRowsCopied / 4; ++i) {
      const int row = kRowsCopied * wave + 4 * i + lane / 16;
      const int chunk = (lane % 16) ^ (row & 15);
      const int64_t src = base + row * kRowBytes + chunk * 16;
      const int dst = (kRowsCopied * wave + 4 * i) * kRowBytes;  // wave-uniform block start
      __builtin_amdgcn_global_load_lds(kcache + src, (lds_void_t*)(kl + dst), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(vcache + src, (lds_void_t*)(vl + dst), 16, 0, 0);
    }
  };

  issue_tile(kt_begin, 0);
  __builtin_amdgcn_s_waitcnt(0);       // vmcnt(0) lgkmcnt(0): this wave's copies landed
  __syncthreads();

  const int grp = lane / 16, gi = lane % 16;
  for (int kt = kt_begin; kt < kt_end; ++kt) {
    const int buf = (kt - kt_begin) & 1;
    if (kt + 1 < kt_end) issue_tile(kt + 1, buf ^ 1);
    const int k0 = kt * kPage;
    const bool skip = !wave_active || k0 > w_max_pos || k0 + kPage - 1 < w_min_lo;
    if (!skip) {
      // MASK: some key of the tile is invisible to some row of the wave; TAIL: the tile
      // holds slots past the sequence end (they may hold NaN; a TAIL tile also masks)
      auto compute = [&](auto mask_c, auto tail_c) {
        constexpr bool MASK = decltype(mask_c)::value;
        constexpr bool TAIL = decltype(tail_c)::value;
        const unsigned char* kt_lds = lds + buf * 2 * kTileBytes;
        const unsigned char* vt_lds = kt_lds + kTileBytes;
  #pragma unroll 1
        for (int kh = 0; kh < 2; ++kh) {         // 32-key halves of the tile
          // ---- S^T = K Q^T for this half, two row blocks
          f32x16_t sc[kRB];
  #pragma unroll
          for (int rb = 0; rb < kRB; ++rb)
  #pragma unroll
            for (int e = 0; e < 16; ++e) sc[rb][e] = 0.f;
          const int krow = 32 * kh + lr;
          __builtin_amdgcn_sched_barrier(0);
          bf16x8_t kop[8];
  #pragma unroll
          for (int i = 0; i < 8; ++i)
            kop[i] = *reinterpret_cast<const bf16x8_t*>(kt_lds + swz(krow, 2 * i + half));
  #pragma unroll
          for (int i = 0; i < 8; ++i)
  #pragma unroll
            for (int rb = 0; rb < kRB; ++rb)
              sc[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[i], qop[rb][i], sc[rb], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
          // ---- mask, online softmax, P^T in bf16
          bf16x8_t pop[kRB][2];
  #pragma unroll
          for (int rb = 0; rb < kRB; ++rb) {
            if (MASK) {
  #pragma unroll
              for (int v = 0; v < 16; ++v) {
                const int j = k0 + 32 * kh + (v / 4) * 8 + half * 4 + (v % 4);
                if (j > row_pos[rb] || j < row_lo[rb]) sc[rb][v] = -INFINITY;
              }
            }
            float mx = fmaxf(sc[rb][0], sc[rb][1]);
  #pragma unroll
            for (int v = 2; v < 16; ++v) mx = fmaxf(mx, sc[rb][v]);
            mx = swap_halves_max(mx) * c;
            // raise the running max only when it grew by more than the slack
            if (__builtin_amdgcn_ballot_w64(mx > m_run[rb] + kRescaleSlack) != 0) {
              const float m_new = fmaxf(m_run[rb], mx);
              // 0 when this row saw no key before; 1 when it still sees none
              const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run[rb] - m_new);
              l_run[rb] *= alpha;
  #pragma unroll
              for (int db = 0; db < 4; ++db) acc[rb][db] *= alpha;
              m_run[rb] = m_new;
            }
            const float m_use = m_run[rb] == -INFINITY ? 0.f : m_run[rb];
            float psum = 0.f;
  #pragma unroll
            for (int cc = 0; cc < 2; ++cc) {
              bf16x8_t pb;
  #pragma unroll
              for (int jj = 0; jj < 8; ++jj) {
                const float p = __builtin_amdgcn_exp2f(fmaf(sc[rb][8 * cc + jj], c, -m_use));
                psum += p;
                pb[jj] = (__bf16)p;
              }
              pop[rb][cc] = pb;
            }
            l_run[rb] += psum;
          }
          __builtin_amdgcn_sched_barrier(0);
          // ---- O^T += V^T P^T over the 32 keys of this half (2 MFMA k-steps of 16)
  #pragma unroll
          for (int cc = 0; cc < 2; ++cc) {
            const int key0 = 32 * kh + 16 * cc + 4 * (grp / 2) + gi / 4;   // row read by this lane
  #pragma unroll
            for (int db = 0; db < 4; ++db) {
              const int col = 32 * db + 16 * (grp % 2) + 4 * (gi % 4);    // bf16 element column
              const int off0 = swz(key0, col / 8) + (col % 8) * 2;
              const int off1 = swz(key0 + 8, col / 8) + (col % 8) * 2;
              i16x4_t t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                  (__attribute__((address_space(3))) i16x4_t*)(vt_lds + off0));
              i16x4_t t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                  (__attribute__((address_space(3))) i16x4_t*)(vt_lds + off1));
              if (TAIL) {
                // this lane received keys key0-(gi/4)+0..3 (t0) and +8 (t1) at one column
                const int kb0 = k0 + 32 * kh + 16 * cc + 4 * (grp / 2);
  #pragma unroll
                for (int e = 0; e < 4; ++e) {
                  if (kb0 + e >= kv) t0[e] = 0;
                  if (kb0 + 8 + e >= kv) t1[e] = 0;
                }
              }
              const u32x2_t u0 = __builtin_bit_cast(u32x2_t, t0), u1 = __builtin_bit_cast(u32x2_t, t1);
              const u32x4_t uv = {u0[0], u0[1], u1[0], u1[1]};
              const bf16x8_t vop = __builtin_bit_cast(bf16x8_t, uv);
  #pragma unroll
              for (int rb = 0; rb < kRB; ++rb)
                acc[rb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pop[rb][cc], acc[rb][db], 0, 0, 0);
            }
          }
        }
      };
      const bool need_mask = (k0 + kPage - 1 > w_min_pos) || (k0 < w_max_lo);
      if (k0 + kPage > kv) compute(std::true_type{}, std::true_type{});
      else if (need_mask) compute(std::true_type{}, std::false_type{});
      else compute(std::false_type{}, std::false_type{});
    }
    __builtin_amdgcn_s_waitcnt(0);     // this wave's copies of the next tile landed
    __syncthreads();                   // ... and everyone's; the current buffer is free
  }

  // ---- epilogue: 1/l, gate, bf16 store (lane owns row lr of each block; d values
  // 32*db + 8*(v/4) + 4*half + (v%4))
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) {
    const float lsum = swap_halves_sum(l_run[rb]);
    const int r = wrow0 + 32 * rb + lr;
    if (!wave_active || (r - wrow0) >= wrows) continue;
    const int t = r / L.G;
    const int h = g * L.G + r % L.G;
    const int64_t tok = q0 + t;
    const float inv = lsum > 0.f ? 1.0f / lsum : 0.f;
    const float bh = gate != nullptr ? bf16_to_f32(gate_bias[h]) : 0.f;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d = 32 * db + 8 * q4 + 4 * half;
        float y[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = acc[rb][db][4 * q4 + e] * inv;
        if (gate != nullptr) {
          const u32x2_t gw = *reinterpret_cast<const u32x2_t*>(gate + tok * gate_stride + (int64_t)h * kHeadDim + d);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float gv = bf16_to_f32((gw[e / 2] >> (16 * (e % 2))) & 0xFFFFu) + bh;
            y[e] *= 1.0f / (1.0f + expf(-gv));
          }
        }
        const u32x2_t o = {pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
        *reinterpret_cast<u32x2_t*>(out + tok * out_stride + (int64_t)h * kHeadDim + d) = o;
      }
  }
}

}  // namespace

hipError_t launch_attn_prefill(const LayerParams& L, const BatchParams& B, const CacheParams& C,
                               const void* q, int64_t q_stride, const void* gate,
                               int64_t gate_stride, const void* gate_bias, void* out,
                               int64_t out_stride, hipStream_t stream) {
  if (B.num_tokens == 0 || B.num_seqs == 0 || B.max_q_len == 0) return hipSuccess;
  const int64_t tiles = ((int64_t)B.max_q_len * L.G + kRowsPerBlock - 1) / kRowsPerBlock;
  const dim3 grid((unsigned)tiles, (unsigned)L.Hkv, (unsigned)B.num_seqs), block(kThreads);
  auto launch = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, grid, block, 0, stream, L, B, C, static_cast<const uint16_t*>(q),
                       q_stride, static_cast<const uint16_t*>(gate), gate_stride,
                       static_cast<const uint16_t*>(gate_bias), static_cast<uint16_t*>(out),
                       out_stride);
  };
  if (L.kind == BEAM_LAYER_SWA) launch(prefill_kernel<BEAM_LAYER_SWA>);
  else launch(prefill_kernel<BEAM_LAYER_FULL>);
  return hipGetLastError();
}

}  // namespace beam
