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
//  * 4 waves x 64 rows; a wave computes S^T = K Q^T with MFMA 32x32x16 bf16 for two
//    32-row blocks that share each K operand read from LDS. After the MFMA, a lane holds
//    32 scores of one row, so the row max/sum need one cross-half swap (permlane32).
//  * O^T = V^T P^T: P^T is the score accumulator packed to bf16 in place (the key order
//    of the accumulator is the MFMA's k-slot order); V^T is read from the row-major V
//    tile with the gfx950 transposing LDS read ds_read_b64_tr_b16.
//  * K/V tiles are one 64-token page per KV head (16 KiB each), double-buffered in LDS;
//    the next page is fetched into registers while the current one is consumed.
//  * Fully visible tiles skip the mask; tiles wholly outside a wave's rows are skipped.
#include "beam_common.h"

namespace beam {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kRowsPerWave = 64;
constexpr int kRowsPerBlock = kWaves * kRowsPerWave;     // 256
constexpr int kRowBytes = kHeadDim * 2 + 16;             // padded LDS row (bf16)
constexpr int kTileBytes = kPage * kRowBytes;            // one K or V page tile
constexpr float kLog2e = 1.4426950408889634f;

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
__global__ __launch_bounds__(kThreads, 1) void prefill_kernel(
    LayerParams L, BatchParams B, CacheParams C, const uint16_t* __restrict__ q, int64_t q_stride,
    const uint16_t* __restrict__ gate, int64_t gate_stride, const uint16_t* __restrict__ gate_bias,
    uint16_t* out, int64_t out_stride) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[2 * 2 * kTileBytes];

  const int tile = blockIdx.x;
  const int g = blockIdx.y;
  const int b = blockIdx.z;
  const int tid = threadIdx.x;
  const int wave = tid / 64;
  const int lane = tid % 64;
  const int half = lane / 32;      // which 8-slice of each 16-wide k step this lane feeds
  const int lr = lane % 32;        // the row (within a 32-row block) this lane owns

  const int64_t q0 = B.q_start[b];
  const int64_t n = (int64_t)B.q_start[b + 1] - q0;
  const int64_t rows_b = n * L.G;
  const int64_t tile_row0 = (int64_t)tile * kRowsPerBlock;
  if (n <= 0 || tile_row0 >= rows_b) return;
  const int64_t kv = B.kv_len[b];
  const int64_t first_pos = kv - n;
  constexpr bool swa = KIND == BEAM_LAYER_SWA;
  const int64_t tile_rows = rows_b - tile_row0 < kRowsPerBlock ? rows_b - tile_row0 : kRowsPerBlock;

  // key range of the workgroup
  const int64_t pos_first = first_pos + tile_row0 / L.G;
  const int64_t pos_last = first_pos + (tile_row0 + tile_rows - 1) / L.G;
  const int64_t key_lo = swa ? (pos_first - L.window + 1 > 0 ? pos_first - L.window + 1 : 0) : 0;
  const int64_t kt_begin = key_lo / kPage;
  const int64_t kt_end = pos_last / kPage + 1;            // exclusive

  // rows of this wave
  const int64_t wrow0 = tile_row0 + wave * kRowsPerWave;
  const int64_t wrows = tile_row0 + tile_rows - wrow0;    // may be <= 0
  const bool wave_active = wrows > 0;
  const int64_t w_min_pos = first_pos + (wave_active ? wrow0 / L.G : 0);
  const int64_t w_max_pos = first_pos + (wave_active ? (wrow0 + (wrows < kRowsPerWave ? wrows : kRowsPerWave) - 1) / L.G : -1);
  const int64_t w_max_lo = swa ? (w_max_pos - L.window + 1 > 0 ? w_max_pos - L.window + 1 : 0) : 0;
  const int64_t w_min_lo = swa ? (w_min_pos - L.window + 1 > 0 ? w_min_pos - L.window + 1 : 0) : 0;

  // per-lane rows: Q^T operand, position, window start
  bf16x8_t qop[2][8];
  int64_t row_pos[2], row_lo[2];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int64_t r = wrow0 + 32 * rb + lr;
    const bool valid = wave_active && (r - wrow0) < wrows;
    const int64_t t = valid ? r / L.G : 0;
    const int h = g * L.G + (int)(valid ? r % L.G : 0);
    row_pos[rb] = valid ? first_pos + t : -1;
    row_lo[rb] = (swa && valid) ? (row_pos[rb] - L.window + 1 > 0 ? row_pos[rb] - L.window + 1 : 0) : 0;
    const uint16_t* qrow = q + (q0 + t) * q_stride + (int64_t)h * kHeadDim;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      u32x4_t v = {0u, 0u, 0u, 0u};
      if (valid) v = *reinterpret_cast<const u32x4_t*>(qrow + 16 * i + 8 * half);
      qop[rb][i] = __builtin_bit_cast(bf16x8_t, v);
    }
  }

  const float c = L.sm_scale * kLog2e;
  float m_run[2] = {-INFINITY, -INFINITY};
  float l_run[2] = {0.f, 0.f};
  f32x16_t acc[2][4];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[rb][db][e] = 0.f;

  // ---- global -> register staging of one K and one V page tile (4 x 16 B each per thread)
  const uint16_t* kcache = static_cast<const uint16_t*>(C.k);
  const uint16_t* vcache = static_cast<const uint16_t*>(C.v);
  const int st_row = tid / 16;          // + 16 * it
  const int st_col = (tid % 16) * 8;    // elements
  u32x4_t stage_k[4], stage_v[4];
  auto fetch = [&](int64_t kt) {
    const int64_t page = B.block_table[(int64_t)b * B.max_pages + kt];
    const int64_t base = (page * L.Hkv + g) * (int64_t)kPage * kHeadDim;
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int r = st_row + 16 * it;
      const int64_t off = base + (int64_t)r * kHeadDim + st_col;
      stage_k[it] = *reinterpret_cast<const u32x4_t*>(kcache + off);
      stage_v[it] = *reinterpret_cast<const u32x4_t*>(vcache + off);
      if (kt * kPage + r >= kv) {   // slots past the sequence may hold NaN
        stage_k[it] = u32x4_t{0u, 0u, 0u, 0u};
        stage_v[it] = u32x4_t{0u, 0u, 0u, 0u};
      }
    }
  };
  auto commit = [&](int buf) {
    unsigned char* kt_lds = lds + buf * 2 * kTileBytes;
    unsigned char* vt_lds = kt_lds + kTileBytes;
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int r = st_row + 16 * it;
      *reinterpret_cast<u32x4_t*>(kt_lds + r * kRowBytes + st_col * 2) = stage_k[it];
      *reinterpret_cast<u32x4_t*>(vt_lds + r * kRowBytes + st_col * 2) = stage_v[it];
    }
  };

  fetch(kt_begin);
  commit(0);
  __syncthreads();

  for (int64_t kt = kt_begin; kt < kt_end; ++kt) {
    const int buf = (int)((kt - kt_begin) & 1);
    const bool has_next = kt + 1 < kt_end;
    if (has_next) fetch(kt + 1);
    const int64_t k0 = kt * kPage;
    const bool skip = !wave_active || k0 > w_max_pos || k0 + kPage - 1 < w_min_lo;
    if (!skip) {
      const unsigned char* kt_lds = lds + buf * 2 * kTileBytes;
      const unsigned char* vt_lds = kt_lds + kTileBytes;
      // ---- S^T = K Q^T for 2 key blocks x 2 row blocks
      f32x16_t sc[2][2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
          for (int e = 0; e < 16; ++e) sc[kb][rb][e] = 0.f;
        const unsigned char* krow = kt_lds + (32 * kb + lr) * kRowBytes + 16 * half;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const bf16x8_t kop = *reinterpret_cast<const bf16x8_t*>(krow + 32 * i);
#pragma unroll
          for (int rb = 0; rb < 2; ++rb)
            sc[kb][rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qop[rb][i], sc[kb][rb], 0, 0, 0);
        }
      }
      const bool need_mask = (k0 + kPage - 1 > w_min_pos) || (k0 < w_max_lo);
      bf16x8_t pop[2][4];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        if (need_mask) {
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              const int64_t j = k0 + 32 * kb + (v / 4) * 8 + half * 4 + (v % 4);
              if (j > row_pos[rb] || j < row_lo[rb]) sc[kb][rb][v] = -INFINITY;
            }
        }
        float mx = sc[0][rb][0];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int v = 0; v < 16; ++v) mx = fmaxf(mx, sc[kb][rb][v]);
        mx = swap_halves_max(mx);
        const float m_new = fmaxf(m_run[rb], mx * c);
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m_run[rb] - m_use);
        float psum = 0.f;
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
          bf16x8_t pb;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float p = __builtin_amdgcn_exp2f(fmaf(sc[cc / 2][rb][8 * (cc % 2) + j], c, -m_use));
            psum += p;
            pb[j] = (__bf16)p;
          }
          pop[rb][cc] = pb;
        }
        l_run[rb] = l_run[rb] * alpha + psum;
        m_run[rb] = m_new;
#pragma unroll
        for (int db = 0; db < 4; ++db) acc[rb][db] *= alpha;
      }
      // ---- O^T += V^T P^T
      const int grp = lane / 16, gi = lane % 16;
      const int hh = grp / 2;
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const int col = 32 * db + 16 * (grp % 2) + 4 * (gi % 4);
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
          const unsigned char* a0 = vt_lds + (16 * cc + 4 * hh + gi / 4) * kRowBytes + col * 2;
          const unsigned char* a1 = a0 + 8 * kRowBytes;
          const i16x4_t t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) i16x4_t*)(a0));
          const i16x4_t t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) i16x4_t*)(a1));
          const u32x2_t u0 = __builtin_bit_cast(u32x2_t, t0), u1 = __builtin_bit_cast(u32x2_t, t1);
          const u32x4_t uv = {u0[0], u0[1], u1[0], u1[1]};
          const bf16x8_t vop = __builtin_bit_cast(bf16x8_t, uv);
#pragma unroll
          for (int rb = 0; rb < 2; ++rb)
            acc[rb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pop[rb][cc], acc[rb][db], 0, 0, 0);
        }
      }
    }
    if (has_next) {
      commit(buf ^ 1);
    }
    __syncthreads();
  }

  // ---- epilogue: 1/l, gate, bf16 store (lane owns row lr of each block; d values
  // 32*db + 8*(v/4) + 4*half + (v%4))
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const float lsum = swap_halves_sum(l_run[rb]);
    const int64_t r = wrow0 + 32 * rb + lr;
    if (!wave_active || (r - wrow0) >= wrows) continue;
    const int64_t t = r / L.G;
    const int h = g * L.G + (int)(r % L.G);
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
