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
//    a workgroup owns 256 (or 128) consecutive rows (about 43 tokens x 6 heads), so every K/V
//    tile it stages in LDS serves all 6 query heads of the group (GQA reuse) and all of
//    its tokens. Grid: (row tile, KV head, sequence), remapped so that the row tiles of
//    one (sequence, KV head) run on one XCD and share its L2.
//  * K/V tiles are one 64-token page of one KV head (16 KiB each), copied straight from
//    global memory into LDS with buffer_load_dwordx4 ... lds (no staging registers)
//    and double-buffered: the next page is in flight while the current one is consumed.
//    Each 256-byte row is stored with its 16-byte chunks XOR-swizzled by the row index so
//    that the operand reads below hit distinct LDS banks. Page numbers come from the
//    block table through scalar loads, one tile ahead.
//  * Full layers: 8 waves (2 per SIMD) x 32 rows = 256 rows per workgroup. Sliding
//    layers: 4 waves x 32 rows, two workgroups per CU, so that one workgroup's start-up
//    (Q rows, first tile) and end (output) overlap the other's compute -- a sliding row
//    tile only spans about 9 key tiles. Rows of q, gate and out pass through LDS, so
//    that every global access moves whole rows (see prefill_rows). Per 32-key half of a
//    tile a wave computes
//    S^T = K Q^T with MFMA 32x32x16 bf16 (K from LDS, Q^T held in registers); a lane
//    then holds 16 scores of one row, so row max/sum take one cross-half swap
//    (permlane32).
//  * O^T += V^T P^T: P^T is the score accumulator packed to bf16 in place (its key order
//    is the MFMA's k-slot order); V^T comes from the row-major V tile through the
//    transposing LDS read ds_read_b64_tr_b16. The V reads and the next half's K reads
//    are issued before the softmax so that their latency hides behind it.
//  * The running maximum is only raised when a row's maximum grows by more than 2^8
//    (log2 domain), so the 128-value output rescale is skipped on almost every tile;
//    the final division by the same running sum keeps the result exact.
//  * Tiles that every row of the workgroup sees whole run in a loop of their own with no
//    mask; the masked tiles at the window start and at the diagonal run in separate
//    loops, where tiles wholly outside a wave's rows skip compute.
//  * One full-layer workgroup runs per CU at a time. When an XCD's share of row tiles
//    would end in a round that leaves at least half of its CUs idle, each tile of that
//    round runs as two workgroups of 128 rows whose waves form two streams over the two
//    halves of the key tiles, merging their partial softmaxes in LDS (prefill_rows,
//    SPLIT).
#include <type_traits>
#include <utility>

#include "beam_common.h"

namespace beam {
namespace {

// Workgroup shape (prefill_waves, prefill_rows_per_block): waves x one 32-row MFMA block
// each; 8 waves (256 rows) for full layers, 4 (128 rows) for sliding ones, 8 over 128 rows
// with the key split. All keep 2 waves per SIMD (at most 256 VGPRs).
constexpr int kRowsPerWave = 32;
constexpr int kRowBytes = kHeadDim * 2;                  // 256-byte bf16 row, swizzled chunks
constexpr int kTileBytes = kPage * kRowBytes;            // one K or V page tile: 16 KiB
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescaleSlack = 8.0f;                    // log2 headroom before rescaling
constexpr int kNumXcds = 8;                              // MI355X: 8 XCDs x 32 CUs

typedef __attribute__((address_space(3))) void lds_void_t;
// 16-byte direct copy global -> LDS (buffer_load_dwordx4 ... lds) through a buffer
// resource over one page tile: the base sits in scalar registers and each lane adds a
// 32-bit offset, so the tile loop does no 64-bit per-lane address arithmetic. Plain
// functions, so that kernel templates whose copy loops depend on template parameters
// still instantiate in the host compilation pass.
constexpr int kRawBufferWord3 = 0x00020000;          // raw buffer, 32-bit data format (CDNA)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const char* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), 0, bytes, kRawBufferWord3);
}
__device__ __forceinline__ void copy16_to_lds(__amdgpu_buffer_rsrc_t r, uint32_t off, lds_void_t* dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, off, 0, 0, 0);
}
// Lane offsets of a row-data buffer resource (rows of q, gate or out) that lie past its
// range: loads through them return zero and stores are dropped.
constexpr uint32_t kRowRange = 0x80000000u;

// Chunk slot of 16-byte chunk c (0..15) of row r in a swizzled tile: c XOR f(r mod 16),
// f swapping the two 2-bit halves of r's low nibble. f is a bijection, so the 16 rows a
// K-operand read touches at one chunk land in 16 distinct slots; and 4 consecutive rows
// get distinct f(r) >> 2, so the 4 rows x 4 chunks of a transposing V read land in 4
// distinct 4-slot bank groups.
__device__ __forceinline__ int swz_key(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
__device__ __forceinline__ int swz(int r, int c) { return r * kRowBytes + ((c ^ swz_key(r)) << 4); }

__device__ __forceinline__ float swap_halves_max(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_elementwise_maximum(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// BUF of a std::integral_constant<int, BUF> argument, -1 for a run-time int
template <typename T> struct const_buf { static constexpr int value = -1; };
template <int N> struct const_buf<std::integral_constant<int, N>> { static constexpr int value = N; };
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
// f(integral_constant<int, i>) for i = 0 .. N-1, so that i can feed immediates
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}
// Transposing 8-byte LDS read (ds_read_b64_tr_b16) at a 32-bit LDS byte address + OFF.
template <int OFF>
__device__ __forceinline__ u32x2_t lds_read_tr(uint32_t addr) {
  u32x2_t r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
  return r;
}
// Wait for every outstanding LDS read; the values are threaded through the wait so that
// no use of them is scheduled before it.
__device__ __forceinline__ void lds_wait_all(u32x2_t (&v)[2][4][2]) {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int c = 0; c < 2; ++c) asm volatile("" : "+v"(v[a][b][c]));
}
__device__ __forceinline__ float swap_halves_sum(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Work list of a launch: `units` row tiles of the full height (prefill_rows_per_block
// without the split), ordered (sequence, KV head, tile). Blocks are dispatched
// round-robin over the 8 XCDs (each with its own L2), so block `lin` runs on XCD lin % 8;
// each XCD takes a contiguous range of the list, in which the row tiles of one (sequence,
// KV head) are consecutive, so that the blocks streaming the same K/V pages share an L2.
// Full layers may run some units as two blocks of half the rows with the key range split
// between two wave streams (prefill_rows, SPLIT): split_mode 1 splits every unit; 2 splits
// as many of the units of an XCD's last round as that round leaves CUs idle (one prefill
// block runs per CU at a time), the last units of the XCD's range first: those are the
// later row tiles of a (sequence, KV head), which see the most keys.
struct PrefillGrid {
  int32_t units;
  int32_t tiles;           // row tiles per (sequence, KV head)
  int32_t split_mode;      // 0 none, 1 all, 2 last-round units, up to its idle CUs
  int32_t cus_per_xcd;
};

// Units of XCD `xcd`: n of them from `base`, of which the last n_split run split.
__host__ __device__ inline void prefill_xcd_plan(const PrefillGrid& P, int xcd, int* n, int* base,
                                                 int* n_split) {
  const int per = P.units / kNumXcds, extra = P.units % kNumXcds;
  *n = per + (xcd < extra ? 1 : 0);
  *base = xcd * per + (xcd < extra ? xcd : extra);
  *n_split = 0;
  if (P.split_mode == 1) {
    *n_split = *n;
  } else if (P.split_mode == 2 && *n > 0) {
    const int rounds = (*n + P.cus_per_xcd - 1) / P.cus_per_xcd;
    const int last = *n - (rounds - 1) * P.cus_per_xcd;
    const int idle = P.cus_per_xcd - last;
    *n_split = last < idle ? last : idle;
  }
}

// One row tile: rows [tile_row0, tile_row0 + rows per block) of the (token, query head)
// rows of KV head g of sequence b. `lds` is the kernel's LDS array.
//
// SPLIT (full layers): the workgroup's 8 waves form two streams of 4 over the same 128
// rows; the first walks the first half of the key tiles, the second the rest, each with
// its own double-buffered tiles, and the second hands its (max, sum, output) to the first
// through LDS at the end, where they combine as two partial softmaxes do.
template <int KIND, int KV, bool SPLIT>
__device__ __forceinline__ void prefill_rows(
    const LayerParams& L, const BatchParams& B, const CacheParams& C, const uint16_t* __restrict__ q,
    int64_t q_stride, const uint16_t* __restrict__ gate, int64_t gate_stride,
    const uint16_t* __restrict__ gate_bias, uint16_t* out, int64_t out_stride, int tile_row0,
    int g, int b, unsigned char* lds) {
  constexpr int kWaves = prefill_waves(KIND);
  constexpr int kStreams = SPLIT ? 2 : 1;                // key-range streams per workgroup
  constexpr int kStreamWaves = kWaves / kStreams;        // waves sharing one tile stream
  constexpr int kStreamThreads = kStreamWaves * 64;
  constexpr int kRowsPerBlock = kStreamWaves * kRowsPerWave;
  constexpr int kStreamLds = 2 * 2 * kTileBytes;         // two buffers of one K and one V tile
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);   // uniform: kept in a scalar register
  const int kstream = SPLIT ? wave / kStreamWaves : 0;   // 1: the second key half
  const int rwave = SPLIT ? wave % kStreamWaves : wave;  // this wave's 32-row block of the tile
  const int stid = SPLIT ? tid % kStreamThreads : tid;   // thread index among its stream's waves
  const int lds_base = kstream * kStreamLds;   // this stream's tile buffers
  const int lane = tid % 64;
  const int half = lane / 32;      // which 8-slice of each 16-wide k step this lane feeds
  const int lr = lane % 32;        // the row (within a 32-row block) this lane owns
  constexpr bool swa = KIND == BEAM_LAYER_SWA;

  const int q0 = B.q_start[b];
  const int n = B.q_start[b + 1] - q0;
  const int rows_b = n * L.G;
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
  // this wave's stream: all of them, or (SPLIT) the first or second half, the second
  // taking the odd one out
  const int kt_mid = kt_begin + (kt_end - kt_begin) / 2;
  const int s_begin = kstream == 1 ? kt_mid : kt_begin;
  const int s_end = (SPLIT && kstream == 0) ? kt_mid : kt_end;

  // rows of this wave
  const int wrow0 = tile_row0 + rwave * kRowsPerWave;
  const int wrows = min(tile_row0 + tile_rows - wrow0, kRowsPerWave);   // may be <= 0
  const bool wave_active = wrows > 0;
  const int w_min_pos = wave_active ? first_pos + wrow0 / L.G : 0;
  const int w_max_pos = wave_active ? first_pos + (wrow0 + wrows - 1) / L.G : -1;
  const int w_max_lo = swa ? max(w_max_pos - L.window + 1, 0) : 0;
  const int w_min_lo = swa ? max(w_min_pos - L.window + 1, 0) : 0;

  // per-lane row: Q^T operand, position, window start
  bf16x8_t qop[8];
  const int my_row = wrow0 + lr;
  const bool row_valid = wave_active && lr < wrows;
  const int row_pos = row_valid ? first_pos + my_row / L.G : -1;
  const int row_lo = (swa && row_valid) ? max(row_pos - L.window + 1, 0) : 0;

  // Rows of q, gate and out go through LDS, so that each global access instruction moves
  // whole 256-byte rows (4 rows, 1 KiB) instead of 16 or 8 bytes of 32 rows. A sliding
  // row tile sees only about nine key tiles, so these moves are a large share of its
  // time. Q is copied straight into LDS with the first tile, the gate during the last
  // tile, and the gated output is assembled in place of the gate, then stored row by
  // row. Each wave moves its own 32 rows, swizzled like the K/V tiles. Row R of the tile
  // is token t_first + (r0m + R) / G, head g G + (r0m + R) % G. Full layers keep them in
  // the upper half of the kernel's LDS (otherwise used only by split blocks' second
  // stream); sliding layers use the second tile buffer for Q and the free buffer of the
  // last tile for the gate. Split blocks load Q into registers and store from them.
  constexpr bool kRowLds = !SPLIT;
  constexpr int kRowRegion = swa ? -1 : 4 * kTileBytes;
  const int t_first = tile_row0 / L.G;
  const int r0m = tile_row0 - t_first * L.G;
  const float inv_g = 1.0f / (float)L.G;
  // byte offset of chunk slot (ln % 16) of row 32 rwave + 4 i + ln / 16 in a row tensor
  // of token stride `stride` (elements), relative to token t_first; past the tile's
  // rows, an offset outside the buffer range. The entry point bounds the strides at
  // 4,194,303 elements, so that the farthest row (255 tokens on, when G = 1) stays below
  // 2^31 bytes. x / G is taken in fp32: x < 2^9, so x + 0.5 over G is at least 0.5 / G
  // from an integer, far beyond the rounding of the product.
  auto row_off = [&](int i, int64_t stride, int ln) -> uint32_t {
    const int r = 32 * rwave + 4 * i + ln / 16;
    const int x = r0m + r;
    const int t = (int)(((float)x + 0.5f) * inv_g);
    const int hh = x - t * L.G;
    const int chunk = (ln % 16) ^ swz_key(r);
    const uint32_t off = (uint32_t)(t * (int)stride + (g * L.G + hh) * kHeadDim) * 2u + chunk * 16;
    return r < tile_rows ? off : kRowRange;
  };
  auto row_rsrc = [&](const uint16_t* base, int64_t stride) {
    return tile_rsrc(reinterpret_cast<const char*>(base + (int64_t)(q0 + t_first) * stride), (int)kRowRange);
  };
  // copy this wave's 32 rows of a row tensor into LDS at `dst` (+ 32 rwave rows)
  auto issue_rows = [&](const uint16_t* base, int64_t stride, int dst) {
    const __amdgpu_buffer_rsrc_t r = row_rsrc(base, stride);
    // the lane index made opaque, so that the offsets are formed here: the gate's copy
    // sits inside the tile loops, which would otherwise keep them in registers throughout
    int ln = lane;
    asm volatile("" : "+v"(ln));
#pragma unroll
    for (int i = 0; i < 8; ++i)
      copy16_to_lds(r, row_off(i, stride, ln), (lds_void_t*)(lds + dst + (32 * rwave + 4 * i) * kRowBytes));
  };
  if constexpr (!kRowLds) {
    const int t = row_valid ? my_row / L.G : 0;
    const int h = g * L.G + (row_valid ? my_row % L.G : 0);
    const uint16_t* qrow = q + (int64_t)(q0 + t) * q_stride + (int64_t)h * kHeadDim;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      u32x4_t v = {0u, 0u, 0u, 0u};
      if (row_valid) v = *reinterpret_cast<const u32x4_t*>(qrow + 16 * i + 8 * half);
      qop[i] = __builtin_bit_cast(bf16x8_t, v);
    }
  }

  // fp8 caches: codes are converted exactly to bf16 on their way into LDS; the K scale
  // folds into the softmax scale and the V scale into the final normalisation
  constexpr bool fp8 = KV == BEAM_KV_FP8_E4M3;
  const float c = L.sm_scale * kLog2e * (fp8 ? C.k_scale : 1.0f);
  float m_run = -INFINITY, l_run = 0.f;
  // Loop-carried forms of the running max, so that the common half tile spends no
  // instruction on them: the exponent offset (0 while the row has seen no key) and the
  // rescale threshold in raw-score units (c > 0: the entry point rejects other scales).
  const float inv_c = 1.0f / c;
  float neg_m = 0.f, thr_raw = -INFINITY;
  f32x16_t acc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[db][e] = 0.f;

  // ---- lane-constant LDS offsets. Every tile row this lane touches has a fixed residue
  // mod 16, so each swizzled offset is a lane constant plus a compile-time immediate
  // (buffer, 32-key half, 16-key step).
  const int grp = lane / 16, gi = lane % 16;
  const uint32_t lds_addr = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)lds;
  int k_off[8];                       // K operand: row lr (+32 per half), chunk 2i + half
#pragma unroll
  for (int i = 0; i < 8; ++i) k_off[i] = lds_base + lr * kRowBytes + (((2 * i + half) ^ swz_key(lr)) << 4);
  // V operand, transposing reads: rows rv (+8) of each 16-key step, columns
  // 32*db + 16*(grp%2) + 4*(gi%4) = chunk 4*db + cv, byte 8*(gi%2) inside the chunk
  const int rv = 4 * (grp / 2) + gi / 4, cv = 2 * (grp % 2) + (gi % 4) / 2;
  int v_off0[4], v_off1[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) {
    v_off0[db] = lds_base + rv * kRowBytes + (((4 * db + cv) ^ swz_key(rv)) << 4) + 8 * (gi % 2);
    v_off1[db] = lds_base + (rv + 8) * kRowBytes + (((4 * db + cv) ^ swz_key(rv + 8)) << 4) + 8 * (gi % 2);
  }

  // ---- direct global -> LDS copy of one K and one V page tile. Wave w of a stream
  // copies rows [Rw, Rw + R) of each, R = 64 / (waves of the stream), with R / 4
  // instructions per tensor; an instruction moves 64 lanes x 16 bytes = 4 rows into one
  // contiguous 1 KiB block: lane l lands at row 4i + l/16, chunk slot l%16, so it fetches
  // that row's chunk (l%16) ^ swz_key(row).
  constexpr int kRowsCopied = kPage / kStreamWaves;
  uint32_t cp_off[kRowsCopied / 4];
#pragma unroll
  for (int i = 0; i < kRowsCopied / 4; ++i) {
    const int row = kRowsCopied * rwave + 4 * i + lane / 16;
    cp_off[i] = row * kRowBytes + (((lane % 16) ^ swz_key(row)) << 4);
  }
  // Physical pages come through scalar loads: the block table is read-only for the
  // kernel's lifetime, so it is read through the constant address space, one scalar
  // load per tile issued a tile ahead of its use.
  typedef __attribute__((address_space(4))) const int32_t const_i32_t;
  const_i32_t* bt_row = (const_i32_t*)(B.block_table + (int64_t)b * B.max_pages);
  int page_ahead = bt_row[s_begin];      // s_begin < kt_end: a page of the sequence
  constexpr int kSrcTileBytes = fp8 ? kTileBytes / 2 : kTileBytes;   // one head's page in the cache
  const int64_t head_off = (int64_t)g * kSrcTileBytes;
  const int64_t page_bytes = (int64_t)L.Hkv * kSrcTileBytes;
  constexpr int kFp8Reps = kPage * 8 / kStreamThreads;   // fp8 rows staged per thread
  u32x4_t k_stage[kFp8Reps], v_stage[kFp8Reps];
#pragma unroll
  for (int r = 0; r < kFp8Reps; ++r) { k_stage[r] = u32x4_t{0u, 0u, 0u, 0u}; v_stage[r] = k_stage[r]; }
  const int fp8_off = (stid / 8) * kHeadDim + (stid % 8) * 16;   // byte offset in an fp8 page tile
  auto issue_tile = [&](int kt, auto buf_c) {
    constexpr int BUF = decltype(buf_c)::value;
    // page_ahead holds tile kt's page (loaded one issue earlier); fetch the next one
    const int page = page_ahead;
    page_ahead = bt_row[kt + 1 < s_end ? kt + 1 : kt];
    const int64_t base = (int64_t)page * page_bytes + head_off;
    const char* kb = static_cast<const char*>(C.k) + base;
    const char* vb = static_cast<const char*>(C.v) + base;
    if constexpr (!fp8) {
      const __amdgpu_buffer_rsrc_t rk = tile_rsrc(kb, kTileBytes), rv = tile_rsrc(vb, kTileBytes);
#pragma unroll
      for (int i = 0; i < kRowsCopied / 4; ++i) {
        const int dst = lds_base + BUF * 2 * kTileBytes + (kRowsCopied * rwave + 4 * i) * kRowBytes;
        copy16_to_lds(rk, cp_off[i], (lds_void_t*)(lds + dst));
        copy16_to_lds(rv, cp_off[i], (lds_void_t*)(lds + dst + kTileBytes));
      }
    } else {
      // thread stid of the stream loads 16 codes (bytes 16 * (stid % 8) ..) of fp8 rows
      // stid / 8 (+ the stream's thread count / 8) of each tensor into registers;
      // store_staged converts and writes them after this tile
#pragma unroll
      for (int r = 0; r < kFp8Reps; ++r) {
        k_stage[r] = *reinterpret_cast<const u32x4_t*>(kb + fp8_off + r * (kStreamThreads / 8) * kHeadDim);
        v_stage[r] = *reinterpret_cast<const u32x4_t*>(vb + fp8_off + r * (kStreamThreads / 8) * kHeadDim);
      }
    }
  };
  // fp8: the staged codes of the next tile, converted to bf16, into LDS buffer BUF at the
  // same swizzled slots the bf16 copy fills (16 codes = bf16 chunks 2j and 2j + 1)
  auto store_staged = [&](auto buf_c) {
    if constexpr (fp8) {
      constexpr int BUF = decltype(buf_c)::value;
      unsigned char* kt_lds = lds + lds_base + BUF * 2 * kTileBytes;
      // sliding layers: the thread index made opaque, so that the slots below are formed
      // here rather than held in registers across the tile loops (which spilled); full
      // layers keep them (1.5% faster there)
      int st = stid;
      if constexpr (swa) asm volatile("" : "+v"(st));
#pragma unroll
      for (int r = 0; r < kFp8Reps; ++r) {
        const int row = st / 8 + r * (kStreamThreads / 8), j = st % 8;
        const int s0 = row * kRowBytes + (((2 * j) ^ swz_key(row)) << 4);
        const int s1 = row * kRowBytes + (((2 * j + 1) ^ swz_key(row)) << 4);
        *reinterpret_cast<bf16x8_t*>(kt_lds + s0) = fp8x8_to_bf16x8(k_stage[r][0], k_stage[r][1]);
        *reinterpret_cast<bf16x8_t*>(kt_lds + s1) = fp8x8_to_bf16x8(k_stage[r][2], k_stage[r][3]);
        *reinterpret_cast<bf16x8_t*>(kt_lds + kTileBytes + s0) = fp8x8_to_bf16x8(v_stage[r][0], v_stage[r][1]);
        *reinterpret_cast<bf16x8_t*>(kt_lds + kTileBytes + s1) = fp8x8_to_bf16x8(v_stage[r][2], v_stage[r][3]);
      }
    }
  };

  // ---- one 64-key tile from LDS buffer BUF: MASK when some key is invisible to some row
  // of the wave, TAIL when the tile holds slots past the sequence end (NaN allowed there)
  auto compute = [&](int k0, auto buf_v, auto mask_c, auto tail_c) {
    constexpr bool MASK = decltype(mask_c)::value;
    constexpr bool TAIL = decltype(tail_c)::value;
    // a compile-time buffer index puts the buffer offset into the LDS reads' immediates
    constexpr int CB = const_buf<decltype(buf_v)>::value;
    const int buf = CB >= 0 ? 0 : (int)buf_v;
    constexpr int kImm = CB >= 0 ? CB * 2 * kTileBytes : 0;
    const unsigned char* tl = lds + kImm + buf * 2 * kTileBytes;   // this tile's K; V follows
    // per-lane LDS byte addresses of this tile's V operand rows (halves and 16-key steps
    // are immediate offsets on top)
    const uint32_t vbase = lds_addr + buf * 2 * kTileBytes + kTileBytes;
    uint32_t va0[4], va1[4];
#pragma unroll
    for (int db = 0; db < 4; ++db) { va0[db] = vbase + v_off0[db]; va1[db] = vbase + v_off1[db]; }
    // K operands of the first half; the second half's are read while the first computes
    bf16x8_t kop[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) kop[i] = *reinterpret_cast<const bf16x8_t*>(tl + k_off[i]);
    static_for<2>([&](auto kh_c) {           // 32-key halves of the tile
      constexpr int kh = decltype(kh_c)::value;
      __builtin_amdgcn_sched_barrier(0);
      // ---- S^T = K Q^T for this half
      f32x16_t sc;
#pragma unroll
      for (int e = 0; e < 16; ++e) sc[e] = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[i], qop[i], sc, 0, 0, 0);
      // V^T operands of this half (transposing reads, inline assembly: the tile has landed,
      // and the compiler would otherwise also wait for the next tile's copy in flight)
      u32x2_t vr[2][4][2];
      static_for<2>([&](auto cc_c) {
        constexpr int cc = decltype(cc_c)::value;
        constexpr int off = (32 * kh + 16 * cc) * kRowBytes;
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          vr[cc][db][0] = lds_read_tr<off + kImm>(va0[db]);
          vr[cc][db][1] = lds_read_tr<off + kImm>(va1[db]);
        }
      });
      if (kh == 0) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
          kop[i] = *reinterpret_cast<const bf16x8_t*>(tl + 32 * kRowBytes + k_off[i]);
      }
      __builtin_amdgcn_sched_barrier(0);
      // ---- mask, online softmax, P^T in bf16 (k-slot order of the two 16-key steps)
      if (MASK) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int j = k0 + 32 * kh + (v / 4) * 8 + half * 4 + (v % 4);
          if (j > row_pos || j < row_lo) sc[v] = -INFINITY;
        }
      }
      float mx = __builtin_elementwise_maximum(__builtin_elementwise_maximum(sc[0], sc[1]), sc[2]);
#pragma unroll
      for (int v = 3; v < 16; v += 2) mx = __builtin_elementwise_maximum(__builtin_elementwise_maximum(mx, sc[v]), sc[v + 1 < 16 ? v + 1 : v]);
      mx = swap_halves_max(mx);
      // raise the running max only when it grew by more than the slack
      if (__builtin_amdgcn_ballot_w64(mx > thr_raw) != 0) {
        const float m_new = fmaxf(m_run, mx * c);
        // 0 when this row saw no key before; 1 when it still sees none
        const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < 4; ++db) acc[db] *= alpha;
        m_run = m_new;
        neg_m = m_new == -INFINITY ? 0.f : -m_new;
        thr_raw = (m_new + kRescaleSlack) * inv_c;
      }
      bf16x8_t pop[2];
      float psum = -0.f;                   // -0 + p folds to p
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          const float p = __builtin_amdgcn_exp2f(fmaf(sc[8 * cc + jj], c, neg_m));
          psum += p;
          pop[cc][jj] = (__bf16)p;
        }
      }
      l_run += psum;
      lds_wait_all(vr);
      __builtin_amdgcn_sched_barrier(0);
      // ---- O^T += V^T P^T over the 32 keys of this half (2 MFMA k-steps of 16)
#pragma unroll
      for (int cc = 0; cc < 2; ++cc)
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          u32x2_t u0 = vr[cc][db][0], u1 = vr[cc][db][1];
          if (TAIL) {
            // this lane received keys kb0 + 0..3 (u0) and kb0 + 8..11 (u1) at one column
            const int kb0 = k0 + 32 * kh + 16 * cc + 4 * (grp / 2);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const uint32_t m = 0xFFFFu << (16 * (e % 2));
              if (kb0 + e >= kv) u0[e / 2] &= ~m;
              if (kb0 + 8 + e >= kv) u1[e / 2] &= ~m;
            }
          }
          const u32x4_t uv = {u0[0], u0[1], u1[0], u1[1]};
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, uv), pop[cc],
                                                           acc[db], 0, 0, 0);
        }
    });
  };

  // Tiles every row of the workgroup sees whole need no mask; they form one contiguous
  // range [plain_begin, plain_end). The masked tiles before it (window start) and after
  // it (diagonal, sequence end) run a separate loop, so that each loop body has a single
  // straight-line compute and the accumulators stay in place across iterations.
  const int blk_max_lo = swa ? max(pos_last - L.window + 1, 0) : 0;
  const int plain_begin = min(max((blk_max_lo + kPage - 1) / kPage, kt_begin), kt_end);
  const int plain_end = max(min((pos_first + 1) / kPage, kt_end), plain_begin);
  int buf = 0;
  int gate_buf = 0;        // (kRowLds) the LDS buffer the gate rows were copied into
  auto issue_gate = [&](int to_buf) {
    if constexpr (kRowLds) {
      if (gate != nullptr) {
        gate_buf = to_buf;
        issue_rows(gate, gate_stride, swa ? to_buf * 2 * kTileBytes : kRowRegion);
      }
    }
  };
  auto advance = [&](int kt) {
    if (kt + 1 < s_end) {
      if (buf == 0) issue_tile(kt + 1, std::integral_constant<int, 1>{});
      else issue_tile(kt + 1, std::integral_constant<int, 0>{});
    } else {
      issue_gate(buf ^ 1);     // the last tile: the gate rows go into the free buffer
    }
  };
  auto finish = [&](int kt) {
    if (fp8 && kt + 1 < s_end) {
      if (buf == 0) store_staged(std::integral_constant<int, 1>{});
      else store_staged(std::integral_constant<int, 0>{});
    }
    __builtin_amdgcn_s_waitcnt(0);     // this wave's copies of the next tile landed
    __syncthreads();                   // ... and everyone's; this buffer is free again
    buf ^= 1;
  };
  auto masked_step = [&](int kt, auto tail_c) {
    advance(kt);
    const int k0 = kt * kPage;
    const bool skip = !wave_active || k0 > w_max_pos || k0 + kPage - 1 < w_min_lo;
    if (!skip) compute(k0, buf, std::true_type{}, tail_c);
    finish(kt);
  };

  // Only the sequence's last tile can hold slots past its end (whose V may be anything);
  // it runs last, on its own, with the V masking. Plain tiles lie wholly before the
  // first new token, so the tail tile is never one of them. Each stream runs the three
  // ranges clipped to its own tiles [s_begin, s_end).
  const bool tail_tile = kt_end * kPage > kv;
  const bool s_tail = tail_tile && s_end == kt_end;
  const int s_stop = s_tail ? s_end - 1 : s_end;
  const int p_begin = min(max(plain_begin, s_begin), s_end);
  const int p_end = min(max(plain_end, p_begin), s_end);
  if (s_end > s_begin) {
    issue_tile(s_begin, std::integral_constant<int, 0>{});
    store_staged(std::integral_constant<int, 0>{});
  }
  if constexpr (kRowLds) issue_rows(q, q_stride, swa ? 2 * kTileBytes : kRowRegion);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if constexpr (kRowLds) {
    // this lane's row of Q; sliding layers then make sure every wave is done with buffer
    // 1 before the second tile is copied there
    constexpr int kQAt = swa ? 2 * kTileBytes : kRowRegion;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      qop[i] = *reinterpret_cast<const bf16x8_t*>(lds + kQAt + (32 * rwave + lr) * kRowBytes +
                                                  (((2 * i + half) ^ swz_key(lr)) << 4));
    if constexpr (swa) __syncthreads();
  }
  for (int kt = s_begin; kt < min(p_begin, s_stop); ++kt) masked_step(kt, std::false_type{});
  {
    // the plain loop runs tile pairs on buffers (0, 1), so that every LDS buffer address
    // is an immediate; a first tile on buffer 1 and a last one on buffer 0 run alone
    int kt = p_begin;
    if (kt < p_end && buf == 1) {
      advance(kt);
      compute(kt * kPage, buf, std::false_type{}, std::false_type{});
      finish(kt);
      ++kt;
    }
    for (; kt + 1 < p_end; kt += 2) {
      if (kt + 1 < s_end) issue_tile(kt + 1, std::integral_constant<int, 1>{});
      compute(kt * kPage, std::integral_constant<int, 0>{}, std::false_type{}, std::false_type{});
      if (fp8 && kt + 1 < s_end) store_staged(std::integral_constant<int, 1>{});
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (kt + 2 < s_end) issue_tile(kt + 2, std::integral_constant<int, 0>{});
      else issue_gate(0);
      compute((kt + 1) * kPage, std::integral_constant<int, 1>{}, std::false_type{}, std::false_type{});
      if (fp8 && kt + 2 < s_end) store_staged(std::integral_constant<int, 0>{});
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
    if (kt < p_end) {
      advance(kt);
      compute(kt * kPage, buf, std::false_type{}, std::false_type{});
      finish(kt);
      ++kt;
    }
  }
  for (int kt = p_end; kt < s_stop; ++kt) masked_step(kt, std::false_type{});
  if (s_tail) masked_step(s_end - 1, std::true_type{});

  if constexpr (SPLIT) {
    // Every wave has passed one barrier per tile of its stream plus the first; the
    // first stream holds at most one tile fewer and passes the missing barrier here,
    // so that both streams meet the barriers below together.
    for (int i = s_end - s_begin; i < kt_end - kt_mid; ++i) __syncthreads();
    __syncthreads();                   // every tile read is done: LDS is free
    // the second stream's per-lane (max, sum, 64 accumulators), lane-contiguous, into
    // 66 x 64 floats per row block (67.6 KB for 4 row blocks)
    float* xch = reinterpret_cast<float*>(lds) + rwave * (66 * 64) + lane;
    if (kstream == 1) {
      xch[0] = m_run;
      xch[64] = l_run;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) xch[(2 + 16 * db + e) * 64] = acc[db][e];
    }
    __syncthreads();
    if (kstream == 1) return;
    // two partial softmaxes of one row over disjoint keys, each relative to its own
    // running max (log2 units): rescale both to the larger; a stream that saw no key of
    // the row (max -inf) contributes nothing
    const float m_o = xch[0], l_o = xch[64];
    const float m_new = fmaxf(m_run, m_o);
    const float s_me = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
    const float s_o = m_o == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_o - m_new);
    l_run = l_run * s_me + l_o * s_o;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[db][e] = acc[db][e] * s_me + xch[(2 + 16 * db + e) * 64] * s_o;
  }

  // ---- epilogue: 1/l, gate, bf16 store (lane owns row lr; d values
  // 32*db + 8*(v/4) + 4*half + (v%4))
  const float lsum = swap_halves_sum(l_run);
  if constexpr (kRowLds) {
    if (!wave_active) return;
    // every tile is done (the last tile's barrier), so the tile buffers are free; this
    // wave's rows: full layers' upper LDS half, or (sliding) the gate's buffer, or buffer
    // 0 without a gate
    const int rows_at = (swa ? (gate != nullptr ? gate_buf * 2 * kTileBytes : 0) : kRowRegion) + 32 * rwave * kRowBytes;
    if (row_valid) {
      const float inv = lsum > 0.f ? (fp8 ? C.v_scale : 1.0f) / lsum : 0.f;
      const int h = g * L.G + my_row % L.G;
      const float bh = gate != nullptr ? bf16_to_f32(gate_bias[h]) : 0.f;
      unsigned char* rl = lds + rows_at + lr * kRowBytes + 8 * half;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          // d = 32 db + 8 q4 + 4 half + e: bytes 8 half.. of chunk 4 db + q4
          u32x2_t* pr = reinterpret_cast<u32x2_t*>(rl + (((4 * db + q4) ^ swz_key(lr)) << 4));
          float y[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) y[e] = acc[db][4 * q4 + e] * inv;
          if (gate != nullptr) {
            const u32x2_t gw = *pr;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float gv = bf16_to_f32((gw[e / 2] >> (16 * (e % 2))) & 0xFFFFu) + bh;
              y[e] *= gate_sigmoid(gv);
            }
          }
          *pr = u32x2_t{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
        }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");    // the wave's output rows are in LDS
    const __amdgpu_buffer_rsrc_t ro = row_rsrc(out, out_stride);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(lds + rows_at + (4 * i + lane / 16) * kRowBytes + (lane % 16) * 16);
      __builtin_amdgcn_raw_buffer_store_b128(v, ro, row_off(i, out_stride, lane), 0, 0);
    }
    return;
  }
  if (!row_valid) return;
  const int t = my_row / L.G;
  const int h = g * L.G + my_row % L.G;
  const int64_t tok = q0 + t;
  const float inv = lsum > 0.f ? (fp8 ? C.v_scale : 1.0f) / lsum : 0.f;
  const float bh = gate != nullptr ? bf16_to_f32(gate_bias[h]) : 0.f;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int d = 32 * db + 8 * q4 + 4 * half;
      float y[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) y[e] = acc[db][4 * q4 + e] * inv;
      if (gate != nullptr) {
        const u32x2_t gw = *reinterpret_cast<const u32x2_t*>(gate + tok * gate_stride + (int64_t)h * kHeadDim + d);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float gv = bf16_to_f32((gw[e / 2] >> (16 * (e % 2))) & 0xFFFFu) + bh;
          y[e] *= gate_sigmoid(gv);
        }
      }
      const u32x2_t o = {pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
      *reinterpret_cast<u32x2_t*>(out + tok * out_stride + (int64_t)h * kHeadDim + d) = o;
    }
}

// Launch bound: 512 threads, which also caps every shape at 256 VGPRs, i.e. 2 waves per
// SIMD. One block per entry of the work list (PrefillGrid), plus idle padding blocks.
template <int KIND, int KV>
__global__ __launch_bounds__(512) void prefill_kernel(
    LayerParams L, BatchParams B, CacheParams C, const uint16_t* __restrict__ q, int64_t q_stride,
    const uint16_t* __restrict__ gate, int64_t gate_stride, const uint16_t* __restrict__ gate_bias,
    uint16_t* out, int64_t out_stride, PrefillGrid P) {
  constexpr bool kCanSplit = KIND == BEAM_LAYER_FULL;
  __shared__ __attribute__((aligned(1024))) unsigned char lds[(kCanSplit ? 2 : 1) * 2 * 2 * kTileBytes];
  const int lin = blockIdx.x;
  const int xcd = lin % kNumXcds, slot = lin / kNumXcds;
  int n, base, n_split;
  prefill_xcd_plan(P, xcd, &n, &base, &n_split);
  const int n_plain = n - n_split;
  if (slot >= n_plain + 2 * n_split) return;             // padding
  const bool split = slot >= n_plain;
  const int j = slot - n_plain;                          // split blocks: 2 per unit
  const int unit = split ? base + n_plain + j / 2 : base + slot;
  const int tile = unit % P.tiles;
  const int g = (unit / P.tiles) % L.Hkv;
  const int b = unit / (P.tiles * L.Hkv);
  constexpr int kRows = prefill_rows_per_block(KIND, false);
  if constexpr (kCanSplit) {
    if (split) {
      prefill_rows<KIND, KV, true>(L, B, C, q, q_stride, gate, gate_stride, gate_bias, out, out_stride,
                                   tile * kRows + (j % 2) * (kRows / 2), g, b, lds);
      return;
    }
  }
  prefill_rows<KIND, KV, false>(L, B, C, q, q_stride, gate, gate_stride, gate_bias, out, out_stride,
                                tile * kRows, g, b, lds);
}

}  // namespace

hipError_t launch_attn_prefill(const LayerParams& L, const BatchParams& B, const CacheParams& C,
                               int split_mode, int cus, const void* q, int64_t q_stride,
                               const void* gate, int64_t gate_stride, const void* gate_bias,
                               void* out, int64_t out_stride, hipStream_t stream) {
  if (B.num_tokens == 0 || B.num_seqs == 0 || B.max_q_len == 0) return hipSuccess;
  const int rows_per_block = prefill_rows_per_block(L.kind, false);
  const int64_t tiles = ((int64_t)B.max_q_len * L.G + rows_per_block - 1) / rows_per_block;
  const int64_t units = tiles * L.Hkv * B.num_seqs;
  if (units > 0x3FFFFFFF) return hipErrorInvalidValue;
  PrefillGrid P;
  P.units = (int32_t)units;
  P.tiles = (int32_t)tiles;
  P.split_mode = L.kind == BEAM_LAYER_FULL ? split_mode : 0;
  P.cus_per_xcd = cus / kNumXcds > 0 ? cus / kNumXcds : 1;
  int per_xcd = 0;
  for (int x = 0; x < kNumXcds; ++x) {
    int n, base, n_split;
    prefill_xcd_plan(P, x, &n, &base, &n_split);
    per_xcd = max(per_xcd, n + n_split);
  }
  const dim3 grid((unsigned)(per_xcd * kNumXcds)), block(prefill_waves(L.kind) * 64);
  auto launch = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, grid, block, 0, stream, L, B, C, static_cast<const uint16_t*>(q),
                       q_stride, static_cast<const uint16_t*>(gate), gate_stride,
                       static_cast<const uint16_t*>(gate_bias), static_cast<uint16_t*>(out),
                       out_stride, P);
  };
  const bool f8 = C.dtype == BEAM_KV_FP8_E4M3;
  if (L.kind == BEAM_LAYER_SWA) {
    if (f8) launch(prefill_kernel<BEAM_LAYER_SWA, BEAM_KV_FP8_E4M3>);
    else launch(prefill_kernel<BEAM_LAYER_SWA, BEAM_KV_BF16>);
  } else {
    if (f8) launch(prefill_kernel<BEAM_LAYER_FULL, BEAM_KV_FP8_E4M3>);
    else launch(prefill_kernel<BEAM_LAYER_FULL, BEAM_KV_BF16>);
  }
  return hipGetLastError();
}

}  // namespace beam
