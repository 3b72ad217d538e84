// bf16 linear layer y = x W^T for the projections on either side of the attention core:
// the packed Q/K/V/gate projection (hidden 5120 -> 6144 + 1024 + 1024 + 6144 = 14336
// columns) and o_proj (6144 -> 5120), "Reflection Beam 1.0 on vLLM", sections
// "Attention: sliding-window layers plus NoPE full-attention layers" (the gate has its
// own full-width projection) and "Agent-driven optimization" (one packed GEMM feeds the
// fused norm/RoPE kernel); "SGLang natively supports Reflection's Beam", section
// "Hybrid attention and output gating".
//
// What it computes: y[m][n] = bf16( sum_k x[m][k] * w[n][k] ), fp32 accumulation, with x
// [M][K] and w [N][K] both row-major (the weight in its [out][in] layout), so every MFMA
// operand is a run of 8 consecutive k of one row.
//
// Design (MFMA-bound for token counts in the hundreds and up, MI355X):
//  * Workgroup tile 256 (n) x 256 (m), 8 waves as 4 (n) x 2 (m), a wave owning 64 x 128
//    outputs = 2 x 4 blocks of MFMA 32x32x16 bf16 (A operand: W rows, B operand: x rows;
//    the accumulator then holds 4 consecutive n per lane, stored as 8 bytes).
//  * K advances 64 at a time through LDS: 256 rows x 128 bytes of each operand per stage
//    (64 KiB), copied straight from global memory with buffer_load_dwordx4 ... lds through
//    one buffer resource per operand and stage (32-bit lane offsets, no per-lane 64-bit
//    addresses: +4-5% against global_load_lds with 64-bit addresses), double-buffered. gfx950's LDS has 64 four-byte banks, so two 128-byte rows fill them;
//    the 16-byte chunk c of row r is stored at slot c ^ ((r / 2) mod 8), so the 16 rows a
//    16-lane group of an operand read touches (one chunk each) cover all 64 banks.
//  * The output tile goes through LDS as bf16 rows and is stored 512 contiguous bytes per
//    32 lanes (+2.6% on both projections against 8-byte stores scattered over 32 rows).
//  * Workgroups are remapped so that each XCD runs a contiguous range of tiles, ordered
//    4 m-tiles at a time: the ~32 workgroups an XCD runs together cover a 4 x 8 block of
//    tiles and share each x and W slab through its L2.
#include "beam_common.h"

namespace beam {
namespace {

constexpr int kBN = 256, kBM = 256, kBK = 64;
constexpr int kLinWaves = 8;
constexpr int kLinThreads = kLinWaves * 64;
constexpr int kLinRowBytes = kBK * 2;                      // 128 bytes of one row per stage
constexpr int kLinTileBytes = 256 * kLinRowBytes;          // 32 KiB per operand per stage
constexpr int kGroupM = 4;
constexpr int kXcds = 8;

typedef __attribute__((address_space(3))) void lds_void_t;

__global__ __launch_bounds__(kLinThreads) void linear_bf16_kernel(
    int64_t M, int64_t N, int64_t K, const uint16_t* __restrict__ x, int64_t x_stride,
    const uint16_t* __restrict__ w, int64_t w_stride, uint16_t* __restrict__ y,
    int64_t y_stride) {
  __shared__ __attribute__((aligned(1024))) unsigned char lds[2 * 2 * kLinTileBytes];

  // ---- tile of this workgroup: XCD-contiguous ranges, then groups of kGroupM m-tiles
  const int tiles_m = (int)((M + kBM - 1) / kBM), tiles_n = (int)((N + kBN - 1) / kBN);
  const int num = tiles_m * tiles_n;
  const int lin = blockIdx.x;
  const int xcd = lin % kXcds, slot = lin / kXcds;
  const int per = num / kXcds, extra = num % kXcds;
  const int pid = xcd * per + min(xcd, extra) + slot;
  const int in_group = kGroupM * tiles_n;
  const int first_m = (pid / in_group) * kGroupM;
  const int gm = min(tiles_m - first_m, kGroupM);
  const int tm = first_m + (pid % in_group) % gm;
  const int tn = (pid % in_group) / gm;
  const int64_t m0 = (int64_t)tm * kBM, n0 = (int64_t)tn * kBN;

  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64;
  const int wn = wave % 4, wm = wave / 4;
  const int half = lane / 32, lr = lane % 32;

  // ---- copy of one stage: wave w moves rows [32w, 32w + 32) of both tiles, 8 rows per
  // instruction; lane l lands at row 8i + l/8, slot l%8, so it fetches that row's chunk
  // (l%8) ^ ((row/2)%8). Rows past M or N read the last valid row (their results are dropped).
  // Each operand's 256 rows are read through one buffer resource per stage (base in scalar
  // registers) plus a 32-bit lane offset, so a copy needs no 64-bit per-lane address.
  const int64_t nk = K / kBK;
  uint32_t wrow_off[4], xrow_off[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 32 * wave + 8 * i + lane / 8;
    const int chunk = (lane % 8) ^ ((row >> 1) & 7);
    const int64_t wr = min(n0 + row, N - 1) - n0, xr = min(m0 + row, M - 1) - m0;
    wrow_off[i] = (uint32_t)(wr * w_stride * 2 + chunk * 16);
    xrow_off[i] = (uint32_t)(xr * x_stride * 2 + chunk * 16);
  }
  const char* w_tile = reinterpret_cast<const char*>(w) + n0 * w_stride * 2;
  const char* x_tile = reinterpret_cast<const char*>(x) + m0 * x_stride * 2;
  const int w_bytes = (int)(min((int64_t)kBN, N - n0) * w_stride * 2);
  const int x_bytes = (int)(min((int64_t)kBM, M - m0) * x_stride * 2);
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  auto issue_stage = [&](int64_t ks, int buf) {
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(w_tile + ks * kBK * 2), 0, w_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(x_tile + ks * kBK * 2), 0, x_bytes, 0x00020000);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int dst = buf * 2 * kLinTileBytes + (32 * wave_s + 8 * i) * kLinRowBytes;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void_t*)(lds + dst), 16, wrow_off[i], 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void_t*)(lds + dst + kLinTileBytes), 16, xrow_off[i], 0, 0, 0);
    }
  };

  // ---- operand offsets: row lr of a 32-row block, chunk 2*kk + half at slot
  // (2*kk + half) ^ ((lr/2) % 8) (block starts are multiples of 32 rows)
  int op_off[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) op_off[kk] = lr * kLinRowBytes + (((2 * kk + half) ^ ((lr >> 1) & 7)) << 4);

  f32x16_t acc[2][4];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb)
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[nb][mb][e] = 0.f;

  auto compute = [&](int buf) {
    const unsigned char* wt = lds + buf * 2 * kLinTileBytes + (64 * wn) * kLinRowBytes;
    const unsigned char* xt = lds + buf * 2 * kLinTileBytes + kLinTileBytes + (128 * wm) * kLinRowBytes;
    // operands of k step kk + 1 are read (second register set) while step kk's MFMAs run;
    // the scheduling barriers keep the two sets apart
    bf16x8_t a[2][2], bop[2][4];
    auto load = [&](int kk, int set) {
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
        a[set][nb] = *reinterpret_cast<const bf16x8_t*>(wt + nb * 32 * kLinRowBytes + op_off[kk]);
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
        bop[set][mb] = *reinterpret_cast<const bf16x8_t*>(xt + mb * 32 * kLinRowBytes + op_off[kk]);
    };
    load(0, 0);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      if (kk + 1 < 4) load(kk + 1, (kk + 1) & 1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
          acc[nb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[kk & 1][nb], bop[kk & 1][mb], acc[nb][mb], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  issue_stage(0, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  // stages in pairs on buffers (0, 1), so that every LDS operand address is a lane
  // constant plus an immediate
  int64_t ks = 0;
  for (; ks + 1 < nk; ks += 2) {
    issue_stage(ks + 1, 1);
    compute(0);
    __builtin_amdgcn_s_waitcnt(0);     // this wave's copies of the next stage landed
    __syncthreads();                   // ... and everyone's; this buffer is free again
    if (ks + 2 < nk) issue_stage(ks + 2, 0);
    compute(1);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
  if (ks < nk) {                       // an odd last stage, on buffer 0
    compute(0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  // ---- epilogue through LDS (free: the last stage ended with a barrier): the tile as bf16
  // rows [256 m][256 n], 16-byte chunk c of row m at slot c ^ (m mod 32), then each wave
  // stores 32 whole rows, 512 contiguous bytes per 32 lanes. A lane holds D[n][m] for m =
  // its column and 4 consecutive n per register quad.
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    const int ml = 128 * wm + 32 * mb + lr;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int c = 8 * wn + 4 * nb + q4;                 // (64 wn + 32 nb + 8 q4) / 8
        const f32x16_t& d = acc[nb][mb];
        const u32x2_t o = {pack_bf16x2(d[4 * q4], d[4 * q4 + 1]), pack_bf16x2(d[4 * q4 + 2], d[4 * q4 + 3])};
        *reinterpret_cast<u32x2_t*>(lds + ml * 512 + ((c ^ (ml & 31)) << 4) + 8 * half) = o;
      }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int ml = 32 * wave + 2 * i + lane / 32, c = lane % 32;
    const int64_t m = m0 + ml, n = n0 + 8 * c;
    if (m < M && n < N) {
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(lds + ml * 512 + ((c ^ (ml & 31)) << 4));
      uint16_t* dst = y + m * y_stride + n;
      if (n + 8 <= N) *reinterpret_cast<u32x4_t*>(dst) = v;
      else *reinterpret_cast<u32x2_t*>(dst) = u32x2_t{v[0], v[1]};   // n % 8 == 4 at the end
    }
  }
}

}  // namespace

hipError_t launch_linear_bf16(int64_t M, int64_t N, int64_t K, const void* x, int64_t x_stride,
                              const void* w, int64_t w_stride, void* y, int64_t y_stride,
                              hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  const int64_t tiles = ((M + kBM - 1) / kBM) * ((N + kBN - 1) / kBN);
  hipLaunchKernelGGL(linear_bf16_kernel, dim3((unsigned)tiles), dim3(kLinThreads), 0, stream, M, N,
                     K, static_cast<const uint16_t*>(x), x_stride, static_cast<const uint16_t*>(w),
                     w_stride, static_cast<uint16_t*>(y), y_stride);
  return hipGetLastError();
}

}  // namespace beam
