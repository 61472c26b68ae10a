// Weight generation for stacked GDPA layers: K (or V) = C W^T, and its weight
// gradient dW = dK^T C.  The Telegram review of the Kunlun paper (layer step 1)
// and the paper summary (section 2.1, interaction block) say K and V are
// generated from the context features; the pages give no further detail, so this
// is read as one linear map per layer, with the weight stored output-major
// ([cols][ctx_dim], the usual layout of a linear layer's weight).
//
// Two kernels compute C[M][N] = sum_k A(m, k) B(n, k) in bf16 with fp32
// accumulation:
//   forward : out[B][cols] = ctx[B][c] . W[cols][c]^T    (gemm_nt_kernel: both operands
//                                                         k-contiguous)
//   gradient: dW[cols][c]  = dK[B][cols]^T . ctx[B][c]   (gemm_tn_kernel: both k-major)
// Both are persistent (one work-group per CU walking 256 x 256 output tiles), stage
// their operands in LDS with asynchronous global->LDS copies, and write whole row
// segments of the output through a per-wave LDS area.
#include "gdpa_device.h"
#include "gdpa_launch.h"

namespace gdpa {

// Forward weight generation, both operands k-contiguous: C[M][N] = A[M][K] . B[N][K]^T.
// Persistent work-groups (one per CU), each walking output tiles of 256 (m) x 256 (n)
// with 8 waves of 128 (m) x 64 (n).  Operands reach LDS by asynchronous global->LDS
// copies into a 2-stage ring of k steps of 64 that runs on across tile boundaries, one
// step (64 MFMAs per SIMD) ahead of the MFMAs; each wave issues eight 1 KiB copies
// (8 rows of 128 bytes) per step, a row's eight 16-byte k chunks stored at positions
// c ^ nt_swz(row) so that 16 consecutive rows of one chunk fall in distinct banks.  The
// MFMA A operand is B's rows (n) and the B operand A's rows (m), so the C tile gives
// each lane four consecutive n of one m.  A finished tile is written 32 rows at a
// time through a 4 KiB LDS area of the wave's own (no barrier) and stored as whole
// 128-byte row segments while the next tile's copies are in flight.  Rows past M / N
// and k past K read clamped valid addresses; k past K is zeroed in the operand
// registers (K is a multiple of 8).
namespace {
constexpr int NT_M = 256, NT_N = 256, NT_K = 64, NT_T = 512, NT_STAGES = 2;
constexpr int NT_ROW_B = NT_K * 2;                 // bytes per staged row (128)
constexpr int NT_TILE_B = NT_M * NT_ROW_B;         // bytes of one operand tile per stage (32 KiB)
constexpr int NT_STAGE_B = 2 * NT_TILE_B;          // A tile then B tile
constexpr int NT_RPI = 1024 / NT_ROW_B;            // rows per 1 KiB copy instruction (8)
constexpr int NT_IPW = NT_M / 8 / NT_RPI;          // copy instructions per wave per tile (4)
constexpr int NT_STORES = 16;                      // 16-byte stores per wave per tile
constexpr int NT_CW_B = 32 * 64 * 2;               // per-wave output staging (32 x 64 bf16)
// Position swizzle of a staged row's 16-byte chunks.  Rows are 128 bytes, half the
// 256-byte bank period, so rows r and r + 2 start on the same banks; XOR-ing the chunk
// with (r / 2) % 8 puts the 16 rows that one 16-lane phase of a ds_read_b128 reads (same
// chunk) in 16 distinct 16-byte bank groups.
__device__ __forceinline__ int nt_swz(int row) { return (row >> 1) & 7; }
}  // namespace

__global__ __launch_bounds__(NT_T, 1) void gemm_nt_kernel(int M, long N, int K,
                                                          const uint16_t* __restrict__ A,
                                                          const uint16_t* __restrict__ Bm,
                                                          uint16_t* __restrict__ C) {
  static_assert(NT_M == NT_N, "one copy pattern serves both tiles");
  static_assert(NT_STAGES == 2, "the wait counts below assume two stages");
  __shared__ __align__(16) uint8_t ring[NT_STAGES * NT_STAGE_B];  // 128 KiB
  __shared__ __align__(16) uint8_t cstage[8 * NT_CW_B];            // 32 KiB

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lr = lane & 31, g = lane >> 5;
  const int mt = (M + NT_M - 1) / NT_M, nt = (int)((N + NT_N - 1) / NT_N), tiles = mt * nt;
  const int first = xcd_remap(blockIdx.x, gridDim.x), stride = gridDim.x;
  if (first >= tiles) return;
  const int nk = (K + NT_K - 1) / NT_K;
  const int my_tiles = (tiles - first + stride - 1) / stride;
  const int wm = (wave & 1) * 128, wn = (wave >> 1) * 64;

  // A position in this work-group's sequence of (tile, k step) pairs, advanced one k
  // step at a time (no divisions in the loop).
  struct Pos {
    int tile, k;      // index into this work-group's tiles, k step
    int m0;           // first row of the tile
    long n0;          // first column of the tile
  };
  auto locate = [&](Pos& p) {
    const int t = first + min(p.tile, my_tiles - 1) * stride;
    p.m0 = (t % mt) * NT_M;
    p.n0 = (long)(t / mt) * NT_N;
  };
  auto advance = [&](Pos& p) {
    if (++p.k == nk) {
      p.k = 0;
      ++p.tile;
      locate(p);
    }
  };
  auto is_cut = [&](const Pos& p) { return p.m0 + NT_M > M || p.n0 + NT_N > N; };

  // Copies of the step at `p` into stage `st`; positions past the last tile re-read the
  // last tile's (valid) addresses so that every wave always has the same number of
  // copies in flight.  Wave w copies rows 32 w .. 32 w + 31 of both tiles: lane i of
  // instruction q -> row 32 w + 8 q + i / 8, position i % 8.
  auto issue = [&](const Pos& p, int st) {
    const int k0 = (p.tile < my_tiles ? p.k : nk - 1) * NT_K;
    const uint32_t sb = lds_addr(ring) + (uint32_t)(st * NT_STAGE_B);
#pragma unroll
    for (int q = 0; q < NT_IPW; ++q) {
      const int row = 32 * wave + NT_RPI * q + lane / (NT_ROW_B / 16);
      const int k = min(k0 + 8 * ((lane % (NT_ROW_B / 16)) ^ nt_swz(row)), K - 8);
      const uint32_t lo = (uint32_t)((32 * wave + NT_RPI * q) * NT_ROW_B);
      dma16(__builtin_amdgcn_readfirstlane(sb + lo), A + (long)min(p.m0 + row, M - 1) * K + k);
      dma16(__builtin_amdgcn_readfirstlane(sb + NT_TILE_B + lo), Bm + min(p.n0 + row, N - 1) * K + k);
    }
  };

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  Pos cur{0, 0, 0, 0}, nxt{0, 0, 0, 0};
  locate(cur);
  locate(nxt);
  issue(nxt, 0);
  advance(nxt);
  bool stored_last = false, cut_last = false;  // did the previous step end a tile (cut by M / N)
  const int total = my_tiles * nk;
  for (int gs = 0; gs < total; ++gs) {
    // The copies for step gs were issued at the top of step gs - 1; only the stores of
    // a tile that ended with step gs - 1 can be newer.  After a cut tile (masked
    // stores, count not fixed) wait for everything.
    if (stored_last && !cut_last) wait_vmcnt<NT_STORES>();
    else wait_vmcnt<0>();
    __syncthreads();  // step gs landed for every wave; the other stage is free
    issue(nxt, (gs + 1) & 1);
    advance(nxt);

    const int kx = cur.k;
    const uint16_t* As = (const uint16_t*)(ring + (gs & 1) * NT_STAGE_B);
    const uint16_t* Bs = As + NT_TILE_B / 2;
    const int lx = opaque(lr), gx = opaque(g);
    const bool tail = (kx + 1) * NT_K > K;
    // Operands of k sub-step kk + 1 are read while the MFMAs of kk run.
    bf16x8 x[2][2], y[2][4];
    auto load = [&](int kk, bf16x8* xs, bf16x8* ys) {
      const int c = 2 * kk + gx;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int row = wn + 32 * j + lx;
        xs[j] = lds_read8(&Bs[row * NT_K + 8 * (c ^ nt_swz(row))]);
        if (tail && kx * NT_K + 8 * c >= K) xs[j] = bf16x8{};
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = wm + 32 * i + lx;
        ys[i] = lds_read8(&As[row * NT_K + 8 * (c ^ nt_swz(row))]);
      }
    };
    load(0, x[0], y[0]);
#pragma unroll
    for (int kk = 0; kk < NT_K / 16; ++kk) {
      if (kk + 1 < NT_K / 16) load(kk + 1, x[(kk + 1) & 1], y[(kk + 1) & 1]);
      // Fences keep the next sub-step's reads ahead of these MFMAs (left alone, the
      // compiler sinks each read next to its first use).
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(x[kk & 1][j], y[kk & 1][i], acc[i][j]);
      __builtin_amdgcn_sched_barrier(0);
    }

    stored_last = kx == nk - 1;
    cut_last = stored_last && is_cut(cur);
    if (stored_last) {
      // Tile done.  Lane (m + 32 g), register r of C tile (i, j) holds column
      // 32 j + 8 (r / 4) + 4 g + r % 4 of row 32 i + (lane % 32) of the wave's block.
      // Per i: 8-byte LDS writes into 32 rows of 128 bytes (16-byte chunk c of row m at
      // position c ^ (m & 7)), then eight lanes per row read 16 bytes each and store
      // whole row segments: exactly NT_STORES stores per wave when the tile is whole.
      const long m0 = cur.m0, n0 = cur.n0;
      const bool whole = !cut_last;
      uint8_t* cw = cstage + wave * NT_CW_B;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int a4 = 0; a4 < 4; ++a4) {
            const int chunk = 4 * j + a4;
            bf16x4 o;
            o[0] = f2bf(acc[i][j][4 * a4]);
            o[1] = f2bf(acc[i][j][4 * a4 + 1]);
            o[2] = f2bf(acc[i][j][4 * a4 + 2]);
            o[3] = f2bf(acc[i][j][4 * a4 + 3]);
            *(GDPA_LDS bf16x4*)(cw + lr * 128 + 16 * (chunk ^ (lr & 7)) + 8 * g) = o;
          }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int row = 8 * u + (lane >> 3), chunk = lane & 7;
          const u32x4 v = *(const GDPA_LDS u32x4*)(cw + row * 128 + 16 * (chunk ^ (row & 7)));
          const long m = m0 + wm + 32 * i + row, n = n0 + wn + 8 * chunk;
          if (whole || (m < M && n < N)) *(u32x4*)(C + m * N + n) = v;
        }
        acc[i][0] = f32x16{};
        acc[i][1] = f32x16{};
      }
    }
    advance(cur);
  }
  wait_vmcnt<0>();  // copies issued past the end land before the work-group releases its LDS
}

// Weight gradient, both operands k-major: C[M][N] = sum_k A[k][M] B[k][N]
// (dW[cols][c] = dK[B][cols]^T ctx[B][c]).  Same organisation as gemm_nt_kernel
// (persistent work-groups, 256 x 256 tiles, 8 waves of 128 (m) x 64 (n), 2-stage
// global->LDS ring of 64-wide k steps, per-wave LDS staging of the output), but the
// staged tiles are k rows of 256 m (or n) values, so the MFMA operands (8 consecutive
// k per lane) are read with ds_read_b64_tr_b16: in each 16-lane group, lane 4 r + c
// addresses row k + r, columns c0 + 4 c .. + 3, and lane i receives column c0 + i of
// rows k .. k + 3.  A row's 16-byte chunks are stored at positions q ^ (4 (k % 4)):
// rows are 512 bytes apart (same bank alignment), and the 32 lanes of one read phase
// (four rows x four chunks, 256 bytes) then cover all 64 four-byte banks once.  Rows
// past K are clamped and their items zeroed.
namespace {
constexpr int TN_K = 64, TN_T = 512;
constexpr int TN_ROW_B = 256 * 2;              // bytes per staged k row (512)
constexpr int TN_TILE_B = TN_K * TN_ROW_B;     // 32 KiB per operand tile per stage
constexpr int TN_STAGE_B = 2 * TN_TILE_B;
constexpr int TN_IPW = TN_K / 8 / 2;           // copy instructions per wave per tile (2 rows each): 4
constexpr int TN_STORES = 16;
constexpr int TN_CW_B = 32 * 64 * 2;
__device__ __forceinline__ int tn_pos(int q, int k) { return q ^ (4 * (k & 3)); }
}  // namespace

__global__ __launch_bounds__(TN_T, 1) void gemm_tn_kernel(int M, long N, int K,
                                                          const uint16_t* __restrict__ A,
                                                          const uint16_t* __restrict__ Bm,
                                                          uint16_t* __restrict__ C) {
  __shared__ __align__(16) uint8_t ring[2 * TN_STAGE_B];  // 128 KiB
  __shared__ __align__(16) uint8_t cstage[8 * TN_CW_B];   // 32 KiB

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lr = lane & 31, g = lane >> 5;
  const int mt = (M + 255) / 256, nt = (int)((N + 255) / 256), tiles = mt * nt;
  const int first = xcd_remap(blockIdx.x, gridDim.x), stride = gridDim.x;
  if (first >= tiles) return;
  const int nk = (K + TN_K - 1) / TN_K;
  const int my_tiles = (tiles - first + stride - 1) / stride;
  const int wm = (wave & 1) * 128, wn = (wave >> 1) * 64;

  struct Pos {
    int tile, k, m0;
    long n0;
  };
  // Tiles sharing m (the same dK columns, the large operand) are consecutive, so the
  // work-groups of one XCD read each dK block from HBM once and share it through L2.
  auto locate = [&](Pos& p) {
    const int t = first + min(p.tile, my_tiles - 1) * stride;
    p.n0 = (long)(t % nt) * 256;
    p.m0 = (t / nt) * 256;
  };
  auto advance = [&](Pos& p) {
    if (++p.k == nk) {
      p.k = 0;
      ++p.tile;
      locate(p);
    }
  };
  auto is_cut = [&](const Pos& p) { return p.m0 + 256 > M || p.n0 + 256 > N; };

  // Copies: wave w takes k rows 8 w .. 8 w + 7 of both tiles, two rows (1 KiB) per
  // instruction; lane i -> row 8 w + 2 q + i / 32, ring position i % 32.
  auto issue = [&](const Pos& p, int st) {
    const int k0 = (p.tile < my_tiles ? p.k : nk - 1) * TN_K;
    const uint32_t sb = lds_addr(ring) + (uint32_t)(st * TN_STAGE_B);
#pragma unroll
    for (int q = 0; q < TN_IPW; ++q) {
      const int row = 8 * wave + 2 * q + (lane >> 5);
      const int kr = min(k0 + row, K - 1);
      const int c = tn_pos(lane & 31, row);  // chunk of 8 columns held at this position
      const uint32_t lo = (uint32_t)((8 * wave + 2 * q) * TN_ROW_B);
      dma16(__builtin_amdgcn_readfirstlane(sb + lo), A + (long)kr * M + min(p.m0 + 8 * c, M - 8));
      dma16(__builtin_amdgcn_readfirstlane(sb + TN_TILE_B + lo), Bm + (long)kr * N + min(p.n0 + 8 * c, N - 8));
    }
  };

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  Pos cur{0, 0, 0, 0}, nxt{0, 0, 0, 0};
  locate(cur);
  locate(nxt);
  issue(nxt, 0);
  advance(nxt);
  bool stored_last = false, cut_last = false;
  const int total = my_tiles * nk;
  for (int gs = 0; gs < total; ++gs) {
    if (stored_last && !cut_last) wait_vmcnt<TN_STORES>();
    else wait_vmcnt<0>();
    __syncthreads();
    issue(nxt, (gs + 1) & 1);
    advance(nxt);

    const int kx = cur.k;
    const uint8_t* As = ring + (gs & 1) * TN_STAGE_B;
    const uint8_t* Bs = As + TN_TILE_B;
    const int lx = opaque(lane), gx = lx >> 5;
    const int grp_hi = (lx >> 4) & 1, li = lx & 15, rr = li >> 2, cc = li & 3;
    const bool tail = (kx + 1) * TN_K > K;
    // Transpose read of 4 k rows (base kb, kb % 4 == 0) x 16 columns starting at col0.
    auto trd = [&](const uint8_t* tile, int kb, int col0) {
      const int row = kb + rr, col = col0 + 16 * grp_hi + 4 * cc;
      const uint8_t* p = tile + row * TN_ROW_B + 16 * tn_pos(col >> 3, row) + 2 * (col & 7);
      bf16x4 v = lds_read_tr4((const uint16_t*)p);
      if (tail && kx * TN_K + kb + 3 >= K) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (kx * TN_K + kb + e >= K) v[e] = (__bf16)0.f;
      }
      return v;
    };
    bf16x8 x[2][2], y[2][4];
    auto load = [&](int kk, bf16x8* xs, bf16x8* ys) {
      const int kb = 16 * kk + 8 * gx;
#pragma unroll
      for (int j = 0; j < 2; ++j) xs[j] = cat8(trd(Bs, kb, wn + 32 * j), trd(Bs, kb + 4, wn + 32 * j));
#pragma unroll
      for (int i = 0; i < 4; ++i) ys[i] = cat8(trd(As, kb, wm + 32 * i), trd(As, kb + 4, wm + 32 * i));
    };
    // Operands of sub-step kk + 1 are read while the MFMAs of kk run (fences as above).
    load(0, x[0], y[0]);
#pragma unroll
    for (int kk = 0; kk < TN_K / 16; ++kk) {
      if (kk + 1 < TN_K / 16) load(kk + 1, x[(kk + 1) & 1], y[(kk + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(x[kk & 1][j], y[kk & 1][i], acc[i][j]);
      __builtin_amdgcn_sched_barrier(0);
    }

    stored_last = kx == nk - 1;
    cut_last = stored_last && is_cut(cur);
    if (stored_last) {
      // As in gemm_nt_kernel: lane (m + 32 g), register r of C tile (i, j) holds column
      // 32 j + 8 (r / 4) + 4 g + r % 4 of row 32 i + (lane % 32) of the wave's block.
      const long m0 = cur.m0, n0 = cur.n0;
      const bool whole = !cut_last;
      uint8_t* cw = cstage + wave * TN_CW_B;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int a4 = 0; a4 < 4; ++a4) {
            const int chunk = 4 * j + a4;
            bf16x4 o;
            o[0] = f2bf(acc[i][j][4 * a4]);
            o[1] = f2bf(acc[i][j][4 * a4 + 1]);
            o[2] = f2bf(acc[i][j][4 * a4 + 2]);
            o[3] = f2bf(acc[i][j][4 * a4 + 3]);
            *(GDPA_LDS bf16x4*)(cw + lr * 128 + 16 * (chunk ^ (lr & 7)) + 8 * g) = o;
          }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int row = 8 * u + (lane >> 3), chunk = lane & 7;
          const u32x4 v = *(const GDPA_LDS u32x4*)(cw + row * 128 + 16 * (chunk ^ (row & 7)));
          const long m = m0 + wm + 32 * i + row, n = n0 + wn + 8 * chunk;
          if (whole || (m < M && n < N)) *(u32x4*)(C + m * N + n) = v;
        }
        acc[i][0] = f32x16{};
        acc[i][1] = f32x16{};
      }
    }
    advance(cur);
  }
  wait_vmcnt<0>();
}

hipError_t launch_gemm_bf16(bool a_kmajor, bool b_kmajor, int M, int64_t N, int K, const void* A,
                            const void* B, void* C, hipStream_t s) {
  if (M == 0 || N == 0) return hipSuccess;
  if (a_kmajor != b_kmajor) return hipErrorInvalidValue;
  const uint16_t* a = (const uint16_t*)A;
  const uint16_t* b = (const uint16_t*)B;
  uint16_t* c = (uint16_t*)C;
  // Persistent kernels: one work-group per CU (or per tile when there are fewer).
  const long tiles = ((N + 255) / 256) * (((long)M + 255) / 256);
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    cus = 256;
  const dim3 grid((unsigned)((min(tiles, (long)cus) + 7) / 8 * 8));
  if (!a_kmajor)
    hipLaunchKernelGGL(gemm_nt_kernel, grid, dim3(NT_T), 0, s, M, (long)N, K, a, b, c);
  else
    hipLaunchKernelGGL(gemm_tn_kernel, grid, dim3(TN_T), 0, s, M, (long)N, K, a, b, c);
  return hipGetLastError();
}

}  // namespace gdpa
