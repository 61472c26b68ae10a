// Weight generation for stacked GDPA layers: K (or V) = C W^T, and its weight
// gradient dW = dK^T C.  The Telegram review of the Kunlun paper (layer step 1)
// and the paper summary (section 2.1, interaction block) say K and V are
// generated from the context features; the pages give no further detail, so this
// is read as one linear map per layer, with the weight stored output-major
// ([cols][ctx_dim], the usual layout of a linear layer's weight).
//
// One kernel computes C[M][N] = sum_k A(m, k) B(n, k) in bf16 with fp32
// accumulation, where each operand is given either k-contiguous ([M][K] / [N][K])
// or k-major ([K][M] / [K][N]):
//   forward : out[B][cols]      = ctx[B][c]  . W[cols][c]^T   (both k-contiguous)
//   gradient: dW[cols][c]       = dK[B][cols]^T . ctx[B][c]   (both k-major)
// Operands are staged in LDS as [row][k] tiles (k-major operands are transposed
// while staging, two k values per 4-byte write), so every MFMA operand read is a
// conflict-free 16-byte LDS read.  Work-group tile 128 x 256, 4 waves of
// 64 x 128 (2 x 4 tiles of 32x32x16 MFMA), k steps of 32, next step's global
// loads issued before the current step's MFMAs, LDS double-buffered.  The 1-D
// grid is remapped so that the tiles sharing an operand tile (all M tiles of one
// N tile, or the reverse, whichever dimension has fewer tiles) run back to back
// on one XCD and read that operand tile from its L2 once.
#include "gdpa_device.h"
#include "gdpa_launch.h"

namespace gdpa {

namespace {
constexpr int GM = 128, GN = 256, GK = 32, GLD = GK + 8;  // tile sizes; LDS row stride
constexpr int GT = 256;                                     // threads

// Global -> register staging of one operand tile with ROWS rows (m or n) for the
// k range [k0, k0 + 32).  k-contiguous operand: a chunk is 8 consecutive k of one
// row.  k-major operand: a chunk is 8 consecutive rows of one k pair (2 x 16 B).
template <int ROWS, bool KMAJOR>
struct Stage {
  static constexpr int CHUNKS = KMAJOR ? (GK / 2) * (ROWS / 8) : ROWS * (GK / 8);
  static constexpr int PER = CHUNKS / GT;  // chunks per thread
  static constexpr int REGS = KMAJOR ? 2 : 1;
  u32x4 r[PER][REGS];

  // rows [row0, row0 + ROWS) of a matrix with `rows_total` rows and `kdim` k;
  // ld = leading dimension in elements.  Rows / k beyond the matrix read a
  // clamped valid address; their values are masked at the LDS write.
  __device__ __forceinline__ void load(const uint16_t* __restrict__ p, long ld, long row0,
                                       long rows_total, int k0, int kdim, int tid) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int c = i * GT + tid;
      if (!KMAJOR) {
        const long row = min(row0 + c / (GK / 8), rows_total - 1);
        const int k = min(k0 + 8 * (c % (GK / 8)), kdim - 8);
        r[i][0] = gload16(p + row * ld + k);
      } else {
        const int kp = c % (GK / 2);             // k pair
        const long row = min(row0 + 8 * (c / (GK / 2)), rows_total - 8);
        const int ka = min(k0 + 2 * kp, kdim - 1), kb = min(k0 + 2 * kp + 1, kdim - 1);
        r[i][0] = gload16(p + (long)ka * ld + row);
        r[i][1] = gload16(p + (long)kb * ld + row);
      }
    }
  }

  __device__ __forceinline__ void store(uint16_t* lds, long row0, long rows_total, int k0,
                                        int kdim, int tid) const {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int c = i * GT + tid;
      if (!KMAJOR) {
        const int rl = c / (GK / 8), kl = 8 * (c % (GK / 8));
        const bool ok = row0 + rl < rows_total && k0 + kl < kdim;
        lds_write16(&lds[rl * GLD + kl], ok ? r[i][0] : u32x4{});
      } else {
        const int kp = c % (GK / 2), rl = 8 * (c / (GK / 2));
        const bool kok0 = k0 + 2 * kp < kdim, kok1 = k0 + 2 * kp + 1 < kdim;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int sh = 16 * (e & 1);
          const uint32_t lo = kok0 ? (r[i][0][e >> 1] >> sh) & 0xffffu : 0u;
          const uint32_t hi = kok1 ? (r[i][1][e >> 1] >> sh) & 0xffffu : 0u;
          const bool rok = row0 + rl + e < rows_total;
          *(GDPA_LDS uint32_t*)(&lds[(rl + e) * GLD + 2 * kp]) = rok ? (lo | (hi << 16)) : 0u;
        }
      }
    }
  }
};
}  // namespace

template <bool AK, bool BK>
__global__ __launch_bounds__(GT, 2) void gemm_bf16_kernel(int M, long N, int K,
                                                          const uint16_t* __restrict__ A, long lda,
                                                          const uint16_t* __restrict__ Bm, long ldb,
                                                          uint16_t* __restrict__ C) {
  __shared__ __align__(16) uint16_t As[2][GM * GLD];
  __shared__ __align__(16) uint16_t Bs[2][GN * GLD];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lr = lane & 31, g = lane >> 5;
  const long mt = (M + GM - 1) / GM, nt = (N + GN - 1) / GN;
  const long wid = xcd_remap(blockIdx.x, gridDim.x);
  if (wid >= mt * nt) return;
  const bool m_inner = mt <= nt;
  const long m0 = (m_inner ? wid % mt : wid / nt) * GM;
  const long n0 = (m_inner ? wid / mt : wid % nt) * GN;
  const int wm = (wave >> 1) * 64, wn = (wave & 1) * 128;

  Stage<GM, AK> sa;
  Stage<GN, BK> sb;
  f32x16 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

  const int nk = (K + GK - 1) / GK;
  sa.load(A, lda, m0, M, 0, K, tid);
  sb.load(Bm, ldb, n0, N, 0, K, tid);
  sa.store(As[0], m0, M, 0, K, tid);
  sb.store(Bs[0], n0, N, 0, K, tid);
  __syncthreads();

  for (int ks = 0; ks < nk; ++ks) {
    const int buf = ks & 1;
    const bool more = ks + 1 < nk;
    if (more) {
      sa.load(A, lda, m0, M, (ks + 1) * GK, K, tid);
      sb.load(Bm, ldb, n0, N, (ks + 1) * GK, K, tid);
    }
    const uint16_t* as = As[buf];
    const uint16_t* bs = Bs[buf];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      bf16x8 af[2], bfr[4];
#pragma unroll
      for (int i = 0; i < 2; ++i) af[i] = lds_read8(&as[(wm + 32 * i + lr) * GLD + 16 * kk + 8 * g]);
#pragma unroll
      for (int j = 0; j < 4; ++j) bfr[j] = lds_read8(&bs[(wn + 32 * j + lr) * GLD + 16 * kk + 8 * g]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma32(af[i], bfr[j], acc[i][j]);
    }
    if (more) {
      sa.store(As[buf ^ 1], m0, M, (ks + 1) * GK, K, tid);
      sb.store(Bs[buf ^ 1], n0, N, (ks + 1) * GK, K, tid);
    }
    __syncthreads();
  }

  // Lane (n + 32 g), register r: row 8 (r / 4) + 4 g + r % 4 of the 32x32 tile.
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const long col = n0 + wn + 32 * j + lr;
      if (col >= N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const long row = m0 + wm + 32 * i + 8 * (r >> 2) + 4 * g + (r & 3);
        if (row < M) C[row * N + col] = __builtin_bit_cast(uint16_t, f2bf(acc[i][j][r]));
      }
    }
}

// Forward weight generation, both operands k-contiguous: C[M][N] = A[M][K] . B[N][K]^T.
// Persistent work-groups (one per CU), each walking output tiles of 256 (m) x 256 (n)
// with 8 waves of 128 (m) x 64 (n).  Operands reach LDS by asynchronous global->LDS
// copies into a 2-stage ring of k steps of 64 that runs on across tile boundaries, one
// step (64 MFMAs per SIMD) ahead of the MFMAs; each wave issues eight 1 KiB copies
// (8 rows of 128 bytes) per step, a row's eight 16-byte k chunks stored at positions
// c ^ (row & 7) so that 8 consecutive rows of one chunk fall in distinct banks.  The
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
constexpr int NT_DMA = 2 * NT_IPW;                 // copies per wave per step (8)
constexpr int NT_STORES = 16;                      // 16-byte stores per wave per tile
constexpr int NT_CW_B = 32 * 64 * 2;               // per-wave output staging (32 x 64 bf16)
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
      const int k = min(k0 + 8 * ((lane % (NT_ROW_B / 16)) ^ (row & 7)), K - 8);
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
        xs[j] = lds_read8(&Bs[row * NT_K + 8 * (c ^ (row & 7))]);
        if (tail && kx * NT_K + 8 * c >= K) xs[j] = bf16x8{};
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = wm + 32 * i + lx;
        ys[i] = lds_read8(&As[row * NT_K + 8 * (c ^ (row & 7))]);
      }
    };
    load(0, x[0], y[0]);
#pragma unroll
    for (int kk = 0; kk < NT_K / 16; ++kk) {
      if (kk + 1 < NT_K / 16) load(kk + 1, x[(kk + 1) & 1], y[(kk + 1) & 1]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(x[kk & 1][j], y[kk & 1][i], acc[i][j]);
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

hipError_t launch_gemm_bf16(bool a_kmajor, bool b_kmajor, int M, int64_t N, int K, const void* A,
                            const void* B, void* C, hipStream_t s) {
  if (M == 0 || N == 0) return hipSuccess;
  const long tiles = ((N + GN - 1) / GN) * (((long)M + GM - 1) / GM);
  const dim3 grid((unsigned)((tiles + 7) / 8 * 8)), blk(GT);
  const uint16_t* a = (const uint16_t*)A;
  const uint16_t* b = (const uint16_t*)B;
  uint16_t* c = (uint16_t*)C;
  const long lda = a_kmajor ? (long)M : (long)K;
  const long ldb = b_kmajor ? (long)N : (long)K;
  if (!a_kmajor && !b_kmajor) {
    const long t2 = ((N + NT_N - 1) / NT_N) * (((long)M + NT_M - 1) / NT_M);
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      cus = 256;
    const long grid = (min(t2, (long)cus) + 7) / 8 * 8;
    hipLaunchKernelGGL(gemm_nt_kernel, dim3((unsigned)grid), dim3(NT_T), 0, s, M, (long)N, K, a, b, c);
  }
  else if (a_kmajor && b_kmajor)
    hipLaunchKernelGGL((gemm_bf16_kernel<true, true>), grid, blk, 0, s, M, (long)N, K, a, lda, b, ldb, c);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace gdpa
