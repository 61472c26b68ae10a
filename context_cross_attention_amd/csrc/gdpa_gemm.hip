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
  if (!a_kmajor && !b_kmajor)
    hipLaunchKernelGGL((gemm_bf16_kernel<false, false>), grid, blk, 0, s, M, (long)N, K, a, lda, b, ldb, c);
  else if (a_kmajor && b_kmajor)
    hipLaunchKernelGGL((gemm_bf16_kernel<true, true>), grid, blk, 0, s, M, (long)N, K, a, lda, b, ldb, c);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace gdpa
