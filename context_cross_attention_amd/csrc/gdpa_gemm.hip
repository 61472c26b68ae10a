// Weight generation for stacked GDPA layers: K (or V) = C W, a plain bf16 GEMM,
// and its weight gradient dW = C^T dK.  The Telegram review of the Kunlun paper
// (layer step 1) and the paper summary (section 2.1, interaction block) say K and
// V are generated from the context features; the pages give no further detail,
// so this is read as one linear map per layer.
//
// C[M][N] = op(A)[M][K] * B[K][N], bf16 operands, fp32 accumulation, bf16 result.
// Work-group tile 128 x 128, 4 waves of 64 x 64 (2 x 2 MFMA 32x32x16 tiles),
// k steps of 32 staged through LDS.  B (and A when transposed) is stored
// row-major in LDS and read column-wise with transpose reads.
#include "gdpa_device.h"
#include "gdpa_launch.h"

namespace gdpa {

template <bool AT>
__global__ __launch_bounds__(256, 2) void gemm_bf16_kernel(int M, long N, int K,
                                                           const uint16_t* __restrict__ A,
                                                           const uint16_t* __restrict__ Bm,
                                                           uint16_t* __restrict__ C) {
  constexpr int BMg = 128, BNg = 128, BK = 32;
  constexpr int LDA = AT ? BMg + 8 : BK + 8;  // A tile: [BK][BMg] if AT else [BMg][BK]
  constexpr int LDB = BNg + 8;                // B tile: [BK][BNg]
  __shared__ __align__(16) uint16_t As[(AT ? BK : BMg) * LDA];
  __shared__ __align__(16) uint16_t Bs[BK * LDB];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lr = lane & 31, g = lane >> 5;
  const int m0 = blockIdx.y * BMg;
  const long n0 = (long)blockIdx.x * BNg;
  const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;

  // Transpose-read lane addressing (contiguous k): lane 16 G + 4 r + c reads row
  // 8 (G / 2) + r (second read + 4), columns 16 (G % 2) + 4 c.
  const int trG = lane >> 4;
  const int tr_row = 8 * (trG >> 1) + ((lane & 15) >> 2), tr_col = 16 * (trG & 1) + 4 * (lane & 3);

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  for (int k0 = 0; k0 < K; k0 += BK) {
    __syncthreads();
    // Stage A: 128 x 32 values = 512 chunks of 8.
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int idx = i * 256 + tid;
      if (AT) {  // A is [K][M]: tile rows k, 16 chunks of 8 along m
        const int kr = idx / 16, c = idx % 16;
        const bool ok = (k0 + kr < K) && (m0 + 8 * c < M);
        lds_write16(&As[kr * LDA + 8 * c],
                    ok ? gload16(A + (size_t)(k0 + kr) * M + m0 + 8 * c) : u32x4{});
      } else {   // A is [M][K]: tile rows m, 4 chunks of 8 along k
        const int mr = idx / 4, c = idx % 4;
        const bool ok = (m0 + mr < M) && (k0 + 8 * c < K);
        lds_write16(&As[mr * LDA + 8 * c],
                    ok ? gload16(A + (size_t)(m0 + mr) * K + k0 + 8 * c) : u32x4{});
      }
    }
    // Stage B: 32 x 128 values.
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int idx = i * 256 + tid;
      const int kr = idx / 16, c = idx % 16;
      const bool ok = (k0 + kr < K) && (n0 + 8 * c < N);
      lds_write16(&Bs[kr * LDB + 8 * c],
                  ok ? gload16(Bm + (size_t)(k0 + kr) * N + n0 + 8 * c) : u32x4{});
    }
    __syncthreads();

#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      bf16x8 af[2], bfr[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        if (AT) {
          const int o = (16 * kk + tr_row) * LDA + wm + 32 * i + tr_col;
          af[i] = cat8(lds_read_tr4(&As[o]), lds_read_tr4(&As[o + 4 * LDA]));
        } else {
          af[i] = lds_read8(&As[(wm + 32 * i + lr) * LDA + 16 * kk + 8 * g]);
        }
        const int ob = (16 * kk + tr_row) * LDB + wn + 32 * i + tr_col;
        bfr[i] = cat8(lds_read_tr4(&Bs[ob]), lds_read_tr4(&Bs[ob + 4 * LDB]));
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(af[i], bfr[j], acc[i][j]);
    }
  }

  // Lane (n + 32 g), register r: row 8 (r / 4) + 4 g + r % 4 of the 32x32 tile.
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const long col = n0 + wn + 32 * j + lr;
      if (col >= N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm + 32 * i + 8 * (r >> 2) + 4 * g + (r & 3);
        if (row < M) C[(size_t)row * N + col] = __builtin_bit_cast(uint16_t, f2bf(acc[i][j][r]));
      }
    }
}

hipError_t launch_gemm_bf16(bool a_trans, int M, int64_t N, int K, const void* A, const void* B,
                            void* C, hipStream_t s) {
  if (M == 0 || N == 0) return hipSuccess;
  const dim3 grid((unsigned)((N + 127) / 128), (unsigned)((M + 127) / 128)), blk(256);
  if (a_trans)
    hipLaunchKernelGGL((gemm_bf16_kernel<true>), grid, blk, 0, s, M, (long)N, K,
                       (const uint16_t*)A, (const uint16_t*)B, (uint16_t*)C);
  else
    hipLaunchKernelGGL((gemm_bf16_kernel<false>), grid, blk, 0, s, M, (long)N, K,
                       (const uint16_t*)A, (const uint16_t*)B, (uint16_t*)C);
  return hipGetLastError();
}

}  // namespace gdpa
