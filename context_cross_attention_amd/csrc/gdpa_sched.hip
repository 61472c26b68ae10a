// Jagged-batch scheduling and small auxiliary passes.
//
// The jagged batch (per-sample user histories of irregular length; Kunlun paper
// summary, section 1, names such uneven shapes as a cause of low hardware
// utilisation) is turned into work lists on the device, so the host never has to
// read the offsets back.
#include "gdpa_device.h"
#include "gdpa_launch.h"

namespace gdpa {

// tile_start[b] = sum_{b' < b} ceil(len(b') / tile_rows), tile_start[B] = total;
// with `order`, the scan runs over the samples order[0], order[1], ... instead.
// One work-group of 1024 threads scans the batch in chunks of 1024 samples.
__global__ __launch_bounds__(1024) void tile_scan_kernel(const int32_t* __restrict__ off, int B,
                                                         int tile_rows,
                                                         int32_t* __restrict__ tile_start,
                                                         const int32_t* __restrict__ order) {
  __shared__ int32_t wave_sums[16];
  __shared__ int32_t carry;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) carry = 0;
  __syncthreads();
  for (int base = 0; base < B; base += 1024) {
    const int b = base + tid;
    int c = 0;
    if (b < B) {
      const int sb = order != nullptr ? order[b] : b;
      const int len = off[sb + 1] - off[sb];
      c = (len + tile_rows - 1) / tile_rows;
    }
    // inclusive scan inside the wave
    int x = c;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int y = __shfl_up(x, d, 64);
      if (lane >= d) x += y;
    }
    if (lane == 63) wave_sums[wave] = x;
    __syncthreads();
    int before = 0;
    for (int w = 0; w < wave; ++w) before += wave_sums[w];
    const int excl = carry + before + x - c;
    if (b < B) tile_start[b] = excl;
    __syncthreads();
    if (tid == 1023) carry = excl + c;
    __syncthreads();
  }
  if (tid == 0) tile_start[B] = carry;
}

// order[] = samples sorted by length, longest first (ties by index), so that
// the hardware dispatcher, which starts work-groups in index order, performs
// longest-processing-time-first list scheduling.  Bitonic sort in LDS.
__global__ __launch_bounds__(1024) void longest_first_kernel(const int32_t* __restrict__ off, int B,
                                                             int32_t* __restrict__ order) {
  __shared__ uint64_t key[kMaxSortBatch];
  const int tid = threadIdx.x;
  int N = 1;
  while (N < B) N <<= 1;
  for (int i = tid; i < N; i += 1024) {
    if (i < B) {
      const uint32_t len = (uint32_t)(off[i + 1] - off[i]);
      key[i] = ((uint64_t)(0x7fffffffu - len) << 32) | (uint32_t)i;
    } else {
      key[i] = ~0ull;
    }
  }
  __syncthreads();
  for (int k = 2; k <= N; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = tid; i < N; i += 1024) {
        const int ixj = i ^ j;
        if (ixj > i) {
          const bool up = (i & k) == 0;
          const uint64_t a = key[i], c = key[ixj];
          if ((a > c) == up) {
            key[i] = c;
            key[ixj] = a;
          }
        }
      }
      __syncthreads();
    }
  }
  for (int i = tid; i < B; i += 1024) order[i] = (int32_t)(key[i] & 0xffffffffu);
}

__global__ void iota_kernel(int32_t* order, int B) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < B) order[i] = i;
}

// dvec[row] = sum_e O[row, e] * dO[row, e] in fp32 (softmax backward term).
// With an output bias ob ([B, H, D]), O holds P V + ob: the term is taken for P V,
// i.e. sum_e (O - ob)[row, e] dO[row, e], row = token * H + head.
// One row of d elements per group of d/8 lanes.
template <int D, bool BF16>
__global__ __launch_bounds__(256) void softmax_dvec_kernel(const void* __restrict__ o,
                                                           const void* __restrict__ d_o, int rows,
                                                           float* __restrict__ dvec, const int32_t* off,
                                                           int B, int H, const float* __restrict__ ob) {
  constexpr int LPR = D / 8;  // lanes per row, 8 elements per lane
  // rows * LPR reaches past 2^31 for large batches (T * H >= 2^27 at d = 128): 64-bit indices.
  const int64_t gtid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t row = gtid / LPR;
  const int part = (int)(gtid % LPR);
  float acc = 0.f;
  if (row < rows) {
    const size_t base = (size_t)row * D + part * 8;
    if (ob != nullptr) {
      const int t = (int)(row / H), h = (int)(row - (int64_t)t * H);
      const float* bp = ob + ((size_t)find_sample(off, B, t) * H + h) * D + part * 8;
      if (BF16) {
        const u32x4 c = *(const u32x4*)((const uint16_t*)d_o + base);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc -= bp[2 * i] * __uint_as_float(c[i] << 16);
          acc -= bp[2 * i + 1] * __uint_as_float(c[i] & 0xffff0000u);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) acc -= bp[i] * ((const float*)d_o)[base + i];
      }
    }
    if (BF16) {
      const u32x4 a = *(const u32x4*)((const uint16_t*)o + base);
      const u32x4 c = *(const u32x4*)((const uint16_t*)d_o + base);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc += __uint_as_float(a[i] << 16) * __uint_as_float(c[i] << 16);
        acc += __uint_as_float(a[i] & 0xffff0000u) * __uint_as_float(c[i] & 0xffff0000u);
      }
    } else {
      const float* a = (const float*)o + base;
      const float* c = (const float*)d_o + base;
#pragma unroll
      for (int i = 0; i < 8; ++i) acc += a[i] * c[i];
    }
  }
#pragma unroll
  for (int d = LPR / 2; d > 0; d >>= 1) acc += __shfl_xor(acc, d, 64);
  if (row < rows && part == 0) dvec[row] = acc;
}

// out = x0 + x1 (+ x2) (+ x3) over n bf16 values (n % 8 == 0), fp32 sums rounded
// once; out may alias any input (each thread reads its 8 values before writing).
__global__ __launch_bounds__(256) void add_bf16_kernel(uint16_t* out, const uint16_t* x0, const uint16_t* x1,
                                                       const uint16_t* x2, const uint16_t* x3, long n8) {
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n8) return;
  const uint16_t* src[4] = {x0, x1, x2, x3};
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    if (src[k] == nullptr) continue;
    const u32x4 v = *(const u32x4*)(src[k] + 8 * i);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[2 * e] += __uint_as_float(v[e] << 16);
      acc[2 * e + 1] += __uint_as_float(v[e] & 0xffff0000u);
    }
  }
  *(bf16x8*)(out + 8 * i) = pack8(acc[0], acc[1], acc[2], acc[3], acc[4], acc[5], acc[6], acc[7]);
}

// Column sums of dO over each sample's tokens: one work-group per (sample, head);
// thread t sums 8 consecutive columns of the rows t / (d / 8), + 256 / (d / 8), ...
template <int D, bool BF16>
__global__ __launch_bounds__(256) void out_bias_grad_kernel(const int32_t* __restrict__ off, const void* __restrict__ d_o,
                                                            int H, float* __restrict__ dob) {
  constexpr int CPR = D / 8, RPS = 256 / CPR;  // threads per row, rows per sweep
  __shared__ float part[RPS][D];
  const int b = blockIdx.x / H, h = blockIdx.x - b * H;
  const int tid = threadIdx.x, c = tid % CPR, r0 = tid / CPR;
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  for (int t = off[b] + r0; t < off[b + 1]; t += RPS) {
    const size_t base = ((size_t)t * H + h) * D + 8 * c;
    if (BF16) {
      const u32x4 v = *(const u32x4*)((const uint16_t*)d_o + base);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] += __uint_as_float(v[e] << 16);
        acc[2 * e + 1] += __uint_as_float(v[e] & 0xffff0000u);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += ((const float*)d_o)[base + e];
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) part[r0][8 * c + e] = acc[e];
  __syncthreads();
  for (int col = tid; col < D; col += 256) {
    float sum = 0.f;
    for (int r = 0; r < RPS; ++r) sum += part[r][col];
    dob[((size_t)b * H + h) * D + col] = sum;
  }
}

hipError_t launch_out_bias_grad(const int32_t* offsets, const void* d_o, int B, int H, int d, bool bf16,
                                float* d_out_bias, hipStream_t s) {
  const dim3 grid((unsigned)((long)B * H)), block(256);
  if ((long)B * H == 0) return hipSuccess;
#define GDPA_OBG(D)                                                                                       \
  if (d == D) {                                                                                           \
    if (bf16) hipLaunchKernelGGL((out_bias_grad_kernel<D, true>), grid, block, 0, s, offsets, d_o, H, d_out_bias); \
    else hipLaunchKernelGGL((out_bias_grad_kernel<D, false>), grid, block, 0, s, offsets, d_o, H, d_out_bias);     \
    return hipGetLastError();                                                                             \
  }
  GDPA_OBG(32) GDPA_OBG(64) GDPA_OBG(128)
#undef GDPA_OBG
  return hipErrorInvalidValue;
}

hipError_t launch_add_bf16(long n, void* out, const void* x0, const void* x1, const void* x2,
                           const void* x3, hipStream_t s) {
  const long n8 = n / 8;
  if (n8 == 0) return hipSuccess;
  hipLaunchKernelGGL(add_bf16_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, s, (uint16_t*)out,
                     (const uint16_t*)x0, (const uint16_t*)x1, (const uint16_t*)x2, (const uint16_t*)x3, n8);
  return hipGetLastError();
}

hipError_t launch_tile_scan(const int32_t* offsets, int B, int tile_rows, int32_t* tile_start,
                            hipStream_t s, const int32_t* order) {
  hipLaunchKernelGGL(tile_scan_kernel, dim3(1), dim3(1024), 0, s, offsets, B, tile_rows,
                     tile_start, order);
  return hipGetLastError();
}

hipError_t launch_longest_first(const int32_t* offsets, int B, int32_t* order, hipStream_t s) {
  if (B <= kMaxSortBatch) {
    hipLaunchKernelGGL(longest_first_kernel, dim3(1), dim3(1024), 0, s, offsets, B, order);
  } else {
    hipLaunchKernelGGL(iota_kernel, dim3((B + 255) / 256), dim3(256), 0, s, order, B);
  }
  return hipGetLastError();
}

hipError_t launch_softmax_dvec(const void* o, const void* d_o, int rows, int d, bool bf16,
                               float* dvec, hipStream_t s, const int32_t* offsets, int B, int H,
                               const float* out_bias) {
  const long threads = (long)rows * (d / 8);
  const dim3 grid((unsigned)((threads + 255) / 256)), block(256);
  if (rows == 0) return hipSuccess;
#define GDPA_DVEC(D)                                                                            \
  if (d == D) {                                                                                 \
    if (bf16) hipLaunchKernelGGL((softmax_dvec_kernel<D, true>), grid, block, 0, s, o, d_o,     \
                                 rows, dvec, offsets, B, H, out_bias);                          \
    else hipLaunchKernelGGL((softmax_dvec_kernel<D, false>), grid, block, 0, s, o, d_o, rows,   \
                            dvec, offsets, B, H, out_bias);                                     \
    return hipGetLastError();                                                                   \
  }
  GDPA_DVEC(32) GDPA_DVEC(64) GDPA_DVEC(128)
#undef GDPA_DVEC
  return hipErrorInvalidValue;
}

}  // namespace gdpa
