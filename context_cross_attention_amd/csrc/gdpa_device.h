// Device-side helpers shared by the GDPA kernels (gfx950 / CDNA4 only).
//
// MFMA operand layouts used throughout (v_mfma_f32_32x32x16_bf16, wave64,
// lane l, g = l / 32):
//   A (32 x 16, M x K): lane l holds A[m = l % 32][k = 8 g + i], i = 0..7
//   B (16 x 32, K x N): lane l holds B[k = 8 g + i][n = l % 32]
//   C (32 x 32):        lane l, register r holds C[m = 8 (r / 4) + 4 g + r % 4][n = l % 32]
// The contraction pairs item i of lane (m + 32 g) of A with item i of lane
// (n + 32 g) of B, so any relabelling of k applied to both operands gives the
// same product; the kernels use that freedom to feed a C tile straight back in
// as an A or B operand.
//
// ds_read_b64_tr_b16 (transpose read from LDS, 4 x 16-bit per lane): within
// each group of 16 lanes, output lane i, item r is element i % 4 of the 8-byte
// chunk addressed by lane 4 r + i / 4 of the group.  If lane 4 r + c of group G
// addresses row R_r(G), columns c0(G) + 4 c .. + 3 of a row-major 16-bit tile,
// lane 16 G + i receives column c0(G) + i of rows R_0..R_3: a column-major
// operand read from a row-major tile.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdpa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define GDPA_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 16-byte LDS read of 8 bf16 (address must be 16-byte aligned).
__device__ __forceinline__ bf16x8 lds_read8(const uint16_t* p) {
  return *(const GDPA_LDS bf16x8*)(p);
}
// Transpose read: see the header comment.  Address must be 8-byte aligned.
__device__ __forceinline__ bf16x4 lds_read_tr4(const uint16_t* p) {
  s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((GDPA_LDS s16x4*)(p));
  return __builtin_bit_cast(bf16x4, v);
}
__device__ __forceinline__ bf16x8 cat8(bf16x4 a, bf16x4 b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ void lds_write16(uint16_t* p, u32x4 v) { *(GDPA_LDS u32x4*)(p) = v; }
__device__ __forceinline__ void lds_write8(uint16_t* p, u32x2 v) { *(GDPA_LDS u32x2*)(p) = v; }

__device__ __forceinline__ u32x4 gload16(const uint16_t* p) { return *(const u32x4*)(p); }
__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// fp32 -> bf16, round to nearest even (finite inputs).
__device__ __forceinline__ __bf16 f2bf(float x) { return (__bf16)x; }
__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

__device__ __forceinline__ bf16x8 pack8(float a0, float a1, float a2, float a3, float a4, float a5,
                                        float a6, float a7) {
  bf16x8 r;
  r[0] = f2bf(a0); r[1] = f2bf(a1); r[2] = f2bf(a2); r[3] = f2bf(a3);
  r[4] = f2bf(a4); r[5] = f2bf(a5); r[6] = f2bf(a6); r[7] = f2bf(a7);
  return r;
}
// Registers 8 kk .. 8 kk + 7 of a 32x32 C tile as a bf16 operand.
__device__ __forceinline__ bf16x8 pack_c8(const f32x16& c, int kk) {
  return pack8(c[8 * kk + 0], c[8 * kk + 1], c[8 * kk + 2], c[8 * kk + 3], c[8 * kk + 4],
               c[8 * kk + 5], c[8 * kk + 6], c[8 * kk + 7]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// sigmoid(s) with one exp2 and one reciprocal; exact limits 0 and 1 at the tails.
__device__ __forceinline__ float fast_sigmoid(float s) {
  return fast_rcp(1.0f + fast_exp2(-s * kLog2e));
}

__device__ __forceinline__ float wave_xor32(float v) { return __shfl_xor(v, 32, 64); }

// Standard normal CDF Phi(s) and the density factor exp(-s^2 / 2), through
// erf(x) = 1 - (a1 t + a2 t^2 + a3 t^3 + a4 t^4 + a5 t^5) exp(-x^2), t = 1 / (1 + p x), x >= 0
// (Abramowitz and Stegun, Handbook of Mathematical Functions, formula 7.1.26;
// |error| <= 1.5e-7), with x = |s| / sqrt(2).
__device__ __forceinline__ float normal_cdf(float s, float& gauss) {
  const float x = fabsf(s) * 0.70710678118654752f;
  const float t = fast_rcp(fmaf(0.3275911f, x, 1.0f));
  const float poly =
      t * fmaf(t, fmaf(t, fmaf(t, fmaf(t, 1.061405429f, -1.453152027f), 1.421413741f), -0.284496736f),
               0.254829592f);
  gauss = fast_exp2(-0.72134752044448170f * s * s);  // exp(-s^2 / 2)
  const float tail = 0.5f * poly * gauss;             // (1 - erf(x)) / 2
  return s >= 0.f ? 1.0f - tail : tail;
}

// Elementwise score maps (phi = 1 .. 4 of gdpa_launch.h): value, and value with its
// derivative.  SiLU s sigmoid(s); ReLU max(s, 0) (derivative 0 at s = 0); GELU
// s Phi(s) (the exact, erf form); identity.  Each maps 0 to 0, so zero-padded
// context rows contribute nothing.
template <int PHI>
__device__ __forceinline__ float phi_value(float s) {
  if (PHI == 1) return s * fast_sigmoid(s);
  if (PHI == 2) return fmaxf(s, 0.f);
  if (PHI == 3) {
    float gauss;
    return s * normal_cdf(s, gauss);
  }
  return s;
}
template <int PHI>
__device__ __forceinline__ float phi_value_grad(float s, float& grad) {
  if (PHI == 1) {
    const float sg = fast_sigmoid(s);
    const float p = s * sg;
    grad = fmaf(s - p, sg, sg);  // sigmoid (1 + s (1 - sigmoid))
    return p;
  }
  if (PHI == 2) {
    grad = s > 0.f ? 1.0f : 0.0f;
    return fmaxf(s, 0.f);
  }
  if (PHI == 3) {
    float gauss;
    const float cdf = normal_cdf(s, gauss);
    grad = fmaf(s * gauss, 0.39894228040143268f, cdf);  // Phi(s) + s exp(-s^2/2) / sqrt(2 pi)
    return s * cdf;
  }
  grad = 1.0f;
  return s;
}

// The value of x, hidden from the optimiser: per-lane index arithmetic derived from
// it inside a loop is recomputed there (a few VALU instructions) instead of being
// hoisted into registers held across the loop.
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// Byte address of an LDS location, as the hardware sees it (M0 / DS addresses).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const GDPA_LDS void*)p;
}

// Asynchronous copy global -> LDS of 16 bytes per lane: lane i's 16 bytes from
// `src` land at LDS byte address `lds_base + 16 i` (lds_base wave-uniform).  No
// VGPR receives data; completion is tracked by the wave's vmcnt like any vector
// memory load, so the caller waits with s_waitcnt vmcnt before a barrier that
// publishes the data.  The copy takes its LDS base from M0: the asm saves M0,
// sets it and restores it, so whatever the compiler keeps in M0 survives.  The
// copy is written as asm rather than with the compiler builtin on purpose: the
// builtin makes the compiler treat the LDS write as possibly aliasing every
// later LDS read (the destination is computed), and it then waits for all
// copies in flight (vmcnt(0)) before such reads, which serialises the prefetch
// ring with HBM latency.  Ordering against readers is the caller's, through
// vmcnt and a barrier.
__device__ __forceinline__ void dma16(uint32_t lds_base, const void* src) {
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %2, off\n\ts_mov_b32 m0, %0"
               : "=&s"(saved) : "s"(lds_base), "v"(src) : "memory");
}
// Same with 4 bytes per lane (lane i -> lds_base + 4 i).
__device__ __forceinline__ void dma4(uint32_t lds_base, const void* src) {
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %2, off\n\ts_mov_b32 m0, %0"
               : "=&s"(saved) : "s"(lds_base), "v"(src) : "memory");
}
// s_waitcnt vmcnt(N) (expcnt and lgkmcnt not waited for); N < 64 (vmcnt is split
// over bits 3:0 and 15:14 of the immediate).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// Work-group id remapped so that the WGs of one XCD (hardware places WG i on
// XCD i % 8) take a contiguous range of the work list; neighbouring work items
// (the q-tiles of one sample and head) then share that XCD's L2.
__device__ __forceinline__ int xcd_remap(int bid, int grid) {  // grid % 8 == 0
  const int per = grid >> 3;  // grid is a multiple of 8
  return (bid & 7) * per + (bid >> 3);
}

// Context rows of sample b: rows row0 .. row0 + n - 1 of the K / V tensors, with
// n returned.  kv_off == nullptr: every sample owns n_fixed rows, stored sample
// after sample ([B, n_fixed, H, d]); otherwise kv_off[B+1] are the row offsets of
// a jagged [total, H, d] context.
__device__ __forceinline__ int kv_rows(const int32_t* kv_off, int b, int n_fixed, size_t& row0) {
  if (kv_off != nullptr) {
    const int r0 = kv_off[b];
    row0 = (size_t)r0;
    return kv_off[b + 1] - r0;
  }
  row0 = (size_t)b * n_fixed;
  return n_fixed;
}

// Largest b in [0, B-1] with tile_start[b] <= tile (tile_start non-decreasing,
// tile_start[0] = 0).
__device__ __forceinline__ int find_sample(const int32_t* __restrict__ tile_start, int B, int tile) {
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (tile_start[mid] <= tile) lo = mid; else hi = mid - 1;
  }
  return lo;
}

}  // namespace gdpa
