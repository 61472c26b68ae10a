// GDPA forward (Kunlun paper summary, section 2.2, GDPA bullet: the personalised
// FFN recast as one fused attention kernel with sequence tokens as queries and
// context-derived weights as keys and values).
//
// bf16 path.  One work-group = 4 waves = one tile of 128 query rows of one
// (sample, head); each wave owns 32 rows.  The sample's K and V are streamed
// through LDS in blocks of 64 context rows and shared by the 4 waves.  Per block:
//   S^T = K Q^T       (32x32x16 bf16 MFMA; A = K rows from LDS, B = the wave's
//                      Q rows, held in registers for the whole tile)
//   P   = phi(S)      (in registers: online softmax in base 2, or an elementwise map)
//   O^T += V^T P^T    (A = V columns via LDS transpose reads, B = P straight
//                      from the C layout of S^T, rounded to bf16)
// Computing S^T rather than S puts one query row per lane, so the softmax row
// max is a register max plus one cross-half exchange, and the C tile of S^T is
// already in the B-operand layout that the second product needs.
//
// fp32 path: plain per-(token, head) loop in fp32, for the small fp32 workload.
#include "gdpa_device.h"
#include "gdpa_launch.h"

namespace gdpa {

// Online softmax with a lazy reference max: a row's reference (the shift of its
// exponentials) moves only when a new score exceeds it by more than this many units
// of log2, as in FlashAttention-4's conditional rescaling, so the unnormalised P stays
// at most 2^8 (exact in fp32 and no coarser in bf16, whose precision is relative) and
// O is rescaled only on the rare tiles that raise some row's max that far.
namespace {
constexpr float kRescaleLog2 = 8.0f;
}  // namespace

// SW: sliding-window self-attention (Kunlun paper summary, section 2.2, Sliding
// Window Attention bullet): K and V are the sample's own token rows, and token i
// (position in its sample) attends to positions i - window < j <= i only; the
// context-row loop covers just that band and out-of-band scores are -inf.
// BIAS: FFN biases (a.score_bias and / or a.out_bias), never with RESID or SW.
template <int D, int PHI, bool RESID, bool SW = false, bool BIAS = false>
__global__ __launch_bounds__(256, 2) void fwd_bf16_kernel(const FwdArgs a) {
  constexpr int BM = kFwdTileRows, BN = 64, KS = D / 16, DT = D / 32;
  // Row strides (elements) for gfx950's 64 LDS banks: K rows are read 16 bytes per
  // lane by 16 consecutive rows per phase (stride = 4 mod 8 dwords: 16 distinct
  // 4-bank groups); V rows by transpose loads, 4 consecutive rows x 64 bytes per
  // 32-lane phase (stride = 16 or 48 mod 64 dwords: the 4 rows fill all 64 banks).
  constexpr int LD = D + 8, LDV = D == 32 ? 32 : D + 32;
  constexpr int CH = D / 8;                   // 16-byte chunks per K/V row
  constexpr int SI = (BN * CH + 255) / 256;   // staging chunks per thread per tensor
  __shared__ __align__(16) uint16_t Ks[BN * LD];
  __shared__ __align__(16) uint16_t Vs[BN * LDV];
  __shared__ __align__(16) float Sbl[BIAS ? BN : 4];  // score bias of the block's rows

  const int H = a.H, B = a.B;
  const int total = a.tile_start[B];
  const int wid = xcd_remap(blockIdx.x, gridDim.x);
  if (wid >= total * H) return;
  const int qtile = wid / H, h = wid - qtile * H;
  const int b = find_sample(a.tile_start, B, qtile);
  const int row0 = a.offsets[b] + (qtile - a.tile_start[b]) * BM;
  const int rows = min(BM, a.offsets[b + 1] - row0);
  const int seq0 = a.offsets[b];
  size_t crow0 = 0;  // first context row of this sample
  const int n = SW ? a.offsets[b + 1] - seq0 : kv_rows(a.kv_offsets, b, a.n, crow0);

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lr = lane & 31, g = lane >> 5;
  const int trow = wave * 32 + lr;
  const bool tvalid = trow < rows;
  const size_t rs = (size_t)H * D;  // token / context row stride in elements

  // This lane's query row, as B operand: items i <-> d = 16 ks + 8 g + i.
  bf16x8 qf[KS];
  {
    const uint16_t* qp = (const uint16_t*)a.q + (size_t)(row0 + trow) * rs + (size_t)h * D + 8 * g;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[ks] = tvalid ? as_bf16x8(gload16(qp + 16 * ks)) : bf16x8{};
  }

  const size_t kv0 = SW ? (size_t)seq0 * H : crow0 * H;
  const uint16_t* Kg = (const uint16_t*)a.k + (kv0 + h) * D;
  const uint16_t* Vg = (const uint16_t*)a.v + (kv0 + h) * D;
  // Context rows this tile needs: all n, or the band of its rows qlo .. qlo + rows - 1.
  const int qlo = row0 - seq0;
  const int jbeg = SW ? max(0, qlo - a.window + 1) : 0;
  const int jend = SW ? min(n, qlo + rows) : n;
  const int irow = qlo + trow;  // this lane's token position in its sample
  u32x4 kreg[SI], vreg[SI];
  auto gload_block = [&](int jb) {
#pragma unroll
    for (int i = 0; i < SI; ++i) {
      const int idx = i * 256 + tid, j = idx / CH, c = idx % CH;
      const bool ok = (idx < BN * CH) && (jb + j < n);
      kreg[i] = ok ? gload16(Kg + (size_t)(jb + j) * rs + 8 * c) : u32x4{};
      vreg[i] = ok ? gload16(Vg + (size_t)(jb + j) * rs + 8 * c) : u32x4{};
    }
  };
  auto store_block = [&](int jb) {
#pragma unroll
    for (int i = 0; i < SI; ++i) {
      const int idx = i * 256 + tid, j = idx / CH, c = idx % CH;
      if (idx < BN * CH) {
        lds_write16(&Ks[j * LD + 8 * c], kreg[i]);
        lds_write16(&Vs[j * LDV + 8 * c], vreg[i]);
      }
    }
    if (BIAS && tid < BN)
      Sbl[tid] = (a.score_bias != nullptr && jb + tid < n) ? a.score_bias[(crow0 + jb + tid) * H + h] : 0.f;
  };

  // Transpose-read addressing: lane 16 G + 4 r + c reads row 4 (G / 2) + r,
  // columns 16 (G % 2) + 4 c of a 32-row slab (second read: rows + 8).  Lane
  // (d + 32 g) then holds V[j][d] for j = 4 g + i (i < 4) and 8 + 4 g + i - 4,
  // matching the row order of the S^T C tile.
  const int trG = lane >> 4;
  const int tr_off = (4 * (trG >> 1) + ((lane & 15) >> 2)) * LDV + 16 * (trG & 1) + 4 * (lane & 3);

  f32x16 O[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) O[dt] = f32x16{};
  // Online softmax in base 2.  With a positive scale and no biases the running max is
  // kept in units of the raw product Q.K (the max commutes with the scale) and the
  // scale enters each exponent through the FMA that subtracts the max: one VALU
  // operation per score fewer.  Otherwise (biases, or a scale <= 0) the scores are
  // scaled first and sm = 1.
  float m_run = -INFINITY, l_run = 0.f;
  const float sl2 = a.scale * kLog2e;
  const bool raw = !BIAS && a.scale > 0.f;
  const float sm = raw ? sl2 : 1.0f;

  gload_block(jbeg);
  for (int jb = jbeg; jb < jend; jb += BN) {
    __syncthreads();
    store_block(jb);
    __syncthreads();
    if (jb + BN < jend) gload_block(jb + BN);
    // SW: none of the wave's 32 query rows sees a key row of this block (all lie after
    // the rows, or all left their windows): it adds nothing (no barrier follows).
    if (SW && (jb > qlo + 32 * wave + 31 || jb + BN - 1 <= qlo + 32 * wave - a.window)) continue;
    // Score bias (BIAS) of rows 32 mt + 8 q + 4 g + {0..3}: register 4 q + i of tile mt.
    float bj[2][16];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4 bv = BIAS ? *(const GDPA_LDS f32x4*)&Sbl[32 * mt + 8 * q + 4 * g] : f32x4{};
#pragma unroll
        for (int i = 0; i < 4; ++i) bj[mt][4 * q + i] = bv[i];
      }

    f32x16 S[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      S[mt] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        S[mt] = mfma32(lds_read8(&Ks[(32 * mt + lr) * LD + 16 * ks + 8 * g]), qf[ks], S[mt]);
    }

    if (PHI == 0) {
      // Online softmax over the context rows, base 2.
      // Only the last block of a context (or a sliding window's band) has scores to
      // mask; the test is wave-uniform, and each case is compiled on its own so that
      // full blocks carry no per-score select.
      const bool tail = jb + BN > n;
      float mx = -INFINITY;
      if (!raw) {  // wave-uniform: scores in base-2 units first (see sm)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            S[mt][r] = BIAS ? fmaf(bj[mt][r], kLog2e, S[mt][r] * sl2) : S[mt][r] * sl2;
      }
      auto mask_max = [&](auto MASK) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            float s = S[mt][r];
            if (decltype(MASK)::value) {
              const int j = jb + 32 * mt + 8 * (r >> 2) + 4 * g + (r & 3);
              if (j >= n || (SW && (j > irow || j <= irow - a.window))) s = -INFINITY;
            }
            S[mt][r] = s;
            mx = fmaxf(mx, s);
          }
      };
      // A sliding window's block needs no mask when it lies inside the window of every
      // row of the wave (and before the end of the sample).
      const int i0 = qlo + 32 * wave;
      const bool inside = SW && jb + BN - 1 <= i0 && jb > i0 + 31 - a.window;
      if (tail || (SW && !inside)) mask_max(std::true_type{});  // wave-uniform
      else mask_max(std::false_type{});
      mx = fmaxf(mx, wave_xor32(mx));
      // m_run is the row's reference max (the shift of its exponentials), moved only
      // when a score exceeds it by more than 2^kRescaleLog2 (wave-uniform test; the
      // first finite block of a row always moves it, and a row with no finite score
      // yet keeps -inf).  A row whose window has missed every block so far (SW) is
      // shifted by 0.
      const float m_new = fmaxf(m_run, mx);
      if (__any((m_new - m_run) * sm > kRescaleLog2)) {
        const float corr = fast_exp2((m_run - ((SW && m_new == -INFINITY) ? 0.f : m_new)) * sm);
        l_run *= corr;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) O[dt] *= corr;
        m_run = m_new;
      }
      const float m_use = (SW && m_run == -INFINITY) ? 0.f : m_run;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = fast_exp2(fmaf(S[mt][r], sm, -m_use * sm));
          l_run += p;
          S[mt][r] = p;
        }
    } else {
      // Elementwise maps; rows past n are zero in K and V, and phi(0) = 0.
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          S[mt][r] = phi_value<PHI>(BIAS ? fmaf(S[mt][r], a.scale, bj[mt][r]) : S[mt][r] * a.scale);
    }

#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const bf16x8 p = pack_c8(S[mt], kk);
        const uint16_t* vb = &Vs[(32 * mt + 16 * kk) * LDV + tr_off];
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const bf16x4 lo = lds_read_tr4(vb + 32 * dt);
          const bf16x4 hi = lds_read_tr4(vb + 8 * LDV + 32 * dt);
          O[dt] = mfma32(cat8(lo, hi), p, O[dt]);
        }
      }
  }

  if (PHI == 0) {
    const float l_tot = l_run + wave_xor32(l_run);
    const float inv = 1.0f / l_tot;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) O[dt] *= inv;
    if (tvalid && g == 0 && a.lse != nullptr)
      a.lse[(size_t)(row0 + trow) * H + h] = fmaf(m_run, sm, __log2f(l_tot)) * kLn2;
  }
  if (tvalid) {
    // Lane (t, g), register r holds O[t][d = 32 dt + 8 (r / 4) + 4 g + r % 4].
    const size_t base = (size_t)(row0 + trow) * rs + (size_t)h * D + 4 * g;
    uint16_t* op = (uint16_t*)a.o + base;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int col = 32 * dt + 8 * q4;
        float v0 = O[dt][4 * q4 + 0], v1 = O[dt][4 * q4 + 1];
        float v2 = O[dt][4 * q4 + 2], v3 = O[dt][4 * q4 + 3];
        if (RESID) {
          const u32x2 rr = *(const u32x2*)((const uint16_t*)a.residual + base + col);
          v0 += __uint_as_float(rr[0] << 16);
          v1 += __uint_as_float(rr[0] & 0xffff0000u);
          v2 += __uint_as_float(rr[1] << 16);
          v3 += __uint_as_float(rr[1] & 0xffff0000u);
        }
        if (BIAS && a.out_bias != nullptr) {
          const f32x4 bv = *(const f32x4*)(a.out_bias + ((size_t)b * H + h) * D + 4 * g + col);
          v0 += bv[0]; v1 += bv[1]; v2 += bv[2]; v3 += bv[3];
        }
        bf16x4 ov;
        ov[0] = f2bf(v0); ov[1] = f2bf(v1); ov[2] = f2bf(v2); ov[3] = f2bf(v3);
        *(bf16x4*)(op + col) = ov;
        if (a.o_plus_q != nullptr) {  // the residual block's sum X + O (X = the queries)
          const u32x2 xq = *(const u32x2*)((const uint16_t*)a.q + base + col);
          bf16x4 yv;
          yv[0] = f2bf(v0 + __uint_as_float(xq[0] << 16));
          yv[1] = f2bf(v1 + __uint_as_float(xq[0] & 0xffff0000u));
          yv[2] = f2bf(v2 + __uint_as_float(xq[1] << 16));
          yv[3] = f2bf(v3 + __uint_as_float(xq[1] & 0xffff0000u));
          *(bf16x4*)((uint16_t*)a.o_plus_q + base + col) = yv;
        }
      }
  }
}

// fp32: one thread per (token, head), online softmax or elementwise-map accumulation
// in fp32 (the device library's expf / erff).
template <int D, int PHI, bool RESID>
__global__ __launch_bounds__(128) void fwd_f32_kernel(const FwdArgs a) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // the grid's last block overhangs T * H
  if (idx >= (int64_t)a.T * a.H) return;
  const int t = (int)(idx / a.H), h = (int)(idx - (int64_t)t * a.H);
  const int b = find_sample(a.offsets, a.B, t);
  const size_t rs = (size_t)a.H * D;
  const float* qp = (const float*)a.q + (size_t)t * rs + (size_t)h * D;
  float q[D], acc[D];
#pragma unroll
  for (int e = 0; e < D; ++e) {
    q[e] = qp[e];
    acc[e] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  size_t crow0;
  const int n = kv_rows(a.kv_offsets, b, a.n, crow0);
  const float* Kb = (const float*)a.k + (crow0 * a.H + h) * D;
  const float* Vb = (const float*)a.v + (crow0 * a.H + h) * D;
  for (int j = 0; j < n; ++j) {
    const float* kj = Kb + (size_t)j * rs;
    const float* vj = Vb + (size_t)j * rs;
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < D; ++e) s = fmaf(q[e], kj[e], s);
    s *= a.scale;
    if (a.score_bias != nullptr) s += a.score_bias[(crow0 + j) * a.H + h];
    if (PHI == 0) {
      const float m_new = fmaxf(m, s);
      const float c = expf(m - m_new), p = expf(s - m_new);
      l = l * c + p;
#pragma unroll
      for (int e = 0; e < D; ++e) acc[e] = fmaf(p, vj[e], acc[e] * c);
      m = m_new;
    } else {
      float p = s;
      if (PHI == kPhiSilu) p = s / (1.0f + expf(-s));
      if (PHI == kPhiRelu) p = fmaxf(s, 0.f);
      if (PHI == kPhiGelu) p = 0.5f * s * (1.0f + erff(s * 0.70710678118654752f));
#pragma unroll
      for (int e = 0; e < D; ++e) acc[e] = fmaf(p, vj[e], acc[e]);
    }
  }
  float* op = (float*)a.o + (size_t)t * rs + (size_t)h * D;
  const float* rp = RESID ? (const float*)a.residual + (size_t)t * rs + (size_t)h * D : nullptr;
  const float inv = (PHI == 0) ? 1.0f / l : 1.0f;
  const float* obp = a.out_bias != nullptr ? a.out_bias + ((size_t)b * a.H + h) * D : nullptr;
#pragma unroll
  for (int e = 0; e < D; ++e) op[e] = acc[e] * inv + (RESID ? rp[e] : 0.f) + (obp != nullptr ? obp[e] : 0.f);
  if (a.o_plus_q != nullptr) {  // the residual block's sum X + O (X = the queries)
    float* yp = (float*)a.o_plus_q + (size_t)t * rs + (size_t)h * D;
    const float* qx = (const float*)a.q + (size_t)t * rs + (size_t)h * D;
    for (int e = 0; e < D; ++e) yp[e] = op[e] + qx[e];
  }
  if (PHI == 0 && a.lse != nullptr) a.lse[(size_t)t * a.H + h] = m + logf(l);
}

int fwd_bf16_grid(int T, int B, int H) {
  // sum_b ceil(L_b / BM) <= floor(T / BM) + B; round up to a multiple of 8 (XCDs).
  const long tiles = (long)T / kFwdTileRows + B;
  const long items = tiles * H;
  return (int)((items + 7) / 8 * 8);
}

template <int D>
static hipError_t fwd_bf16_d(const FwdArgs& a, int phi, bool resid, int grid, hipStream_t s) {
  const dim3 g(grid), blk(256);
  const bool biased = a.score_bias != nullptr || a.out_bias != nullptr;  // never with a residual
  return dispatch_phi(phi, [&](auto P) {
    constexpr int PH = decltype(P)::value;
    if (biased) hipLaunchKernelGGL((fwd_bf16_kernel<D, PH, false, false, true>), g, blk, 0, s, a);
    else if (resid) hipLaunchKernelGGL((fwd_bf16_kernel<D, PH, true>), g, blk, 0, s, a);
    else hipLaunchKernelGGL((fwd_bf16_kernel<D, PH, false>), g, blk, 0, s, a);
    return hipGetLastError();
  });
}

template <int D>
static hipError_t fwd_swa_d(const FwdArgs& a, int grid, hipStream_t s) {
  hipLaunchKernelGGL((fwd_bf16_kernel<D, kPhiSoftmax, false, true>), dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_fwd_swa(const FwdArgs& a, int d, int grid, hipStream_t s) {
  if (grid == 0) return hipSuccess;
  switch (d) {
    case 32: return fwd_swa_d<32>(a, grid, s);
    case 64: return fwd_swa_d<64>(a, grid, s);
    case 128: return fwd_swa_d<128>(a, grid, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_fwd_bf16(const FwdArgs& a, int d, int phi, bool resid, int grid, hipStream_t s) {
  if (grid == 0) return hipSuccess;
  switch (d) {
    case 32: return fwd_bf16_d<32>(a, phi, resid, grid, s);
    case 64: return fwd_bf16_d<64>(a, phi, resid, grid, s);
    case 128: return fwd_bf16_d<128>(a, phi, resid, grid, s);
  }
  return hipErrorInvalidValue;
}

template <int D>
static hipError_t fwd_f32_d(const FwdArgs& a, int phi, bool resid, hipStream_t s) {
  const long items = (long)a.T * a.H;
  const dim3 g((unsigned)((items + 127) / 128)), blk(128);
  return dispatch_phi(phi, [&](auto P) {
    constexpr int PH = decltype(P)::value;
    if (resid) hipLaunchKernelGGL((fwd_f32_kernel<D, PH, true>), g, blk, 0, s, a);
    else hipLaunchKernelGGL((fwd_f32_kernel<D, PH, false>), g, blk, 0, s, a);
    return hipGetLastError();
  });
}

hipError_t launch_fwd_f32(const FwdArgs& a, int d, int phi, bool resid, hipStream_t s) {
  if ((long)a.T * a.H == 0) return hipSuccess;
  switch (d) {
    case 32: return fwd_f32_d<32>(a, phi, resid, s);
    case 64: return fwd_f32_d<64>(a, phi, resid, s);
    case 128: return fwd_f32_d<128>(a, phi, resid, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace gdpa
