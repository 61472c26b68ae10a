// GDPA backward for d = 128 and n <= 256: one work-group covers all of a
// (sample, head)'s context rows, so dQ needs no cross-work-group reduction.
//
// Same mathematics as gdpa_bwd.hip (Kunlun paper summary section 2.2, GDPA
// bullet: keys and values are per-sample weights, so dK and dV are sums over the
// sample's own tokens).  Organisation:
//   * 8 waves (two per SIMD, so one wave's LDS reads overlap the other's MFMAs);
//     wave w owns context rows 32 w .. 32 w + 31 and keeps their dK, dV fp32
//     accumulators (32 x 128 each) for the whole sample, with their K and V rows
//     in registers as MFMA B operands.  Rows past n are zero.
//   * K^T is resident in LDS ([d][j]) for the dQ product.
//   * Per 32-row query step the work-group stages Q and dO both row-major (A
//     operands of S = Q K^T and dP = dO V^T) and transposed with the tokens in
//     C-tile order (B operands of dK += dS^T Q and dV += P^T dO), and writes dS
//     row-major (operand of dQ).  Every MFMA operand read is a 16-byte,
//     bank-conflict-free LDS read; there are no transpose loads in the loop.
//   * Waves 0..3 then compute dQ^T for head columns 32 w .. 32 w + 31 over all
//     context rows (dQ^T = K^T dS^T), whose C tile gives each lane four
//     consecutive columns of one token: 8-byte stores, residual dO added in fp32.
//   * The score scale is applied once, to dQ per step and to dK at the end.
//   * Global loads are unconditional (rows clamped into the sample); the next
//     step's Q / dO are loaded during the dK / dV and dQ products of this one.
// Work-groups are launched longest sample first.
#include "gdpa_device.h"
#include "gdpa_launch.h"

namespace gdpa {

namespace {
// Position of token t of a 32-token step in the transposed tiles: the C tile of
// S holds, for lane group g and register r, token 8 (r / 4) + 4 g + r % 4, and
// k-step kk of a P^T / dS^T A operand takes registers 8 kk .. 8 kk + 7, so token
// t = 16 kk + 8 a + 4 g + c goes to 16 kk + 8 g + 4 a + c.
__device__ __forceinline__ int tok_pos(int t) { return (t & ~12) | ((t & 4) << 1) | ((t & 8) >> 1); }

__device__ __forceinline__ uint16_t half_of(const u32x4& v, int i) {
  return (uint16_t)(v[i >> 1] >> (16 * (i & 1)));
}
__device__ __forceinline__ float lo_f(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_f(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
}  // namespace

// DQB: 0 dQ = result, 1 dQ = dO + result (dO from LDS), 2 dQ = dQ + result.
template <int PHI, int DQB>
__global__ __launch_bounds__(512, 1) void bwd_res_kernel(const BwdArgs a) {
  constexpr int D = 128, NT = 512, NJ = 256, BQ = 32, KS = D / 16, DT = D / 32;
  constexpr int LDQ = D + 8;    // Qs, dOs rows (68 dwords: 8 consecutive rows conflict free)
  constexpr int LDT = BQ + 8;   // Qt, dOt rows (20 dwords: likewise)
  constexpr int LDJ = NJ + 8;   // Kt and dS rows (132 dwords)
  constexpr int LDE = D;        // bf16 dK / dV rows in the epilogue
  static_assert(BQ * D / 8 == NT, "one 16-byte staging chunk per thread and tensor");
  __shared__ __align__(16) uint16_t Kt[D * LDJ];
  __shared__ __align__(16) uint16_t Qs[BQ * LDQ];
  __shared__ __align__(16) uint16_t dOs[BQ * LDQ];
  __shared__ __align__(16) uint16_t Qt[D * LDT];
  __shared__ __align__(16) uint16_t dOt[D * LDT];
  __shared__ __align__(16) uint16_t dSs[BQ * LDJ];
  __shared__ __align__(16) float lse_s[BQ], dvec_s[BQ];
  static_assert(8 * 32 * LDE <= D * LDJ, "epilogue tiles must fit in Kt");

  const int H = a.H, n = a.n;
  const int item = blockIdx.x;
  const int rank = item / H, h = item - rank * H;
  const int b = a.order[rank];
  const int seq0 = a.offsets[b], L = a.offsets[b + 1] - seq0;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lr = lane & 31, g = lane >> 5;
  const size_t rs = (size_t)H * D;
  const int j = 32 * wave + lr;  // this lane's context row in the S / dP C tiles
  const bool jvalid = j < n;

  // K and V rows of this wave as B operands (lane (j + 32 g), items d = 16 ks + 8 g + i),
  // zero past n; K^T written into LDS from the same registers (32 consecutive j per
  // half-wave: each 2-byte write instruction covers two contiguous 64-byte runs).
  bf16x8 kf[KS], vf[KS];
  {
    const size_t row = ((size_t)b * n + min(j, n - 1)) * rs + (size_t)h * D + 8 * g;
    u32x4 kr[KS], vr[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      kr[ks] = gload16((const uint16_t*)a.k + row + 16 * ks);
      vr[ks] = gload16((const uint16_t*)a.v + row + 16 * ks);
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (!jvalid) {
        kr[ks] = u32x4{};
        vr[ks] = u32x4{};
      }
      kf[ks] = as_bf16x8(kr[ks]);
      vf[ks] = as_bf16x8(vr[ks]);
#pragma unroll
      for (int i = 0; i < 8; ++i) Kt[(16 * ks + 8 * g + i) * LDJ + j] = half_of(kr[ks], i);
    }
  }

  f32x16 dK[DT], dV[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    dK[dt] = f32x16{};
    dV[dt] = f32x16{};
  }

  const float scale = a.scale, sl2 = scale * kLog2e, c1 = -scale * kLog2e;
  const uint16_t* Qg = (const uint16_t*)a.q + (size_t)h * D;
  const uint16_t* dOg = (const uint16_t*)a.d_o + (size_t)h * D;

  // Staging: thread tid -> token t = tid % 32, column chunk c = tid / 32 (consecutive
  // lanes take consecutive tokens).
  const int st_t = tid % BQ, st_c = tid / BQ;
  u32x4 qn, dn;
  float lse_n = 0.f, dvec_n = 0.f;
  auto load_step = [&](int tq) {
    const size_t off = (size_t)(seq0 + min(tq + st_t, L - 1)) * rs + 8 * st_c;
    qn = gload16(Qg + off);
    dn = gload16(dOg + off);
    if (PHI == 0) {
      const size_t r = (size_t)(seq0 + min(tq + (tid & (BQ - 1)), L - 1)) * H + h;
      lse_n = a.lse[r] * kLog2e;
      dvec_n = a.dvec[r];
    }
  };
  if (L > 0) load_step(0);

  for (int tq = 0; tq < L; tq += BQ) {
    const int rows = min(BQ, L - tq);
    __syncthreads();  // previous step finished with the step buffers
    {
      const bool ok = st_t < rows;
      const u32x4 qv = ok ? qn : u32x4{}, dv = ok ? dn : u32x4{};
      lds_write16(&Qs[st_t * LDQ + 8 * st_c], qv);
      lds_write16(&dOs[st_t * LDQ + 8 * st_c], dv);
      const int p = tok_pos(st_t);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        Qt[(8 * st_c + e) * LDT + p] = half_of(qv, e);
        dOt[(8 * st_c + e) * LDT + p] = half_of(dv, e);
      }
      if (PHI == 0 && tid < BQ) {
        lse_s[tid] = tid < rows ? lse_n : INFINITY;
        dvec_s[tid] = tid < rows ? dvec_n : 0.f;
      }
    }
    __syncthreads();

    // S and dP for this wave's 32 context rows (M = tokens, N = context rows).
    f32x16 S = f32x16{}, dP = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int o = lr * LDQ + 16 * ks + 8 * g;
      S = mfma32(lds_read8(&Qs[o]), kf[ks], S);
      dP = mfma32(lds_read8(&dOs[o]), vf[ks], dP);
    }
    // Lane (j + 32 g), register r: token t = 8 (r / 4) + 4 g + r % 4.  S becomes P
    // and dP becomes dS / scale.
    if (PHI == 0) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const f32x4 ls = *(const GDPA_LDS f32x4*)&lse_s[8 * q4 + 4 * g];
        const f32x4 dvv = *(const GDPA_LDS f32x4*)&dvec_s[8 * q4 + 4 * g];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int r = 4 * q4 + c;
          float p = fast_exp2(fmaf(S[r], sl2, -ls[c]));
          if (!jvalid) p = 0.f;
          S[r] = p;
          dP[r] = p * (dP[r] - dvv[c]);
        }
      }
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float sg = fast_rcp(1.0f + fast_exp2(S[r] * c1));
        const float sv = S[r] * scale;
        const float p = sv * sg;
        S[r] = p;
        dP[r] = dP[r] * fmaf(sv - p, sg, sg);
      }
    }
    bf16x8 pa[2], sa[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      pa[kk] = pack_c8(S, kk);
      sa[kk] = pack_c8(dP, kk);
      // dS row-major for the dQ product: item i of k-step kk is token
      // 16 kk + 8 (i / 4) + 4 g + i % 4.
      const u32x4 sw = __builtin_bit_cast(u32x4, sa[kk]);
#pragma unroll
      for (int i = 0; i < 8; ++i)
        dSs[(16 * kk + 8 * (i >> 2) + 4 * g + (i & 3)) * LDJ + j] = half_of(sw, i);
    }
    // The next step's Q / dO are loaded here, where S and dP are no longer live.
    if (tq + BQ < L) load_step(tq + BQ);
    // dV += P^T dO, dK += dS^T Q over the 32 tokens.
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int o = (32 * dt + lr) * LDT + 16 * kk + 8 * g;
        dV[dt] = mfma32(pa[kk], lds_read8(&dOt[o]), dV[dt]);
        dK[dt] = mfma32(sa[kk], lds_read8(&Qt[o]), dK[dt]);
      }
    __syncthreads();  // dS complete

    if (wave < 4) {
      // dQ^T[32 w .. 32 w + 31, tokens] = K^T dS^T over all 256 context rows.
      f32x16 dq = f32x16{};
      const int oa = (32 * wave + lr) * LDJ + 8 * g, ob = lr * LDJ + 8 * g;
#pragma unroll
      for (int ks = 0; ks < NJ / 16; ++ks)
        dq = mfma32(lds_read8(&Kt[oa + 16 * ks]), lds_read8(&dSs[ob + 16 * ks]), dq);
      // Lane (t + 32 g), register r: column 32 w + 8 (r / 4) + 4 g + r % 4 of token t = lr.
      if (lr < rows) {
        uint16_t* dst = (uint16_t*)a.dq + (size_t)(seq0 + tq + lr) * rs + (size_t)h * D + 32 * wave + 4 * g;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          float v0 = dq[4 * q4] * scale, v1 = dq[4 * q4 + 1] * scale;
          float v2 = dq[4 * q4 + 2] * scale, v3 = dq[4 * q4 + 3] * scale;
          u32x2 base = u32x2{0u, 0u};
          if (DQB == 1) base = *(const GDPA_LDS u32x2*)&dOs[lr * LDQ + 32 * wave + 8 * q4 + 4 * g];
          if (DQB == 2) base = *(const u32x2*)(dst + 8 * q4);
          if (DQB != 0) {
            v0 += lo_f(base[0]);
            v1 += hi_f(base[0]);
            v2 += lo_f(base[1]);
            v3 += hi_f(base[1]);
          }
          bf16x4 o4;
          o4[0] = f2bf(v0);
          o4[1] = f2bf(v1);
          o4[2] = f2bf(v2);
          o4[3] = f2bf(v3);
          *(bf16x4*)(dst + 8 * q4) = o4;
        }
      }
    }
  }

  // dK (times the scale) and dV through LDS (Kt's space, once every wave is done
  // with it) as bf16 32 x 128 tiles per wave, then 16-byte stores of rows j < n.
  __syncthreads();
  uint16_t* Ew = Kt + wave * 32 * LDE;
#pragma unroll
  for (int which = 0; which < 2; ++which) {
    // Lane (d + 32 g), register r: context row 8 (r / 4) + 4 g + r % 4 of this wave.
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        Ew[(8 * (r >> 2) + 4 * g + (r & 3)) * LDE + 32 * dt + lr] =
            __builtin_bit_cast(uint16_t, f2bf(which == 0 ? dK[dt][r] * scale : dV[dt][r]));
    uint16_t* dst = (uint16_t*)(which == 0 ? a.dk : a.dv) + ((size_t)b * n * H + h) * D;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int row = 4 * u + (lane >> 4), c = lane & 15;
      const int jr = 32 * wave + row;
      const u32x4 v = *(const GDPA_LDS u32x4*)&Ew[row * LDE + 8 * c];
      if (jr < n) *(u32x4*)(dst + (size_t)jr * rs + 8 * c) = v;
    }
    asm volatile("" ::: "memory");  // dV reuses this wave's region
  }
}

bool bwd_res_supported(int d, int n) { return d == 128 && n <= 256; }

hipError_t launch_bwd_res(const BwdArgs& a, int phi, hipStream_t s) {
  const long items = (long)a.B * a.H;
  if (items == 0) return hipSuccess;
  const dim3 g((unsigned)items), blk(512);
  const int mode = a.dq_base == nullptr ? 0 : (a.dq_base == a.d_o ? 1 : 2);
#define GDPA_BWD_RES(P, M) hipLaunchKernelGGL((bwd_res_kernel<P, M>), g, blk, 0, s, a)
  if (phi == 0) {
    if (mode == 0) GDPA_BWD_RES(0, 0); else if (mode == 1) GDPA_BWD_RES(0, 1); else GDPA_BWD_RES(0, 2);
  } else {
    if (mode == 0) GDPA_BWD_RES(1, 0); else if (mode == 1) GDPA_BWD_RES(1, 1); else GDPA_BWD_RES(1, 2);
  }
#undef GDPA_BWD_RES
  return hipGetLastError();
}

}  // namespace gdpa
