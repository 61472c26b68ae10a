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
//   * Q and dO (and, for softmax, the row LSE and rowsum(dO O)) of each 32-row
//     query step reach LDS by asynchronous global->LDS copies issued by waves
//     4..7 two steps ahead into a 3-slot ring: no registers hold staged data and
//     HBM latency is covered by two steps of compute.  Each copying wave brings in
//     one 32-column block of both tiles (rows of 64 bytes, 16-byte chunks XOR-
//     swizzled by row quad so that 16 consecutive rows of one chunk, one 16-lane
//     phase of a ds_read_b128, hit distinct banks).  The row-major tiles are the A operands of S = Q K^T and dP = dO V^T.
//   * The same wave writes its block transposed, with the tokens in C-tile order
//     (B operands of dK += dS^T Q and dV += P^T dO; zero past the sample's last
//     row), for the next step while waves 0..3 compute dQ: it waits only for its
//     own copies, and the transposition costs the step no barrier.  Every MFMA
//     operand read is a 16-byte, bank-conflict-free LDS read; there are no
//     transpose loads in the loop.
//   * Waves 0..3 then compute dQ^T for head columns 32 w .. 32 w + 31 over all
//     context rows (dQ^T = K^T dS^T), whose C tile (rows permuted) gives each lane
//     16 consecutive columns of one token: 16-byte stores, residual added in fp32.
//   * The score scale is applied once, to dQ per step and to dK at the end.
//   * Global addresses are clamped into the sample (copies past its last step
//     re-read valid rows into the free slot, which keeps every wave's count of
//     outstanding copies fixed for its s_waitcnt).
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

// dQ^T = K^T dS^T: the A operand's row i = 8 a + 4 b + c of each 32-column block is
// head column kt_row(i) = 16 b + 4 a + c, so that C-tile lane group g holds the 16
// consecutive columns 16 g .. 16 g + 15 in register order (two 16-byte stores).
// K^T rows are 528 bytes apart, so row d starts at bank group d % 16 (16-byte groups of
// the 64 4-byte banks); the 16-byte chunk q of row d is stored at chunk
// q ^ (8 (d / 16 % 2)) so that the rows {0..3, 16..19, 4..7, 20..23} + 8 k read by one
// 16-lane phase of a ds_read_b128 fall in distinct bank groups.
__device__ __forceinline__ int kt_row(int i) { return 16 * ((i >> 2) & 1) + 4 * (i >> 3) + (i & 3); }
__device__ __forceinline__ int kt_col(int j, int d) { return 8 * ((j >> 3) ^ (((d >> 4) & 1) << 3)) + (j & 7); }

__device__ __forceinline__ uint16_t half_of(const u32x4& v, int i) {
  return (uint16_t)(v[i >> 1] >> (16 * (i & 1)));
}
__device__ __forceinline__ float lo_f(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_f(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
}  // namespace

// DQB: 0 dQ = result, 1 dQ = dO + result (dO from LDS), 2 dQ = dQ + result,
// 3 dQ = result with the FFN score bias (a.score_bias, gradient into a.d_score_bias).
template <int PHI, int DQB>
__global__ __launch_bounds__(512, 1) void bwd_res_kernel(const BwdArgs a) {
  constexpr int D = 128, NT = 512, NJ = 256, BQ = 32, KS = D / 16, DT = D / 32;
  constexpr int LDT = BQ + 8;   // Qt, dOt rows (20 dwords: likewise)
  constexpr int LDJ = NJ + 8;   // Kt and dS rows (132 dwords)
  constexpr int LDE = D;        // bf16 dK / dV rows in the epilogue
  // Ring slot: Q tile and dO tile (bf16, each 4 blocks of 32 rows x 64 bytes: block G
  // holds head columns 32 G .. 32 G + 31 of every token, the 16-byte chunk q of row t at
  // position q ^ ((t / 4) % 4)), then LSE[32] and rowsum(dO O)[32] (fp32, softmax only).
  constexpr int NSLOT = 3, TILE_B = BQ * D * 2, SLOT_B = 2 * TILE_B + 2 * BQ * 4;
  constexpr int DMA_OPS = PHI == 0 ? 5 : 4;  // copies per step issued by each of waves 4..7
  static_assert(BQ * D / 8 == NT, "one 16-byte chunk per thread and tensor");
  __shared__ __align__(16) uint16_t Kt[D * LDJ];
  __shared__ __align__(16) uint8_t ring[NSLOT * SLOT_B];
  __shared__ __align__(16) uint16_t QdT[2 * D * LDT];  // Q^T then dO^T (one base address)
  uint16_t* const Qt = QdT;
  uint16_t* const dOt = QdT + D * LDT;
  __shared__ __align__(16) uint16_t dSs[BQ * LDJ];
  static_assert(8 * 32 * LDE <= D * LDJ, "epilogue tiles must fit in Kt");

  const int H = a.H;
  const int item = blockIdx.x;
  const int rank = item / H, h = item - rank * H;
  const int b = a.order[rank];
  size_t crow0;
  const int n = kv_rows(a.kv_offsets, b, a.n, crow0);  // 1 <= n <= a.n
  const int seq0 = a.offsets[b], L = a.offsets[b + 1] - seq0;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lr = lane & 31, g = lane >> 5;
  const size_t rs = (size_t)H * D;
  const int j = 32 * wave + lr;  // this lane's context row in the S / dP C tiles
  const bool jvalid = j < n;
  // FFN score bias of this lane's row (DQB 3), and the running sum of its score gradient.
  const float sbj = (DQB == 3 && a.score_bias != nullptr && jvalid) ? a.score_bias[(crow0 + j) * H + h] : 0.f;
  const float sbj2 = sbj * kLog2e;
  float dsb = 0.f;

  // K and V rows of this wave as B operands (lane (j + 32 g), items d = 16 ks + 8 g + i),
  // zero past n; K^T written into LDS from the same registers (32 consecutive j per
  // half-wave: each 2-byte write instruction covers two contiguous 64-byte runs).
  bf16x8 kf[KS], vf[KS];
  {
    const size_t row = (crow0 + min(j, n - 1)) * rs + (size_t)h * D + 8 * g;
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
      for (int i = 0; i < 8; ++i) {
        const int d = 16 * ks + 8 * g + i;
        Kt[d * LDJ + kt_col(j, d)] = half_of(kr[ks], i);
      }
    }
  }

  f32x16 dK[DT], dV[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    dK[dt] = f32x16{};
    dV[dt] = f32x16{};
  }

  const float scale = a.scale, sl2 = scale * kLog2e, c1 = -scale * kLog2e;

  // Ring copies for step `st` (waves 4..7): wave w copies block G = w - 4 (columns
  // 32 G .. 32 G + 31 of all 32 rows) of the Q and dO tiles, 16 rows (1 KiB) per
  // instruction; lane i takes row 16 k + i / 4 and position i % 4.
  const int nsteps = (L + BQ - 1) / BQ;
  auto slot_off = [](int t, int cl) { return t * 32 + 8 * (cl ^ ((t >> 2) & 3)); };  // halves
  auto issue = [&](int st) {
    const int tq = st * BQ, G = wave - 4;
    const uint32_t sb = lds_addr(ring) + (uint32_t)((st % NSLOT) * SLOT_B + G * 2048);
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int t = 16 * k + (lane >> 2);
      const int c = 4 * G + ((lane & 3) ^ ((t >> 2) & 3));
      const size_t off = (size_t)(seq0 + min(tq + t, L - 1)) * rs + (size_t)h * D + 8 * c;
      dma16(__builtin_amdgcn_readfirstlane(sb + 1024 * k), (const uint16_t*)a.q + off);
      dma16(__builtin_amdgcn_readfirstlane(sb + TILE_B + 1024 * k), (const uint16_t*)a.d_o + off);
    }
    if (PHI == 0) {  // lanes 0..31: LSE of rows 0..31; lanes 32..63: rowsum(dO O) (every copying wave)
      const size_t r = (size_t)(seq0 + min(tq + lr, L - 1)) * H + h;
      dma4(__builtin_amdgcn_readfirstlane(lds_addr(ring) + (uint32_t)((st % NSLOT) * SLOT_B + 2 * TILE_B)),
           g == 0 ? (const void*)(a.lse + r) : (const void*)(a.dvec + r));
    }
  };

  // Transposed copies of the block a copying wave brought in itself (so it only waits
  // for its own copies): lane -> token t = lane % 32, local chunks lane / 32 and + 2;
  // rows past the sample are zero.
  auto transpose = [&](int st) {
    const int tq = st * BQ, rows = min(BQ, L - tq), G = wave - 4;
    const uint16_t* Qs = (const uint16_t*)(ring + (st % NSLOT) * SLOT_B) + G * 1024;
    const uint16_t* dOs = Qs + TILE_B / 2;
    const int t = opaque(lr), p = tok_pos(t);
    const bool ok = t < rows;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int cl = (lane >> 5) + 2 * u, c = 4 * G + cl;
      const int o = slot_off(t, cl);
      const u32x4 qv = ok ? *(const GDPA_LDS u32x4*)&Qs[o] : u32x4{};
      const u32x4 dv = ok ? *(const GDPA_LDS u32x4*)&dOs[o] : u32x4{};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        Qt[(8 * c + e) * LDT + p] = half_of(qv, e);
        dOt[(8 * c + e) * LDT + p] = half_of(dv, e);
      }
    }
  };

  // Waves 4..7: copies for steps 0 and 1, then step 0's transposed tiles.
  if (L > 0 && wave >= 4) {
    issue(0);
    issue(1);
    wait_vmcnt<DMA_OPS>();  // this wave's copies for step 0 landed (step 1's may remain)
    transpose(0);
  }

  for (int s = 0; s < nsteps; ++s) {
    const int tq = s * BQ, rows = min(BQ, L - tq);
    const uint8_t* slot = ring + (s % NSLOT) * SLOT_B;
    const uint16_t* Qs = (const uint16_t*)slot;
    const uint16_t* dOs = (const uint16_t*)(slot + TILE_B);
    const float* lse_s = (const float*)(slot + 2 * TILE_B);
    const float* dvec_s = lse_s + BQ;
    const int lx = opaque(lr), gx = opaque(g);
    // Step s's slot landed (waited for by waves 4..7 before they built Qt / dOt for it)
    // and Qt / dOt hold step s; step s - 1 is finished with dSs and its slot.
    __syncthreads();
    if (wave >= 4) issue(s + 2);

    // S and dP for this wave's 32 context rows (M = tokens, N = context rows).
    f32x16 S = f32x16{}, dP = f32x16{};
    // k-step ks reads chunk (2 ks + g) % 4 of block ks / 2: two base offsets (even and
    // odd ks) plus immediates.
    const int oe = slot_off(lx, gx), oo = slot_off(lx, gx + 2);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int o = (ks >> 1) * 1024 + ((ks & 1) ? oo : oe);
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
          float p = fast_exp2(fmaf(S[r], sl2, DQB == 3 ? fmaf(-ls[c], kLog2e, sbj2) : -ls[c] * kLog2e));
          if (!jvalid) p = 0.f;
          S[r] = p;
          dP[r] = p * (dP[r] - dvv[c]);
        }
      }
    } else if (PHI == kPhiSilu) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float sv = DQB == 3 ? fmaf(S[r], scale, sbj) : S[r] * scale;
        const float sg = fast_rcp(1.0f + fast_exp2(DQB == 3 ? -sv * kLog2e : S[r] * c1));
        const float p = sv * sg;
        S[r] = p;
        dP[r] = dP[r] * fmaf(sv - p, sg, sg);
      }
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float gr;
        S[r] = phi_value_grad<PHI>(DQB == 3 ? fmaf(S[r], scale, sbj) : S[r] * scale, gr);
        dP[r] *= gr;
      }
    }
    if (DQB == 3) {  // score-bias gradient: the sample's tokens of this step (register r: token 8 (r/4) + 4 g + r%4)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (8 * (r >> 2) + 4 * g + (r & 3) < rows) dsb += dP[r];
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
    // dV += P^T dO, dK += dS^T Q over the 32 tokens.
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int o = (32 * dt + lr) * LDT + 16 * kk + 8 * g;
        dV[dt] = mfma32(pa[kk], lds_read8(&dOt[o]), dV[dt]);
        dK[dt] = mfma32(sa[kk], lds_read8(&Qt[o]), dK[dt]);
      }
    __syncthreads();  // dS complete; Qt and dOt are free

    if (wave >= 4 && s + 1 < nsteps) {
      // Next step's transposed tiles, overlapping the dQ product of waves 0..3.
      wait_vmcnt<DMA_OPS>();  // this wave's copies for step s + 1 landed (step s + 2's may remain)
      transpose(s + 1);
    }
    if (wave < 4) {
      // dQ^T[32 w .. 32 w + 31, tokens] = K^T dS^T over all 256 context rows.
      f32x16 dq = f32x16{};
      // Row kr of K^T, columns 16 ks + 8 g .. + 7: the chunk swizzle moves them by
      // +-64 (sign from bit 2 of ks) on rows with bit 4 set, so two base addresses plus
      // immediate offsets cover all k-steps.
      const int lxd = opaque(lr);
      const int kr = 32 * wave + kt_row(lxd);
      const int sw = ((kr >> 4) & 1) * 64;
      const int oa_p = kr * LDJ + 8 * g + sw, oa_m = kr * LDJ + 8 * g - sw;
      const int ob = lxd * LDJ + 8 * g;
#pragma unroll
      for (int ks = 0; ks < NJ / 16; ++ks)
        dq = mfma32(lds_read8(&Kt[((ks >> 2) & 1 ? oa_m : oa_p) + 16 * ks]), lds_read8(&dSs[ob + 16 * ks]), dq);
      // Lane (t + 32 g), register r: column 32 w + 16 g + r of token t = lr.
      if (lr < rows) {
        uint16_t* dst = (uint16_t*)a.dq + (size_t)(seq0 + tq + lr) * rs + (size_t)h * D + 32 * wave + 16 * g;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          float v[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = dq[8 * hh + e] * scale;
          u32x4 base = u32x4{0u, 0u, 0u, 0u};
          if (DQB == 1)
            base = *(const GDPA_LDS u32x4*)&dOs[wave * 1024 + slot_off(lxd, 2 * g + hh)];
          if (DQB == 2) base = gload16(dst + 8 * hh);
          if (DQB == 1 || DQB == 2) {
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] += bf2f(half_of(base, e));
          }
          *(bf16x8*)(dst + 8 * hh) = pack8(v[0], v[1], v[2], v[3], v[4], v[5], v[6], v[7]);
        }
      }
    }
  }

  // dK (times the scale) and dV through LDS (Kt's space, once every wave is done
  // with it) as bf16 32 x 128 tiles per wave, then 16-byte stores of rows j < n.
  // The copies issued for the two steps past the end land before the work-group
  // releases its LDS.
  if (DQB == 3 && a.d_score_bias != nullptr) {
    dsb += wave_xor32(dsb);
    if (g == 0 && jvalid) a.d_score_bias[(crow0 + j) * H + h] = dsb;
  }
  if (wave >= 4) wait_vmcnt<0>();
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
    uint16_t* dst = (uint16_t*)(which == 0 ? a.dk : a.dv) + (crow0 * H + h) * D;
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
  const int mode = a.score_bias != nullptr || a.d_score_bias != nullptr ? 3
                   : (a.dq_base == nullptr ? 0 : (a.dq_base == a.d_o ? 1 : 2));
  return dispatch_phi(phi, [&](auto P) {
    constexpr int PH = decltype(P)::value;
    if (mode == 0) hipLaunchKernelGGL((bwd_res_kernel<PH, 0>), g, blk, 0, s, a);
    else if (mode == 1) hipLaunchKernelGGL((bwd_res_kernel<PH, 1>), g, blk, 0, s, a);
    else if (mode == 2) hipLaunchKernelGGL((bwd_res_kernel<PH, 2>), g, blk, 0, s, a);
    else hipLaunchKernelGGL((bwd_res_kernel<PH, 3>), g, blk, 0, s, a);
    return hipGetLastError();
  });
}

}  // namespace gdpa
