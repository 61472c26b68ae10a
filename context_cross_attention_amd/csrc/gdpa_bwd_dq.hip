// dQ of the GDPA / sliding-window backward, one work-group per 128-row query tile:
// dQ = scale dS K over the tile's context rows, with S, P and dP recomputed, so
// dQ needs no reduction across work-groups (the key-chunk kernel of gdpa_bwd.hip
// then computes dK and dV only).  Same mathematics as gdpa_bwd.hip (Kunlun paper
// summary section 2.2, GDPA bullet; for SW the Sliding Window Attention bullet).
//
// Organisation (as the streaming forward): 4 waves x 32 query rows; each lane
// holds its query row and its dO row as MFMA B operands, and the context rows
// stream through LDS in 64-row blocks shared by the 4 waves:
//   S^T  = K Q^T,  dP^T = V dO^T      (A = K / V rows, 16-byte LDS reads)
//   dS^T = P (dP - rowsum(dO O)) (softmax) or dP phi'(S)      (registers)
//   dQ^T += K^T dS^T                  (A = K columns via LDS transpose reads,
//                                      B = dS^T straight from its C tile)
// One token per lane, so LSE and rowsum(dO O) are one value per lane.
#include "gdpa_device.h"
#include "gdpa_launch.h"

namespace gdpa {

// BIAS: FFN score bias a.score_bias added to the scaled scores (never with SW).
template <int D, int PHI, bool SW, bool BIAS = false>
__global__ __launch_bounds__(256, 2) void bwd_dq_kernel(const BwdArgs a) {
  constexpr int BM = kFwdTileRows, BN = 64, KS = D / 16, DT = D / 32;
  constexpr int LD = D + 8;                   // K and V rows (16-byte reads of 16 rows: distinct banks)
  constexpr int kHalves = (PHI == kPhiGelu || PHI == kPhiIdentity) ? 2 : 1;  // unrolled 32-row halves
  constexpr int CH = D / 8;
  constexpr int SI = (BN * CH + 255) / 256;   // staging chunks per thread per tensor
  __shared__ __align__(16) uint16_t Ks[BN * LD];
  __shared__ __align__(16) uint16_t Vs[BN * LD];
  __shared__ __align__(16) float Sbl[BIAS ? BN : 4];  // score bias of the block's rows

  const int H = a.H, B = a.B;
  const int total = a.tile_start[B];
  const int wid = xcd_remap(blockIdx.x, gridDim.x);
  if (wid >= total * H) return;
  const int qtile = wid / H, h = wid - qtile * H;
  const int b = find_sample(a.tile_start, B, qtile);
  const int seq0 = a.offsets[b];
  const int row0 = seq0 + (qtile - a.tile_start[b]) * BM;
  const int rows = min(BM, a.offsets[b + 1] - row0);
  size_t crow0 = 0;  // first context row of this sample
  const int n = SW ? a.offsets[b + 1] - seq0 : kv_rows(a.kv_offsets, b, a.n, crow0);

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lr = lane & 31, g = lane >> 5;
  const int trow = wave * 32 + lr;
  const bool tvalid = trow < rows;
  const size_t rs = (size_t)H * D;
  const size_t qrow = (size_t)(row0 + (tvalid ? trow : 0)) * rs + (size_t)h * D;

  // Query and dO rows as B operands: items i <-> d = 16 ks + 8 g + i.
  bf16x8 qf[KS], dof[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    qf[ks] = tvalid ? as_bf16x8(gload16((const uint16_t*)a.q + qrow + 16 * ks + 8 * g)) : bf16x8{};
    dof[ks] = tvalid ? as_bf16x8(gload16((const uint16_t*)a.d_o + qrow + 16 * ks + 8 * g)) : bf16x8{};
  }
  const size_t th = (size_t)(row0 + (tvalid ? trow : 0)) * H + h;
  const float lse2 = (PHI == kPhiSoftmax) ? a.lse[th] * kLog2e : 0.f;
  const float dvec = (PHI == kPhiSoftmax) ? a.dvec[th] : 0.f;

  const size_t kv0 = SW ? (size_t)seq0 * H : crow0 * H;
  const uint16_t* Kg = (const uint16_t*)a.k + (kv0 + h) * D;
  const uint16_t* Vg = (const uint16_t*)a.v + (kv0 + h) * D;
  const int qlo = row0 - seq0;
  const int jbeg = SW ? max(0, qlo - a.window + 1) : 0;
  const int jend = SW ? min(n, qlo + rows) : n;
  const int irow = qlo + trow;
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
        lds_write16(&Vs[j * LD + 8 * c], vreg[i]);
      }
    }
    if (BIAS && tid < BN)
      Sbl[tid] = (a.score_bias != nullptr && jb + tid < n) ? a.score_bias[(crow0 + jb + tid) * H + h] : 0.f;
  };
  // Transpose reads of K (as in the forward's V^T): lane 16 G + 4 r + c reads row
  // 4 (G / 2) + r, columns 16 (G % 2) + 4 c of a 32-row slab (second read: rows + 8),
  // so lane (d + 32 g) holds K[j][d] for the j order of the dS^T C tile.
  const int trG = lane >> 4;
  const int tr_off = (4 * (trG >> 1) + ((lane & 15) >> 2)) * LD + 16 * (trG & 1) + 4 * (lane & 3);

  f32x16 dQ[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) dQ[dt] = f32x16{};
  const float sl2 = a.scale * kLog2e;

  if (jbeg < jend) gload_block(jbeg);
  for (int jb = jbeg; jb < jend; jb += BN) {
    __syncthreads();
    store_block(jb);
    __syncthreads();
    if (jb + BN < jend) gload_block(jb + BN);

    // Both 32-row halves unrolled for the maps with more elementwise work to
    // overlap; softmax and ReLU keep one half live (unrolled, they spill).
#pragma unroll kHalves
    for (int mt = 0; mt < 2; ++mt) {
      f32x16 S = f32x16{}, dP = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int o = (32 * mt + lr) * LD + 16 * ks + 8 * g;
        S = mfma32(lds_read8(&Ks[o]), qf[ks], S);
        dP = mfma32(lds_read8(&Vs[o]), dof[ks], dP);
      }
      // Lane (t + 32 g), register r: context row jb + 32 mt + 8 (r / 4) + 4 g + r % 4.
      float bj[16];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4 bv = BIAS ? *(const GDPA_LDS f32x4*)&Sbl[32 * mt + 8 * q + 4 * g] : f32x4{};
#pragma unroll
        for (int i = 0; i < 4; ++i) bj[4 * q + i] = bv[i];
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int j = jb + 32 * mt + 8 * (r >> 2) + 4 * g + (r & 3);
        float ds;
        if (PHI == kPhiSoftmax) {
          // P <= 1 for the sample's rows; the cap keeps rows past n finite when every
          // score of the token is very negative (their P would overflow).
          const float p = fminf(fast_exp2(fmaf(S[r], sl2, BIAS ? fmaf(bj[r], kLog2e, -lse2) : -lse2)), 1.0f);
          ds = p * (dP[r] - dvec);
        } else {
          float gr;
          phi_value_grad<PHI>(BIAS ? fmaf(S[r], a.scale, bj[r]) : S[r] * a.scale, gr);
          ds = dP[r] * gr;
        }
        // Rows past n hold zero K and V in LDS (finite scores and P, and zero products
        // with K), so only a sliding window's band needs masking.
        if (SW && (j >= n || j > irow || j <= irow - a.window)) ds = 0.f;
        S[r] = ds;
      }
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const bf16x8 sb = pack_c8(S, kk);
        const uint16_t* kb = &Ks[(32 * mt + 16 * kk) * LD + tr_off];
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const bf16x8 ka = cat8(lds_read_tr4(kb + 32 * dt), lds_read_tr4(kb + 8 * LD + 32 * dt));
          dQ[dt] = mfma32(ka, sb, dQ[dt]);
        }
      }
    }
  }

  if (tvalid) {
    // Lane (t, g), register r holds dQ[t][d = 32 dt + 8 (r / 4) + 4 g + r % 4].
    const size_t base = (size_t)(row0 + trow) * rs + (size_t)h * D + 4 * g;
    uint16_t* op = (uint16_t*)a.dq + base;
    const uint16_t* bp = (const uint16_t*)a.dq_base;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int col = 32 * dt + 8 * q4;
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = dQ[dt][4 * q4 + e] * a.scale;
        if (bp != nullptr) {
          const u32x2 rr = *(const u32x2*)(bp + base + col);
          v[0] += __uint_as_float(rr[0] << 16);
          v[1] += __uint_as_float(rr[0] & 0xffff0000u);
          v[2] += __uint_as_float(rr[1] << 16);
          v[3] += __uint_as_float(rr[1] & 0xffff0000u);
        }
        bf16x4 ov;
        ov[0] = f2bf(v[0]); ov[1] = f2bf(v[1]); ov[2] = f2bf(v[2]); ov[3] = f2bf(v[3]);
        *(bf16x4*)(op + col) = ov;
      }
  }
}

template <int D, bool SW>
static hipError_t bwd_dq_d(const BwdArgs& a, int phi, int grid, hipStream_t s) {
  const bool biased = !SW && a.score_bias != nullptr;
  return dispatch_phi(phi, [&](auto P) {
    if (biased) hipLaunchKernelGGL((bwd_dq_kernel<D, decltype(P)::value, false, true>), dim3(grid), dim3(256), 0, s, a);
    else hipLaunchKernelGGL((bwd_dq_kernel<D, decltype(P)::value, SW>), dim3(grid), dim3(256), 0, s, a);
    return hipGetLastError();
  });
}

hipError_t launch_bwd_dq(const BwdArgs& a, int d, int phi, bool sliding_window, int grid, hipStream_t s) {
  if (grid == 0) return hipSuccess;
  switch (d) {
    case 32: return sliding_window ? bwd_dq_d<32, true>(a, phi, grid, s) : bwd_dq_d<32, false>(a, phi, grid, s);
    case 64: return sliding_window ? bwd_dq_d<64, true>(a, phi, grid, s) : bwd_dq_d<64, false>(a, phi, grid, s);
    case 128: return sliding_window ? bwd_dq_d<128, true>(a, phi, grid, s) : bwd_dq_d<128, false>(a, phi, grid, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace gdpa
