// GDPA forward with the sample's K and V resident in LDS (bf16, n * d <= 32768).
//
// Same contraction as gdpa_fwd.hip (Kunlun paper summary, section 2.2, GDPA
// bullet), organised for the case where one (sample, head)'s context fits in
// LDS: K [n][d] row-major and V^T [d][n] (transposed, with the context rows
// permuted into the order of the S^T C tile) are loaded once per work-group and
// every query row of the sample streams past them.  All MFMA operand reads are
// 16-byte LDS reads with conflict-free strides; there are no barriers in the
// main loop: each of the 8 waves walks its own 32-row query chunks and
// prefetches the next chunk's Q while computing the current one.
//
// One work-group per (sample, head), launched longest sample first.
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

// Position of context row j inside V^T rows: the S^T C tile holds, in lane group g,
// register r, row 8 (r / 4) + 4 g + r % 4 of a 32-row tile; a B-operand k-step kk
// takes registers 8 kk .. 8 kk + 7.  Storing j = 32 t + 16 kk + 8 a + 4 g + c at
// 32 t + 16 kk + 8 g + 4 a + c makes each lane's 8 operand values contiguous.
__device__ __forceinline__ int vt_pos(int j) { return (j & ~12) | ((j & 4) << 1) | ((j & 8) >> 1); }

// Head columns.  The contraction over d of S^T = K Q^T takes, in k-step ks and lane
// group g, the 8 consecutive columns 32 (ks / 2) + 16 g + 8 (ks % 2) .. + 7 (one
// 16-byte read of a K row, one 16-byte load of a Q row).  In O^T += V^T P^T the
// A operand's row i = 8 a + 4 b + c of each 32-column block is column
// vt_row(i) = 16 b + 4 a + c, so that C-tile lane group g holds the 16 consecutive
// columns 16 g .. 16 g + 15 in register order: two 16-byte stores per block, and
// the residual Q columns of the same lane are exactly its Q operand items.
__device__ __forceinline__ int vt_row(int i) { return 16 * ((i >> 2) & 1) + 4 * (i >> 3) + (i & 3); }
// V^T rows are 16 bytes (mod 256) apart, so row d starts at bank group d % 16 (16-byte
// groups of the 64 4-byte banks); the 16-byte chunk q of row d is stored at chunk
// q ^ (8 (d / 16 % 2)) so that the rows {0..3, 16..19, 4..7, 20..23} + 8 k read by one
// 16-lane phase of a ds_read_b128 fall in distinct bank groups.
__device__ __forceinline__ int vt_chunk(int q, int d) { return q ^ (((d >> 4) & 1) << 3); }

// RESID: 0 none, 1 residual is the query tensor, 2 a separate residual tensor,
// 3 FFN biases (a.score_bias and / or a.out_bias; no residual), 4 residual block:
// O to a.o and O + Q to a.o_plus_q (the layer output X + GDPA(X) with its GDPA term
// kept, which the softmax backward needs).
template <int D, int NMAX, int PHI, int RESID>
__global__ __launch_bounds__(512, 1) void fwd_res_kernel(const FwdArgs a, const int32_t* __restrict__ order) {
  constexpr int NW = 8, NT = NW * 64, KS = D / 16, DT = D / 32, CH = D / 8;
  constexpr int LDK = D + 8;      // K rows: 4 mod 32 dwords -> 8 consecutive rows conflict free
  constexpr int LDV = NMAX + 8;   // V^T rows: likewise for 8 consecutive d rows
  __shared__ __align__(16) uint16_t Kc[NMAX * LDK];
  __shared__ __align__(16) uint16_t Vt[D * LDV];
  __shared__ __align__(16) float Sb[RESID == 3 ? NMAX : 4];  // score bias of the sample's rows

  const int H = a.H;
  const int item = blockIdx.x;
  const int rank = item / H, h = item - rank * H;
  const int b = order[rank];
  const int seq0 = a.offsets[b], L = a.offsets[b + 1] - seq0;
  if (L == 0) return;
  size_t crow0;
  const int n = kv_rows(a.kv_offsets, b, a.n, crow0);  // 1 <= n <= a.n <= NMAX
  const int npad = (n + 63) & ~63;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lr = lane & 31, g = lane >> 5;
  const size_t rs = (size_t)H * D;
  const uint16_t* Kg = (const uint16_t*)a.k + (crow0 * H + h) * D;
  const uint16_t* Vg = (const uint16_t*)a.v + (crow0 * H + h) * D;

  // Stage K row-major and V^T.  Every load is unconditional (row index clamped
  // into the sample) so the compiler keeps them in flight together; padding rows
  // are zeroed afterwards with selects.
  const int nlast = n - 1;
  {
    constexpr int KI = NMAX * CH / NT;   // K chunks per thread (upper bound)
    u32x4 kr[KI];
#pragma unroll
    for (int i = 0; i < KI; ++i) {
      const int idx = i * NT + tid, j = idx / CH, c = idx % CH;
      kr[i] = gload16(Kg + (size_t)min(j, nlast) * rs + 8 * c);
    }
#pragma unroll
    for (int i = 0; i < KI; ++i) {
      const int idx = i * NT + tid, j = idx / CH, c = idx % CH;
      if (j < npad) {
        lds_write16(&Kc[j * LDK + 8 * c], j < n ? kr[i] : u32x4{});
      }
    }
  }
  // V^T: a task is 4 context rows x 8 columns; consecutive lanes take
  // consecutive row groups so the 8-byte LDS writes land on distinct banks.
  {
    constexpr int VI = NMAX / 4 * CH / NT;  // tasks per thread (upper bound)
    const int nq = npad / 4;
    u32x4 vr[VI][4];
#pragma unroll
    for (int i = 0; i < VI; ++i) {
      const int idx = i * NT + tid, jq = idx % nq, dc = min(idx / nq, CH - 1), j0 = 4 * jq;
#pragma unroll
      for (int c = 0; c < 4; ++c) vr[i][c] = gload16(Vg + (size_t)min(j0 + c, nlast) * rs + 8 * dc);
    }
#pragma unroll
    for (int i = 0; i < VI; ++i) {
      const int idx = i * NT + tid, jq = idx % nq, dc = idx / nq, j0 = 4 * jq;
      if (dc >= CH) continue;
      const int pos = vt_pos(j0);
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if (j0 + c >= n) vr[i][c] = u32x4{};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int sh = 16 * (e & 1);
        const uint32_t h0 = (vr[i][0][e >> 1] >> sh) & 0xffffu, h1 = (vr[i][1][e >> 1] >> sh) & 0xffffu;
        const uint32_t h2 = (vr[i][2][e >> 1] >> sh) & 0xffffu, h3 = (vr[i][3][e >> 1] >> sh) & 0xffffu;
        const int d = 8 * dc + e;
        lds_write8(&Vt[d * LDV + 8 * vt_chunk(pos >> 3, d) + (pos & 7)], u32x2{h0 | (h1 << 16), h2 | (h3 << 16)});
      }
    }
  }
  const bool sbias = RESID == 3 && a.score_bias != nullptr;
  if (RESID == 3) {
    for (int j = tid; j < npad; j += NT) Sb[j] = (sbias && j < n) ? a.score_bias[(crow0 + j) * H + h] : 0.f;
  }
  __syncthreads();

  const float scl = a.scale, sl2 = scl * kLog2e, nsl2 = -sl2;
  // Softmax: with a positive scale and no biases the running max is kept in raw Q.K
  // units (see mix); the chunk loop is compiled for both cases (RAW below).
  const bool raw_max = PHI == 0 && RESID != 3 && scl > 0.f;
  const int nchunks = (L + 31) / 32;
  // Query rows past the sample are read from its last row (clamped, always a
  // valid address) and never stored: each lane's row is independent.  k-step ks of
  // lane group g takes columns 32 (ks / 2) + 16 g + 8 (ks % 2) .. + 7.
  const uint16_t* Qg = (const uint16_t*)a.q + (size_t)h * D + 16 * g;
  auto load_q = [&](int ch, bf16x8* dst) {
    const int t = min(32 * ch + lr, L - 1);
    const uint16_t* qp = Qg + (size_t)(seq0 + t) * rs;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) dst[ks] = as_bf16x8(gload16(qp + 32 * (ks >> 1) + 8 * (ks & 1)));
  };

  // One 32-row chunk with Q already in qc; prefetches the Q of chunk ch + NW into qn.
  auto do_chunk = [&](int ch, const bf16x8* qc, bf16x8* qn, auto RAW) {
    constexpr bool raw = decltype(RAW)::value;
    const float sm = raw ? sl2 : 1.0f;
    const int t = 32 * ch + lr;
    const bool tvalid = t < L;
    load_q(ch + NW, qn);
    const size_t obase = (size_t)(seq0 + min(t, L - 1)) * rs + (size_t)h * D + 16 * g;
    // O is first written by the first tile's products (zero accumulator operand), so
    // it needs no zeroing.
    f32x16 O[DT];
    float m_run = -INFINITY, l_run = 0.f;

    // S^T for the 32 context rows j0 .. j0 + 31.
    auto scores = [&](int j0, f32x16& S) {
      S = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        S = mfma32(lds_read8(&Kc[(j0 + lr) * LDK + 32 * (ks >> 1) + 16 * g + 8 * (ks & 1)]), qc[ks], S);
    };
    // phi of one 32-row tile, then O^T += V^T P^T.
    // FIRST: the chunk's first tile (O not yet written, no running max to rescale).
    auto mix = [&](int j0, f32x16& S, auto FIRST) {
      constexpr bool first = decltype(FIRST)::value;
      // Score bias of rows j0 + 8 q + 4 g + {0..3} (register 4 q + i): the scaled
      // score becomes S * scale + b, applied in each map's own units below.
      float bj[16];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4 bv = RESID == 3 ? *(const GDPA_LDS f32x4*)&Sb[j0 + 8 * q + 4 * g] : f32x4{};
#pragma unroll
        for (int i = 0; i < 4; ++i) bj[4 * q + i] = bv[i];
      }
      if (PHI == 0) {
        // With a positive scale and no biases the running max is kept in units of the
        // raw product Q.K and the scale enters each exponent through the FMA that
        // subtracts the max (one VALU operation per score fewer); otherwise (biases, or
        // a scale <= 0) the scores are scaled first and sm = 1.
        // Only a tile that runs past n has scores to mask (wave-uniform test); each case
        // is compiled on its own so that full tiles carry no per-score select.
        const bool tail = j0 + 32 > n;
        float mx = -INFINITY;
        auto mask_max = [&](auto score, auto MASK) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            float s = score(r);
            if (decltype(MASK)::value && j0 + 8 * (r >> 2) + 4 * g + (r & 3) >= n) s = -INFINITY;
            S[r] = s;
            mx = fmaxf(mx, s);
          }
        };
        auto raw_score = [&](int r) { return S[r]; };
        auto scaled_score = [&](int r) { return RESID == 3 ? fmaf(bj[r], kLog2e, S[r] * sl2) : S[r] * sl2; };
        if (raw) {
          if (tail) mask_max(raw_score, std::true_type{});
          else mask_max(raw_score, std::false_type{});
        } else {
          if (tail) mask_max(scaled_score, std::true_type{});
          else mask_max(scaled_score, std::false_type{});
        }
        mx = fmaxf(mx, wave_xor32(mx));
        if (first) {
          m_run = mx;
        } else if (__any((mx - m_run) * sm > kRescaleLog2)) {  // lazy reference max (wave-uniform test)
          const float m_new = fmaxf(m_run, mx);
          const float corr = fast_exp2((m_run - m_new) * sm);
          l_run *= corr;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) O[dt] *= corr;
          m_run = m_new;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = fast_exp2(fmaf(S[r], sm, -m_run * sm));
          l_run += p;
          S[r] = p;
        }
      } else if (PHI == kPhiSilu) {
        // SiLU(s) with s = scale * S: with t = -log2(e) * s, silu(s) = -ln(2) * t / (1 + 2^t).
        // The constant -ln(2) is applied once to O after the last tile.
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float t = RESID == 3 ? fmaf(-bj[r], kLog2e, S[r] * nsl2) : S[r] * nsl2;
          S[r] = t * fast_rcp(1.0f + fast_exp2(t));
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) S[r] = phi_value<PHI>(RESID == 3 ? fmaf(S[r], scl, bj[r]) : S[r] * scl);
      }
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const bf16x8 p = pack_c8(S, kk);
        const int vr = vt_row(lr);  // V^T row within each 32-column block
        const uint16_t* vb = &Vt[vr * LDV + 8 * vt_chunk((j0 >> 3) + 2 * kk + g, vr)];
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
          O[dt] = mfma32(lds_read8(vb + 32 * dt * LDV), p, first && kk == 0 ? f32x16{} : O[dt]);
      }
    };

    // Software pipeline: the MFMAs for the next tile's scores are issued before
    // this tile's phi, so the VALU work overlaps matrix-core time.
    // npad is a multiple of 64, so the tiles come in pairs (at least one).
    const int ntile = npad / 32;
    f32x16 Sa, Sb;
    scores(0, Sa);
    scores(32, Sb);
    mix(0, Sa, std::true_type{});
    __builtin_amdgcn_sched_barrier(0);
    if (2 < ntile) scores(64, Sa);
    mix(32, Sb, std::false_type{});
    __builtin_amdgcn_sched_barrier(0);
    for (int jt = 2; jt < ntile; jt += 2) {
      scores(32 * (jt + 1), Sb);
      mix(32 * jt, Sa, std::false_type{});
      if (jt + 2 < ntile) scores(32 * (jt + 2), Sa);
      mix(32 * (jt + 1), Sb, std::false_type{});
    }
    // The output is O times a per-row factor (SiLU: the constant -ln 2; softmax: 1 / the
    // row sum), applied in the epilogue together with the residual (one FMA per item).
    float oscale = PHI == kPhiSilu ? -kLn2 : 1.0f;
    if (PHI == 0) {
      const float l_tot = l_run + wave_xor32(l_run);
      oscale = 1.0f / l_tot;
      if (tvalid && g == 0 && a.lse != nullptr)
        a.lse[(size_t)(seq0 + t) * H + h] = fmaf(m_run, sm, __log2f(l_tot)) * kLn2;
    }
    if (tvalid) {
      // Lane group g holds columns 32 dt + 16 g + r in register r (see vt_row).
      uint16_t* op = (uint16_t*)a.o + obase;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          float v[8];
          if (RESID == 1) {
            // Residual is Q itself: the same columns are items of the Q operand.
            const bf16x8 qv = qc[2 * dt + hh];
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = fmaf(O[dt][8 * hh + e], oscale, (float)qv[e]);
          } else if (RESID == 2) {
            const u32x4 rr = gload16((const uint16_t*)a.residual + obase + 32 * dt + 8 * hh);
#pragma unroll
            for (int e = 0; e < 8; ++e)
              v[e] = fmaf(O[dt][8 * hh + e], oscale, bf2f((uint16_t)(rr[e >> 1] >> (16 * (e & 1)))));
          } else if (RESID == 3 && a.out_bias != nullptr) {
            const float* bp = a.out_bias + ((size_t)b * H + h) * D + 32 * dt + 16 * g + 8 * hh;
            const f32x4 b0 = *(const f32x4*)bp, b1 = *(const f32x4*)(bp + 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              v[e] = fmaf(O[dt][8 * hh + e], oscale, b0[e]);
              v[4 + e] = fmaf(O[dt][8 * hh + 4 + e], oscale, b1[e]);
            }
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = O[dt][8 * hh + e] * oscale;
          }
          if (RESID == 4) {
            const bf16x8 qv = qc[2 * dt + hh];
            float y[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) y[e] = v[e] + (float)qv[e];
            *(bf16x8*)((uint16_t*)a.o_plus_q + obase + 32 * dt + 8 * hh) =
                pack8(y[0], y[1], y[2], y[3], y[4], y[5], y[6], y[7]);
          }
          *(bf16x8*)(op + 32 * dt + 8 * hh) = pack8(v[0], v[1], v[2], v[3], v[4], v[5], v[6], v[7]);
        }
    }
  };

  // Two register sets for Q alternate between "current" and "prefetch".
  auto chunks = [&](auto RAW) {
    bf16x8 qa[KS], qb[KS];
    load_q(wave, qa);
    for (int ch = wave; ch < nchunks; ch += 2 * NW) {
      do_chunk(ch, qa, qb, RAW);
      if (ch + NW < nchunks) do_chunk(ch + NW, qb, qa, RAW);
    }
  };
  if constexpr (PHI == 0) {
    if (raw_max) chunks(std::true_type{});  // wave-uniform
    else chunks(std::false_type{});
  } else {
    chunks(std::false_type{});
  }
}

bool fwd_res_supported(int d, int n) { return (long)n * d <= 32768 && (d == 32 || d == 64 || d == 128); }

template <int D, int NMAX, int PHI>
static void fwd_res_launch(const FwdArgs& a, const int32_t* order, int resid, hipStream_t s) {
  const dim3 g((unsigned)((long)a.B * a.H)), blk(512);
  if (resid == 0) hipLaunchKernelGGL((fwd_res_kernel<D, NMAX, PHI, 0>), g, blk, 0, s, a, order);
  else if (resid == 1) hipLaunchKernelGGL((fwd_res_kernel<D, NMAX, PHI, 1>), g, blk, 0, s, a, order);
  else if (resid == 2) hipLaunchKernelGGL((fwd_res_kernel<D, NMAX, PHI, 2>), g, blk, 0, s, a, order);
  else if (resid == 3) hipLaunchKernelGGL((fwd_res_kernel<D, NMAX, PHI, 3>), g, blk, 0, s, a, order);
  else hipLaunchKernelGGL((fwd_res_kernel<D, NMAX, PHI, 4>), g, blk, 0, s, a, order);
}

template <int D, int NMAX>
static hipError_t fwd_res_d(const FwdArgs& a, const int32_t* order, int phi, bool resid, hipStream_t s) {
  const bool biased = a.score_bias != nullptr || a.out_bias != nullptr;  // never with a residual
  const int mode = a.o_plus_q != nullptr ? 4 : biased ? 3 : (!resid ? 0 : (a.residual == a.q ? 1 : 2));
  return dispatch_phi(phi, [&](auto P) {
    fwd_res_launch<D, NMAX, decltype(P)::value>(a, order, mode, s);
    return hipGetLastError();
  });
}

hipError_t launch_fwd_res(const FwdArgs& a, const int32_t* order, int d, int phi, bool resid,
                          hipStream_t s) {
  if ((long)a.B * a.H == 0) return hipSuccess;
  switch (d) {
    case 32: return fwd_res_d<32, 1024>(a, order, phi, resid, s);
    case 64: return fwd_res_d<64, 512>(a, order, phi, resid, s);
    case 128: return fwd_res_d<128, 256>(a, order, phi, resid, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace gdpa
