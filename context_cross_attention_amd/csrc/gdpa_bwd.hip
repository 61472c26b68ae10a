// GDPA backward: dQ, dK, dV of sum(O * dO), with dK and dV summed over each
// sample's own tokens (the keys and values are per-sample weights derived from
// that sample's context; Kunlun paper summary section 2.2, GDPA bullet).
//
// bf16 path.  One work-group owns (sample b, head h, a chunk of 32 * NW context
// rows); wave w owns 32 of those rows and keeps their dK and dV accumulators in
// registers while the work-group walks all of the sample's query rows, 32 at a
// time.  So dK and dV are reduced per sample without atomics.  Per 32-row query
// tile (Q and dO staged in LDS, row-major):
//   S  = Q K^T,  dP = dO V^T      (M = tokens, N = the wave's context rows)
//   P  = phi(S); dS = softmax: P (dP - rowsum(dO O)),  elementwise maps: dP phi'(S)
//   dV += P^T dO, dK += scale dS^T Q   (A = P^T / dS^T straight from the C tile,
//                                       B = dO / Q columns via LDS transpose reads)
//   dQ  = scale dS K over all the work-group's context rows: dS^T goes to LDS and
//         every wave computes 16x16 output tiles from it.
// When the context rows need more than one work-group, this kernel computes dK and
// dV only and dQ comes from the query-tile kernel of gdpa_bwd_dq.hip (S, P, dP
// recomputed there), so nothing is reduced across work-groups.
//
// Work-groups are launched longest sample first (longest-processing-time list
// scheduling by the hardware dispatcher).
//
// fp32 path: plain loops in fp32, for the small fp32 workload.
#include "gdpa_device.h"
#include "gdpa_launch.h"

namespace gdpa {

// Storage row of token t (0..31) of a query tile: inside each group of 8 rows,
// tokens 0..3 go to even rows and 4..7 to odd rows.
__device__ __forceinline__ int qpos(int t) { return (t & ~7) | ((t & 3) << 1) | ((t >> 2) & 1); }

// SW: sliding-window self-attention (Kunlun paper summary, section 2.2, Sliding
// Window Attention bullet).  The work-group's key rows are a chunk of its sample's
// own tokens, only the query steps whose windows reach them are visited, pairs
// outside i - window < j <= i get P = dS = 0.
// DQ = false: dK and dV only (dQ comes from the query-tile kernel of gdpa_bwd_dq.hip,
// used whenever several key chunks feed a query row).
// BIAS: FFN score bias a.score_bias (per context row, added to the scaled score)
// and its gradient a.d_score_bias (the sum of the score gradient over the tokens).
// KVSUM (self-attention block, with SW): dk receives a.kv_sum_base + dK + dV, dv is
// not written.
template <int D, int PHI, int NW, bool SW = false, bool DQ = true, bool BIAS = false, bool KVSUM = false>
__global__ __launch_bounds__(NW * 64, 8 / NW) void bwd_bf16_kernel(const BwdArgs a) {
  constexpr int NJ = 32 * NW;          // context rows per work-group
  constexpr int BQ = kBwdRowsPerWave;  // query rows per step
  constexpr int KS = D / 16, DT = D / 32, LD = D + 8, CH = D / 8;
  constexpr int LDT = BQ + 8;          // dS^T row stride
  // LDS bank layout (32 banks of 4 bytes).  Row strides D + 8 and BQ + 8 are 4 mod 32
  // dwords (20 for BQ + 8), so 16-byte reads by 8 consecutive rows are conflict
  // free, and transpose loads over rows spaced by 2 are too.  Q and dO tile rows
  // are stored at qpos(t), which spreads each run of 4 consecutive tokens over
  // rows 2 apart while keeping any 8 consecutive tokens on distinct banks.
  constexpr int NT = NW * 64;
  constexpr int DQ_TILES = (BQ / 16) * (D / 16);
  constexpr int TPW = DQ_TILES / NW;   // 16x16 dQ tiles per wave
  static_assert(TPW * NW == DQ_TILES && TPW >= 1, "dQ tiles must split evenly over waves");

  __shared__ __align__(16) uint16_t Kc[NJ * LD];
  __shared__ __align__(16) uint16_t Qs[BQ * LD];
  __shared__ __align__(16) uint16_t dOs[BQ * LD];
  __shared__ __align__(16) uint16_t dSt[DQ ? NJ * LDT : 8];
  __shared__ float lse_s[BQ], dvec_s[BQ];

  const int H = a.H, nch = a.n_chunks;
  const int item = blockIdx.x;
  int b, h, jc;
  if (SW) {
    const int c = item / H;  // the grid is an upper bound on the number of chunks
    if (c >= a.chunk_start[a.B]) return;
    h = item - c * H;
    b = find_sample(a.chunk_start, a.B, c);
    jc = c - a.chunk_start[b];
  } else {
    // The nch chunks of one (sample, head) read the same Q and dO rows.  Blocks are
    // dealt to the 8 XCDs round robin, so block 8 s + x runs on XCD x: the chunks
    // of pair 8 s' + x take slots s = nch s' .. nch s' + nch - 1 of XCD x, and their
    // Q / dO reads after the first hit that XCD's L2.  Pairs stay in longest-first
    // order across slots; the grid is padded to whole groups of 8 pairs.
    const int x = item & 7, slot = item >> 3;
    const int grp = slot / nch;
    jc = slot - grp * nch;
    const int pair = 8 * grp + x;
    if (pair >= a.B * H) return;
    const int rank = pair / H;
    h = pair - rank * H;
    b = a.order[rank];
  }
  const int seq0 = a.offsets[b], L = a.offsets[b + 1] - seq0;
  size_t crow0 = 0;  // first context row of this sample
  const int n = SW ? L : kv_rows(a.kv_offsets, b, a.n, crow0);  // key rows of this sample
  const int j0 = jc * NJ;
  if (j0 >= n) return;  // a jagged context with fewer rows than the largest

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lr = lane & 31, g = lane >> 5;
  const size_t rs = (size_t)H * D;
  const size_t kv0 = SW ? (size_t)seq0 * H : crow0 * H;
  const uint16_t* Kg = (const uint16_t*)a.k + (kv0 + h) * D;
  const uint16_t* Vg = (const uint16_t*)a.v + (kv0 + h) * D;

  // K chunk, row-major, into LDS (zero rows past n); loads first, then writes.
  {
    constexpr int KI = NJ * CH / NT;
    u32x4 kr[KI];
#pragma unroll
    for (int i = 0; i < KI; ++i) {
      const int idx = i * NT + tid, j = idx / CH, c = idx % CH;
      kr[i] = (j0 + j < n) ? gload16(Kg + (size_t)(j0 + j) * rs + 8 * c) : u32x4{};
    }
#pragma unroll
    for (int i = 0; i < KI; ++i) {
      const int idx = i * NT + tid, j = idx / CH, c = idx % CH;
      lds_write16(&Kc[j * LD + 8 * c], kr[i]);
    }
  }
  // The wave's V rows as B operand of dP = dO V^T: lane (j + 32 g), items d = 16 ks + 8 g + i.
  const int jl = 32 * wave + lr;  // local context row of this lane
  const int jw = j0 + jl;
  const bool jvalid = jw < n;
  const float sbj = (BIAS && a.score_bias != nullptr && jvalid) ? a.score_bias[(crow0 + jw) * H + h] : 0.f;
  float dsb = 0.f;  // sum over the tokens of the score gradient of row jw (BIAS)
  bf16x8 vf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    vf[ks] = jvalid ? as_bf16x8(gload16(Vg + (size_t)jw * rs + 16 * ks + 8 * g)) : bf16x8{};

  f32x16 dK[DT], dV[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    dK[dt] = f32x16{};
    dV[dt] = f32x16{};
  }

  // Transpose-read addressing for the dV / dK products (row order of the C tile,
  // as in the forward kernel) and for the dQ product (contiguous rows, 16x16x32).
  const int trG = lane >> 4, trr = (lane & 15) >> 2;
  // dV / dK B operand: lane 16 G + 4 r + c reads token row 16 kk + 4 (G / 2) + r
  // (second read + 8), columns 32 dt + 16 (G % 2) + 4 c.
  const int tr_tok = 4 * (trG >> 1) + trr, tr_col = 16 * (trG & 1) + 4 * (lane & 3);
  // dQ operands (16x16x32): lane 16 G + 4 r + c reads context row 8 G + 2 r (second
  // read + 1), columns base + 4 c; item i <-> context row 8 G + 2 (i % 4) + i / 4.
  const int q16_row = 8 * trG + 2 * trr, q16_col = 4 * (lane & 3);

  const float sl2 = a.scale * kLog2e, nsl2 = -sl2;
  const uint16_t* Qg = (const uint16_t*)a.q + (size_t)h * D;
  const uint16_t* dOg = (const uint16_t*)a.d_o + (size_t)h * D;

  // Each thread stages SPT 16-byte chunks of the Q and dO tiles per step; the
  // next step's chunks are loaded while the current step computes.
  constexpr int SPT = (BQ * CH + NT - 1) / NT;
  u32x4 q_next[SPT], do_next[SPT];
  float lse_next = INFINITY, dvec_next = 0.f;
  auto load_step = [&](int tq) {
    const int rows_ = min(BQ, L - tq);
#pragma unroll
    for (int i = 0; i < SPT; ++i) {
      const int idx = i * NT + tid, t = idx / CH, c = idx % CH;
      const bool ok = idx < BQ * CH && t < rows_;
      const size_t off = (size_t)(seq0 + tq + t) * rs + 8 * c;
      q_next[i] = ok ? gload16(Qg + off) : u32x4{};
      do_next[i] = ok ? gload16(dOg + off) : u32x4{};
    }
    if (PHI == 0 && tid < BQ) {
      const bool ok = tid < rows_;
      const size_t r = (size_t)(seq0 + tq + tid) * H + h;
      lse_next = ok ? a.lse[r] * kLog2e : INFINITY;
      dvec_next = ok ? a.dvec[r] : 0.f;
    }
  };
  // Query steps: every token, or (SW) the tokens whose windows reach key rows
  // j0 .. j0 + NJ - 1, i.e. j0 .. j0 + NJ + window - 2.
  const int tq_beg = SW ? min(j0, L) : 0;
  const int tq_end = SW ? min(L, j0 + NJ - 1 + a.window) : L;
  if (tq_beg < tq_end) load_step(tq_beg);

  for (int tq = tq_beg; tq < tq_end; tq += BQ) {
    const int rows = min(BQ, L - tq);
    __syncthreads();  // previous step is done with Qs, dOs, dSt
#pragma unroll
    for (int i = 0; i < SPT; ++i) {
      const int idx = i * NT + tid, t = idx / CH, c = idx % CH;
      if (idx < BQ * CH) {
        lds_write16(&Qs[qpos(t) * LD + 8 * c], q_next[i]);
        lds_write16(&dOs[qpos(t) * LD + 8 * c], do_next[i]);
      }
    }
    if (PHI == 0 && tid < BQ) {
      lse_s[tid] = lse_next;
      dvec_s[tid] = dvec_next;
    }
    __syncthreads();
    if (tq + BQ < tq_end) load_step(tq + BQ);
    // SW: no token of this step sees any of the wave's 32 key rows (all are after the
    // tokens, or all left their windows): nothing to add (no barrier follows in the
    // step without dQ).
    if (SW && !DQ && (tq + BQ - 1 < j0 + 32 * wave || tq - a.window >= j0 + 32 * wave + 31)) continue;

    // S = Q K^T and dP = dO V^T for the wave's 32 context rows.
    f32x16 S = f32x16{}, dP = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 qa = lds_read8(&Qs[qpos(lr) * LD + 16 * ks + 8 * g]);
      const bf16x8 kb = lds_read8(&Kc[jl * LD + 16 * ks + 8 * g]);
      S = mfma32(qa, kb, S);
      const bf16x8 da = lds_read8(&dOs[qpos(lr) * LD + 16 * ks + 8 * g]);
      dP = mfma32(da, vf[ks], dP);
    }

    // Lane (j + 32 g), register r: token t = 8 (r / 4) + 4 g + r % 4 of the step.
    f32x16 P, dS;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int t = 8 * (r >> 2) + 4 * g + (r & 3);
      float p, ds;
      if (PHI == 0) {
        // P <= 1 for the sample's rows; the cap keeps rows past n finite when every
        // score of the token is very negative (their P would overflow).
        p = fminf(fast_exp2(BIAS ? fmaf(sbj, kLog2e, S[r] * sl2) - lse_s[t] : fmaf(S[r], sl2, -lse_s[t])), 1.0f);
        ds = p * (dP[r] - dvec_s[t]);
      } else if (PHI == kPhiSilu && !BIAS) {
        // With sg = sigmoid(scale S) and q = S sg: P = scale q (the scale is applied to dV
        // at the end) and ds / dP = sg + scale q (1 - sg).
        const float sg = fast_rcp(1.0f + fast_exp2(S[r] * nsl2));
        p = S[r] * sg;
        ds = dP[r] * fmaf(a.scale, fmaf(-p, sg, p), sg);
      } else {
        float gr;
        p = phi_value_grad<PHI>(BIAS ? fmaf(S[r], a.scale, sbj) : S[r] * a.scale, gr);
        ds = dP[r] * gr;
      }
      // Rows past n (lanes with !jvalid) have zero K and V: their scores and P are
      // finite, their dK, dV and score-bias gradients are never stored, and they add
      // nothing to dQ (zero K rows), so only a sliding window's band needs masking.
      if (SW && (!jvalid || jw > tq + t || jw <= tq + t - a.window)) {
        p = 0.f;
        ds = 0.f;
      }
      P[r] = p;
      if (BIAS) dsb += ds;  // rows past the sample have dO = 0, so ds = 0 there
      dS[r] = ds;  // the score scale is applied to dK and dQ at the end
    }

    // dS^T rows of this wave into LDS: row jl, tokens 8 q + 4 g .. + 3.
#pragma unroll
    for (int q4 = 0; q4 < (DQ ? 4 : 0); ++q4) {
      bf16x4 v;
      v[0] = f2bf(dS[4 * q4 + 0]); v[1] = f2bf(dS[4 * q4 + 1]);
      v[2] = f2bf(dS[4 * q4 + 2]); v[3] = f2bf(dS[4 * q4 + 3]);
      *(GDPA_LDS bf16x4*)(&dSt[jl * LDT + 8 * q4 + 4 * g]) = v;
    }

    // dV += P^T dO, dK += dS^T Q (contraction over the 32 tokens of the step).
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const bf16x8 pa = pack_c8(P, kk);
      const bf16x8 sa = pack_c8(dS, kk);
      const int r0 = qpos(16 * kk + tr_tok) * LD + tr_col, r1 = qpos(16 * kk + 8 + tr_tok) * LD + tr_col;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const bf16x8 dob = cat8(lds_read_tr4(&dOs[r0 + 32 * dt]), lds_read_tr4(&dOs[r1 + 32 * dt]));
        dV[dt] = mfma32(pa, dob, dV[dt]);
        const bf16x8 qb = cat8(lds_read_tr4(&Qs[r0 + 32 * dt]), lds_read_tr4(&Qs[r1 + 32 * dt]));
        dK[dt] = mfma32(sa, qb, dK[dt]);
      }
    }
    if (!DQ) continue;
    __syncthreads();  // dS^T complete

    // dQ[32 x D] = dS[32 x NJ] K[NJ x D] with 16x16x32 tiles; wave w takes TPW tiles.
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int tile = wave * TPW + i;
      const int t0 = 16 * (tile / (D / 16)), d0 = 16 * (tile % (D / 16));
      f32x4 acc = f32x4{};
#pragma unroll 4
      for (int js = 0; js < NJ; js += 32) {
        const int ra = (js + q16_row) * LDT + t0 + q16_col;
        const bf16x8 av = cat8(lds_read_tr4(&dSt[ra]), lds_read_tr4(&dSt[ra + LDT]));
        const int rb = (js + q16_row) * LD + d0 + q16_col;
        const bf16x8 bv = cat8(lds_read_tr4(&Kc[rb]), lds_read_tr4(&Kc[rb + LD]));
        acc = mfma16(av, bv, acc);
      }
      // Lane (d + 16 q), register r: token t0 + 4 q + r, column d0 + lane % 16.
      const int d = d0 + (lane & 15);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = t0 + 4 * (lane >> 4) + r;
        if (t < rows) {
          const size_t idx = (size_t)(seq0 + tq + t) * rs + (size_t)h * D + d;
          float v = acc[r] * a.scale;
          if (a.dq_base != nullptr) v += bf2f(((const uint16_t*)a.dq_base)[idx]);
          ((uint16_t*)a.dq)[idx] = __builtin_bit_cast(uint16_t, f2bf(v));
        }
      }
    }
  }

  if (BIAS && a.d_score_bias != nullptr) {
    dsb += wave_xor32(dsb);
    if (g == 0 && jvalid) a.d_score_bias[(crow0 + jw) * H + h] = dsb;
  }
  // dK takes the score scale here, and so does dV when P was kept without it (SiLU).
  constexpr bool dv_scaled = PHI == kPhiSilu && !BIAS;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dK[dt][r] *= a.scale;
      if (dv_scaled) dV[dt][r] *= a.scale;
    }
  // dK, dV: lane (d + 32 g), register r holds context row 32 w + 8 (r / 4) + 4 g + r % 4.
  uint16_t* dkp = (uint16_t*)a.dk + (kv0 + h) * D;
  uint16_t* dvp = (uint16_t*)a.dv + (kv0 + h) * D;
  if (KVSUM) {  // self-attention block: base + dK + dV in one tensor
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) dK[dt][r] += dV[dt][r];
    // A column block's base values are loaded before its stores: the compiler
    // cannot prove that the stores leave the base alone, so interleaved, every
    // load would wait for the store before it.
    const uint16_t* bp = (const uint16_t*)a.kv_sum_base + (kv0 + h) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      uint16_t base[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int j = min(j0 + 32 * wave + 8 * (r >> 2) + 4 * g + (r & 3), n - 1);
        base[r] = bp[(size_t)j * rs + 32 * dt + lr];
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int j = j0 + 32 * wave + 8 * (r >> 2) + 4 * g + (r & 3);
        if (j < n)
          dkp[(size_t)j * rs + 32 * dt + lr] = __builtin_bit_cast(uint16_t, f2bf(bf2f(base[r]) + dK[dt][r]));
      }
    }
    return;
  }
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int j = j0 + 32 * wave + 8 * (r >> 2) + 4 * g + (r & 3);
      if (j < n) {
        const size_t idx = (size_t)j * rs + 32 * dt + lr;
        dkp[idx] = __builtin_bit_cast(uint16_t, f2bf(dK[dt][r]));
        dvp[idx] = __builtin_bit_cast(uint16_t, f2bf(dV[dt][r]));
      }
    }
}

// ---------------------------------------------------------------------------
// fp32 path
// ---------------------------------------------------------------------------

template <int D, int PHI>
__device__ __forceinline__ void f32_ds(float s_raw, float dp, float scale, float lse, float dvec,
                                       float& p, float& ds, float bias = 0.f) {
  const float s = fmaf(s_raw, scale, bias);
  if (PHI == 0) {
    p = expf(s - lse);
    ds = p * (dp - dvec);
  } else if (PHI == kPhiSilu) {
    const float sg = 1.0f / (1.0f + expf(-s));
    p = s * sg;
    ds = dp * sg * (1.0f + s * (1.0f - sg));
  } else if (PHI == kPhiRelu) {
    p = fmaxf(s, 0.f);
    ds = s > 0.f ? dp : 0.f;
  } else if (PHI == kPhiGelu) {
    const float cdf = 0.5f * (1.0f + erff(s * 0.70710678118654752f));
    p = s * cdf;
    ds = dp * (cdf + s * expf(-0.5f * s * s) * 0.39894228040143268f);
  } else {
    p = s;
    ds = dp;
  }
}

// dQ: one thread per (token, head).
template <int D, int PHI>
__global__ __launch_bounds__(128) void bwd_f32_dq_kernel(const BwdArgs a) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // the grid's last block overhangs T * H
  if (idx >= (int64_t)a.T * a.H) return;
  const int t = (int)(idx / a.H), h = (int)(idx - (int64_t)t * a.H);
  const int b = find_sample(a.offsets, a.B, t);
  const size_t rs = (size_t)a.H * D;
  const float* qp = (const float*)a.q + (size_t)t * rs + (size_t)h * D;
  const float* dop = (const float*)a.d_o + (size_t)t * rs + (size_t)h * D;
  const float lse = PHI == 0 ? a.lse[(size_t)t * a.H + h] : 0.f;
  const float dvec = PHI == 0 ? a.dvec[(size_t)t * a.H + h] : 0.f;
  float acc[D];
#pragma unroll
  for (int e = 0; e < D; ++e) acc[e] = 0.f;
  size_t crow0;
  const int n = kv_rows(a.kv_offsets, b, a.n, crow0);
  const float* Kb = (const float*)a.k + (crow0 * a.H + h) * D;
  const float* Vb = (const float*)a.v + (crow0 * a.H + h) * D;
  for (int j = 0; j < n; ++j) {
    const float* kj = Kb + (size_t)j * rs;
    const float* vj = Vb + (size_t)j * rs;
    float s = 0.f, dp = 0.f;
#pragma unroll
    for (int e = 0; e < D; ++e) {
      s = fmaf(qp[e], kj[e], s);
      dp = fmaf(dop[e], vj[e], dp);
    }
    float p, ds;
    f32_ds<D, PHI>(s, dp, a.scale, lse, dvec, p, ds,
                   a.score_bias != nullptr ? a.score_bias[(crow0 + j) * a.H + h] : 0.f);
    ds *= a.scale;
#pragma unroll
    for (int e = 0; e < D; ++e) acc[e] = fmaf(ds, kj[e], acc[e]);
  }
  const size_t row = (size_t)t * rs + (size_t)h * D;
  const float* basep = a.dq_base != nullptr ? (const float*)a.dq_base + row : nullptr;
  float* dqp = (float*)a.dq + row;
#pragma unroll
  for (int e = 0; e < D; ++e) dqp[e] = acc[e] + (basep != nullptr ? basep[e] : 0.f);
}

// dK, dV: one thread per (sample, context row, head, 32-column slice).
template <int D, int PHI>
__global__ __launch_bounds__(128) void bwd_f32_dkdv_kernel(const BwdArgs a) {
  constexpr int DS = D / 32;
  const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (long)a.B * a.n * a.H * DS) return;
  const int sl = idx % DS;
  const long bjh = idx / DS;
  const int h = bjh % a.H;
  const long bj = bjh / a.H;
  const int j = bj % a.n;
  const int b = (int)(bj / a.n);
  size_t crow0;
  if (j >= kv_rows(a.kv_offsets, b, a.n, crow0)) return;  // past a jagged sample's rows
  const size_t rs = (size_t)a.H * D;
  const float* kj = (const float*)a.k + (crow0 + j) * rs + (size_t)h * D;
  const float* vj = (const float*)a.v + (crow0 + j) * rs + (size_t)h * D;
  const float sbj = a.score_bias != nullptr ? a.score_bias[(crow0 + j) * a.H + h] : 0.f;
  float dsb = 0.f;
  float gk[32], gv[32];
#pragma unroll
  for (int e = 0; e < 32; ++e) {
    gk[e] = 0.f;
    gv[e] = 0.f;
  }
  for (int t = a.offsets[b]; t < a.offsets[b + 1]; ++t) {
    const float* qp = (const float*)a.q + (size_t)t * rs + (size_t)h * D;
    const float* dop = (const float*)a.d_o + (size_t)t * rs + (size_t)h * D;
    float s = 0.f, dp = 0.f;
#pragma unroll
    for (int e = 0; e < D; ++e) {
      s = fmaf(qp[e], kj[e], s);
      dp = fmaf(dop[e], vj[e], dp);
    }
    const float lse = PHI == 0 ? a.lse[(size_t)t * a.H + h] : 0.f;
    const float dvec = PHI == 0 ? a.dvec[(size_t)t * a.H + h] : 0.f;
    float p, ds;
    f32_ds<D, PHI>(s, dp, a.scale, lse, dvec, p, ds, sbj);
    dsb += ds;
    ds *= a.scale;
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      gv[e] = fmaf(p, dop[32 * sl + e], gv[e]);
      gk[e] = fmaf(ds, qp[32 * sl + e], gk[e]);
    }
  }
  if (sl == 0 && a.d_score_bias != nullptr) a.d_score_bias[(crow0 + j) * a.H + h] = dsb;
  float* dkp = (float*)a.dk + (crow0 + j) * rs + (size_t)h * D + 32 * sl;
  float* dvp = (float*)a.dv + (crow0 + j) * rs + (size_t)h * D + 32 * sl;
#pragma unroll
  for (int e = 0; e < 32; ++e) {
    dkp[e] = gk[e];
    dvp[e] = gv[e];
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

int bwd_bf16_waves(int d, int n) {
  // 8 waves (256 context rows) per work-group; 4 when the context is short
  // or the head is narrow.
  if (d == 32) return 4;
  return n <= 128 ? 4 : 8;
}

template <int D, int NW>
static hipError_t bwd_bf16_dw(const BwdArgs& a, int phi, bool with_dq, hipStream_t s) {
  const long pairs = (long)a.B * a.H;
  if (pairs == 0 || a.n_chunks == 0) return hipSuccess;
  const long items = (pairs + 7) / 8 * 8 * a.n_chunks;  // whole groups of 8 pairs (see the kernel)
  const dim3 g((unsigned)items), blk(NW * 64);
  const bool biased = a.score_bias != nullptr || a.d_score_bias != nullptr;
  return dispatch_phi(phi, [&](auto P) {
    constexpr int PH = decltype(P)::value;
    if (biased && with_dq) hipLaunchKernelGGL((bwd_bf16_kernel<D, PH, NW, false, true, true>), g, blk, 0, s, a);
    else if (biased) hipLaunchKernelGGL((bwd_bf16_kernel<D, PH, NW, false, false, true>), g, blk, 0, s, a);
    else if (with_dq) hipLaunchKernelGGL((bwd_bf16_kernel<D, PH, NW, false, true>), g, blk, 0, s, a);
    else hipLaunchKernelGGL((bwd_bf16_kernel<D, PH, NW, false, false>), g, blk, 0, s, a);
    return hipGetLastError();
  });
}

// Sliding window: 4-wave work-groups of 128 key rows.  Without the dS^T tile
// (dQ comes from the query-tile kernel) one takes 52 KiB of LDS, so two share a
// CU and one's barriers and staging overlap the other's MFMAs.  The 8-wave form
// fills a CU alone and spills registers (measured: window-512 backward 23.3 ->
// 18.7 ms on a batch of 1.44 M tokens, H = 8, d = 128).
int swa_bwd_waves(int d) { (void)d; return 4; }

template <int D, int NW>
static hipError_t bwd_swa_dw(const BwdArgs& a, int max_chunks, hipStream_t s) {
  const long items = (long)max_chunks * a.H;
  if (items == 0) return hipSuccess;
  if (a.kv_sum_base != nullptr)
    hipLaunchKernelGGL((bwd_bf16_kernel<D, kPhiSoftmax, NW, true, false, false, true>), dim3((unsigned)items),
                       dim3(NW * 64), 0, s, a);
  else
    hipLaunchKernelGGL((bwd_bf16_kernel<D, kPhiSoftmax, NW, true, false>), dim3((unsigned)items), dim3(NW * 64),
                       0, s, a);
  return hipGetLastError();
}

hipError_t launch_bwd_swa(const BwdArgs& a, int d, int max_chunks, hipStream_t s) {
  switch (d) {
    case 32: return bwd_swa_dw<32, 4>(a, max_chunks, s);
    case 64: return bwd_swa_dw<64, 4>(a, max_chunks, s);
    case 128: return bwd_swa_dw<128, 4>(a, max_chunks, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_bf16(const BwdArgs& a, int d, int phi, int waves, bool with_dq, hipStream_t s) {
  if (d == 32 && waves == 4) return bwd_bf16_dw<32, 4>(a, phi, with_dq, s);
  if (d == 64 && waves == 4) return bwd_bf16_dw<64, 4>(a, phi, with_dq, s);
  if (d == 64 && waves == 8) return bwd_bf16_dw<64, 8>(a, phi, with_dq, s);
  if (d == 128 && waves == 4) return bwd_bf16_dw<128, 4>(a, phi, with_dq, s);
  if (d == 128 && waves == 8) return bwd_bf16_dw<128, 8>(a, phi, with_dq, s);
  return hipErrorInvalidValue;
}

template <int D>
static hipError_t bwd_f32_d(const BwdArgs& a, int phi, hipStream_t s) {
  const long nq = (long)a.T * a.H;
  const long nkv = (long)a.B * a.n * a.H * (D / 32);
  // dK/dV first: the dQ buffer may be the dO buffer itself.
  if (nkv > 0) {
    const dim3 g((unsigned)((nkv + 127) / 128)), blk(128);
    const hipError_t e = dispatch_phi(phi, [&](auto P) {
      hipLaunchKernelGGL((bwd_f32_dkdv_kernel<D, decltype(P)::value>), g, blk, 0, s, a);
      return hipGetLastError();
    });
    if (e != hipSuccess) return e;
  }
  if (nq > 0) {
    const dim3 g((unsigned)((nq + 127) / 128)), blk(128);
    return dispatch_phi(phi, [&](auto P) {
      hipLaunchKernelGGL((bwd_f32_dq_kernel<D, decltype(P)::value>), g, blk, 0, s, a);
      return hipGetLastError();
    });
  }
  return hipGetLastError();
}

hipError_t launch_bwd_f32(const BwdArgs& a, int d, int phi, hipStream_t s) {
  switch (d) {
    case 32: return bwd_f32_d<32>(a, phi, s);
    case 64: return bwd_f32_d<64>(a, phi, s);
    case 128: return bwd_f32_d<128>(a, phi, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace gdpa
