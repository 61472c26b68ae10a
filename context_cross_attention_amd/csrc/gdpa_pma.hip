// Seed pooling attention over a jagged batch: the attention core of Pooling by
// Multihead Attention, whose learnable seed queries Hierarchical Seed Pooling
// builds on (Kunlun paper summary, section 2.2, HSP bullet; Telegram review,
// layer step 3).  For sample b (tokens offsets[b] .. offsets[b+1]-1 of K, V
// [T,H,d]), seed s < m and head h:
//   O[b,s,h,:] = sum_j softmax_j(scale <Seeds[s,h,:], K[j,h,:]>) V[j,h,:]
// and the backward gives dK, dV per token and dSeeds summed over the batch.
// bf16 in and out, fp32 accumulation, d in {32, 64, 128}, m <= 32.
//
// Work: one single-wave work-group per (chunk of up to a.chunk tokens of one
// sample, head), several per CU, so that one work-group's start and epilogue
// overlap the others' streaming.  The 32 (zero-padded) seeds stay in registers
// as MFMA operands; the chunk's 32-token blocks stream through two LDS slots
// filled by global->LDS DMA two blocks ahead, so each slot is in flight except
// while the wave computes on it.  Per byte of K/V the operation does at most m
// flops, far below the MFMA/HBM balance point of the chip, so the kernels are
// organised around keeping HBM busy; the MFMA work hides under the copies.
//
// LDS tiles are dense row-major [rows][d] bf16 with the 16-byte chunks of a row
// permuted (chunk c of row r stored at position c ^ swz(r)), so that both the
// 16-byte row reads (16 consecutive rows per phase) and the transpose reads
// (4 rows x 64 bytes per 32-lane phase) hit distinct banks.
//
// Forward layout: S^T = K Seeds^T (lane = seed, registers = tokens), so the
// softmax statistics are per lane; O^T += V^T P^T (A = V^T by transpose reads).
// Backward layout: S = Seeds K^T and dP = dO V^T (lane = token, registers =
// seeds); dV^T = dO^T P and dK^T = scale Seeds^T dS (A operands by transpose
// reads of the seed and dO tiles); dSeeds^T += K^T dS^T with dS^T read back
// transposed from a per-wave LDS tile.
#include <math.h>

#include "gdpa_device.h"
#include "gdpa_launch.h"

namespace gdpa {

namespace {

constexpr int kPmaBlock = 32;  // tokens per LDS slot (one wave's MFMA tile)

// Chunk position permutation of a [rows][D] tile (see the header comment).
template <int D>
__device__ __forceinline__ int pma_swz(int row) {
  if constexpr (D == 128) return 4 * (row & 3) + ((row >> 2) & 3);
  else if constexpr (D == 64) return 4 * ((row >> 1) & 1) + ((row >> 2) & 3);
  else return (row >> 2) & 3;
}
// Element offset of 16-byte chunk c (elements 8 c .. 8 c + 7) of `row`.
template <int D>
__device__ __forceinline__ int tile_off(int row, int c) {
  return row * D + 8 * (c ^ pma_swz<D>(row));
}

// DMA of tokens tok0 .. tok0 + 31 (rows past `last` repeat row `last`, so every
// row holds finite data) of K and V into the [32][D] tiles Kt, Vt, by one wave.
// Kg / Vg point at token 0 of the sample, head h; rs is the token stride in
// elements.  D / 8 copies of 1 KiB, tracked by the wave's vmcnt.
template <int D>
__device__ __forceinline__ void pma_issue(uint16_t* Kt, uint16_t* Vt, const uint16_t* Kg,
                                          const uint16_t* Vg, size_t rs, int tok0, int last, int lane) {
  constexpr int NQ = kPmaBlock * D / 512;  // 1 KiB wave copies per tensor
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int e = q * 512 + 8 * lane;
    const int row = e / D, pos = (e % D) / 8;
    const size_t src = (size_t)min(tok0 + row, last) * rs + 8 * (pos ^ pma_swz<D>(row));
    dma16(__builtin_amdgcn_readfirstlane(lds_addr(Kt + q * 512)), Kg + src);
    dma16(__builtin_amdgcn_readfirstlane(lds_addr(Vt + q * 512)), Vg + src);
  }
}

// Waits until the wave's older slot has landed: at most N copies outstanding
// (N = those of the newer slot, or 0), then keeps the compiler from moving LDS
// reads of the slot above the wait.
template <int N>
__device__ __forceinline__ void slot_wait() {
  wait_vmcnt<N>();
  asm volatile("" ::: "memory");
}

// A operand of a [32][D] (or wider) tile read column-wise: lane (x + 32 g) gets
// column 32 dt + x of rows r0 + 16 kk + 4 g + {0..3} and r0 + 16 kk + 8 + 4 g + {0..3},
// the row order of pack_c8(C, kk) for a C tile whose rows are those rows.
template <int D>
__device__ __forceinline__ bf16x8 tile_cols(const uint16_t* t, int r0, int kk, int dt, int lane) {
  const int G = lane >> 4, rr = (lane >> 2) & 3, cc = lane & 3;
  const int R = r0 + 16 * kk + 4 * (G >> 1) + rr;
  const int c8 = 4 * dt + 2 * (G & 1) + (cc >> 1);
  return cat8(lds_read_tr4(t + tile_off<D>(R, c8) + 4 * (cc & 1)),
              lds_read_tr4(t + tile_off<D>(R + 8, c8) + 4 * (cc & 1)));
}

// Epilogue staging of a 32 x D fp32 C tile held as lane (s + 32 g), register r of
// C[dt] <-> row s, column 32 dt + 8 (r / 4) + 4 g + r % 4: rows of D + 4 floats
// in LDS (16-byte writes of 16 consecutive rows fall in distinct banks), each
// value times `mul`.  Waits for the wave's LDS traffic on both sides.
template <int D>
__device__ __forceinline__ void stage_rows(float* st, const f32x16* C, float mul, int lane) {
  const int lr = lane & 31, g = lane >> 5;
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      f32x4 v;
      v[0] = C[dt][4 * q] * mul; v[1] = C[dt][4 * q + 1] * mul;
      v[2] = C[dt][4 * q + 2] * mul; v[3] = C[dt][4 * q + 3] * mul;
      *(GDPA_LDS f32x4*)(st + lr * (D + 4) + 32 * dt + 8 * q + 4 * g) = v;
    }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}
// Rows 0 .. nrows-1 of the staged tile to dst + row * stride as bf16: each lane
// converts 8 consecutive columns, so a wave store covers whole 2 D-byte rows.
template <int D>
__device__ __forceinline__ void store_rows_bf16(const float* st, uint16_t* dst, size_t stride, int nrows, int lane) {
  constexpr int CH = D / 8, RPI = 64 / CH;
  const int c = lane % CH;
#pragma unroll
  for (int i = 0; i < 32 / RPI; ++i) {
    const int row = RPI * i + lane / CH;
    const f32x4 x = *(const GDPA_LDS f32x4*)(st + row * (D + 4) + 8 * c);
    const f32x4 y = *(const GDPA_LDS f32x4*)(st + row * (D + 4) + 8 * c + 4);
    if (row < nrows) {
      bf16x8 v;
      v[0] = f2bf(x[0]); v[1] = f2bf(x[1]); v[2] = f2bf(x[2]); v[3] = f2bf(x[3]);
      v[4] = f2bf(y[0]); v[5] = f2bf(y[1]); v[6] = f2bf(y[2]); v[7] = f2bf(y[3]);
      *(bf16x8*)(dst + (size_t)row * stride + 8 * c) = v;
    }
  }
}
// All 32 rows of the staged tile to the dense [32][D] fp32 array dst.
template <int D>
__device__ __forceinline__ void store_rows_f32(const float* st, float* dst, int lane) {
  constexpr int CH = D / 4, RPI = 64 / CH;
  const int c = lane % CH;
#pragma unroll
  for (int i = 0; i < 32 / RPI; ++i) {
    const int row = RPI * i + lane / CH;
    *(f32x4*)(dst + (size_t)row * D + 4 * c) = *(const GDPA_LDS f32x4*)(st + row * (D + 4) + 4 * c);
  }
}

struct ChunkInfo {
  int b, h, seq0, c0, c1, nch, chunk;
};

__device__ __forceinline__ bool decode_chunk(const PmaArgs& a, ChunkInfo& ci) {
  const int nchunks = a.chunk_start[a.B];
  // Work items in launch order: the dispatcher deals consecutive work-groups to
  // the 8 XCDs in turn, so the longest-first order stays balanced across them.
  const int wid = blockIdx.x;
  if (wid >= nchunks * a.H) return false;
  ci.chunk = wid / a.H;
  ci.h = wid - ci.chunk * a.H;
  const int r = find_sample(a.chunk_start, a.B, ci.chunk);  // rank in the longest-first order
  ci.b = a.order[r];
  ci.seq0 = a.offsets[ci.b];
  const int len = a.offsets[ci.b + 1] - ci.seq0;
  ci.c0 = (ci.chunk - a.chunk_start[r]) * a.chunk;
  ci.c1 = min(len, ci.c0 + a.chunk);
  ci.nch = a.chunk_start[r + 1] - a.chunk_start[r];
  return true;
}

template <int D>
__global__ __launch_bounds__(64) void pma_fwd_kernel(const PmaArgs a) {
  constexpr int KS = D / 16, DT = D / 32, TS = kPmaBlock * D, NPB = D / 8;
  __shared__ __align__(1024) uint16_t ring[4 * TS];  // [slot][K | V][TS]

  ChunkInfo ci;
  if (!decode_chunk(a, ci)) return;
  const int H = a.H, h = ci.h;
  const int lane = threadIdx.x, lr = lane & 31, g = lane >> 5;
  const size_t rs = (size_t)H * D;
  const uint16_t* Kg = (const uint16_t*)a.k + (size_t)ci.seq0 * rs + (size_t)h * D;
  const uint16_t* Vg = (const uint16_t*)a.v + (size_t)ci.seq0 * rs + (size_t)h * D;
  const int len = ci.c1 - ci.c0, last = ci.c1 - 1;
  const int nb = (len + kPmaBlock - 1) / kPmaBlock;  // >= 1

  // Seeds as B operands: lane (s + 32 g) holds Seeds[s][16 ks + 8 g .. + 7].  They
  // are waited for before the first copy is issued, so that no wait for them is
  // left inside the loop (it would also wait for every copy in flight).
  bf16x8 sb[KS];
  {
    const uint16_t* sp = (const uint16_t*)a.seeds + ((size_t)(lr < a.m ? lr : 0) * H + h) * D + 8 * g;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) sb[ks] = lr < a.m ? as_bf16x8(gload16(sp + 16 * ks)) : bf16x8{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) asm volatile("" :: "v"(sb[ks]));
  }
  pma_issue<D>(ring, ring + TS, Kg, Vg, rs, ci.c0, last, lane);
  if (nb > 1) pma_issue<D>(ring + 2 * TS, ring + 3 * TS, Kg, Vg, rs, ci.c0 + kPmaBlock, last, lane);

  const float sl2 = a.scale * kLog2e;
  float m_run = -INFINITY, l_run = 0.f;
  f32x16 O[DT];  // O^T: lane (s + 32 g), register r <-> d = 32 dt + 8 (r / 4) + 4 g + r % 4
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) O[dt] = f32x16{};

  for (int j = 0; j < nb; ++j) {
    if (j + 1 < nb) slot_wait<NPB>(); else slot_wait<0>();
    uint16_t* Kt = ring + (j & 1) * 2 * TS;
    const uint16_t* Vt = Kt + TS;
    const int nvalid = min(kPmaBlock, len - kPmaBlock * j);

    // S^T[t][s]: lane (s + 32 g), register r <-> token 8 (r / 4) + 4 g + r % 4.
    f32x16 S = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) S = mfma32(lds_read8(Kt + tile_off<D>(lr, 2 * ks + g)), sb[ks], S);
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int t = 8 * (r >> 2) + 4 * g + (r & 3);
      S[r] = t < nvalid ? S[r] * sl2 : -INFINITY;
      mx = fmaxf(mx, S[r]);
    }
    mx = fmaxf(mx, wave_xor32(mx));  // finite: token 0 of the block is valid
    // Lazy rescale: the reference maximum moves only when a score exceeds it by
    // more than 2^8, so P <= 256 and the O / l rescale is rare (first block).
    if (__builtin_amdgcn_ballot_w64(mx > m_run + 8.0f) != 0) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = fast_exp2(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) O[dt] *= alpha;
      m_run = m_new;
    }
    float ls = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      S[r] = fast_exp2(S[r] - m_run);
      ls += S[r];
    }
    l_run += ls;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const bf16x8 pb = pack_c8(S, kk);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) O[dt] = mfma32(tile_cols<D>(Vt, 0, kk, dt, lane), pb, O[dt]);
    }
    // The slot's LDS reads have completed (their data fed the MFMAs): refill it.
    if (j + 2 < nb) pma_issue<D>(Kt, Kt + TS, Kg, Vg, rs, ci.c0 + kPmaBlock * (j + 2), last, lane);
  }

  // Epilogue: O^T goes through LDS (the ring is idle now) so that it leaves as
  // whole rows; scattered 8- or 16-byte pieces of 32 rows cost HBM transactions
  // far beyond their bytes.
  const float L = l_run + wave_xor32(l_run);
  const bool single = ci.nch == 1;
  stage_rows<D>((float*)ring, O, single ? 1.0f / L : 1.0f, lane);
  if (single) {
    store_rows_bf16<D>((const float*)ring, (uint16_t*)a.o + ((size_t)ci.b * a.m * H + h) * D, rs, a.m, lane);
    if (lane < a.m) a.lse[((size_t)ci.b * a.m + lane) * H + h] = (m_run + log2f(L)) * kLn2;
  } else {
    store_rows_f32<D>((const float*)ring, a.part + ((size_t)ci.chunk * H + h) * 32 * D, lane);
    if (g == 0) {
      float* mp = a.part_ml + (((size_t)ci.chunk * H + h) * 32 + lr) * 2;
      mp[0] = m_run;
      mp[1] = L;
    }
  }
}

// O and LSE of samples with no chunk (empty: zeros, -inf) or several chunks
// (merge of the chunks' partial max / sum / O); one work-group per (sample, head),
// samples taken by their rank in the longest-first order.
template <int D>
__global__ __launch_bounds__(256) void pma_combine_kernel(const PmaArgs a) {
  constexpr int NC = D / 8;
  const int r = blockIdx.x / a.H, h = blockIdx.x - r * a.H;
  const int b = a.order[r];
  const int c_beg = a.chunk_start[r], nch = a.chunk_start[r + 1] - c_beg;
  if (nch == 1) return;
  const int tid = threadIdx.x, s = tid >> 3, cb = (tid & 7) * NC;
  if (s >= a.m) return;
  uint16_t* op = (uint16_t*)a.o + (((size_t)b * a.m + s) * a.H + h) * D + cb;
  float* lp = a.lse + ((size_t)b * a.m + s) * a.H + h;
  if (nch == 0) {
#pragma unroll
    for (int j = 0; j < NC; j += 4) *(u32x2*)(op + j) = u32x2{};
    if ((tid & 7) == 0) *lp = -INFINITY;
    return;
  }
  float M = -INFINITY;
  for (int c = 0; c < nch; ++c) M = fmaxf(M, a.part_ml[(((size_t)(c_beg + c) * a.H + h) * 32 + s) * 2]);
  float L = 0.f, o[NC];
#pragma unroll
  for (int j = 0; j < NC; ++j) o[j] = 0.f;
  for (int c = 0; c < nch; ++c) {
    const size_t slot = (size_t)(c_beg + c) * a.H + h;
    const float w = fast_exp2(a.part_ml[(slot * 32 + s) * 2] - M);
    L = fmaf(a.part_ml[(slot * 32 + s) * 2 + 1], w, L);
    const float* pp = a.part + slot * 32 * D + (size_t)s * D + cb;
#pragma unroll
    for (int j = 0; j < NC; j += 4) {
      const f32x4 v = *(const f32x4*)(pp + j);
      o[j] = fmaf(v[0], w, o[j]); o[j + 1] = fmaf(v[1], w, o[j + 1]);
      o[j + 2] = fmaf(v[2], w, o[j + 2]); o[j + 3] = fmaf(v[3], w, o[j + 3]);
    }
  }
  const float inv = 1.0f / L;
#pragma unroll
  for (int j = 0; j < NC; j += 4) {
    bf16x4 v;
    v[0] = f2bf(o[j] * inv); v[1] = f2bf(o[j + 1] * inv); v[2] = f2bf(o[j + 2] * inv); v[3] = f2bf(o[j + 3] * inv);
    *(bf16x4*)(op + j) = v;
  }
  if ((tid & 7) == 0) *lp = (M + log2f(L)) * kLn2;
}

// KVSUM: the sequence is pooled with itself (K = V); dK + dV leave as one tensor.
template <int D, bool KVSUM>
__global__ __launch_bounds__(64) void pma_bwd_kernel(const PmaArgs a) {
  constexpr int KS = D / 16, DT = D / 32, TS = kPmaBlock * D, NPB = D / 8;
  __shared__ __align__(1024) uint16_t ring[4 * TS];  // [slot][K | V][TS]
  __shared__ __align__(16) uint16_t dst[32 * 32];    // dS as [token][seed]

  ChunkInfo ci;
  if (!decode_chunk(a, ci)) return;
  const int H = a.H, h = ci.h, m = a.m;
  const int lane = threadIdx.x, lr = lane & 31, g = lane >> 5;
  const size_t rs = (size_t)H * D;
  const uint16_t* Kg = (const uint16_t*)a.k + (size_t)ci.seq0 * rs + (size_t)h * D;
  const uint16_t* Vg = (const uint16_t*)a.v + (size_t)ci.seq0 * rs + (size_t)h * D;
  const int len = ci.c1 - ci.c0, last = ci.c1 - 1;
  const int nb = (len + kPmaBlock - 1) / kPmaBlock;  // >= 1
  pma_issue<D>(ring, ring + TS, Kg, Vg, rs, ci.c0, last, lane);

  // Seeds and dO of (b, h), zero-padded to 32 rows, as [32][D] tiles in the
  // second slot (filled only after the set-up).  The set-up's loads wait for the
  // first slot's copies too (they were issued earlier); the second slot's copies
  // are issued after the set-up so that no wait inside the loop covers them.
  uint16_t* St = ring + 2 * TS;
  uint16_t* Dt = ring + 3 * TS;
  for (int i = lane; i < 32 * (D / 8); i += 64) {
    const int s = i / (D / 8), c = i % (D / 8);
    u32x4 sv = u32x4{}, dv = u32x4{};
    if (s < m) {
      sv = gload16((const uint16_t*)a.seeds + ((size_t)s * H + h) * D + 8 * c);
      dv = gload16((const uint16_t*)a.d_o + (((size_t)ci.b * m + s) * H + h) * D + 8 * c);
    }
    lds_write16(St + tile_off<D>(s, c), sv);
    lds_write16(Dt + tile_off<D>(s, c), dv);
  }
  __syncthreads();

  // Row operands, lane (s + 32 g): Seeds / dO [s][16 ks + 8 g .. + 7].
  bf16x8 seA[KS], doA[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    seA[ks] = lds_read8(St + tile_off<D>(lr, 2 * ks + g));
    doA[ks] = lds_read8(Dt + tile_off<D>(lr, 2 * ks + g));
  }
  // Column operands, lane (x + 32 g): Seeds / dO [seeds of pack_c8(., kk)][32 dt + x].
  bf16x8 seT[2][DT], doT[2][DT];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      seT[kk][dt] = tile_cols<D>(St, 0, kk, dt, lane);
      doT[kk][dt] = tile_cols<D>(Dt, 0, kk, dt, lane);
    }
  // rowsum(dO * O) and the log2-scaled LSE of seed lr; padded seeds get P = 0.
  float dv_s = 0.f;
  if (lr < m) {
    const uint16_t* op = (const uint16_t*)a.o + (((size_t)ci.b * m + lr) * H + h) * D + 8 * g;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const u32x4 ov = gload16(op + 16 * ks);
      const u32x4 dw = __builtin_bit_cast(u32x4, doA[ks]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        dv_s = fmaf(__uint_as_float(ov[e] << 16), __uint_as_float(dw[e] << 16), dv_s);
        dv_s = fmaf(__uint_as_float(ov[e] & 0xffff0000u), __uint_as_float(dw[e] & 0xffff0000u), dv_s);
      }
    }
  }
  dv_s += wave_xor32(dv_s);
  const float lse2_s = lr < m ? a.lse[((size_t)ci.b * m + lr) * H + h] * kLog2e : INFINITY;
  // Per register of the lane = token layout: register r <-> seed 8 (r / 4) + 4 g + r % 4.
  float lse2r[16], dvr[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int src = 8 * (r >> 2) + 4 * g + (r & 3);
    lse2r[r] = __shfl(lse2_s, src, 64);
    dvr[r] = __shfl(dv_s, src, 64);
  }

  asm volatile("" :: "v"(dv_s), "v"(lse2_s));
  __syncthreads();  // the tile reads have completed: the second slot may be filled
  if (nb > 1) pma_issue<D>(ring + 2 * TS, ring + 3 * TS, Kg, Vg, rs, ci.c0 + kPmaBlock, last, lane);

  const float sl2 = a.scale * kLog2e;
  uint16_t* myds = dst;
  f32x16 dSd[DT];  // dSeeds^T: lane (s + 32 g), register r <-> d = 32 dt + 8 (r / 4) + 4 g + r % 4
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) dSd[dt] = f32x16{};
  const int G = lane >> 4, rr = (lane >> 2) & 3, cc = lane & 3;

  // vmcnt counts this wave's copies and stores together, in issue order.  Issued
  // after block j's copies: the previous block's NST row stores, then block
  // j + 1's NPB copies; waiting for exactly block j keeps both in flight (the
  // stores of a full block are NST instructions; only the last block can be
  // partial, and nothing waits past it).
  constexpr int NST = (KVSUM ? 1 : 2) * (D / 16);
  for (int j = 0; j < nb; ++j) {
    if (j == 0) {
      if (nb > 1) slot_wait<NPB>(); else slot_wait<0>();
    } else {
      if (j + 1 < nb) slot_wait<NPB + NST>(); else slot_wait<NST>();
    }
    uint16_t* Kt = ring + (j & 1) * 2 * TS;
    const uint16_t* Vt = Kt + TS;
    const int tok0 = ci.c0 + kPmaBlock * j;  // sample-local
    const int nvalid = min(kPmaBlock, ci.c1 - tok0);
    const int r0 = 0;

    // S = Seeds K^T, dP = dO V^T: lane (t + 32 g), register r <-> seed 8 (r / 4) + 4 g + r % 4.
    f32x16 S = f32x16{}, dP = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int off = tile_off<D>(r0 + lr, 2 * ks + g);
      S = mfma32(seA[ks], lds_read8(Kt + off), S);
      dP = mfma32(doA[ks], lds_read8(Vt + off), dP);
    }
    const bool tv = lr < nvalid;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = tv ? fast_exp2(fmaf(S[r], sl2, -lse2r[r])) : 0.f;
      S[r] = p;
      dP[r] = p * (dP[r] - dvr[r]);
    }
    // dV^T = dO^T P, dK^T = scale Seeds^T dS: lane (t + 32 g), register r <-> d = 32 dt + 8 (r / 4) + 4 g + r % 4.
    // Both go out through the slot's own tiles (V is no longer needed once dP is
    // formed, K once the dSeeds products have read it), as whole rows.
    uint16_t* Vw = Kt + TS;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      f32x16 acc = f32x16{};
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) acc = mfma32(doT[kk][dt], pack_c8(S, kk), acc);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        bf16x4 v;
        v[0] = f2bf(acc[4 * q]); v[1] = f2bf(acc[4 * q + 1]); v[2] = f2bf(acc[4 * q + 2]); v[3] = f2bf(acc[4 * q + 3]);
        *(GDPA_LDS bf16x4*)(Vw + tile_off<D>(lr, 4 * dt + q) + 4 * g) = v;
      }
    }
    // dS into the wave's tile as [token][seed]: 4-seed (8-byte) unit u of row t at u ^ ((t >> 2) & 7).
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      bf16x4 v;
      v[0] = f2bf(dP[4 * q]); v[1] = f2bf(dP[4 * q + 1]); v[2] = f2bf(dP[4 * q + 2]); v[3] = f2bf(dP[4 * q + 3]);
      *(GDPA_LDS bf16x4*)(myds + 32 * lr + 4 * ((2 * q + g) ^ ((lr >> 2) & 7))) = v;
    }
    // dSeeds^T += K^T dS^T: B = dS^T read back transposed, lane (s + 32 g) gets the
    // tokens 16 kk + 4 g + {0..3}, 16 kk + 8 + 4 g + {0..3} of seed s.
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int R = 16 * kk + 4 * (G >> 1) + rr, u = 4 * (G & 1) + cc;
      const bf16x8 bs = cat8(lds_read_tr4(myds + 32 * R + 4 * (u ^ ((R >> 2) & 7))),
                             lds_read_tr4(myds + 32 * (R + 8) + 4 * (u ^ (((R + 8) >> 2) & 7))));
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) dSd[dt] = mfma32(tile_cols<D>(Kt, r0, kk, dt, lane), bs, dSd[dt]);
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      f32x16 acc = f32x16{};
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) acc = mfma32(seT[kk][dt], pack_c8(dP, kk), acc);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        bf16x4 v;
        v[0] = f2bf(acc[4 * q] * a.scale); v[1] = f2bf(acc[4 * q + 1] * a.scale);
        v[2] = f2bf(acc[4 * q + 2] * a.scale); v[3] = f2bf(acc[4 * q + 3] * a.scale);
        *(GDPA_LDS bf16x4*)(Kt + tile_off<D>(lr, 4 * dt + q) + 4 * g) = v;
      }
    }
    // Rows out: lane l takes 16-byte chunk l % (D / 8) of row RPI i + l / (D / 8).
    {
      constexpr int CH = D / 8, RPI = 64 / CH;
      const int c = lane % CH;
      uint16_t* dvg = KVSUM ? nullptr : (uint16_t*)a.dv + (size_t)(ci.seq0 + tok0) * rs + (size_t)h * D + 8 * c;
      uint16_t* dkg = (uint16_t*)a.dk + (size_t)(ci.seq0 + tok0) * rs + (size_t)h * D + 8 * c;
#pragma unroll
      for (int i2 = 0; i2 < 32 / RPI; ++i2) {
        const int row = RPI * i2 + lane / CH;
        const u32x4 vv = __builtin_bit_cast(u32x4, lds_read8(Vw + tile_off<D>(row, c)));
        const u32x4 kv = __builtin_bit_cast(u32x4, lds_read8(Kt + tile_off<D>(row, c)));
        if (KVSUM) {
          bf16x8 sv;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            sv[2 * e] = f2bf(__uint_as_float(vv[e] << 16) + __uint_as_float(kv[e] << 16));
            sv[2 * e + 1] = f2bf(__uint_as_float(vv[e] & 0xffff0000u) + __uint_as_float(kv[e] & 0xffff0000u));
          }
          if (row < nvalid) *(bf16x8*)(dkg + (size_t)row * rs) = sv;
        } else if (row < nvalid) {
          *(u32x4*)(dvg + (size_t)row * rs) = vv;
          *(u32x4*)(dkg + (size_t)row * rs) = kv;
        }
      }
    }
    // The slot's LDS reads have completed (their data fed the MFMAs): refill it.
    if (j + 2 < nb) pma_issue<D>(Kt, Kt + TS, Kg, Vg, rs, ci.c0 + kPmaBlock * (j + 2), last, lane);
  }

  // This chunk's dSeeds^T partial [32][D] (unscaled), as whole rows through LDS.
  stage_rows<D>((float*)ring, dSd, 1.0f, lane);
  store_rows_f32<D>((const float*)ring, a.part + ((size_t)ci.chunk * H + h) * 32 * D, lane);
}

// dSeeds, first level: slice sl sums the partials of chunks sl, sl + kPmaSlices, ...
// (4 consecutive elements of one (head, seed, d) row per thread).
__global__ __launch_bounds__(256) void pma_reduce1_kernel(const float* __restrict__ part, const int32_t* chunk_start,
                                                          int B, int per_chunk, float* __restrict__ part2) {
  const int sl = blockIdx.y;
  const int e = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (e >= per_chunk) return;
  const int nchunks = chunk_start[B];
  f32x4 acc = f32x4{};
  for (int c = sl; c < nchunks; c += kPmaSlices) acc += *(const f32x4*)(part + (size_t)c * per_chunk + e);
  *(f32x4*)(part2 + (size_t)sl * per_chunk + e) = acc;
}

// dSeeds, second level: sum of the slices, times scale, into d_seeds [m][H][D] bf16.
template <int D>
__global__ __launch_bounds__(256) void pma_reduce2_kernel(const float* __restrict__ part2, int H, int m,
                                                          float scale, uint16_t* __restrict__ d_seeds) {
  const int per_chunk = H * 32 * D;
  const int e = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (e >= per_chunk) return;
  const int hs = e / D, d = e % D, h = hs / 32, s = hs % 32;
  if (s >= m) return;
  f32x4 acc = f32x4{};
  for (int sl = 0; sl < kPmaSlices; ++sl) acc += *(const f32x4*)(part2 + (size_t)sl * per_chunk + e);
  bf16x4 v;
  v[0] = f2bf(acc[0] * scale); v[1] = f2bf(acc[1] * scale); v[2] = f2bf(acc[2] * scale); v[3] = f2bf(acc[3] * scale);
  *(bf16x4*)(d_seeds + ((size_t)s * H + h) * D + d) = v;
}

}  // namespace

int pma_chunk(int T, int H) {
  int c = 1024;
  while (c < 8192 && (int64_t)T * H / (2 * c) >= 2560) c *= 2;
  return c;
}

int pma_grid(int T, int B, int H, int chunk) {
  const long chunks = (long)T / chunk + B;  // >= sum_b ceil(L_b / chunk)
  const long g = (chunks * H + 7) / 8 * 8;
  return (int)g;
}

hipError_t launch_pma_fwd(const PmaArgs& a, int d, int grid, hipStream_t s) {
  if (grid > 0) {
    switch (d) {
      case 32: hipLaunchKernelGGL(pma_fwd_kernel<32>, dim3(grid), dim3(64), 0, s, a); break;
      case 64: hipLaunchKernelGGL(pma_fwd_kernel<64>, dim3(grid), dim3(64), 0, s, a); break;
      case 128: hipLaunchKernelGGL(pma_fwd_kernel<128>, dim3(grid), dim3(64), 0, s, a); break;
      default: return hipErrorInvalidValue;
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const dim3 cg((unsigned)(a.B * a.H));
  switch (d) {
    case 32: hipLaunchKernelGGL(pma_combine_kernel<32>, cg, dim3(256), 0, s, a); break;
    case 64: hipLaunchKernelGGL(pma_combine_kernel<64>, cg, dim3(256), 0, s, a); break;
    case 128: hipLaunchKernelGGL(pma_combine_kernel<128>, cg, dim3(256), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_pma_bwd(const PmaArgs& a, int d, int grid, float* part2, bool kv_sum, hipStream_t s) {
  if (grid > 0) {
#define GDPA_PMA_BWD(DD)                                                                               \
  case DD:                                                                                             \
    if (kv_sum) hipLaunchKernelGGL((pma_bwd_kernel<DD, true>), dim3(grid), dim3(64), 0, s, a);        \
    else hipLaunchKernelGGL((pma_bwd_kernel<DD, false>), dim3(grid), dim3(64), 0, s, a);              \
    break;
    switch (d) {
      GDPA_PMA_BWD(32)
      GDPA_PMA_BWD(64)
      GDPA_PMA_BWD(128)
      default: return hipErrorInvalidValue;
    }
#undef GDPA_PMA_BWD
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int per_chunk = a.H * 32 * d;
  const unsigned nb = (unsigned)((per_chunk / 4 + 255) / 256);
  hipLaunchKernelGGL(pma_reduce1_kernel, dim3(nb, kPmaSlices), dim3(256), 0, s, a.part, a.chunk_start, a.B,
                     per_chunk, part2);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  switch (d) {
    case 32: hipLaunchKernelGGL(pma_reduce2_kernel<32>, dim3(nb), dim3(256), 0, s, part2, a.H, a.m, a.scale, (uint16_t*)a.d_seeds); break;
    case 64: hipLaunchKernelGGL(pma_reduce2_kernel<64>, dim3(nb), dim3(256), 0, s, part2, a.H, a.m, a.scale, (uint16_t*)a.d_seeds); break;
    case 128: hipLaunchKernelGGL(pma_reduce2_kernel<128>, dim3(nb), dim3(256), 0, s, part2, a.H, a.m, a.scale, (uint16_t*)a.d_seeds); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace gdpa
