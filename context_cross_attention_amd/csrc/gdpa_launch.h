// Internal launch interface between the C ABI (gdpa_api.cpp) and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <type_traits>

namespace gdpa {

// Forward q-tile height of the bf16 MFMA kernel (4 waves x 32 rows).
constexpr int kFwdTileRows = 128;
// Backward: each wave owns 32 context rows; q rows are visited 32 at a time.
constexpr int kBwdRowsPerWave = 32;
// Largest batch the on-device longest-first ordering sorts (larger: natural order).
constexpr int kMaxSortBatch = 4096;

// Score maps (the gdpa_phi values of the C ABI).  Softmax normalises over a row;
// the others are elementwise (their values and derivatives are in gdpa_device.h).
constexpr int kPhiSoftmax = 0, kPhiSilu = 1, kPhiRelu = 2, kPhiGelu = 3, kPhiIdentity = 4;
constexpr int kPhiCount = 5;

// Calls f(std::integral_constant<int, phi>{}) for a run-time phi (kernel templates
// take phi as a compile-time parameter).
template <class F>
inline hipError_t dispatch_phi(int phi, F&& f) {
  switch (phi) {
    case kPhiSoftmax: return f(std::integral_constant<int, kPhiSoftmax>{});
    case kPhiSilu: return f(std::integral_constant<int, kPhiSilu>{});
    case kPhiRelu: return f(std::integral_constant<int, kPhiRelu>{});
    case kPhiGelu: return f(std::integral_constant<int, kPhiGelu>{});
    case kPhiIdentity: return f(std::integral_constant<int, kPhiIdentity>{});
  }
  return hipErrorInvalidValue;
}

struct FwdArgs {
  const int32_t* offsets;     // [B+1]
  const int32_t* tile_start;  // [B+1] q-tile prefix sums (bf16 path)
  const void* q;
  const void* k;
  const void* v;
  const void* residual;
  void* o;
  float* lse;
  int B, T, n, H;
  float scale;
  int window;                 // sliding-window self-attention: token i sees i - window < j <= i
  const int32_t* kv_offsets;  // [B+1] jagged context rows (n = the largest count), or nullptr
  // FFN biases, fp32, or nullptr: score_bias[(row0 + j) * H + h] is added to the
  // scaled score of context row j before phi; out_bias[(b * H + h) * d + c] to O.
  const float* score_bias;
  const float* out_bias;
  // Self-attention block (Q = K = V = X, sliding-window forward only): when
  // non-null, O + Q (the block's residual output) is written here as well.
  void* o_plus_q;
};

struct BwdArgs {
  const int32_t* offsets;  // [B+1]
  const int32_t* order;    // [B] samples, longest first
  const void* q;
  const void* k;
  const void* v;
  const void* d_o;
  const float* lse;   // [T*H] softmax
  const float* dvec;  // [T*H] softmax: rowsum(dO * O)
  void* dq;
  void* dk;
  void* dv;
  int B, T, n, H;
  int n_chunks;       // work-groups per (sample, head)
  float scale;
  const void* dq_base;  // dq = dq_base + dQ when non-null (may alias dq or d_o)
  // Self-attention block (K = V, bf16 key-chunk kernel): when non-null, dk receives
  // kv_sum_base + dK + dV and dv is not written.
  const void* kv_sum_base;
  // Sliding-window self-attention: K, V, dK, dV are [T,H,d] token tensors,
  // chunk_start[B+1] the prefix sums of each sample's 32 * waves-row chunks.
  const int32_t* chunk_start;
  int window;
  const int32_t* tile_start;  // [B+1] query-tile prefix sums (dQ kernel)
  const int32_t* kv_offsets;  // [B+1] jagged context rows (n = the largest count), or nullptr
  const float* score_bias;    // as in FwdArgs, or nullptr
  float* d_score_bias;        // gradient of score_bias (written by the dK / dV kernels), or nullptr
};

// Scheduling and small passes (gdpa_sched.hip).
// Prefix sums of ceil(len / tile_rows) over the samples in index order, or in the
// order order[0..B-1] when `order` is given.
hipError_t launch_tile_scan(const int32_t* offsets, int B, int tile_rows, int32_t* tile_start,
                            hipStream_t s, const int32_t* order = nullptr);
hipError_t launch_longest_first(const int32_t* offsets, int B, int32_t* order, hipStream_t s);
// d_out_bias[(b * H + h) * d + c] = sum over the tokens t of sample b of dO[t, h, c].
hipError_t launch_out_bias_grad(const int32_t* offsets, const void* d_o, int B, int H, int d, bool bf16,
                                float* d_out_bias, hipStream_t s);
// out = x0 + x1 (+ x2) (+ x3), bf16, n % 8 == 0; null x2 / x3 are skipped.
hipError_t launch_add_bf16(long n, void* out, const void* x0, const void* x1, const void* x2,
                           const void* x3, hipStream_t s);
// rowsum(dO * O) per (token, head) row; with out_bias, rowsum(dO * (O - out_bias)).
hipError_t launch_softmax_dvec(const void* o, const void* d_o, int rows, int d, bool bf16,
                               float* dvec, hipStream_t s, const int32_t* offsets = nullptr, int B = 0,
                               int H = 1, const float* out_bias = nullptr);

// Forward (gdpa_fwd.hip).
int fwd_bf16_grid(int T, int B, int H);
hipError_t launch_fwd_bf16(const FwdArgs& a, int d, int phi, bool residual, int grid,
                           hipStream_t s);
hipError_t launch_fwd_f32(const FwdArgs& a, int d, int phi, bool residual, hipStream_t s);

// Forward with the context resident in LDS (gdpa_fwd_res.hip), for n * d <= 32768.
bool fwd_res_supported(int d, int n);
hipError_t launch_fwd_res(const FwdArgs& a, const int32_t* order, int d, int phi, bool residual,
                          hipStream_t s);

// Backward (gdpa_bwd.hip).
int bwd_bf16_waves(int d, int n);
// with_dq = false: dK and dV only (dQ from launch_bwd_dq).
hipError_t launch_bwd_bf16(const BwdArgs& a, int d, int phi, int waves, bool with_dq, hipStream_t s);
// dQ over 128-row query tiles (gdpa_bwd_dq.hip), grid as launch_fwd_bf16 (a.tile_start
// over kFwdTileRows-row tiles); sliding_window selects the window mode.
hipError_t launch_bwd_dq(const BwdArgs& a, int d, int phi, bool sliding_window, int grid, hipStream_t s);

// Seed pooling attention (gdpa_pma.hip): m <= 32 seeds [m,H,d] attend over each
// sample's tokens K, V [T,H,d].  One single-wave work-group per (chunk of
// a.chunk tokens, head) over a grid of pma_grid(T, B, H, chunk) (an upper bound;
// surplus work-groups exit).  Samples are visited longest first: order[B]
// (launch_longest_first) and chunk_start[B+1], the prefix sums of
// ceil(L / chunk) over that order.
constexpr int kPmaSlices = 32;  // first-level slices of the dSeeds reduction
// Chunk length for T tokens and H heads: the longest power of two in
// [1024, 8192] that still leaves about 2 work-groups per resident slot of the
// chip (T H / chunk >= 2560).  Longer chunks mean fewer partial results to
// merge; the longest-first order keeps the long ones from forming the tail.
int pma_chunk(int T, int H);
struct PmaArgs {
  const int32_t* offsets;      // [B+1]
  const int32_t* order;        // [B] samples, longest first
  const int32_t* chunk_start;  // [B+1] over the order
  int chunk;                   // tokens per chunk
  const void* seeds;           // [m,H,d]
  const void* k;               // [T,H,d]
  const void* v;
  void* o;                     // [B,m,H,d] (backward: read)
  float* lse;                  // [B,m,H] natural log (backward: read)
  const void* d_o;             // [B,m,H,d]
  void* d_seeds;               // [m,H,d]
  void* dk;                    // [T,H,d]
  void* dv;
  float* part;                 // [chunks][H][32][d]: forward O partials / backward dSeeds partials
  float* part_ml;              // [chunks][H][32][2]: forward (max in log2 units, sum)
  int B, H, m;
  float scale;
};
int pma_grid(int T, int B, int H, int chunk);
// Forward: chunk kernel, then the merge of multi-chunk and empty samples.
hipError_t launch_pma_fwd(const PmaArgs& a, int d, int grid, hipStream_t s);
// Backward: chunk kernel (dK, dV, dSeeds partials), then the two-level dSeeds
// reduction through part2 [kPmaSlices][H][32][d] fp32.
// kv_sum: a.dk receives dK + dV (a.dv unused).
hipError_t launch_pma_bwd(const PmaArgs& a, int d, int grid, float* part2, bool kv_sum, hipStream_t s);

// Sliding-window self-attention on the jagged sequence (softmax, bf16): the
// streaming kernels with K and V taken from the sample's own tokens and the
// context rows limited to each token's window.  The forward grid is that of
// launch_fwd_bf16 (tile_start over kFwdTileRows-row query tiles); the backward
// runs one work-group per (chunk of 32 * swa_bwd_waves(d) key rows, head) over a
// grid of max_chunks * H (an upper bound; surplus work-groups exit) for dK and dV;
// dQ comes from launch_bwd_dq.
hipError_t launch_fwd_swa(const FwdArgs& a, int d, int grid, hipStream_t s);
int swa_bwd_waves(int d);
hipError_t launch_bwd_swa(const BwdArgs& a, int d, int max_chunks, hipStream_t s);
hipError_t launch_bwd_f32(const BwdArgs& a, int d, int phi, hipStream_t s);

// Backward with one work-group per (sample, head) for d = 128, n <= 256 (gdpa_bwd_res.hip).
bool bwd_res_supported(int d, int n);
hipError_t launch_bwd_res(const BwdArgs& a, int phi, hipStream_t s);

// Weight-generation GEMM (gdpa_gemm.hip): C[M][N] = sum_k A(m,k) B(n,k), bf16 in/out,
// fp32 accumulate.  A is [M][K] (a_kmajor = false) or [K][M] (true); B is [N][K] or
// [K][N].  Rows of the operands with k-major layout must be a multiple of 8; with
// k-contiguous layout K must be a multiple of 8.
hipError_t launch_gemm_bf16(bool a_kmajor, bool b_kmajor, int M, int64_t N, int K, const void* A,
                            const void* B, void* C, hipStream_t s);

}  // namespace gdpa
