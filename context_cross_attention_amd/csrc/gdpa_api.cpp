// C ABI of the GDPA library: argument checks, workspace layout and launches.
// Every check happens on the host before the first HIP call, so invalid
// arguments are reported without touching the device.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <map>
#include <mutex>
#include <vector>

#include "gdpa.h"
#include "gdpa_launch.h"

namespace {

static_assert(GDPA_PHI_SOFTMAX == gdpa::kPhiSoftmax && GDPA_PHI_SILU == gdpa::kPhiSilu &&
                  GDPA_PHI_RELU == gdpa::kPhiRelu && GDPA_PHI_GELU == gdpa::kPhiGelu &&
                  GDPA_PHI_IDENTITY == gdpa::kPhiIdentity,
              "ABI score-map values are the kernels' template parameters");

thread_local int g_last_hip_error = 0;

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

gdpa_status hip_status(hipError_t e) {
  if (e == hipSuccess) return GDPA_OK;
  g_last_hip_error = (int)e;
  return GDPA_ERR_HIP;
}

gdpa_status check_problem(const gdpa_problem* p) {
  if (p == nullptr) return GDPA_ERR_INVALID_ARGUMENT;
  if (p->batch < 1 || p->total_tokens < 0 || p->max_seqlen < 0 || p->n_kv < 1 || p->heads < 1 ||
      p->head_dim < 1)
    return GDPA_ERR_INVALID_ARGUMENT;
  if (p->phi < GDPA_PHI_SOFTMAX || p->phi > GDPA_PHI_IDENTITY) return GDPA_ERR_INVALID_ARGUMENT;
  if (p->dtype != GDPA_F32 && p->dtype != GDPA_BF16) return GDPA_ERR_INVALID_ARGUMENT;
  if (!std::isfinite(p->scale)) return GDPA_ERR_INVALID_ARGUMENT;
  // Element counts index with 32-bit token and row numbers and 64-bit offsets.
  if ((int64_t)p->total_tokens * p->heads > INT32_MAX) return GDPA_ERR_INVALID_ARGUMENT;
  if ((int64_t)p->batch * p->n_kv * p->heads > INT32_MAX) return GDPA_ERR_INVALID_ARGUMENT;
  if (p->head_dim != 32 && p->head_dim != 64 && p->head_dim != 128) return GDPA_ERR_UNSUPPORTED;
  if (p->flags & ~(uint32_t)(GDPA_FWD_RESIDUAL | GDPA_BWD_ACCUM_DQ | GDPA_BWD_RESIDUAL))
    return GDPA_ERR_UNSUPPORTED;
  return GDPA_OK;
}

// Workspace layouts (each region 256-byte aligned).
//   forward : tile_start [B+1] int32 (streaming kernel) | order [B] int32 (resident kernel)
//   backward: order [B] int32 | dvec [T*H] fp32 (softmax, except in the one-work-group
//             backward, which sums the row term itself) | tile_start [B+1] int32 (bf16,
//             when the context rows span several work-groups: dQ per query tile)
struct BwdPlan {
  int waves = 0, chunks = 0;
  size_t order_off = 0, dvec_off = 0, tile_off = 0, total = 0;
  bool split_dq = false;  // several key chunks per (sample, head): dQ from the query-tile kernel
};

// The one-work-group-per-(sample, head) backward (bf16, d = 128, n <= 256): it sums the
// softmax row term from P and dP itself, so it needs neither O nor the row-dot pass.
bool bwd_one_wg(const gdpa_problem* p) {
  return p->dtype == GDPA_BF16 && gdpa::bwd_res_supported(p->head_dim, p->n_kv);
}

BwdPlan bwd_plan(const gdpa_problem* p) {
  BwdPlan pl;
  const size_t TH = (size_t)p->total_tokens * p->heads;
  if (bwd_one_wg(p)) {
    pl.waves = 4;
    pl.chunks = 1;
  } else if (p->dtype == GDPA_BF16) {
    pl.waves = gdpa::bwd_bf16_waves(p->head_dim, p->n_kv);
    const int nj = 32 * pl.waves;
    pl.chunks = (p->n_kv + nj - 1) / nj;
    pl.split_dq = pl.chunks > 1;
  }
  size_t off = 0;
  pl.order_off = off;
  off += align_up(sizeof(int32_t) * (size_t)p->batch);
  pl.dvec_off = off;
  if (p->phi == GDPA_PHI_SOFTMAX && !bwd_one_wg(p)) off += align_up(sizeof(float) * TH);
  pl.tile_off = off;
  if (pl.split_dq) off += align_up(sizeof(int32_t) * ((size_t)p->batch + 1));
  pl.total = off;
  return pl;
}

size_t fwd_workspace(const gdpa_problem* p) {
  return align_up(sizeof(int32_t) * ((size_t)p->batch + 1)) + align_up(sizeof(int32_t) * (size_t)p->batch);
}

// Biased backward, softmax, bf16, with an output bias: the softmax row term
// sum_e (P V)[e] dO[e] cannot come from the bf16 O = P V + b_o (its rounding is
// relative to |P V + b_o|, which a large bias makes far coarser than |P V|), so the
// backward recomputes P V once without the bias into its workspace.  Layout after
// the backward plan: forward workspace | P V [T*H*d] bf16 | LSE [T*H] fp32.
struct RecomputePlan {
  bool on = false;
  size_t fwd_off = 0, o_off = 0, lse_off = 0, total = 0;
};

RecomputePlan recompute_plan(const gdpa_problem* p, size_t base, bool out_bias) {
  RecomputePlan r;
  r.total = base;
  r.on = out_bias && p->dtype == GDPA_BF16 && p->phi == GDPA_PHI_SOFTMAX && !bwd_one_wg(p);
  if (!r.on) return r;
  const size_t TH = (size_t)p->total_tokens * p->heads;
  r.fwd_off = base;
  r.o_off = r.fwd_off + fwd_workspace(p);
  r.lse_off = r.o_off + align_up(TH * p->head_dim * 2);
  r.total = r.lse_off + align_up(TH * sizeof(float));
  return r;
}

}  // namespace

extern "C" {

size_t gdpa_workspace_bytes(const gdpa_problem* p, int backward) {
  if (check_problem(p) != GDPA_OK) return 0;
  return backward ? bwd_plan(p).total : fwd_workspace(p);
}

size_t gdpa_biased_workspace_bytes(const gdpa_problem* p, int backward, int out_bias) {
  if (check_problem(p) != GDPA_OK) return 0;
  if (!backward) return fwd_workspace(p);
  return recompute_plan(p, bwd_plan(p).total, out_bias != 0).total;
}

}  // extern "C"

namespace {

// Forward and backward of the dense ([B, n_kv, H, d]) and jagged ([rows, H, d]
// with kv_offsets) context forms; kv_offsets == nullptr selects the dense one.
gdpa_status fwd_impl(const gdpa_problem* p, const int32_t* offsets, const int32_t* kv_offsets,
                     const void* q, const void* k, const void* v, const void* residual, void* o,
                     float* lse, void* workspace, size_t workspace_bytes, void* stream,
                     const float* score_bias = nullptr, const float* out_bias = nullptr,
                     bool launch = true, void* o_plus_q = nullptr) {
  const gdpa_status st = check_problem(p);
  if (st != GDPA_OK) return st;
  if (offsets == nullptr || k == nullptr || v == nullptr) return GDPA_ERR_INVALID_ARGUMENT;
  if (p->total_tokens > 0 && (q == nullptr || o == nullptr)) return GDPA_ERR_INVALID_ARGUMENT;
  const bool resid = (p->flags & GDPA_FWD_RESIDUAL) != 0;
  if (resid && residual == nullptr && p->total_tokens > 0) return GDPA_ERR_INVALID_ARGUMENT;
  if (p->flags & (GDPA_BWD_ACCUM_DQ | GDPA_BWD_RESIDUAL)) return GDPA_ERR_INVALID_ARGUMENT;
  if (resid && residual == o && residual != q) return GDPA_ERR_INVALID_ARGUMENT;
  if (o != nullptr && (o == q || o == k || o == v)) return GDPA_ERR_INVALID_ARGUMENT;
  const size_t need = fwd_workspace(p);
  if (p->dtype == GDPA_BF16 && (workspace == nullptr || workspace_bytes < need))
    return GDPA_ERR_WORKSPACE_TOO_SMALL;
  if (!launch || p->total_tokens == 0) return GDPA_OK;

  hipStream_t s = (hipStream_t)stream;
  gdpa::FwdArgs a{};
  a.offsets = offsets;
  a.q = q;
  a.k = k;
  a.v = v;
  a.residual = residual;
  a.o = o;
  a.lse = (p->phi == GDPA_PHI_SOFTMAX) ? lse : nullptr;
  a.kv_offsets = kv_offsets;
  a.score_bias = score_bias;
  a.out_bias = out_bias;
  a.o_plus_q = o_plus_q;
  a.B = p->batch;
  a.T = p->total_tokens;
  a.n = p->n_kv;
  a.H = p->heads;
  a.scale = p->scale;
  if (p->dtype == GDPA_F32) return hip_status(gdpa::launch_fwd_f32(a, p->head_dim, p->phi, resid, s));

  if (gdpa::fwd_res_supported(p->head_dim, p->n_kv)) {
    int32_t* order = (int32_t*)((char*)workspace + align_up(sizeof(int32_t) * ((size_t)p->batch + 1)));
    hipError_t e = gdpa::launch_longest_first(offsets, p->batch, order, s);
    if (e != hipSuccess) return hip_status(e);
    return hip_status(gdpa::launch_fwd_res(a, order, p->head_dim, p->phi, resid, s));
  }
  int32_t* tile_start = (int32_t*)workspace;
  hipError_t e = gdpa::launch_tile_scan(offsets, p->batch, gdpa::kFwdTileRows, tile_start, s);
  if (e != hipSuccess) return hip_status(e);
  a.tile_start = tile_start;
  const int grid = gdpa::fwd_bf16_grid(p->total_tokens, p->batch, p->heads);
  return hip_status(gdpa::launch_fwd_bf16(a, p->head_dim, p->phi, resid, grid, s));
}

gdpa_status bwd_impl(const gdpa_problem* p, const int32_t* offsets, const int32_t* kv_offsets,
                     const void* q, const void* k, const void* v, const void* o, const float* lse,
                     const void* d_o, void* dq, void* dk, void* dv, void* workspace,
                     size_t workspace_bytes, void* stream, const float* score_bias = nullptr,
                     const float* out_bias = nullptr, float* d_score_bias = nullptr,
                     float* d_out_bias = nullptr, bool launch = true) {
  const gdpa_status st = check_problem(p);
  if (st != GDPA_OK) return st;
  if (offsets == nullptr || k == nullptr || v == nullptr || dk == nullptr || dv == nullptr)
    return GDPA_ERR_INVALID_ARGUMENT;
  if (p->total_tokens > 0 && (q == nullptr || d_o == nullptr || dq == nullptr))
    return GDPA_ERR_INVALID_ARGUMENT;
  const bool softmax = p->phi == GDPA_PHI_SOFTMAX;
  const bool one_wg = bwd_one_wg(p);  // then O is not read
  if (softmax && p->total_tokens > 0 && (lse == nullptr || (o == nullptr && !one_wg)))
    return GDPA_ERR_INVALID_ARGUMENT;
  if (p->flags & GDPA_FWD_RESIDUAL) return GDPA_ERR_INVALID_ARGUMENT;
  const bool accum = (p->flags & GDPA_BWD_ACCUM_DQ) != 0;
  const bool dq_resid = (p->flags & GDPA_BWD_RESIDUAL) != 0;
  if (accum && dq_resid) return GDPA_ERR_INVALID_ARGUMENT;
  if (dq != nullptr && dq == d_o && !accum && !dq_resid) return GDPA_ERR_INVALID_ARGUMENT;
  if (dk == dv || dk == k || dk == v || dv == k || dv == v) return GDPA_ERR_INVALID_ARGUMENT;
  const BwdPlan pl = bwd_plan(p);
  const RecomputePlan rp = recompute_plan(p, pl.total, out_bias != nullptr);
  if (workspace == nullptr || workspace_bytes < rp.total) return GDPA_ERR_WORKSPACE_TOO_SMALL;
  if (!launch) return GDPA_OK;

  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;
  gdpa::BwdArgs a{};
  a.offsets = offsets;
  a.order = (const int32_t*)(ws + pl.order_off);
  a.q = q;
  a.k = k;
  a.v = v;
  a.d_o = d_o;
  a.lse = lse;
  a.dvec = softmax && !one_wg ? (const float*)(ws + pl.dvec_off) : nullptr;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.tile_start = pl.split_dq ? (const int32_t*)(ws + pl.tile_off) : nullptr;
  a.kv_offsets = kv_offsets;
  a.score_bias = score_bias;
  a.d_score_bias = d_score_bias;
  a.B = p->batch;
  a.T = p->total_tokens;
  a.n = p->n_kv;
  a.H = p->heads;
  a.n_chunks = pl.chunks;
  a.scale = p->scale;
  a.dq_base = accum ? (const void*)dq : (dq_resid ? d_o : nullptr);

  const size_t TH = (size_t)p->total_tokens * p->heads;
  hipError_t e = hipSuccess;
  if (softmax && TH > 0 && rp.on) {
    gdpa_problem fp = *p;
    fp.flags = 0;
    const gdpa_status fs = fwd_impl(&fp, offsets, kv_offsets, q, k, v, nullptr, ws + rp.o_off,
                                    (float*)(ws + rp.lse_off), ws + rp.fwd_off, fwd_workspace(p), stream,
                                    score_bias, nullptr);
    if (fs != GDPA_OK) return fs;
    e = gdpa::launch_softmax_dvec(ws + rp.o_off, d_o, (int)TH, p->head_dim, true, (float*)(ws + pl.dvec_off),
                                  s);
    if (e != hipSuccess) return hip_status(e);
  } else if (softmax && TH > 0 && !one_wg) {
    e = gdpa::launch_softmax_dvec(o, d_o, (int)TH, p->head_dim, p->dtype == GDPA_BF16,
                                  (float*)(ws + pl.dvec_off), s, offsets, p->batch, p->heads, out_bias);
    if (e != hipSuccess) return hip_status(e);
  }
  if (d_out_bias != nullptr) {
    e = gdpa::launch_out_bias_grad(offsets, d_o, p->batch, p->heads, p->head_dim, p->dtype == GDPA_BF16,
                                   d_out_bias, s);
    if (e != hipSuccess) return hip_status(e);
  }
  if (p->dtype == GDPA_F32) return hip_status(gdpa::launch_bwd_f32(a, p->head_dim, p->phi, s));

  e = gdpa::launch_longest_first(offsets, p->batch, (int32_t*)(ws + pl.order_off), s);
  if (e != hipSuccess) return hip_status(e);
  if (gdpa::bwd_res_supported(p->head_dim, p->n_kv))
    e = gdpa::launch_bwd_res(a, p->phi, s);
  else
    e = gdpa::launch_bwd_bf16(a, p->head_dim, p->phi, pl.waves, !pl.split_dq, s);
  if (e != hipSuccess || !pl.split_dq) return hip_status(e);
  // Several key chunks per (sample, head): dQ per 128-row query tile (no reduction
  // across work-groups), after the key-chunk kernel, which reads every dO row - dq
  // may be d_o itself (GDPA_BWD_RESIDUAL, GDPA_BWD_ACCUM_DQ); each dQ work-group
  // reads the dO rows it overwrites before writing them.
  e = gdpa::launch_tile_scan(offsets, p->batch, gdpa::kFwdTileRows, (int32_t*)(ws + pl.tile_off), s);
  if (e != hipSuccess) return hip_status(e);
  return hip_status(gdpa::launch_bwd_dq(a, p->head_dim, p->phi, false,
                                        gdpa::fwd_bf16_grid(p->total_tokens, p->batch, p->heads), s));
}

}  // namespace

extern "C" {

gdpa_status gdpa_fwd(const gdpa_problem* p, const int32_t* offsets, const void* q, const void* k,
                     const void* v, const void* residual, void* o, float* lse, void* workspace,
                     size_t workspace_bytes, void* stream) {
  return fwd_impl(p, offsets, nullptr, q, k, v, residual, o, lse, workspace, workspace_bytes, stream);
}

gdpa_status gdpa_bwd(const gdpa_problem* p, const int32_t* offsets, const void* q, const void* k,
                     const void* v, const void* o, const float* lse, const void* d_o, void* dq,
                     void* dk, void* dv, void* workspace, size_t workspace_bytes, void* stream) {
  return bwd_impl(p, offsets, nullptr, q, k, v, o, lse, d_o, dq, dk, dv, workspace, workspace_bytes,
                  stream);
}

gdpa_status gdpa_fwd_jagged_kv(const gdpa_problem* p, const int32_t* offsets, const int32_t* kv_offsets,
                               const void* q, const void* k, const void* v, const void* residual,
                               void* o, float* lse, void* workspace, size_t workspace_bytes,
                               void* stream) {
  if (kv_offsets == nullptr) return GDPA_ERR_INVALID_ARGUMENT;
  return fwd_impl(p, offsets, kv_offsets, q, k, v, residual, o, lse, workspace, workspace_bytes, stream);
}

gdpa_status gdpa_bwd_jagged_kv(const gdpa_problem* p, const int32_t* offsets, const int32_t* kv_offsets,
                               const void* q, const void* k, const void* v, const void* o,
                               const float* lse, const void* d_o, void* dq, void* dk, void* dv,
                               void* workspace, size_t workspace_bytes, void* stream) {
  if (kv_offsets == nullptr) return GDPA_ERR_INVALID_ARGUMENT;
  return bwd_impl(p, offsets, kv_offsets, q, k, v, o, lse, d_o, dq, dk, dv, workspace, workspace_bytes,
                  stream);
}

gdpa_status gdpa_fwd_block(const gdpa_problem* p, const int32_t* offsets, const void* x, const void* k,
                           const void* v, void* o, void* y, float* lse, void* workspace, size_t workspace_bytes,
                           void* stream) {
  if (p != nullptr && p->flags != 0) return GDPA_ERR_UNSUPPORTED;
  if (p != nullptr && p->total_tokens > 0 &&
      (y == nullptr || o == nullptr || y == x || y == o || y == k || y == v))
    return GDPA_ERR_INVALID_ARGUMENT;
  return fwd_impl(p, offsets, nullptr, x, k, v, nullptr, o, lse, workspace, workspace_bytes, stream, nullptr,
                  nullptr, true, y);
}

gdpa_status gdpa_add_bf16(int64_t count, void* out, const void* x0, const void* x1, const void* x2,
                          const void* x3, void* stream) {
  if (count < 0 || (count > 0 && (out == nullptr || x0 == nullptr || x1 == nullptr)))
    return GDPA_ERR_INVALID_ARGUMENT;
  if (count % 8 != 0 || count / 8 >= (int64_t)INT32_MAX * 256) return GDPA_ERR_UNSUPPORTED;
  return hip_status(gdpa::launch_add_bf16((long)count, out, x0, x1, x2, x3, (hipStream_t)stream));
}

gdpa_status gdpa_fwd_biased(const gdpa_problem* p, const int32_t* offsets, const int32_t* kv_offsets,
                            const void* q, const void* k, const void* v, const float* score_bias,
                            const float* out_bias, void* o, float* lse, void* workspace,
                            size_t workspace_bytes, void* stream) {
  if (p != nullptr && p->flags != 0) return GDPA_ERR_UNSUPPORTED;  // no residual with biases
  return fwd_impl(p, offsets, kv_offsets, q, k, v, nullptr, o, lse, workspace, workspace_bytes, stream,
                  score_bias, out_bias);
}

gdpa_status gdpa_bwd_biased(const gdpa_problem* p, const int32_t* offsets, const int32_t* kv_offsets,
                            const void* q, const void* k, const void* v, const float* score_bias,
                            const float* out_bias, const void* o, const float* lse, const void* d_o,
                            void* dq, void* dk, void* dv, float* d_score_bias, float* d_out_bias,
                            void* workspace, size_t workspace_bytes, void* stream) {
  if (p != nullptr && p->flags != 0) return GDPA_ERR_UNSUPPORTED;  // plain dQ with biases
  if (d_score_bias != nullptr && (d_score_bias == score_bias || (const void*)d_score_bias == k ||
                                  (const void*)d_score_bias == v))
    return GDPA_ERR_INVALID_ARGUMENT;
  if (d_out_bias != nullptr && (d_out_bias == out_bias || (const void*)d_out_bias == d_o))
    return GDPA_ERR_INVALID_ARGUMENT;
  return bwd_impl(p, offsets, kv_offsets, q, k, v, o, lse, d_o, dq, dk, dv, workspace, workspace_bytes,
                  stream, score_bias, out_bias, d_score_bias, d_out_bias);
}

}  // extern "C"

namespace {

// Event-level personalisation (Kunlun paper summary, section 2.3): each event type
// runs GDPA with its own heads, head width, context size and batch.  One grouped
// call spreads the groups over the caller's stream and kLanes - 1 library-owned
// streams of the current device (default priority, created on first use and kept
// until the process ends), so that small problems share the machine instead of
// running one after another.  The fork and the join are stream events, so the
// call stays asynchronous and capturable; the enqueue is serialised per process.
constexpr int kLanes = 4;

struct Lanes {
  hipStream_t s[kLanes - 1] = {};
  hipEvent_t fork = nullptr, join[kLanes - 1] = {};
};

std::mutex g_lanes_mu;
std::map<int, Lanes> g_lanes;

hipError_t lanes_for_device(Lanes*& out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  auto it = g_lanes.find(dev);
  if (it != g_lanes.end()) {
    out = &it->second;
    return hipSuccess;
  }
  Lanes l;
  for (int i = 0; i < kLanes - 1 && e == hipSuccess; ++i) {
    e = hipStreamCreateWithFlags(&l.s[i], hipStreamNonBlocking);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&l.join[i], hipEventDisableTiming);
  }
  if (e == hipSuccess) e = hipEventCreateWithFlags(&l.fork, hipEventDisableTiming);
  if (e != hipSuccess) return e;  // a partial set is leaked, not half-used
  out = &(g_lanes[dev] = l);
  return hipSuccess;
}

size_t group_workspace(const gdpa_group& g, bool backward) {
  if (check_problem(&g.problem) != GDPA_OK) return 0;
  return backward ? bwd_plan(&g.problem).total : fwd_workspace(&g.problem);
}

double group_cost(const gdpa_group& g) {  // work estimate for the lane assignment
  const gdpa_problem& p = g.problem;
  return (double)p.total_tokens * p.heads * p.n_kv * p.head_dim + 1.0;
}

gdpa_status group_call(const gdpa_group& g, bool backward, char* ws, size_t bytes, void* stream, bool launch) {
  const gdpa_problem* p = &g.problem;
  if (!backward)
    return fwd_impl(p, g.offsets, g.kv_offsets, g.q, g.k, g.v, g.residual, g.o, g.lse, ws, bytes, stream,
                    nullptr, nullptr, launch);
  return bwd_impl(p, g.offsets, g.kv_offsets, g.q, g.k, g.v, g.o, g.lse, g.d_o, g.dq, g.dk, g.dv, ws, bytes,
                  stream, nullptr, nullptr, nullptr, nullptr, launch);
}

gdpa_status grouped_impl(int32_t groups, const gdpa_group* g, bool backward, void* workspace,
                         size_t workspace_bytes, void* stream) {
  if (groups < 1 || g == nullptr) return GDPA_ERR_INVALID_ARGUMENT;
  // Every group's arguments are checked before anything is launched; each group
  // works in its own slice of the workspace (they run concurrently).
  std::vector<size_t> off((size_t)groups + 1, 0);
  for (int32_t i = 0; i < groups; ++i) {
    const gdpa_status st = check_problem(&g[i].problem);
    if (st != GDPA_OK) return st;
    off[i + 1] = off[i] + align_up(group_workspace(g[i], backward));
  }
  if (workspace == nullptr || workspace_bytes < off[groups]) return GDPA_ERR_WORKSPACE_TOO_SMALL;
  // Groups run concurrently: no output may be another group's output or input.
  auto outs_of = [&](const gdpa_group& x, const void* (&o)[3]) {
    o[0] = backward ? x.dq : x.o;
    o[1] = backward ? x.dk : (const void*)x.lse;
    o[2] = backward ? x.dv : nullptr;
  };
  for (int32_t i = 0; i < groups; ++i) {
    const void* oi[3];
    outs_of(g[i], oi);
    for (int32_t j = 0; j < groups; ++j) {
      if (j == i) continue;
      const void* oj[3];
      outs_of(g[j], oj);
      const void* ins[8] = {g[j].q, g[j].k, g[j].v, g[j].residual, g[j].d_o, g[j].offsets, g[j].kv_offsets,
                            backward ? (const void*)g[j].o : nullptr};
      for (const void* p : oi) {
        if (p == nullptr) continue;
        for (const void* q : oj)
          if (p == q) return GDPA_ERR_INVALID_ARGUMENT;
        for (const void* q : ins)
          if (p == q) return GDPA_ERR_INVALID_ARGUMENT;
      }
    }
  }
  char* ws = (char*)workspace;
  for (int32_t i = 0; i < groups; ++i) {
    const gdpa_status st = group_call(g[i], backward, ws + off[i], off[i + 1] - off[i], stream, false);
    if (st != GDPA_OK) return st;
  }
  if (groups == 1) return group_call(g[0], backward, ws, off[1], stream, true);

  // Largest groups first, each to the lane with the least work so far.
  std::vector<int32_t> order(groups);
  for (int32_t i = 0; i < groups; ++i) order[i] = i;
  std::stable_sort(order.begin(), order.end(),
                   [&](int32_t a, int32_t b) { return group_cost(g[a]) > group_cost(g[b]); });
  std::lock_guard<std::mutex> lock(g_lanes_mu);
  Lanes* lanes = nullptr;
  hipError_t e = lanes_for_device(lanes);
  if (e != hipSuccess) return hip_status(e);
  hipStream_t caller = (hipStream_t)stream;
  const int used = groups < kLanes ? groups : kLanes;
  e = hipEventRecord(lanes->fork, caller);
  for (int l = 1; l < used && e == hipSuccess; ++l) e = hipStreamWaitEvent(lanes->s[l - 1], lanes->fork, 0);
  if (e != hipSuccess) return hip_status(e);
  double load[kLanes] = {};
  gdpa_status result = GDPA_OK;
  for (int32_t i : order) {
    int l = 0;
    for (int c = 1; c < used; ++c)
      if (load[c] < load[l]) l = c;
    load[l] += group_cost(g[i]);
    void* st = l == 0 ? stream : (void*)lanes->s[l - 1];
    const gdpa_status r = group_call(g[i], backward, ws + off[i], off[i + 1] - off[i], st, true);
    if (r != GDPA_OK && result == GDPA_OK) result = r;
  }
  // The join is enqueued whatever happened above, so the caller's stream never
  // runs ahead of work already queued on a lane.
  for (int l = 1; l < used; ++l) {
    hipError_t j = hipEventRecord(lanes->join[l - 1], lanes->s[l - 1]);
    if (j == hipSuccess) j = hipStreamWaitEvent(caller, lanes->join[l - 1], 0);
    if (j != hipSuccess && result == GDPA_OK) result = hip_status(j);
  }
  return result;
}

}  // namespace

extern "C" {

size_t gdpa_grouped_workspace_bytes(int32_t groups, const gdpa_group* g, int backward) {
  if (groups < 1 || g == nullptr) return 0;
  size_t total = 0;
  for (int32_t i = 0; i < groups; ++i) {
    if (check_problem(&g[i].problem) != GDPA_OK) return 0;
    total += align_up(group_workspace(g[i], backward != 0));
  }
  return total;
}

gdpa_status gdpa_fwd_grouped(int32_t groups, const gdpa_group* g, void* workspace, size_t workspace_bytes,
                             void* stream) {
  return grouped_impl(groups, g, false, workspace, workspace_bytes, stream);
}

gdpa_status gdpa_bwd_grouped(int32_t groups, const gdpa_group* g, void* workspace, size_t workspace_bytes,
                             void* stream) {
  return grouped_impl(groups, g, true, workspace, workspace_bytes, stream);
}

}  // extern "C"

// Scratch of gdpa_bwd_noalloc: the backward's workspace (longest-first order,
// softmax row dots, query-tile prefix sums) for callers that cannot allocate.
// One copy per GPU, created when the library's device code is loaded there and
// kept until the process ends.  In host code `scratch` only names the variable;
// its device address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) unsigned char scratch[GDPA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch (looked up on its first use).
gdpa_status scratch_of_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  if (dev < 0 || dev >= kMaxDevices) return GDPA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e);
    if (p == nullptr) return hip_status(hipErrorInvalidSymbol);
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return GDPA_OK;
}

}  // namespace

extern "C" {

gdpa_status gdpa_bwd_noalloc(const gdpa_problem* p, const int32_t* offsets, const void* q, const void* k,
                             const void* v, const void* o, const float* lse, const void* d_o, void* dq,
                             void* dk, void* dv, void* stream) {
  // Every argument check first, against the scratch size (no device call yet):
  // a problem whose workspace exceeds it fails with GDPA_ERR_WORKSPACE_TOO_SMALL.
  void* const unchecked = (void*)(uintptr_t)kAlign;  // stands in for the scratch address while checking
  gdpa_status st = bwd_impl(p, offsets, nullptr, q, k, v, o, lse, d_o, dq, dk, dv, unchecked,
                            GDPA_NOALLOC_SCRATCH_BYTES, stream, nullptr, nullptr, nullptr, nullptr, false);
  if (st != GDPA_OK) return st;
  void* ws = nullptr;
  st = scratch_of_current_device(&ws);
  if (st != GDPA_OK) return st;
  return bwd_impl(p, offsets, nullptr, q, k, v, o, lse, d_o, dq, dk, dv, ws, GDPA_NOALLOC_SCRATCH_BYTES,
                  stream);
}

gdpa_status gdpa_check_kv_offsets(const int32_t* host_kv_offsets, int32_t batch, int32_t n_kv) {
  if (host_kv_offsets == nullptr || batch < 0 || n_kv < 1) return GDPA_ERR_INVALID_ARGUMENT;
  if (host_kv_offsets[0] != 0) return GDPA_ERR_INVALID_ARGUMENT;
  for (int32_t b = 0; b < batch; ++b) {
    const int64_t rows = (int64_t)host_kv_offsets[b + 1] - host_kv_offsets[b];
    if (rows < 1 || rows > n_kv) return GDPA_ERR_INVALID_ARGUMENT;
  }
  return GDPA_OK;
}

gdpa_status gdpa_weightgen_fwd(int32_t batch, int32_t ctx_dim, int64_t cols, const void* ctx,
                               const void* w, void* out, void* stream) {
  if (batch < 1 || ctx_dim < 1 || cols < 1 || ctx == nullptr || w == nullptr || out == nullptr)
    return GDPA_ERR_INVALID_ARGUMENT;
  if (cols % 8 != 0 || ctx_dim % 8 != 0) return GDPA_ERR_UNSUPPORTED;
  if ((cols / 256 + 1) * (batch / 128 + 1) >= INT32_MAX / 2) return GDPA_ERR_UNSUPPORTED;
  return hip_status(gdpa::launch_gemm_bf16(false, false, batch, cols, ctx_dim, ctx, w, out,
                                           (hipStream_t)stream));
}

gdpa_status gdpa_weightgen_bwd_w(int32_t batch, int32_t ctx_dim, int64_t cols, const void* ctx,
                                 const void* d_out, void* d_w, void* stream) {
  if (batch < 1 || ctx_dim < 1 || cols < 1 || ctx == nullptr || d_out == nullptr || d_w == nullptr)
    return GDPA_ERR_INVALID_ARGUMENT;
  if (cols % 8 != 0 || ctx_dim % 8 != 0) return GDPA_ERR_UNSUPPORTED;
  if (cols >= INT32_MAX || (cols / 128 + 1) * (ctx_dim / 256 + 1) >= INT32_MAX / 2)
    return GDPA_ERR_UNSUPPORTED;
  return hip_status(gdpa::launch_gemm_bf16(true, true, (int)cols, ctx_dim, batch, d_out, ctx, d_w,
                                           (hipStream_t)stream));
}

}  // extern "C"

namespace {

gdpa_status check_swa(const gdpa_swa_problem* p) {
  if (p == nullptr) return GDPA_ERR_INVALID_ARGUMENT;
  if (p->batch < 1 || p->total_tokens < 0 || p->max_seqlen < 0 || p->heads < 1 || p->head_dim < 1 ||
      p->window < 1)
    return GDPA_ERR_INVALID_ARGUMENT;
  if (p->dtype != GDPA_F32 && p->dtype != GDPA_BF16) return GDPA_ERR_INVALID_ARGUMENT;
  if (!std::isfinite(p->scale)) return GDPA_ERR_INVALID_ARGUMENT;
  if ((int64_t)p->total_tokens * p->heads > INT32_MAX) return GDPA_ERR_INVALID_ARGUMENT;
  if (p->head_dim != 32 && p->head_dim != 64 && p->head_dim != 128) return GDPA_ERR_UNSUPPORTED;
  if (p->dtype != GDPA_BF16 || p->flags != 0) return GDPA_ERR_UNSUPPORTED;
  return GDPA_OK;
}

struct SwaBwdPlan {
  int waves, max_chunks;
  size_t chunk_off, tile_off, dvec_off, total;
};

SwaBwdPlan swa_bwd_plan(const gdpa_swa_problem* p) {
  SwaBwdPlan pl{};
  pl.waves = gdpa::swa_bwd_waves(p->head_dim);
  const int nj = 32 * pl.waves;
  // sum_b ceil(L_b / nj) <= T / nj + B
  pl.max_chunks = p->total_tokens / nj + p->batch;
  const size_t TH = (size_t)p->total_tokens * p->heads;
  size_t off = 0;
  pl.chunk_off = off;
  off += align_up(sizeof(int32_t) * ((size_t)p->batch + 1));
  pl.tile_off = off;
  off += align_up(sizeof(int32_t) * ((size_t)p->batch + 1));
  pl.dvec_off = off;
  off += align_up(sizeof(float) * TH);
  pl.total = off;
  return pl;
}

}  // namespace

extern "C" {

size_t gdpa_swa_workspace_bytes(const gdpa_swa_problem* p, int backward) {
  if (check_swa(p) != GDPA_OK) return 0;
  return backward ? swa_bwd_plan(p).total : align_up(sizeof(int32_t) * ((size_t)p->batch + 1));
}

}  // extern "C"

namespace {

// Sliding-window forward; o_plus_q != nullptr (self-attention block, q == k == v)
// also writes the block's residual output O + Q there.
gdpa_status swa_fwd_impl(const gdpa_swa_problem* p, const int32_t* offsets, const void* q, const void* k,
                         const void* v, void* o, float* lse, void* workspace, size_t workspace_bytes,
                         void* stream, void* o_plus_q) {
  const gdpa_status st = check_swa(p);
  if (st != GDPA_OK) return st;
  if (offsets == nullptr) return GDPA_ERR_INVALID_ARGUMENT;
  if (p->total_tokens > 0 && (q == nullptr || k == nullptr || v == nullptr || o == nullptr))
    return GDPA_ERR_INVALID_ARGUMENT;
  if (o != nullptr && (o == q || o == k || o == v)) return GDPA_ERR_INVALID_ARGUMENT;
  if (workspace == nullptr || workspace_bytes < gdpa_swa_workspace_bytes(p, 0))
    return GDPA_ERR_WORKSPACE_TOO_SMALL;
  if (p->total_tokens == 0) return GDPA_OK;
  hipStream_t s = (hipStream_t)stream;
  gdpa::FwdArgs a{};
  a.offsets = offsets;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.B = p->batch;
  a.T = p->total_tokens;
  a.H = p->heads;
  a.scale = p->scale;
  a.window = p->window;
  a.o_plus_q = o_plus_q;
  int32_t* tile_start = (int32_t*)workspace;
  hipError_t e = gdpa::launch_tile_scan(offsets, p->batch, gdpa::kFwdTileRows, tile_start, s);
  if (e != hipSuccess) return hip_status(e);
  a.tile_start = tile_start;
  const int grid = gdpa::fwd_bf16_grid(p->total_tokens, p->batch, p->heads);
  return hip_status(gdpa::launch_fwd_swa(a, p->head_dim, grid, s));
}

// Sliding-window backward; block (self-attention block, q == k == v, dk == dv ==
// dq): dq receives d_o + dQ + dK + dV (the residual's gradient plus the three
// attention inputs'), through the key-chunk kernel's summed epilogue and the
// dQ kernel accumulating onto it.
gdpa_status swa_bwd_impl(const gdpa_swa_problem* p, const int32_t* offsets, const void* q, const void* k,
                         const void* v, const void* o, const float* lse, const void* d_o, void* dq, void* dk,
                         void* dv, void* workspace, size_t workspace_bytes, void* stream, bool block) {
  const gdpa_status st = check_swa(p);
  if (st != GDPA_OK) return st;
  if (offsets == nullptr) return GDPA_ERR_INVALID_ARGUMENT;
  if (p->total_tokens > 0 &&
      (q == nullptr || k == nullptr || v == nullptr || o == nullptr || lse == nullptr ||
       d_o == nullptr || dq == nullptr || dk == nullptr || dv == nullptr))
    return GDPA_ERR_INVALID_ARGUMENT;
  if (block) {
    if (q != k || q != v || dq != dk || dq != dv || dq == q || dq == o || dq == d_o)
      return GDPA_ERR_INVALID_ARGUMENT;
  } else {
  const void* outs[3] = {dq, dk, dv};
  const void* ins[5] = {q, k, v, o, d_o};
  for (int i = 0; i < 3; ++i) {
    for (int j = 0; j < 5; ++j)
      if (outs[i] != nullptr && outs[i] == ins[j]) return GDPA_ERR_INVALID_ARGUMENT;
    for (int j = i + 1; j < 3; ++j)
      if (outs[i] != nullptr && outs[i] == outs[j]) return GDPA_ERR_INVALID_ARGUMENT;
  }
  }
  const SwaBwdPlan pl = swa_bwd_plan(p);
  if (workspace == nullptr || workspace_bytes < pl.total) return GDPA_ERR_WORKSPACE_TOO_SMALL;
  if (p->total_tokens == 0) return GDPA_OK;
  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;
  gdpa::BwdArgs a{};
  a.offsets = offsets;
  a.q = q;
  a.k = k;
  a.v = v;
  a.d_o = d_o;
  a.lse = lse;
  a.dvec = (const float*)(ws + pl.dvec_off);
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.B = p->batch;
  a.T = p->total_tokens;
  a.H = p->heads;
  a.n_chunks = 0;
  a.scale = p->scale;
  a.chunk_start = (const int32_t*)(ws + pl.chunk_off);
  a.tile_start = (const int32_t*)(ws + pl.tile_off);
  a.window = p->window;
  a.kv_sum_base = block ? d_o : nullptr;
  a.dq_base = block ? dq : nullptr;
  const size_t TH = (size_t)p->total_tokens * p->heads;
  hipError_t e = gdpa::launch_softmax_dvec(o, d_o, (int)TH, p->head_dim, true, (float*)(ws + pl.dvec_off), s);
  if (e != hipSuccess) return hip_status(e);
  e = gdpa::launch_tile_scan(offsets, p->batch, 32 * pl.waves, (int32_t*)(ws + pl.chunk_off), s);
  if (e != hipSuccess) return hip_status(e);
  e = gdpa::launch_tile_scan(offsets, p->batch, gdpa::kFwdTileRows, (int32_t*)(ws + pl.tile_off), s);
  if (e != hipSuccess) return hip_status(e);
  // dK / dV per key chunk, dQ per query tile: no cross-work-group reduction.
  e = gdpa::launch_bwd_swa(a, p->head_dim, pl.max_chunks, s);
  if (e != hipSuccess) return hip_status(e);
  return hip_status(gdpa::launch_bwd_dq(a, p->head_dim, gdpa::kPhiSoftmax, true,
                                        gdpa::fwd_bf16_grid(p->total_tokens, p->batch, p->heads), s));
}

}  // namespace

extern "C" {

gdpa_status gdpa_swa_fwd(const gdpa_swa_problem* p, const int32_t* offsets, const void* q,
                         const void* k, const void* v, void* o, float* lse, void* workspace,
                         size_t workspace_bytes, void* stream) {
  return swa_fwd_impl(p, offsets, q, k, v, o, lse, workspace, workspace_bytes, stream, nullptr);
}

gdpa_status gdpa_swa_bwd(const gdpa_swa_problem* p, const int32_t* offsets, const void* q,
                         const void* k, const void* v, const void* o, const float* lse,
                         const void* d_o, void* dq, void* dk, void* dv, void* workspace,
                         size_t workspace_bytes, void* stream) {
  return swa_bwd_impl(p, offsets, q, k, v, o, lse, d_o, dq, dk, dv, workspace, workspace_bytes, stream, false);
}

gdpa_status gdpa_swa_block_fwd(const gdpa_swa_problem* p, const int32_t* offsets, const void* x, void* o,
                               void* y, float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  if (p != nullptr && p->total_tokens > 0 && (y == nullptr || y == x || y == o))
    return GDPA_ERR_INVALID_ARGUMENT;
  return swa_fwd_impl(p, offsets, x, x, x, o, lse, workspace, workspace_bytes, stream, y);
}

gdpa_status gdpa_swa_block_bwd(const gdpa_swa_problem* p, const int32_t* offsets, const void* x, const void* o,
                               const float* lse, const void* d_y, void* d_x, void* workspace,
                               size_t workspace_bytes, void* stream) {
  return swa_bwd_impl(p, offsets, x, x, x, o, lse, d_y, d_x, d_x, d_x, workspace, workspace_bytes, stream, true);
}

}  // extern "C"

namespace {

gdpa_status check_pma(const gdpa_pma_problem* p) {
  if (p == nullptr) return GDPA_ERR_INVALID_ARGUMENT;
  if (p->batch < 1 || p->total_tokens < 0 || p->max_seqlen < 0 || p->heads < 1 || p->head_dim < 1 ||
      p->seeds < 1)
    return GDPA_ERR_INVALID_ARGUMENT;
  if (p->dtype != GDPA_F32 && p->dtype != GDPA_BF16) return GDPA_ERR_INVALID_ARGUMENT;
  if (!std::isfinite(p->scale)) return GDPA_ERR_INVALID_ARGUMENT;
  if ((int64_t)p->total_tokens * p->heads > INT32_MAX) return GDPA_ERR_INVALID_ARGUMENT;
  if ((int64_t)p->batch * p->seeds * p->heads > INT32_MAX) return GDPA_ERR_INVALID_ARGUMENT;
  if (p->head_dim != 32 && p->head_dim != 64 && p->head_dim != 128) return GDPA_ERR_UNSUPPORTED;
  if (p->seeds > 32 || p->dtype != GDPA_BF16 || (p->flags & ~GDPA_PMA_BWD_KV_SUM) != 0) return GDPA_ERR_UNSUPPORTED;
  // Work-group ids: (chunks upper bound) x heads must fit a grid dimension.
  if (((int64_t)p->total_tokens / 1024 + p->batch) * p->heads + 8 > INT32_MAX)
    return GDPA_ERR_UNSUPPORTED;
  return GDPA_OK;
}

// Workspace: order [B] int32 | chunk_start [B+1] int32 | part [chunks][H][32][d]
// fp32 | forward: part_ml [chunks][H][32][2] fp32, backward: part2 [slices][H][32][d] fp32.
struct PmaPlan {
  size_t order_off, chunk_off, part_off, extra_off, total;
};

PmaPlan pma_plan(const gdpa_pma_problem* p, bool backward) {
  PmaPlan pl{};
  const size_t chunks = (size_t)p->total_tokens / gdpa::pma_chunk(p->total_tokens, p->heads) + p->batch;
  const size_t per_chunk = (size_t)p->heads * 32 * p->head_dim;
  size_t off = 0;
  pl.order_off = off;
  off += align_up(sizeof(int32_t) * (size_t)p->batch);
  pl.chunk_off = off;
  off += align_up(sizeof(int32_t) * ((size_t)p->batch + 1));
  pl.part_off = off;
  off += align_up(sizeof(float) * chunks * per_chunk);
  pl.extra_off = off;
  off += backward ? align_up(sizeof(float) * gdpa::kPmaSlices * per_chunk)
                  : align_up(sizeof(float) * chunks * p->heads * 32 * 2);
  pl.total = off;
  return pl;
}

gdpa::PmaArgs pma_args(const gdpa_pma_problem* p, const int32_t* offsets, char* ws, const PmaPlan& pl) {
  gdpa::PmaArgs a{};
  a.offsets = offsets;
  a.order = (const int32_t*)(ws + pl.order_off);
  a.chunk_start = (const int32_t*)(ws + pl.chunk_off);
  a.part = (float*)(ws + pl.part_off);
  a.B = p->batch;
  a.H = p->heads;
  a.m = p->seeds;
  a.scale = p->scale;
  a.chunk = gdpa::pma_chunk(p->total_tokens, p->heads);
  return a;
}

// Longest-first sample order and the chunk prefix sums over it.
hipError_t pma_schedule(const gdpa_pma_problem* p, const int32_t* offsets, char* ws, const PmaPlan& pl,
                        hipStream_t s) {
  int32_t* order = (int32_t*)(ws + pl.order_off);
  const hipError_t e = gdpa::launch_longest_first(offsets, p->batch, order, s);
  if (e != hipSuccess) return e;
  return gdpa::launch_tile_scan(offsets, p->batch, gdpa::pma_chunk(p->total_tokens, p->heads),
                                (int32_t*)(ws + pl.chunk_off), s, order);
}

}  // namespace

extern "C" {

size_t gdpa_pma_workspace_bytes(const gdpa_pma_problem* p, int backward) {
  if (check_pma(p) != GDPA_OK) return 0;
  return pma_plan(p, backward != 0).total;
}

gdpa_status gdpa_pma_fwd(const gdpa_pma_problem* p, const int32_t* offsets, const void* seeds,
                         const void* k, const void* v, void* o, float* lse, void* workspace,
                         size_t workspace_bytes, void* stream) {
  const gdpa_status st = check_pma(p);
  if (st != GDPA_OK) return st;
  if (p->flags != 0) return GDPA_ERR_UNSUPPORTED;  // the one flag is the backward's
  if (offsets == nullptr || seeds == nullptr || o == nullptr || lse == nullptr)
    return GDPA_ERR_INVALID_ARGUMENT;
  if (p->total_tokens > 0 && (k == nullptr || v == nullptr)) return GDPA_ERR_INVALID_ARGUMENT;
  if (o == seeds || o == k || o == v) return GDPA_ERR_INVALID_ARGUMENT;
  const PmaPlan pl = pma_plan(p, false);
  if (workspace == nullptr || workspace_bytes < pl.total) return GDPA_ERR_WORKSPACE_TOO_SMALL;
  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;
  gdpa::PmaArgs a = pma_args(p, offsets, ws, pl);
  a.seeds = seeds;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.part_ml = (float*)(ws + pl.extra_off);
  hipError_t e = pma_schedule(p, offsets, ws, pl, s);
  if (e != hipSuccess) return hip_status(e);
  const int grid = p->total_tokens > 0 ? gdpa::pma_grid(p->total_tokens, p->batch, p->heads, a.chunk) : 0;
  return hip_status(gdpa::launch_pma_fwd(a, p->head_dim, grid, s));
}

gdpa_status gdpa_pma_bwd(const gdpa_pma_problem* p, const int32_t* offsets, const void* seeds,
                         const void* k, const void* v, const void* o, const float* lse,
                         const void* d_o, void* d_seeds, void* dk, void* dv, void* workspace,
                         size_t workspace_bytes, void* stream) {
  const gdpa_status st = check_pma(p);
  if (st != GDPA_OK) return st;
  if (offsets == nullptr || seeds == nullptr || o == nullptr || lse == nullptr || d_o == nullptr ||
      d_seeds == nullptr)
    return GDPA_ERR_INVALID_ARGUMENT;
  const bool kv_sum = (p->flags & GDPA_PMA_BWD_KV_SUM) != 0;
  if (kv_sum && (dv != nullptr || k != v)) return GDPA_ERR_INVALID_ARGUMENT;  // one sequence as K and V
  if (p->total_tokens > 0 && (k == nullptr || v == nullptr || dk == nullptr || (!kv_sum && dv == nullptr)))
    return GDPA_ERR_INVALID_ARGUMENT;
  const void* outs[3] = {d_seeds, dk, dv};
  const void* ins[6] = {seeds, k, v, o, d_o, lse};
  for (int i = 0; i < 3; ++i) {
    for (int j = 0; j < 6; ++j)
      if (outs[i] != nullptr && outs[i] == ins[j]) return GDPA_ERR_INVALID_ARGUMENT;
    for (int j = i + 1; j < 3; ++j)
      if (outs[i] != nullptr && outs[i] == outs[j]) return GDPA_ERR_INVALID_ARGUMENT;
  }
  const PmaPlan pl = pma_plan(p, true);
  if (workspace == nullptr || workspace_bytes < pl.total) return GDPA_ERR_WORKSPACE_TOO_SMALL;
  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;
  gdpa::PmaArgs a = pma_args(p, offsets, ws, pl);
  a.seeds = seeds;
  a.k = k;
  a.v = v;
  a.o = const_cast<void*>(o);
  a.lse = const_cast<float*>(lse);
  a.d_o = d_o;
  a.d_seeds = d_seeds;
  a.dk = dk;
  a.dv = dv;
  hipError_t e = pma_schedule(p, offsets, ws, pl, s);
  if (e != hipSuccess) return hip_status(e);
  const int grid = p->total_tokens > 0 ? gdpa::pma_grid(p->total_tokens, p->batch, p->heads, a.chunk) : 0;
  return hip_status(gdpa::launch_pma_bwd(a, p->head_dim, grid, (float*)(ws + pl.extra_off), kv_sum, s));
}

gdpa_status gdpa_check_offsets(const int32_t* host_offsets, int32_t batch, int32_t total_tokens,
                               int32_t max_seqlen) {
  if (host_offsets == nullptr || batch < 0 || total_tokens < 0 || max_seqlen < 0)
    return GDPA_ERR_INVALID_ARGUMENT;
  if (host_offsets[0] != 0 || host_offsets[batch] != total_tokens) return GDPA_ERR_INVALID_ARGUMENT;
  for (int32_t b = 0; b < batch; ++b) {
    const int64_t len = (int64_t)host_offsets[b + 1] - host_offsets[b];
    if (len < 0 || len > max_seqlen) return GDPA_ERR_INVALID_ARGUMENT;
  }
  return GDPA_OK;
}

const char* gdpa_status_str(gdpa_status s) {
  switch (s) {
    case GDPA_OK: return "GDPA_OK";
    case GDPA_ERR_INVALID_ARGUMENT: return "GDPA_ERR_INVALID_ARGUMENT";
    case GDPA_ERR_UNSUPPORTED: return "GDPA_ERR_UNSUPPORTED";
    case GDPA_ERR_WORKSPACE_TOO_SMALL: return "GDPA_ERR_WORKSPACE_TOO_SMALL";
    case GDPA_ERR_HIP: return "GDPA_ERR_HIP";
  }
  return "GDPA_ERR_UNKNOWN";
}

int gdpa_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
