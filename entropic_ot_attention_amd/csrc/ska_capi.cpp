// C ABI of libsinkhorn_attn.so: argument validation, workspace sizing, launch sequencing.
// The declarations and the contract (layouts, ownership, errors) are in include/sinkhorn_attn.h.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <mutex>
#include <cstdint>
#include <string>
#include <utility>
#include <vector>

#include "sinkhorn_attn.h"
#include "ska_internal.h"

namespace {

thread_local std::string g_err;

ska_status fail(ska_status s, const std::string& msg) {
  g_err = msg;
  return s;
}

// ---------------------------------------------------------------------------------------------
// optional per-launch timing with HIP events, process-wide (launches from any thread, e.g. an
// autograd engine's backward thread, are counted); the lock is taken only while timing is on
// ---------------------------------------------------------------------------------------------
struct TimedBracket {
  std::pair<hipEvent_t, hipEvent_t> ev;
  int64_t launches;   // launches of the family between the two events
};
struct Timing {
  std::atomic<bool> on{false};
  std::mutex mu;
  std::vector<TimedBracket> pending[ska::kTimedKinds];
  std::vector<std::pair<hipEvent_t, hipEvent_t>> free_pairs;
  double total_ms[ska::kTimedKinds] = {};
  int64_t launches[ska::kTimedKinds] = {};
};
Timing g_timing;

std::pair<hipEvent_t, hipEvent_t> timing_begin(int kind, hipStream_t st) {
  std::pair<hipEvent_t, hipEvent_t> ev{nullptr, nullptr};
  if (!g_timing.on.load(std::memory_order_relaxed)) return ev;
  std::lock_guard<std::mutex> lock(g_timing.mu);
  if (!g_timing.free_pairs.empty()) {
    ev = g_timing.free_pairs.back();
    g_timing.free_pairs.pop_back();
  } else {
    if (hipEventCreate(&ev.first) != hipSuccess || hipEventCreate(&ev.second) != hipSuccess)
      return {nullptr, nullptr};
  }
  (void)hipEventRecord(ev.first, st);
  (void)kind;
  return ev;
}

// `launches`: how many launches of the family the bracket covers (consecutive launches on one
// stream may share a bracket; the short gaps between them are then included)
void timing_end(int kind, std::pair<hipEvent_t, hipEvent_t> ev, hipStream_t st,
                int64_t launches = 1) {
  if (!ev.first) return;
  (void)hipEventRecord(ev.second, st);
  std::lock_guard<std::mutex> lock(g_timing.mu);
  g_timing.pending[kind].push_back(TimedBracket{ev, launches});
}

// ---------------------------------------------------------------------------------------------
// validation
// ---------------------------------------------------------------------------------------------
struct Plan {
  ska::Geometry g;
  int elt;
  int R, T;
  bool empty;
};

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

ska_status check_problem(const ska_problem* p, ska_op op, Plan* out) {
  if (!p) return fail(SKA_ERR_INVALID, "problem pointer is NULL");
  if (p->bh < 0) return fail(SKA_ERR_INVALID, "bh must be >= 0");
  if (p->L < 0) return fail(SKA_ERR_INVALID, "L must be >= 0");
  if (p->W < 0 || (p->W & 1)) return fail(SKA_ERR_INVALID, "W must be even and >= 0");
  if (p->T < 0) return fail(SKA_ERR_INVALID, "T must be >= 0");
  if (!(p->epsilon > 0.f) || !std::isfinite(p->epsilon))
    return fail(SKA_ERR_INVALID, "epsilon must be finite and > 0");
  if (p->dtype != SKA_F32 && p->dtype != SKA_BF16) return fail(SKA_ERR_INVALID, "unknown dtype");
  const bool vjp = (op == SKA_OP_VJP || op == SKA_OP_DUSTBIN_BLOCK_VJP);
  const bool dustbin = (op == SKA_OP_DUSTBIN_BLOCK_FWD || op == SKA_OP_DUSTBIN_BLOCK_VJP ||
                        op == SKA_OP_DUSTBIN_BLOCK_CONTRACTION);
  if (op < SKA_OP_FWD || op > SKA_OP_DUSTBIN_BLOCK_CONTRACTION) return fail(SKA_ERR_INVALID, "unknown op");
  if (p->R < 0) return fail(SKA_ERR_INVALID, "R must be >= 0");
  if (p->R == 0 && p->T < 1)
    return fail(SKA_ERR_INVALID, "R = 0 needs T >= 1: the output plan's duals come from the base");
  if (vjp && p->R > ska::kTailMaxR) return fail(SKA_ERR_UNSUPPORTED, "the VJP is built for R <= 256");
  if (op == SKA_OP_TAIL_REMAINDER && (int64_t)p->T + p->R > ska::kTailMaxR)
    return fail(SKA_ERR_UNSUPPORTED, "the tail remainder runs the adjoint at depth T + R <= 256");
  if (p->d != ska::kD) return fail(SKA_ERR_UNSUPPORTED, "head dimension d must be 64");
  const int64_t Lr = p->L + (dustbin ? 1 : 0);
  if (Lr > (int64_t(1) << 30)) return fail(SKA_ERR_UNSUPPORTED, "L above 2^30 tokens");
  if (p->bh > 65535) return fail(SKA_ERR_UNSUPPORTED, "bh above 65535");
  int64_t h = p->W / 2;
  if (dustbin && h < p->L) h = p->L;  // widened band: every token reaches the dustbin
  if (h > Lr) h = Lr;                 // wider than the sequence changes nothing
  out->elt = p->dtype;
  out->R = p->R;
  out->T = p->T;
  out->empty = (p->bh == 0 || Lr == 0);
  out->g.bh = p->bh;
  out->g.Lr = (int)Lr;
  out->g.Lpad = (int)ska::pad_tokens(Lr);
  out->g.h = (int)h;
  const double s = 1.0 / (std::sqrt((double)p->d) * (double)p->epsilon);
  out->g.s = (float)s;
  out->g.c2 = (float)(s * 1.4426950408889634);
  return SKA_OK;
}

// Forward workspace, fused path (bands up to half-width 192): two column-dual and two row-dual
// buffers [bh][Lpad] plus two column-partial buffers [bh][nseg][64 seg_len + 32 H16] (about one
// float per token).  Wide path (wider windows up to 8 x 33 tiles, e.g. the dense dustbin
// support): two dual buffers plus one partial row of 16 x (window tiles) floats per 16-token row
// tile, about bh L (W + 32) / 16 floats.  Split path (wider still): two dual buffers.  VJP:
// kVjpVecs vectors [bh][Lpad], plus the streaming passes' dv1 column partials (about one float
// per token).
struct RemLayout {
  size_t o, dq_r, dk_r, dv_r, dq_f, dk_f, dv_f, duals_r, duals_f, part, inner, inner_bytes, total;
};
RemLayout rem_layout(const Plan& pl);
int64_t wide_part_floats(const Plan& pl);
int64_t wide_plane_floats(const Plan& pl);

size_t workspace_for(const Plan& pl, ska_op op) {
  if (pl.empty) return 0;
  if (op == SKA_OP_TAIL_REMAINDER) return rem_layout(pl).total;
  if (op == SKA_OP_CONTRACTION || op == SKA_OP_DUSTBIN_BLOCK_CONTRACTION) return 0;
  const bool vjp = (op == SKA_OP_VJP || op == SKA_OP_DUSTBIN_BLOCK_VJP);
  const int64_t vs = pl.g.bh * (int64_t)pl.g.Lpad;
  if (vjp && pl.R != 2) {
    // general depth: the tail vectors; on the streaming engine also two column-partial buffers
    int64_t part = 0;
    int nt = 0;
    const int nw = ska::vjp_stream_waves(pl.elt, pl.g.h, &nt);
    if (nw > 0) {
      int seg_len = 0, nseg = 0;
      ska::vjp_stream_segments(pl.g.bh, pl.g.Lr, nw, nt, &seg_len, &nseg);
      part = 2 * pl.g.bh * (int64_t)nseg * (16 * nw * seg_len + 16 * (nt - 1));
    }
    return (size_t)(ska::tail_vecs(pl.R) * vs + part) * sizeof(float);
  }
  if (vjp) {
    // streaming passes (both schedules, bands LDS holds) add dv1 column partials
    int nt = 0;
    const int nw = ska::vjp_stream_waves(pl.elt, pl.g.h, &nt);
    int64_t part = 0;
    if (nw > 0) {
      int seg_len = 0, nseg = 0;
      ska::vjp_stream_segments(pl.g.bh, pl.g.Lr, nw, nt, &seg_len, &nseg);
      part = pl.g.bh * (int64_t)nseg * (16 * nw * seg_len + 16 * (nt - 1));
    }
    return (size_t)(ska::kVjpVecs * vs + part) * sizeof(float);
  }
  const int nt = ska::fused_tiles_for(pl.g.h);
  if (nt == 0) {
    // wide path: row and column duals plus one partial row per 16-token row tile (fp32: then Q
    // and K as bf16 planes); split path (windows wider than the wide step holds in registers):
    // the two duals
    return (size_t)(ska::kFwdVecs * vs + wide_part_floats(pl) + wide_plane_floats(pl)) * sizeof(float);
  }
  int seg_len = 0, nseg = 0;
  ska::fused_segments(pl.g.bh, pl.g.Lr, nt, &seg_len, &nseg);
  const int64_t ps = pl.g.bh * (int64_t)nseg * ska::fused_pstride(nt, seg_len);
  return (size_t)(4 * vs + 2 * ps) * sizeof(float);
}

// Wide forward path: floats of the column partials (one partial row per 16-token row tile),
// rounded up to 256 bytes, and of the fp32 step's bf16 planes of Q and K that follow them.
int64_t wide_part_floats(const Plan& pl) {
  if (ska::fused_tiles_for(pl.g.h) != 0 || ska::wide_step_tiles(pl.g.Lr, pl.g.h) <= 0) return 0;
  const int64_t n = pl.g.bh * ((pl.g.Lr + 15) / 16) * (16 * (int64_t)ska::wide_window_tiles(pl.g.Lr, pl.g.h));
  return (n + 63) / 64 * 64;
}
int64_t wide_plane_floats(const Plan& pl) {
  if (pl.elt == SKA_BF16 || wide_part_floats(pl) == 0) return 0;
  return 2 * pl.g.bh * (int64_t)pl.g.Lr * (ska::kPlaneRowElems / 2);
}

// Tail-remainder workspace: O, the two gradient sets (tail at depth R, full at depth T + R),
// both dual sets, the reduction's block sums, then the larger inner workspace of the forward and
// VJP calls; every piece 256-byte aligned.
RemLayout rem_layout(const Plan& pl) {
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  const size_t elems = (size_t)pl.g.bh * pl.g.Lr * ska::kD;
  const size_t tb = up(elems * (pl.elt == 1 ? 2 : 4));
  RemLayout L{};
  size_t at = 0;
  L.o = at; at += tb;
  L.dq_r = at; at += tb;
  L.dk_r = at; at += tb;
  L.dv_r = at; at += tb;
  L.dq_f = at; at += tb;
  L.dk_f = at; at += tb;
  L.dv_f = at; at += tb;
  L.duals_r = at; at += up((size_t)ska::n_duals(pl.R) * pl.g.bh * pl.g.Lr * sizeof(float));
  L.duals_f = at; at += up((size_t)ska::n_duals(pl.T + pl.R) * pl.g.bh * pl.g.Lr * sizeof(float));
  L.part = at; at += up(2 * ska::kSqPartials * sizeof(double));
  Plan a = pl, b = pl;
  b.R = pl.T + pl.R;
  size_t inner = workspace_for(a, SKA_OP_FWD);
  for (size_t x : {workspace_for(b, SKA_OP_FWD), workspace_for(a, SKA_OP_VJP), workspace_for(b, SKA_OP_VJP)})
    inner = x > inner ? x : inner;
  L.inner = at;
  L.inner_bytes = up(inner);
  L.total = at + L.inner_bytes;
  return L;
}

ska_status check_ptr(const void* ptr, const char* name) {
  if (!ptr) return fail(SKA_ERR_INVALID, std::string(name) + " is NULL");
  if (!aligned16(ptr)) return fail(SKA_ERR_INVALID, std::string(name) + " is not 16-byte aligned");
  return SKA_OK;
}

#define SKA_TRY(expr)                  \
  do {                                 \
    ska_status _s = (expr);            \
    if (_s != SKA_OK) return _s;       \
  } while (0)

#define SKA_LAUNCH(kind, st, expr)                                                   \
  do {                                                                               \
    auto _ev = timing_begin(kind, st);                                               \
    hipError_t _e = (expr);                                                          \
    timing_end(kind, _ev, st);                                                       \
    if (_e != hipSuccess)                                                            \
      return fail(SKA_ERR_HIP, std::string("kernel launch failed: ") + hipGetErrorString(_e)); \
  } while (0)

ska::WideArgs wide_args(const Plan& pl, const void* Q, const void* K, const void* V, const void* dO) {
  ska::WideArgs a{};
  a.Q = Q;
  a.K = K;
  a.V = V;
  a.dO = dO;
  a.bh = pl.g.bh;
  a.Lr = pl.g.Lr;
  a.Lpad = pl.g.Lpad;
  a.h = pl.g.h;
  a.nrt = (pl.g.Lr + 15) / 16;
  a.pw = 16 * ska::wide_window_tiles(pl.g.Lr, pl.g.h);
  a.c2 = pl.g.c2;
  a.s = pl.g.s;
  return a;
}

ska_status run_fwd(const ska_problem* p, ska_op op, const void* Q, const void* K, const void* V,
                   void* O, float* duals, void* workspace, size_t workspace_bytes,
                   hipStream_t st) {
  Plan pl;
  SKA_TRY(check_problem(p, op, &pl));
  if (pl.empty) return SKA_OK;
  SKA_TRY(check_ptr(Q, "Q"));
  SKA_TRY(check_ptr(K, "K"));
  SKA_TRY(check_ptr(V, "V"));
  SKA_TRY(check_ptr(O, "O"));
  if (!duals) return fail(SKA_ERR_INVALID, "duals is NULL");
  if ((reinterpret_cast<uintptr_t>(duals) & 3u) != 0) return fail(SKA_ERR_INVALID, "duals misaligned");
  const size_t need = workspace_for(pl, op);
  if (!workspace || workspace_bytes < need)
    return fail(SKA_ERR_WORKSPACE, "workspace smaller than ska_workspace_bytes()");
  if (!aligned16(workspace)) return fail(SKA_ERR_INVALID, "workspace is not 16-byte aligned");

  const ska::Geometry& g = pl.g;
  const int64_t vs = g.bh * (int64_t)g.Lpad;
  const int64_t nd = ska::n_duals(p->R);
  const int64_t dstride = nd * g.Lr;
  // the saved row of u_k / v_k, or none
  auto save_at = [&](int slot) -> float* { return slot >= 0 ? duals + slot * (int64_t)g.Lr : nullptr; };
  float* wsf = static_cast<float*>(workspace);
  const int nt = ska::fused_tiles_for(g.h);
  if (nt > 0) {
    // fused path: one launch per full Sinkhorn step, column update finished by the next launch
    const int nblk = (g.Lr + 63) / 64;
    int seg_len = 0, nseg = 0;
    ska::fused_segments(g.bh, g.Lr, nt, &seg_len, &nseg);
    const int pst = ska::fused_pstride(nt, seg_len);
    const int64_t ps = g.bh * (int64_t)nseg * pst;
    float* vbuf[2] = {wsf, wsf + vs};
    float* ubuf[2] = {wsf + 2 * vs, wsf + 3 * vs};
    float* part[2] = {wsf + 4 * vs, wsf + 4 * vs + ps};
    // no initialisation: the first step reads no duals (it starts from v = 0 and needs no row
    // shift), every step writes its row duals for all Lpad rows (0 past the sequence), and column
    // duals are read only inside the sequence
    hipError_t e = hipSuccess;
    ska::StepArgs a{};
    a.Q = Q;
    a.K = K;
    a.bh = g.bh;
    a.Lr = g.Lr;
    a.Lpad = g.Lpad;
    a.h = g.h;
    a.nblk = nblk;
    a.seg_len = seg_len;
    a.nseg = nseg;
    a.pstride = pst;
    a.H16 = (nt - 1) / 2;
    a.c2 = g.c2;
    a.save_v_stride = dstride;
    a.save_u_stride = dstride;
    const int K_steps = p->T + p->R;
    // the T + R step launches run back to back: one timing bracket covers them all
    const auto run_ev = timing_begin(ska::kTimedStep, st);
    for (int k = 1; k <= K_steps; ++k) {
      a.v_prev = vbuf[(k - 1) % 2];
      a.part_prev = (k > 1) ? part[(k - 1) % 2] : nullptr;
      a.u_prev = ubuf[(k - 1) % 2];
      a.v_next = vbuf[k % 2];
      a.u_out = ubuf[k % 2];
      a.part_out = part[k % 2];
      a.save_v = save_at(ska::dual_slot_v(k - 1, p->T, p->R));
      a.save_u = save_at(ska::dual_slot_u(k, p->T, p->R));
      // alternate the walk direction: each step starts where the previous one ended, on data
      // still in the last-level cache
      const hipError_t le = ska::launch_fused_step(pl.elt, nt, a, (k % 2) == 0, st);
      if (le != hipSuccess) {
        timing_end(ska::kTimedStep, run_ev, st, k - 1);
        return fail(SKA_ERR_HIP, std::string("kernel launch failed: ") + hipGetErrorString(le));
      }
    }
    timing_end(ska::kTimedStep, run_ev, st, K_steps);
    a.v_prev = vbuf[K_steps % 2];
    a.part_prev = part[K_steps % 2];
    a.u_prev = ubuf[K_steps % 2];
    a.v_next = vbuf[(K_steps + 1) % 2];
    a.u_out = nullptr;
    a.part_out = nullptr;
    a.save_v = save_at(ska::dual_slot_v(K_steps, p->T, p->R));
    a.save_u = nullptr;
    e = ska::launch_finish_columns(pl.elt, a, st);
    if (e != hipSuccess) return fail(SKA_ERR_HIP, hipGetErrorString(e));
    int ont = 0;
    const int onw = ska::vjp_stream_waves(pl.elt, g.h, &ont);
    if (onw > 0) {
      // output on the streaming engine (its pass 0)
      ska::VjpArgs o{};
      o.Q = Q;
      o.K = K;
      o.V = V;
      o.dO = nullptr;
      o.out0 = O;
      o.fu = ubuf[K_steps % 2];
      o.fv = vbuf[(K_steps + 1) % 2];
      o.bh = g.bh;
      o.Lr = g.Lr;
      o.Lpad = g.Lpad;
      o.h = g.h;
      o.nblk = (g.Lr + 16 * onw - 1) / (16 * onw);
      ska::vjp_stream_segments(g.bh, g.Lr, onw, ont, &o.seg_len, &o.nseg);
      o.pstride = 16 * onw * o.seg_len + 16 * (ont - 1);
      o.c2 = g.c2;
      o.s = g.s;
      SKA_LAUNCH(ska::kTimedOut, st, ska::launch_vjp_stream_pass(pl.elt, ont, onw, 0, false, o, st));
    } else {
      ska::WideArgs o = wide_args(pl, Q, K, V, nullptr);
      o.out0 = O;
      o.fu = ubuf[K_steps % 2];
      o.fv = vbuf[(K_steps + 1) % 2];
      SKA_LAUNCH(ska::kTimedOut, st, ska::launch_wide_pass(pl.elt, 0, false, o, st));
    }
    return SKA_OK;
  }
  const int kt = ska::wide_step_tiles(g.Lr, g.h);
  if (kt > 0) {
    // wide path: one fused step launch per Sinkhorn step (row update and column partials of each
    // 16-token row tile), then the column finish
    float* u = wsf;
    float* v = u + vs;
    ska::WideArgs a = wide_args(pl, Q, K, V, nullptr);
    a.part = v + vs;
    a.save_stride = dstride;
    hipError_t e = ska::launch_fill(u, 2 * vs, 0.f, st);
    if (e != hipSuccess) return fail(SKA_ERR_HIP, hipGetErrorString(e));
    if (pl.elt != SKA_BF16) {
      // the fp32 step's matrix-core operands: Q and K as bf16 planes, after the partial rows
      float* planes = a.part + wide_part_floats(pl);
      const int64_t rows = g.bh * (int64_t)g.Lr;
      a.Qs = planes;
      a.Ks = planes + rows * (ska::kPlaneRowElems / 2);
      e = ska::launch_split3(static_cast<const float*>(Q), const_cast<void*>(a.Qs), rows, st);
      if (e == hipSuccess) e = ska::launch_split3(static_cast<const float*>(K), const_cast<void*>(a.Ks), rows, st);
      if (e != hipSuccess) return fail(SKA_ERR_HIP, hipGetErrorString(e));
    }
    const int K_steps = p->T + p->R;
    for (int k = 1; k <= K_steps; ++k) {
      // step k: u_k from v_{k-1}; saves u_k and v_{k-1} where the layout keeps them
      a.v_in = v;
      a.u_out = u;
      a.save_u = save_at(ska::dual_slot_u(k, p->T, p->R));
      a.save_v = save_at(ska::dual_slot_v(k - 1, p->T, p->R));
      SKA_LAUNCH(ska::kTimedStep, st, ska::launch_wide_step(pl.elt, kt, k == 1, a, st));
      // finish k: v_k (saved by the next step, or here after the last one)
      a.v_out = v;
      a.save_u = nullptr;
      a.save_v = (k == K_steps) ? save_at(ska::dual_slot_v(k, p->T, p->R)) : nullptr;
      e = ska::launch_wide_finish(pl.elt, a, st);
      if (e != hipSuccess) return fail(SKA_ERR_HIP, hipGetErrorString(e));
    }
    ska::WideArgs o = wide_args(pl, Q, K, V, nullptr);
    o.out0 = O;
    o.fu = u;
    o.fv = v;
    SKA_LAUNCH(ska::kTimedOut, st, ska::launch_wide_pass(pl.elt, 0, false, o, st));
    return SKA_OK;
  }
  // split path (windows wider than the wide step holds): separate row and column half-steps
  float* u = wsf;
  float* v = u + vs;
  hipError_t e = ska::launch_fill(u, 2 * vs, 0.f, st);
  if (e != hipSuccess) return fail(SKA_ERR_HIP, hipGetErrorString(e));
  // stopped base: T full (row, column) steps from u = v = 0
  for (int t = 0; t < p->T; ++t) {
    SKA_LAUNCH(ska::kTimedStep, st, ska::launch_lse(pl.elt, Q, K, v, u, nullptr, 0, g, st));
    SKA_LAUNCH(ska::kTimedStep, st, ska::launch_lse(pl.elt, K, Q, u, v, nullptr, 0, g, st));
  }
  if (p->R == 0) {
    e = ska::launch_save_duals(u, save_at(ska::dual_slot_u(p->T, p->T, 0)), dstride, g, st);
    if (e != hipSuccess) return fail(SKA_ERR_HIP, hipGetErrorString(e));
  }
  e = ska::launch_save_duals(v, save_at(ska::dual_slot_v(p->T, p->T, p->R)), dstride, g, st);
  if (e != hipSuccess) return fail(SKA_ERR_HIP, hipGetErrorString(e));
  // tail: u^(a) from v^(a-1), v^(a) from u^(a); saved as slots 2a-1, 2a
  for (int a = 1; a <= p->R; ++a) {
    SKA_LAUNCH(ska::kTimedStep, st,
               ska::launch_lse(pl.elt, Q, K, v, u, duals + (2 * a - 1) * (int64_t)g.Lr, dstride, g, st));
    SKA_LAUNCH(ska::kTimedStep, st,
               ska::launch_lse(pl.elt, K, Q, u, v, duals + (2 * a) * (int64_t)g.Lr, dstride, g, st));
  }
  ska::WideArgs o = wide_args(pl, Q, K, V, nullptr);
  o.out0 = O;
  o.fu = u;
  o.fv = v;
  SKA_LAUNCH(ska::kTimedOut, st, ska::launch_wide_pass(pl.elt, 0, false, o, st));
  return SKA_OK;
}

ska_status run_vjp(const ska_problem* p, ska_op op, const void* Q, const void* K, const void* V,
                   const float* duals, const void* dO, const void* O, void* dQ, void* dK, void* dV,
                   ska_schedule sched, void* workspace, size_t workspace_bytes, hipStream_t st) {
  Plan pl;
  SKA_TRY(check_problem(p, op, &pl));
  if (sched != SKA_ONE_REFERENCE && sched != SKA_DIRECT_FOUR)
    return fail(SKA_ERR_INVALID, "unknown schedule");
  if (sched == SKA_DIRECT_FOUR && p->R != 2)
    return fail(SKA_ERR_UNSUPPORTED, "the direct-four schedule is the R == 2 adjoint");
  if (pl.empty) return SKA_OK;
  SKA_TRY(check_ptr(Q, "Q"));
  SKA_TRY(check_ptr(K, "K"));
  SKA_TRY(check_ptr(V, "V"));
  SKA_TRY(check_ptr(dO, "dO"));
  if (O) SKA_TRY(check_ptr(O, "O"));
  SKA_TRY(check_ptr(dQ, "dQ"));
  SKA_TRY(check_ptr(dK, "dK"));
  SKA_TRY(check_ptr(dV, "dV"));
  if (!duals) return fail(SKA_ERR_INVALID, "duals is NULL");
  if ((reinterpret_cast<uintptr_t>(duals) & 3u) != 0) return fail(SKA_ERR_INVALID, "duals misaligned");
  const size_t need = workspace_for(pl, op);
  if (!workspace || workspace_bytes < need)
    return fail(SKA_ERR_WORKSPACE, "workspace smaller than ska_workspace_bytes()");
  if (!aligned16(workspace)) return fail(SKA_ERR_INVALID, "workspace is not 16-byte aligned");

  const ska::Geometry& g = pl.g;
  float* ws = static_cast<float*>(workspace);
  const bool d4 = (sched == SKA_DIRECT_FOUR);
  if (p->R != 2) {
    hipError_t e = ska::launch_tail_prep(duals, ws, p->R, g, st);
    if (e != hipSuccess) return fail(SKA_ERR_HIP, hipGetErrorString(e));
    int snt = 0;
    const int snw = ska::vjp_stream_waves(pl.elt, g.h, &snt);
    if (snw > 0) {
      // general tail depth on the streaming engine, R + 3 passes: dV and dv^(R) = V . dV (1);
      // du^(R) and its column partials (2); each level a = R-1 .. 1 (5), the partials alternating
      // between two buffers; dQ (6); dK (7).  R = 0: passes 6 and 7 alone (M = g), pass 7 also
      // giving dV.  Beyond R = 4 (the
      // deep adjoint of full backpropagation) the wide engine's pass A (dv^(R), dV) replaces pass
      // 1, and its dQ and dK passes, which accumulate the 2 R modifier terms level by level,
      // replace passes 6 and 7.
      ska::VjpArgs a{};
      a.Q = Q;
      a.K = K;
      a.V = V;
      a.dO = dO;
      a.O = O;        // optional: du^(R) from delta = dO . O in pass 2
      a.ws = ws;
      a.vec_stride = g.bh * (int64_t)g.Lpad;
      a.bh = g.bh;
      a.Lr = g.Lr;
      a.Lpad = g.Lpad;
      a.h = g.h;
      a.nblk = (g.Lr + 16 * snw - 1) / (16 * snw);
      ska::vjp_stream_segments(g.bh, g.Lr, snw, snt, &a.seg_len, &a.nseg);
      a.pstride = 16 * snw * a.seg_len + 16 * (snt - 1);
      a.c2 = g.c2;
      a.s = g.s;
      a.R = p->R;
      const int64_t ps = g.bh * (int64_t)a.nseg * a.pstride;
      float* parts[2] = {ws + ska::tail_vecs(p->R) * a.vec_stride,
                         ws + ska::tail_vecs(p->R) * a.vec_stride + ps};
      a.part = parts[0];
      a.part_out = parts[1];
      const bool deep = p->R > ska::kStreamMaxR;
      ska::WideArgs w = wide_args(pl, Q, K, V, dO);
      w.ws = ws;
      w.vec_stride = g.bh * (int64_t)g.Lpad;
      w.R = p->R;
      if (p->R >= 1) {
        if (deep) {
          // the wide pass A gives dv^(R) and dV (the streaming dK pass is not run)
          w.out0 = dV;
          SKA_LAUNCH(ska::kTimedVjp, st, ska::launch_tail_pass(pl.elt, 0, w, st));
        } else {
          a.out1 = dV;
          SKA_LAUNCH(ska::kTimedVjp, st, ska::launch_vjp_stream_general(pl.elt, snt, snw, 1, a, st));
        }
        SKA_LAUNCH(ska::kTimedVjp, st, ska::launch_vjp_stream_general(pl.elt, snt, snw, 2, a, st));
      }
      for (int lev = p->R - 1, k = 0; lev >= 1; --lev, ++k) {
        a.level = lev;
        a.part = parts[k % 2];
        a.part_out = parts[(k + 1) % 2];
        SKA_LAUNCH(ska::kTimedVjp, st, ska::launch_vjp_stream_general(pl.elt, snt, snw, 5, a, st));
      }
      if (!deep) {
        a.out0 = dQ;
        SKA_LAUNCH(ska::kTimedVjp, st, ska::launch_vjp_stream_general(pl.elt, snt, snw, 6, a, st));
        a.out0 = dK;
        a.out1 = dV;
        SKA_LAUNCH(ska::kTimedVjp, st, ska::launch_vjp_stream_general(pl.elt, snt, snw, 7, a, st));
        return SKA_OK;
      }
      w.out0 = dQ;
      SKA_LAUNCH(ska::kTimedVjp, st, ska::launch_tail_pass(pl.elt, 4, w, st));
      w.out0 = dK;
      SKA_LAUNCH(ska::kTimedVjp, st, ska::launch_tail_pass(pl.elt, 5, w, st));
      return SKA_OK;
    }
    // general tail depth: one-reference-tile adjoint, 2R + 2 passes on the wide decomposition
    // (A: dv^(R) and dV; B: du^(R); C, D for each level a = R-1 .. 1; then dQ and dK); R = 0
    // differentiates the stopped base plan alone: A (dV), then dQ and dK with M = g
    ska::WideArgs w = wide_args(pl, Q, K, V, dO);
    w.ws = ws;
    w.vec_stride = g.bh * (int64_t)g.Lpad;
    w.R = p->R;
    w.out0 = dV;
    SKA_LAUNCH(ska::kTimedVjp, st, ska::launch_tail_pass(pl.elt, 0, w, st));
    if (p->R > 0) SKA_LAUNCH(ska::kTimedVjp, st, ska::launch_tail_pass(pl.elt, 1, w, st));
    for (int lev = p->R - 1; lev >= 1; --lev) {
      w.level = lev;
      SKA_LAUNCH(ska::kTimedVjp, st, ska::launch_tail_pass(pl.elt, 2, w, st));
      SKA_LAUNCH(ska::kTimedVjp, st, ska::launch_tail_pass(pl.elt, 3, w, st));
    }
    w.out0 = dQ;
    SKA_LAUNCH(ska::kTimedVjp, st, ska::launch_tail_pass(pl.elt, 4, w, st));
    w.out0 = dK;
    SKA_LAUNCH(ska::kTimedVjp, st, ska::launch_tail_pass(pl.elt, 5, w, st));
    return SKA_OK;
  }
  hipError_t e = ska::launch_vjp_prep(duals, ws, g, st);
  if (e != hipSuccess) return fail(SKA_ERR_HIP, hipGetErrorString(e));
  int nt = 0;
  const int nw = ska::vjp_stream_waves(pl.elt, g.h, &nt);
  if (nw > 0) {
    // streaming passes: dV and dv2 = V . dV (owns keys), du2 + dv1 column sums (owns queries),
    // du1 + dQ (owns queries), dK (owns keys)
    ska::VjpArgs a{};
    a.Q = Q;
    a.K = K;
    a.V = V;
    a.dO = dO;
    a.O = O;          // optional: du2 from delta = dO . O in the second pass
    a.ws = ws;
    a.vec_stride = g.bh * (int64_t)g.Lpad;
    a.part = ws + ska::kVjpVecs * a.vec_stride;
    a.bh = g.bh;
    a.Lr = g.Lr;
    a.Lpad = g.Lpad;
    a.h = g.h;
    a.nblk = (g.Lr + 16 * nw - 1) / (16 * nw);
    ska::vjp_stream_segments(g.bh, g.Lr, nw, nt, &a.seg_len, &a.nseg);
    a.pstride = 16 * nw * a.seg_len + 16 * (nt - 1);
    a.c2 = g.c2;
    a.s = g.s;
    // the four passes run back to back: one timing bracket covers them all
    const auto run_ev = timing_begin(ska::kTimedVjp, st);
    for (int pass = 1; pass <= 4; ++pass) {
      a.out0 = (pass == 3) ? dQ : dK;
      a.out1 = dV;
      const hipError_t le = ska::launch_vjp_stream_pass(pl.elt, nt, nw, pass, d4, a, st);
      if (le != hipSuccess) {
        timing_end(ska::kTimedVjp, run_ev, st, pass - 1);
        return fail(SKA_ERR_HIP, std::string("kernel launch failed: ") + hipGetErrorString(le));
      }
    }
    timing_end(ska::kTimedVjp, run_ev, st, 4);
    return SKA_OK;
  }
  // wide passes A..E (bands wider than the streaming passes hold): each owns the side it reduces
  ska::WideArgs w = wide_args(pl, Q, K, V, dO);
  w.O = O;          // optional: du2 from delta = dO . O in pass B
  w.ws = ws;
  w.vec_stride = g.bh * (int64_t)g.Lpad;
  void* outs[6] = {nullptr, dV, nullptr, nullptr, dQ, dK};
  for (int pass = 1; pass <= 5; ++pass) {
    w.out0 = outs[pass];
    SKA_LAUNCH(ska::kTimedVjp, st, ska::launch_wide_pass(pl.elt, pass, d4, w, st));
  }
  return SKA_OK;
}

}  // namespace

ska_status ska::set_error(ska_status s, const std::string& msg) { return fail(s, msg); }

extern "C" {

ska_status ska_workspace_bytes(const ska_problem* p, ska_op op, size_t* bytes) {
  Plan pl;
  SKA_TRY(check_problem(p, op, &pl));
  if (!bytes) return fail(SKA_ERR_INVALID, "bytes pointer is NULL");
  *bytes = workspace_for(pl, op);
  return SKA_OK;
}

ska_status sinkhorn_attn_fwd(const ska_problem* p, const void* Q, const void* K, const void* V,
                             void* O, float* duals, void* workspace, size_t workspace_bytes,
                             hipStream_t stream) {
  g_err.clear();
  return run_fwd(p, SKA_OP_FWD, Q, K, V, O, duals, workspace, workspace_bytes, stream);
}

ska_status sinkhorn_attn_vjp(const ska_problem* p, const void* Q, const void* K, const void* V,
                             const float* duals, const void* dO, const void* O, void* dQ, void* dK,
                             void* dV, ska_schedule schedule, void* workspace,
                             size_t workspace_bytes, hipStream_t stream) {
  g_err.clear();
  return run_vjp(p, SKA_OP_VJP, Q, K, V, duals, dO, O, dQ, dK, dV, schedule, workspace,
                 workspace_bytes, stream);
}

ska_status sinkhorn_attn_dustbin_block_fwd(const ska_problem* p, const void* Q, const void* K,
                                           const void* V, void* O, float* duals, void* workspace,
                                           size_t workspace_bytes, hipStream_t stream) {
  g_err.clear();
  return run_fwd(p, SKA_OP_DUSTBIN_BLOCK_FWD, Q, K, V, O, duals, workspace, workspace_bytes,
                 stream);
}

ska_status sinkhorn_attn_dustbin_block_vjp(const ska_problem* p, const void* Q, const void* K,
                                           const void* V, const float* duals, const void* dO,
                                           const void* O, void* dQ, void* dK, void* dV,
                                           ska_schedule schedule, void* workspace,
                                           size_t workspace_bytes, hipStream_t stream) {
  g_err.clear();
  return run_vjp(p, SKA_OP_DUSTBIN_BLOCK_VJP, Q, K, V, duals, dO, O, dQ, dK, dV, schedule,
                 workspace, workspace_bytes, stream);
}

ska_status sinkhorn_attn_tail_remainder(const ska_problem* p, const void* Q, const void* K,
                                        const void* V, const void* dO, double* sums,
                                        void* workspace, size_t workspace_bytes,
                                        hipStream_t stream) {
  g_err.clear();
  Plan pl;
  SKA_TRY(check_problem(p, SKA_OP_TAIL_REMAINDER, &pl));
  if (pl.empty) return SKA_OK;
  SKA_TRY(check_ptr(Q, "Q"));
  SKA_TRY(check_ptr(K, "K"));
  SKA_TRY(check_ptr(V, "V"));
  SKA_TRY(check_ptr(dO, "dO"));
  if (!sums || (reinterpret_cast<uintptr_t>(sums) & 7u) != 0)
    return fail(SKA_ERR_INVALID, "sums must be an 8-byte aligned device pointer");
  const RemLayout L = rem_layout(pl);
  if (!workspace || workspace_bytes < L.total)
    return fail(SKA_ERR_WORKSPACE, "workspace smaller than ska_workspace_bytes()");
  if (!aligned16(workspace)) return fail(SKA_ERR_INVALID, "workspace is not 16-byte aligned");
  char* w = static_cast<char*>(workspace);
  void* inner = w + L.inner;
  // the stopped-base surrogate at depth R, then full backpropagation: depth T + R from u = v = 0
  ska_problem pr = *p, pf = *p;
  pf.T = 0;
  pf.R = p->T + p->R;
  float* dr = reinterpret_cast<float*>(w + L.duals_r);
  float* df = reinterpret_cast<float*>(w + L.duals_f);
  SKA_TRY(run_fwd(&pr, SKA_OP_FWD, Q, K, V, w + L.o, dr, inner, L.inner_bytes, stream));
  SKA_TRY(run_vjp(&pr, SKA_OP_VJP, Q, K, V, dr, dO, w + L.o, w + L.dq_r, w + L.dk_r, w + L.dv_r,
                  SKA_ONE_REFERENCE, inner, L.inner_bytes, stream));
  SKA_TRY(run_fwd(&pf, SKA_OP_FWD, Q, K, V, w + L.o, df, inner, L.inner_bytes, stream));
  SKA_TRY(run_vjp(&pf, SKA_OP_VJP, Q, K, V, df, dO, nullptr, w + L.dq_f, w + L.dk_f, w + L.dv_f,
                  SKA_ONE_REFERENCE, inner, L.inner_bytes, stream));
  const int64_t n = pl.g.bh * (int64_t)pl.g.Lr * ska::kD;
  double* part = reinterpret_cast<double*>(w + L.part);
  hipError_t e = ska::launch_sq_diff(pl.elt, w + L.dq_f, w + L.dq_r, n, part, sums, stream);
  if (e == hipSuccess) e = ska::launch_sq_diff(pl.elt, w + L.dk_f, w + L.dk_r, n, part, sums + 2, stream);
  if (e != hipSuccess) return fail(SKA_ERR_HIP, hipGetErrorString(e));
  return SKA_OK;
}

namespace {

ska_status contraction_layout(const ska_problem* p, ska_op op, int32_t block, Plan* pl,
                              int64_t* nb, int32_t* m) {
  if (op != SKA_OP_CONTRACTION && op != SKA_OP_DUSTBIN_BLOCK_CONTRACTION)
    return fail(SKA_ERR_INVALID, "not a contraction-certificate op");
  SKA_TRY(check_problem(p, op, pl));
  if (block != 16 && block != 32 && block != 64 && block != 128)
    return fail(SKA_ERR_INVALID, "block must be 16, 32, 64 or 128 tokens");
  const int64_t n = (pl->g.Lr + block - 1) / block;
  *nb = n;
  const int64_t mm = pl->g.h / block;
  *m = (int32_t)std::max<int64_t>(0, std::min<int64_t>(mm, n - 1));
  if (n * (2 * (int64_t)*m + 1) >= (int64_t(1) << 31))
    return fail(SKA_ERR_UNSUPPORTED, "more than 2^31 block pairs per problem");
  return SKA_OK;
}

ska_status run_contraction(const ska_problem* p, ska_op op, int32_t block, const void* Q,
                           const void* K, float* delta, float* kappa, float* delta_max,
                           hipStream_t st) {
  Plan pl;
  int64_t nb = 0;
  int32_t m = 0;
  SKA_TRY(contraction_layout(p, op, block, &pl, &nb, &m));
  if (pl.empty) return SKA_OK;
  SKA_TRY(check_ptr(Q, "Q"));
  SKA_TRY(check_ptr(K, "K"));
  if (!delta || (reinterpret_cast<uintptr_t>(delta) & 3u) != 0)
    return fail(SKA_ERR_INVALID, "delta is NULL or misaligned");
  if (kappa && (reinterpret_cast<uintptr_t>(kappa) & 3u) != 0)
    return fail(SKA_ERR_INVALID, "kappa misaligned");
  if (delta_max && (reinterpret_cast<uintptr_t>(delta_max) & 3u) != 0)
    return fail(SKA_ERR_INVALID, "delta_max misaligned");
  ska::ContractionArgs a{};
  a.Q = Q;
  a.K = K;
  a.delta = delta;
  a.kappa = kappa;
  a.delta_max = delta_max;
  a.bh = pl.g.bh;
  a.Lr = pl.g.Lr;
  a.h = pl.g.h;
  a.B = block;
  a.nb = (int)nb;
  a.m = m;
  a.s = pl.g.s;
  SKA_LAUNCH(ska::kTimedCert, st, ska::launch_contraction(pl.elt, a, st));
  if (delta_max) {
    const hipError_t e = ska::launch_contraction_max(a, st);
    if (e != hipSuccess)
      return fail(SKA_ERR_HIP, std::string("kernel launch failed: ") + hipGetErrorString(e));
  }
  return SKA_OK;
}

}  // namespace

ska_status ska_contraction_layout(const ska_problem* p, ska_op op, int32_t block, int64_t* nb,
                                  int32_t* m) {
  g_err.clear();
  if (!nb || !m) return fail(SKA_ERR_INVALID, "nb and m must not be NULL");
  Plan pl;
  return contraction_layout(p, op, block, &pl, nb, m);
}

ska_status sinkhorn_attn_contraction_certificate(const ska_problem* p, int32_t block,
                                                 const void* Q, const void* K, float* delta,
                                                 float* kappa, float* delta_max,
                                                 hipStream_t stream) {
  g_err.clear();
  return run_contraction(p, SKA_OP_CONTRACTION, block, Q, K, delta, kappa, delta_max, stream);
}

ska_status sinkhorn_attn_dustbin_block_contraction_certificate(const ska_problem* p,
                                                               int32_t block, const void* Q,
                                                               const void* K, float* delta,
                                                               float* kappa, float* delta_max,
                                                               hipStream_t stream) {
  g_err.clear();
  return run_contraction(p, SKA_OP_DUSTBIN_BLOCK_CONTRACTION, block, Q, K, delta, kappa,
                         delta_max, stream);
}

const char* ska_status_string(ska_status s) {
  switch (s) {
    case SKA_OK: return "ok";
    case SKA_ERR_INVALID: return "invalid argument";
    case SKA_ERR_UNSUPPORTED: return "unsupported problem";
    case SKA_ERR_WORKSPACE: return "workspace too small";
    case SKA_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

const char* ska_last_error(void) { return g_err.c_str(); }

ska_status ska_timing_enable(int on) {
  Timing& t = g_timing;
  std::lock_guard<std::mutex> lock(t.mu);
  // launches still pending from an earlier enable are dropped from the counts (their events go
  // back to the pool)
  for (int k = 0; k < ska::kTimedKinds; ++k) {
    for (auto& br : t.pending[k]) {
      (void)hipEventSynchronize(br.ev.second);
      t.free_pairs.push_back(br.ev);
    }
    t.pending[k].clear();
  }
  if (on) {
    t.on = true;
    for (int k = 0; k < ska::kTimedKinds; ++k) {
      t.total_ms[k] = 0;
      t.launches[k] = 0;
    }
    return SKA_OK;
  }
  t.on = false;
  // the event pairs stay in the pool for the next enable: creating events between timed
  // launches would stall the host
  return SKA_OK;
}

ska_status ska_timing_read(int kernel, double* total_ms, int64_t* launches) {
  if (kernel < 0 || kernel >= ska::kTimedKinds || !total_ms || !launches)
    return fail(SKA_ERR_INVALID, "bad timing query");
  Timing& t = g_timing;
  std::lock_guard<std::mutex> lock(t.mu);
  for (auto& br : t.pending[kernel]) {
    if (hipEventSynchronize(br.ev.second) != hipSuccess) return fail(SKA_ERR_HIP, "event sync failed");
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, br.ev.first, br.ev.second) != hipSuccess)
      return fail(SKA_ERR_HIP, "event elapsed time failed");
    t.total_ms[kernel] += ms;
    t.launches[kernel] += br.launches;
    t.free_pairs.push_back(br.ev);
  }
  t.pending[kernel].clear();
  *total_ms = t.total_ms[kernel];
  *launches = t.launches[kernel];
  return SKA_OK;
}

}  // extern "C"
