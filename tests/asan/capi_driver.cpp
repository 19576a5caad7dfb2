// Host-only driver of the C ABI's validation, workspace sizing and launch sequencing, built with
// AddressSanitizer and UndefinedBehaviorSanitizer by tests/test_capi_asan.py (g++, no device
// code).  The kernel launchers are replaced by counting stubs, so every entry point runs its whole
// host path (argument checks, geometry, per-step pointer arithmetic, timing-off brackets) on fake
// 16-byte-aligned device addresses that are never dereferenced.  Exits non-zero on the first
// unexpected status.

#include <cstdio>
#include <cstdint>
#include <cstring>
#include <vector>

#include "sinkhorn_attn.h"
#include "ska_internal.h"

namespace {
long g_launches = 0;
hipError_t stub() {
  ++g_launches;
  return hipSuccess;
}
}  // namespace

namespace ska {
hipError_t launch_fill(float*, int64_t, float, hipStream_t) { return stub(); }
hipError_t launch_save_duals(const float*, float*, int64_t, const Geometry&, hipStream_t) { return stub(); }
hipError_t launch_lse(int, const void*, const void*, const float*, float*, float*, int64_t,
                      const Geometry&, hipStream_t) { return stub(); }
hipError_t launch_fused_step(int, int, const StepArgs&, bool, hipStream_t) { return stub(); }
hipError_t launch_finish_columns(int, const StepArgs&, hipStream_t) { return stub(); }
hipError_t launch_vjp_stream_pass(int, int, int, int, bool, const VjpArgs&, hipStream_t) { return stub(); }
hipError_t launch_vjp_stream_general(int, int, int, int, const VjpArgs&, hipStream_t) { return stub(); }
hipError_t launch_wide_step(int, int, bool, const WideArgs&, hipStream_t) { return stub(); }
hipError_t launch_wide_finish(int, const WideArgs&, hipStream_t) { return stub(); }
hipError_t launch_split3(const float*, void*, int64_t, hipStream_t) { return stub(); }
hipError_t launch_wide_pass(int, int, bool, const WideArgs&, hipStream_t) { return stub(); }
hipError_t launch_vjp_prep(const float*, float*, const Geometry&, hipStream_t) { return stub(); }
hipError_t launch_sq_diff(int, const void*, const void*, int64_t, double*, double*, hipStream_t) { return stub(); }
hipError_t launch_tail_prep(const float*, float*, int, const Geometry&, hipStream_t) { return stub(); }
hipError_t launch_tail_pass(int, int, const WideArgs&, hipStream_t) { return stub(); }
hipError_t launch_contraction(int, const ContractionArgs&, hipStream_t) { return stub(); }
hipError_t launch_contraction_max(const ContractionArgs&, hipStream_t) { return stub(); }
}  // namespace ska

static int g_fail = 0;
#define EXPECT(cond, ...)                        \
  do {                                           \
    if (!(cond)) {                               \
      std::fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
      std::fprintf(stderr, __VA_ARGS__);         \
      std::fprintf(stderr, " [%s]\n", ska_last_error()); \
      ++g_fail;                                  \
    }                                            \
  } while (0)

static void* fake(uintptr_t k) { return reinterpret_cast<void*>(uintptr_t(1) << 40 | (k << 24)); }

int main() {
  void* Q = fake(1);
  void* K = fake(2);
  void* V = fake(3);
  void* O = fake(4);
  void* dO = fake(5);
  void* dQ = fake(6);
  void* dK = fake(7);
  void* dV = fake(8);
  float* duals = static_cast<float*>(fake(9));
  void* ws = fake(10);
  double* sums = static_cast<double*>(fake(11));
  float* delta = static_cast<float*>(fake(12));
  hipStream_t st = nullptr;

  // every band class and engine, both dtypes, tail depths 0..4 and a deep one, empty problems
  const int64_t Ls[] = {0, 1, 17, 97, 512, 1000, 4097, 70000};
  const int64_t Ws[] = {0, 8, 64, 128, 256, 384, 600, 2000, 9000};
  int valid = 0;
  for (int64_t L : Ls)
    for (int64_t W : Ws)
      for (int dt = 0; dt < 2; ++dt)
        for (int R : {0, 1, 2, 3, 4, 9}) {
          for (int dust = 0; dust < 2; ++dust) {
            ska_problem p{3, L, 64, W, 4, R, 0.7f, dt};
            const ska_op fop = dust ? SKA_OP_DUSTBIN_BLOCK_FWD : SKA_OP_FWD;
            const ska_op vop = dust ? SKA_OP_DUSTBIN_BLOCK_VJP : SKA_OP_VJP;
            size_t nf = 0, nv = 0;
            EXPECT(ska_workspace_bytes(&p, fop, &nf) == SKA_OK, "fwd ws L=%lld W=%lld", (long long)L, (long long)W);
            EXPECT(ska_workspace_bytes(&p, vop, &nv) == SKA_OK, "vjp ws L=%lld W=%lld", (long long)L, (long long)W);
            const size_t n = nf > nv ? nf : nv;
            ska_status s = dust ? sinkhorn_attn_dustbin_block_fwd(&p, Q, K, V, O, duals, ws, n, st)
                                : sinkhorn_attn_fwd(&p, Q, K, V, O, duals, ws, n, st);
            EXPECT(s == SKA_OK, "fwd L=%lld W=%lld R=%d dt=%d dust=%d: %d", (long long)L, (long long)W, R, dt, dust, s);
            for (int sch = 0; sch < 2; ++sch) {
              s = dust ? sinkhorn_attn_dustbin_block_vjp(&p, Q, K, V, duals, dO, O, dQ, dK, dV,
                                                         (ska_schedule)sch, ws, n, st)
                       : sinkhorn_attn_vjp(&p, Q, K, V, duals, dO, O, dQ, dK, dV, (ska_schedule)sch, ws,
                                           n, st);
              const ska_status want = (sch == 1 && R != 2) ? SKA_ERR_UNSUPPORTED : SKA_OK;
              EXPECT(s == want, "vjp L=%lld W=%lld R=%d sch=%d: %d", (long long)L, (long long)W, R, sch, s);
              if (nv > 0) {
                // one byte short of the VJP's workspace
                s = dust ? sinkhorn_attn_dustbin_block_vjp(&p, Q, K, V, duals, dO, nullptr, dQ, dK, dV,
                                                           (ska_schedule)sch, ws, nv - 1, st)
                         : sinkhorn_attn_vjp(&p, Q, K, V, duals, dO, nullptr, dQ, dK, dV,
                                             (ska_schedule)sch, ws, nv - 1, st);
                EXPECT(s == (want == SKA_OK ? SKA_ERR_WORKSPACE : want), "short vjp ws: %d", s);
              }
            }
            ++valid;
          }
          if (R <= 4) {
            ska_problem p{2, L, 64, W, 4, R, 1.0f, dt};
            size_t nr = 0;
            if (ska_workspace_bytes(&p, SKA_OP_TAIL_REMAINDER, &nr) == SKA_OK) {
              EXPECT(sinkhorn_attn_tail_remainder(&p, Q, K, V, dO, sums, ws, nr, st) == SKA_OK,
                     "tail remainder L=%lld W=%lld R=%d", (long long)L, (long long)W, R);
            }
            for (int B : {16, 32, 64, 128}) {
              int64_t nb = 0;
              int32_t m = 0;
              if (ska_contraction_layout(&p, SKA_OP_CONTRACTION, B, &nb, &m) == SKA_OK)
                EXPECT(sinkhorn_attn_contraction_certificate(&p, B, Q, K, delta, nullptr, nullptr, st) == SKA_OK,
                       "contraction L=%lld W=%lld B=%d", (long long)L, (long long)W, B);
            }
          }
        }

  // argument errors, returned before anything is enqueued
  const long before = g_launches;
  ska_problem good{2, 100, 64, 16, 3, 2, 1.0f, SKA_F32};
  size_t need = 0;
  EXPECT(ska_workspace_bytes(&good, SKA_OP_FWD, &need) == SKA_OK && need > 0, "good ws");
  struct Bad {
    ska_problem p;
    ska_status want;
  } bad[] = {
      {{-1, 100, 64, 16, 3, 2, 1.0f, SKA_F32}, SKA_ERR_INVALID},
      {{2, -5, 64, 16, 3, 2, 1.0f, SKA_F32}, SKA_ERR_INVALID},
      {{2, 100, 32, 16, 3, 2, 1.0f, SKA_F32}, SKA_ERR_UNSUPPORTED},
      {{2, 100, 64, 15, 3, 2, 1.0f, SKA_F32}, SKA_ERR_INVALID},
      {{2, 100, 64, -2, 3, 2, 1.0f, SKA_F32}, SKA_ERR_INVALID},
      {{2, 100, 64, 16, -1, 2, 1.0f, SKA_F32}, SKA_ERR_INVALID},
      {{2, 100, 64, 16, 3, -1, 1.0f, SKA_F32}, SKA_ERR_INVALID},
      {{2, 100, 64, 16, 0, 0, 1.0f, SKA_F32}, SKA_ERR_INVALID},
      {{2, 100, 64, 16, 3, 2, 0.0f, SKA_F32}, SKA_ERR_INVALID},
      {{2, 100, 64, 16, 3, 2, -1.0f, SKA_F32}, SKA_ERR_INVALID},
      {{2, 100, 64, 16, 3, 2, 1.0f / 0.0f, SKA_F32}, SKA_ERR_INVALID},
      {{2, 100, 64, 16, 3, 2, 1.0f, 7}, SKA_ERR_INVALID},
      {{70000, 100, 64, 16, 3, 2, 1.0f, SKA_F32}, SKA_ERR_UNSUPPORTED},
      {{2, (int64_t(1) << 31), 64, 16, 3, 2, 1.0f, SKA_F32}, SKA_ERR_UNSUPPORTED},
  };
  for (const Bad& b : bad) {
    size_t n = 0;
    EXPECT(ska_workspace_bytes(&b.p, SKA_OP_FWD, &n) == b.want, "bad problem ws");
    EXPECT(sinkhorn_attn_fwd(&b.p, Q, K, V, O, duals, ws, need, st) == b.want, "bad problem fwd");
    EXPECT(std::strlen(ska_last_error()) > 0, "error detail");
  }
  ska_problem deep{2, 100, 64, 16, 3, 257, 1.0f, SKA_F32};
  EXPECT(sinkhorn_attn_vjp(&deep, Q, K, V, duals, dO, nullptr, dQ, dK, dV, SKA_ONE_REFERENCE, ws, 1 << 30, st) ==
             SKA_ERR_UNSUPPORTED, "R above 256");
  EXPECT(ska_workspace_bytes(nullptr, SKA_OP_FWD, &need) == SKA_ERR_INVALID, "null problem");
  EXPECT(ska_workspace_bytes(&good, SKA_OP_FWD, nullptr) == SKA_ERR_INVALID, "null out");
  EXPECT(ska_workspace_bytes(&good, (ska_op)99, &need) == SKA_ERR_INVALID, "bad op");
  EXPECT(sinkhorn_attn_fwd(&good, nullptr, K, V, O, duals, ws, need, st) == SKA_ERR_INVALID, "null Q");
  EXPECT(sinkhorn_attn_fwd(&good, static_cast<char*>(Q) + 4, K, V, O, duals, ws, need, st) ==
             SKA_ERR_INVALID, "misaligned Q");
  EXPECT(sinkhorn_attn_fwd(&good, Q, K, V, O, nullptr, ws, need, st) == SKA_ERR_INVALID, "null duals");
  EXPECT(sinkhorn_attn_fwd(&good, Q, K, V, O, duals, nullptr, need, st) == SKA_ERR_WORKSPACE, "null ws");
  EXPECT(sinkhorn_attn_fwd(&good, Q, K, V, O, duals, ws, need - 1, st) == SKA_ERR_WORKSPACE, "short ws");
  EXPECT(sinkhorn_attn_vjp(&good, Q, K, V, duals, dO, nullptr, dQ, dK, dV, (ska_schedule)5, ws, 1 << 30, st) ==
             SKA_ERR_INVALID, "bad schedule");
  EXPECT(sinkhorn_attn_vjp(&good, Q, K, V, duals, dO, static_cast<char*>(O) + 4, dQ, dK, dV, SKA_ONE_REFERENCE,
                           ws, 1 << 30, st) == SKA_ERR_INVALID, "misaligned O");
  EXPECT(sinkhorn_attn_tail_remainder(&good, Q, K, V, dO, reinterpret_cast<double*>(static_cast<char*>(fake(11)) + 4),
                                      ws, 1 << 30, st) == SKA_ERR_INVALID, "misaligned sums");
  int64_t nb = 0;
  int32_t m = 0;
  EXPECT(ska_contraction_layout(&good, SKA_OP_CONTRACTION, 48, &nb, &m) == SKA_ERR_INVALID, "bad block");
  EXPECT(ska_contraction_layout(&good, SKA_OP_FWD, 16, &nb, &m) == SKA_ERR_INVALID, "not a contraction op");
  EXPECT(g_launches == before, "an argument error enqueued work");
  for (int s = -5; s <= 0; ++s) EXPECT(std::strlen(ska_status_string((ska_status)s)) > 0, "status string");
  std::printf("valid calls %d, stub launches %ld, failures %d\n", valid, g_launches, g_fail);
  return g_fail == 0 ? 0 : 1;
}
