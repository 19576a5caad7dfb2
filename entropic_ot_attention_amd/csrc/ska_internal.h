// Internal declarations shared by the C ABI layer and the HIP kernels of libsinkhorn_attn.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ska {

constexpr int kD = 64;          // head dimension the kernels are built for
constexpr int kWaves = 4;       // waves per workgroup; each wave owns 16 tokens
constexpr int kOwnPerBlock = 64;

// Vectors kept per head in the workspace are padded to a multiple of this many tokens.
inline int64_t pad_tokens(int64_t Lr) { return (Lr + 63) / 64 * 64; }

// Forward workspace: u, v (log2 units), per head Lpad floats each.
constexpr int kFwdVecs = 2;

// VJP workspace vectors, each [bh][Lpad] fp32.
enum VjpVec : int {
  kV0 = 0, kU1, kV1, kU2, kV2,   // duals in log2 units
  kEB,                           // exp(u1 - u2)            (row factor)
  kEE,                           // exp(v1 - v2)            (column factor)
  kEG,                           // exp(v0 - v2)            (column factor)
  kDV2, kDU2, kDV1,              // vector cotangents (natural units)
  kFF,                           // dv1 * exp(v1 - v2)
  kDU1,                          //
  kCC,                           // du1 * exp(u1 - u2)
  kVjpVecs
};

struct Geometry {
  int64_t bh;     // problems
  int Lr;         // token rows per problem
  int Lpad;       // padded vector length
  int h;          // band half-width
  float c2;       // score scale in log2 units: log2(e) / (sqrt(d) * eps)
  float s;        // score scale in natural units: 1 / (sqrt(d) * eps)
};

enum TimedKernel : int { kTimedStep = 0, kTimedOut = 1, kTimedVjp = 2, kTimedKinds = 3 };

// Launchers (return the hipGetLastError() of their launches).  `elt` is 0 for fp32, 1 for bf16.
hipError_t launch_fill(float* p, int64_t n, float value, hipStream_t st);
hipError_t launch_save_duals(const float* vec_log2, float* duals, int64_t dual_stride_head,
                             const Geometry& g, hipStream_t st);
hipError_t launch_lse(int elt, const void* own, const void* win, const float* vin, float* vout,
                      float* vsave, int64_t save_stride, const Geometry& g, hipStream_t st);
hipError_t launch_out(int elt, const void* Q, const void* K, const void* V, const float* u2,
                      const float* v2, void* O, const Geometry& g, hipStream_t st);
hipError_t launch_vjp_prep(const float* duals, float* ws, const Geometry& g, hipStream_t st);
hipError_t launch_vjp_pass(int elt, int pass, bool direct4, const void* Q, const void* K,
                           const void* V, const void* dO, void* out, float* ws, const Geometry& g,
                           hipStream_t st);

}  // namespace ska
