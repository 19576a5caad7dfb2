// Internal declarations shared by the C ABI layer and the HIP kernels of libsinkhorn_attn.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>

#include "sinkhorn_attn.h"

namespace ska {

// Records `msg` as the calling thread's ska_last_error() detail and returns `s`.
ska_status set_error(ska_status s, const std::string& msg);

constexpr int kD = 64;          // head dimension the kernels are built for
constexpr int kWaves = 4;       // waves per workgroup; each wave owns 16 tokens
constexpr int kOwnPerBlock = 64;
constexpr int kBf16StreamWaves = 8;   // waves per workgroup of the bf16 streaming passes
constexpr int kWideWaves = 8;         // waves per workgroup of the wide-band engine

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

// Arguments of one fused Sinkhorn step launch (see ska_fused.hip).  Vectors are [bh][Lpad] fp32
// in log2 units.  A launch splits each problem's 64-row blocks into segments of seg_len
// consecutive blocks, one workgroup per segment; column partial sums are stored per segment,
// [bh][nseg][pstride] fp32 with pstride = 64 seg_len + 32 H16 (H16 = band halo in 16-key tiles).
struct StepArgs {
  const void* Q;
  const void* K;
  const float* v_prev;     // column duals before the previous launch's column update
  const float* part_prev;  // previous launch's column partials, or nullptr (v_prev is final)
  const float* u_prev;     // previous launch's row duals (exact fallback of the column finish)
  float* v_next;           // finished column duals of the owned tokens
  float* u_out;            // row duals of this step
  float* part_out;         // column partials of this step
  float* save_v;           // optional copies in natural units (saved duals), or nullptr
  int64_t save_v_stride;
  float* save_u;
  int64_t save_u_stride;
  int64_t bh;
  int Lr, Lpad, h, nblk, seg_len, nseg, pstride, H16;
  float c2;
};

// Register-resident step width (16-key tiles per wave, 1 + 2 H16 with H16 even) for half-width h,
// or 0 when the band is too wide for the fused step (the split row/column kernels handle it).
int fused_tiles_for(int h);
// Segment geometry of the fused step for a problem: blocks per segment and segments per problem.
void fused_segments(int64_t bh, int Lr, int nt, int* seg_len, int* nseg);
inline int fused_pstride(int nt, int seg_len) { return 64 * seg_len + 16 * (nt - 1); }

// Arguments of the streaming VJP passes (see ska_vjp_stream.hip).  Workgroups of NW waves own
// blocks of 16 NW rows; segments of seg_len blocks per workgroup as in the forward step.  dv1
// column partials are [bh][nseg][pstride] with pstride = 16 NW seg_len + 32 H16.
struct VjpArgs {
  const void* Q;
  const void* K;
  const void* V;
  const void* dO;
  const void* O;         // R = 2 pass 2: the forward's output for delta = dO . O, or null
  void* out0;            // pass 0: O; passes 3 and 6: dQ; passes 4 and 7: dK
  void* out1;            // pass 1 (and general pass 7 at R = 0): dV
  float* ws;             // kVjpVecs vectors [bh][Lpad]
  const float* fu;       // pass 0 (forward output): row duals u^(R), log2 units [bh][Lpad]
  const float* fv;       // pass 0: column duals v^(R), log2 units [bh][Lpad]
  float* part;           // dv1 column partials (general depth: partials read by a level pass,
                         // written by pass 2)
  float* part_out;       // general depth: partials a level pass writes for the next level
  int64_t vec_stride;    // floats between consecutive workspace vectors (bh * Lpad)
  int64_t bh;
  int Lr, Lpad, h, nblk, seg_len, nseg, pstride;
  float c2, s;
  int R, level;          // general depth: tail depth, and the level a of a level pass
};

// Streaming VJP geometry for (dtype, h): waves per workgroup (0 if the streaming passes do not
// cover this band; the chunked passes handle it) and the register-resident tile count.
int vjp_stream_waves(int elt, int h, int* nt);
// General tail depth on the streaming engine, vectors in the general-depth layout of
// tail_vecs(R): pass 1 (dV, dv^(R)) and pass 2 (du^(R), column partials) as for R = 2, then for
// a = R-1 .. 1 a level pass 5 (F_a from the partials, C_a, the next partials) (any R up to
// kTailMaxR), then pass 6 (dQ) and pass 7 (dK; and dV at R = 0) with the 2 R-term modifier on the
// matrix cores (R <= kStreamMaxR).
constexpr int kStreamMaxR = 4;
hipError_t launch_vjp_stream_general(int elt, int nt, int nw, int pass, const VjpArgs& a,
                                     hipStream_t st);
void vjp_stream_segments(int64_t bh, int Lr, int nw, int nt, int* seg_len, int* nseg);

// Arguments of the wide-band engine (see ska_wide.hip): one workgroup per 16-token row tile
// of one problem, its band window split over the workgroup's waves.  Column partials of the
// fused step are [bh][nrt][pw] fp32: row tile rt (nrt = ceil(Lr / 16)) keeps the partial of key
// j at j - 16 t0(rt), t0(rt) = max(0, 16 rt - h) / 16 its first window tile, pw = 16 x the
// widest window in tiles.
struct WideArgs {
  const void* Q;
  const void* K;
  const void* V;
  const void* dO;
  const void* O;           // R = 2 pass B: the forward's output for delta = dO . O, or null
  const void* Qs;          // fp32 step: Q and K as three bf16 planes per row, [bh][Lr][192]
  const void* Ks;
  void* out0;              // output pass: O; pass A: dV; pass D: dQ; pass E: dK
  const float* v_in;       // step / finish: column duals before the step (log2) [bh][Lpad]
  float* u_out;            // step: row duals of the step (log2); finish: read by the exact fallback
  float* v_out;            // finish: column duals after the step (may alias v_in)
  float* part;             // step column partials
  float* save_u;           // optional natural-unit copies (saved duals), head stride save_stride
  float* save_v;
  int64_t save_stride;
  float* ws;               // VJP: kVjpVecs vectors [bh][Lpad]
  int64_t vec_stride;
  const float* fu;         // output pass: u^(R), v^(R) (log2) [bh][Lpad]
  const float* fv;
  int64_t bh;
  int Lr, Lpad, h, nrt, pw;
  float c2, s;
  int R, level;            // general tail depth passes: the depth, and the level a of passes C/D
};

// VJP workspace of a general tail depth R (any band), each [bh][Lpad] fp32: u^(R), v^(R) (log2
// units), the orbit factors EU_a = exp(u^(a) - u^(R)) (a = 1..R) and EV_b = exp(v^(b) - v^(R))
// (b = 0..R), and the scaled cotangents F_a = dv^(a) EV_a and C_a = du^(a) EU_a (a = 1..R).
inline int tail_vecs(int R) { return 3 + 4 * R; }
// Saved duals per head, [n_duals(R)][Lr]: v^(0), u^(1), v^(1), .., u^(R), v^(R) for R >= 1; the
// stopped base pair u^(0), v^(0) for R = 0.  The last two rows are the output plan's duals.
inline int n_duals(int R) { return R == 0 ? 2 : 2 * R + 1; }
// Row of u_k and of v_k (the duals after Sinkhorn step k = 1 .. T + R, counted from u = v = 0),
// or -1 when that dual is not saved.
inline int dual_slot_u(int k, int T, int R) {
  const int off = (R == 0);
  return (k - T >= 1 - off) ? 2 * (k - T) - 1 + off : -1;
}
inline int dual_slot_v(int k, int T, int R) {
  const int off = (R == 0);
  return (k >= T) ? 2 * (k - T) + off : -1;
}
// Deepest tail the general passes run (a full backpropagation through T + R steps from u = v = 0
// is the general adjoint at depth T + R): the workspace holds 3 + 4 R vectors.
constexpr int kTailMaxR = 256;

// Register tiles per wave of the wide fused step for half-width h (its window of at most 8 KT
// tiles stays in registers), or 0 when the window is wider than that.
int wide_step_tiles(int Lr, int h);
// Widest window of a row tile in 16-token tiles.
inline int wide_window_tiles(int Lr, int h) {
  const int64_t all = ((int64_t)Lr + 15) / 16, band = ((2 * (int64_t)h + 15) >> 4) + 2;
  return (int)(all < band ? all : band);
}

enum TimedKernel : int { kTimedStep = 0, kTimedOut = 1, kTimedVjp = 2, kTimedCert = 3, kTimedKinds = 4 };

// Launchers (return the hipGetLastError() of their launches).  `elt` is 0 for fp32, 1 for bf16.
hipError_t launch_fill(float* p, int64_t n, float value, hipStream_t st);
hipError_t launch_save_duals(const float* vec_log2, float* duals, int64_t dual_stride_head,
                             const Geometry& g, hipStream_t st);
hipError_t launch_lse(int elt, const void* own, const void* win, const float* vin, float* vout,
                      float* vsave, int64_t save_stride, const Geometry& g, hipStream_t st);
// rev: walk each segment from its last block down (consecutive steps alternate)
hipError_t launch_fused_step(int elt, int nt, const StepArgs& a, bool rev, hipStream_t st);
hipError_t launch_finish_columns(int elt, const StepArgs& a, hipStream_t st);
hipError_t launch_vjp_stream_pass(int elt, int nt, int nw, int pass, bool d4, const VjpArgs& a,
                                  hipStream_t st);
// first: the first step of the iteration (u = v = 0), which takes the exact row maximum; later
// steps shift the row log-sum-exp by the previous row duals (read from u_out before it is rewritten)
hipError_t launch_wide_step(int elt, int kt, bool first, const WideArgs& a, hipStream_t st);
hipError_t launch_wide_finish(int elt, const WideArgs& a, hipStream_t st);
// x [rows][64] fp32 -> out [rows][192] bf16: the planes (h, m, l) of x = h + m + l (the fp32
// wide step's matrix-core operands)
hipError_t launch_split3(const float* x, void* out, int64_t rows, hipStream_t st);
// bf16 elements of one tensor's planes per row
constexpr int kPlaneRowElems = 3 * 64;
// pass: 0 output, 1..5 the VJP passes A..E
hipError_t launch_wide_pass(int elt, int pass, bool d4, const WideArgs& a, hipStream_t st);
hipError_t launch_vjp_prep(const float* duals, float* ws, const Geometry& g, hipStream_t st);
// out2[0] = sum (a - b)^2, out2[1] = sum a^2 over n elements (double, fixed order); part holds
// 2 x kSqPartials doubles of block sums
constexpr int kSqPartials = 256;
hipError_t launch_sq_diff(int elt, const void* a, const void* b, int64_t n, double* part,
                          double* out2, hipStream_t st);
// General tail depth (0 <= R <= kTailMaxR), one-reference-tile adjoint on the wide decomposition:
// the vector preparation, then passes 0 (A: dv^(R), dV), 1 (B: du^(R)), 2 (C: dv^(a)),
// 3 (D: du^(a)), 4 (dQ), 5 (dK).  R = 0 runs A (dV only), dQ and dK.
hipError_t launch_tail_prep(const float* duals, float* ws, int R, const Geometry& g, hipStream_t st);
hipError_t launch_tail_pass(int elt, int pass, const WideArgs& a, hipStream_t st);

// Projective contraction certificate: the diameter (and Birkhoff-Hopf coefficient) of every active
// B x B block pair, [bh][nb][2 m + 1] by (row block, column-block offset + m), -1 where no block
// pair is active; delta_max[b], if given, the largest entry of problem b (-1 if none is active).
struct ContractionArgs {
  const void* Q;
  const void* K;
  float* delta;
  float* kappa;            // may be null
  float* delta_max;        // may be null
  int64_t bh;
  int Lr, h, B, nb, m;
  float s;                 // 1 / (sqrt(d) epsilon)
};
// diameters and coefficients of every block pair (the timed kernel), then, separately, the
// per-problem maximum into delta_max
hipError_t launch_contraction(int elt, const ContractionArgs& a, hipStream_t st);
hipError_t launch_contraction_max(const ContractionArgs& a, hipStream_t st);
}  // namespace ska
