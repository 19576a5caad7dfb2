/*
 * sinkhorn_attn.h -- C ABI of the MI355X (gfx950) banded balanced Sinkhorn attention library
 * (libsinkhorn_attn.so).
 *
 * Method: arXiv 2605.08123, "Block-Wise Differentiable Sinkhorn Attention: Tail-Refinement
 * Gradients with a Gap-Aware Dustbin Bridge", as summarised on the pages cited per entry point
 * (abstract; technical summaries on gist.science, German "Technische Zusammenfassung" and
 * French "Résumé Technique", §2.1-§2.3; atlas.scime.ai summary, Approach / Key results /
 * Limitations).
 *
 * Problem (one independent problem per batch*head index b, 0 <= b < bh):
 *   tokens 0..Lr-1 with query/key/value rows q_i, k_i, v_i in R^d (Lr = L, or L+1 for the
 *   dustbin_block entry points), band half-width h = W/2, scores on the support
 *   Omega = {(i,j): |i-j| <= h}:  S_ij = q_i . k_j / (sqrt(d) * epsilon).
 *   Base: u = v = 0, then T steps of  u_i = -log sum_j exp(S_ij + v_j),
 *                                     v_j = -log sum_i exp(S_ij + u_i);   v^(0) := v (stopped).
 *   Tail: for a = 1..R:  u^(a) from v^(a-1), then v^(a) from u^(a) (same two updates).
 *   Output: O = P V with P_ij = exp(S_ij + u^(R)_i + v^(R)_j) on Omega.
 *   R = 0 (no tail, T >= 1): the output plan is the base's own, with u^(0), v^(0) the duals of
 *   the last base step, both under stop-gradient.
 *   VJP (0 <= R <= 256): exact gradient of <O, dO> with respect to Q, K, V through the tail,
 *   with v^(0) held fixed (stop-gradient on the base), and u^(0) too when R = 0.
 *
 * Tensor layout: Q, K, V, O, dO, dQ, dK, dV are [bh][Lr][d] row-major (d contiguous), element
 * type given by ska_problem.dtype.  Duals are fp32 [bh][n_d][Lr] in natural-log units: for
 * R >= 1, n_d = 2R+1 rows in the order v^(0), u^(1), v^(1), ..., u^(R), v^(R); for R = 0,
 * n_d = 2 rows u^(0), v^(0).  The last two rows are always the output plan's duals.
 *
 * Ownership and memory: every pointer is a device pointer owned by the caller, including the
 * workspace (size from ska_workspace_bytes).  The library allocates and frees nothing and never
 * synchronises: work is enqueued on `stream` and completes asynchronously.  Between calls it
 * keeps only the allocation-free forward's static scratch and the timing functions' event pool.
 * The compute entry points enqueue kernels only (no memset or copy nodes, no waits; timing, when
 * enabled, adds events), so they can be captured into a HIP graph.  Tensor pointers must be
 * 16-byte aligned; outputs must not alias inputs or the workspace.  Calls on different streams
 * must use different workspaces.
 *
 * Errors: argument errors are detected on the host before anything is enqueued and return
 * SKA_ERR_INVALID / SKA_ERR_UNSUPPORTED / SKA_ERR_WORKSPACE; a failed kernel launch returns
 * SKA_ERR_HIP.  ska_last_error() gives a human-readable detail for the calling thread.  An
 * empty problem (bh == 0 or L == 0, dustbin entry points: bh == 0) returns SKA_OK and
 * enqueues nothing.  Non-finite inputs are not screened: they propagate as NaN/Inf.
 */
#ifndef SINKHORN_ATTN_H
#define SINKHORN_ATTN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { SKA_F32 = 0, SKA_BF16 = 1 } ska_dtype;

/* Adjoint schedule of the VJP.
 * SKA_ONE_REFERENCE: only the reference plan P^(R,R) is exponentiated; the other staircase
 *   plans enter through the orbit factors exp(u^(a)-u^(R)), exp(v^(b)-v^(R)) (abstract;
 *   technical summaries §2.2, orbit equation).  Any R from 0 to 256 (R = 0: the stopped base's
 *   own last plan, with u^(0) and v^(0) both held fixed).
 * SKA_DIRECT_FOUR: R = 2 only; every staircase plan P^(2,2), P^(2,1), P^(1,1), P^(1,0) is
 *   exponentiated on its own (the direct four-plan adjoint, atlas.scime.ai Key results); kept
 *   for comparison.  Other R return SKA_ERR_UNSUPPORTED. */
typedef enum { SKA_ONE_REFERENCE = 0, SKA_DIRECT_FOUR = 1 } ska_schedule;

typedef enum {
  SKA_OK = 0,
  SKA_ERR_INVALID = -1,     /* malformed argument (null/misaligned pointer, W odd, eps <= 0, ...) */
  SKA_ERR_UNSUPPORTED = -2, /* well-formed but not built: d != 64, VJP with R > 256, huge L     */
  SKA_ERR_WORKSPACE = -3,   /* workspace missing or smaller than ska_workspace_bytes()          */
  SKA_ERR_HIP = -4          /* a HIP runtime call or kernel launch failed                        */
} ska_status;

typedef enum {
  SKA_OP_FWD = 0,
  SKA_OP_VJP = 1,
  SKA_OP_DUSTBIN_BLOCK_FWD = 2,
  SKA_OP_DUSTBIN_BLOCK_VJP = 3,
  SKA_OP_TAIL_REMAINDER = 4,
  SKA_OP_CONTRACTION = 5,                /* projective contraction certificate, band support   */
  SKA_OP_DUSTBIN_BLOCK_CONTRACTION = 6   /* the same on the dustbin_block (dense) support      */
} ska_op;

typedef struct {
  int64_t bh;      /* independent problems (batch * heads), >= 0                                 */
  int64_t L;       /* tokens per problem, >= 0 (dustbin_block: real tokens; tensors hold L + 1)  */
  int64_t d;       /* head dimension; 64 is built                                               */
  int64_t W;       /* band width, even, >= 0; support |i - j| <= W / 2                          */
  int32_t T;       /* stopped base steps, >= 0                                                  */
  int32_t R;       /* tail steps >= 0 (R = 0 needs T >= 1); VJP <= 256; direct-four: 2          */
  float epsilon;   /* entropic temperature, finite and > 0                                      */
  int32_t dtype;   /* ska_dtype of Q, K, V, O, dO, dQ, dK, dV (duals are always fp32)           */
} ska_problem;

/* Workspace bytes the entry point `op` needs for problem *p: O(bh * L) floats (dual and cotangent
 * vectors plus per-segment column sums over the band window, about one float per token).
 * Returns SKA_OK and writes *bytes, or an error status for an invalid problem. */
ska_status ska_workspace_bytes(const ska_problem* p, ska_op op, size_t* bytes);

/* Forward pass: stopped T-step balanced Sinkhorn base, R-step tail, O = P^(R,R) V.
 * Writes O [bh][L][d] and duals [bh][n_d][L] (n_d = 2R+1, or 2 when R = 0).
 * (technical summaries §2.1: fixed band support, epsilon absorbed into S, stopped base solve
 * then differentiable tail; abstract: block-wise cost O((T+R) L W), O(L) extra HBM.) */
ska_status sinkhorn_attn_fwd(const ska_problem* p, const void* Q, const void* K, const void* V,
                             void* O, float* duals, void* workspace, size_t workspace_bytes,
                             hipStream_t stream);

/* Exact tail VJP (0 <= R <= 256): given the forward's duals and an arbitrary cotangent dO, writes
 * dQ, dK, dV [bh][L][d].  O is optional (NULL, or the [bh][L][d] output sinkhorn_attn_fwd wrote
 * for the same problem, Q, K, V and duals; it is only read): the row cotangent
 * sum_j P_ij (dO_i . V_j) of the last tail level is then taken as dO_i . O_i, so that pass reads
 * neither V's window nor forms dO . V^T (every R >= 1 on bands the streaming passes hold, R = 2
 * on wider bands and the dustbin_block support; elsewhere O is not read), and the results agree
 * either way within rounding.  An O that is not that output gives wrong gradients.  Scores are recomputed per band
 * tile; extra memory is O(L) vectors (3 + 4 R of them for R != 2).  R = 2 runs the two-level passes (both schedules); other R run
 * 2 R + 2 passes of the one-reference adjoint, the modifier field then holding 2 R terms; R = 0
 * runs dV, dQ and dK of the base plan with both duals fixed (score cotangent P * g)
 * (technical summaries §2.1: R differentiable tail steps; §4.1: tail gradients from R = 0 up).
 * (abstract: one-reference-tile schedule, dS = P^(R,R) * M with M formed from the vector
 * cotangents and the exp(u^(a) - u^(R)), exp(v^(b) - v^(R)) factors; atlas.scime.ai Key
 * results: complete arbitrary-cotangent Q/K/V VJP.) */
ska_status sinkhorn_attn_vjp(const ska_problem* p, const void* Q, const void* K, const void* V,
                             const float* duals, const void* dO, const void* O, void* dQ, void* dK,
                             void* dV, ska_schedule schedule, void* workspace,
                             size_t workspace_bytes, hipStream_t stream);

/* Forward pass that allocates nothing, for callers that cannot allocate device memory around the
 * call (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * Same arguments, results and errors as sinkhorn_attn_fwd, with no workspace argument: the
 * workspace is a static device array of the library, SKA_NOALLOC_SCRATCH_BYTES bytes (32 MiB) per
 * GPU, which every GPU the library runs on holds from module load until the process ends.  A
 * problem whose forward workspace (ska_workspace_bytes with SKA_OP_FWD) is larger is rejected
 * with SKA_ERR_UNSUPPORTED before anything is enqueued; 4 problems of 262,144 tokens at W = 256
 * (about 26.7 MB) fit.  The entry point calls no hipMalloc, hipFree or other allocating routine;
 * on its first call on a device (the current device, which must be the stream's) it looks up
 * that device's copy of the array once.  All calls on one GPU share its array: calls that may
 * overlap on one GPU (other streams, other host threads) race and must be ordered by the caller. */
#define SKA_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
ska_status sinkhorn_attn_fwd_noalloc(const ska_problem* p, const void* Q, const void* K,
                                     const void* V, void* O, float* duals, hipStream_t stream);

/* dustbin_block forward: tensors hold L real tokens followed by the learned dustbin token at
 * row L ([bh][L+1][d]); duals are [bh][n_d][L+1].  Tile padding beyond row L acts as the
 * inactive fill tokens (no support, zero target).  The support is every pair of the L+1 active
 * tokens within the widened half-width max(W/2, L), so the dustbin row and column connect to
 * every token; all active tokens, the dustbin included, have unit row and column targets.  The
 * same balanced surrogate then runs unchanged; cost O(L * max(W, L)).
 * (technical summaries §2.3; searcharxiv abstract: unit-target surrogate on an augmented
 * support with a single active dustbin; atlas.scime.ai Limitations: widened band cost.) */
ska_status sinkhorn_attn_dustbin_block_fwd(const ska_problem* p, const void* Q, const void* K,
                                           const void* V, void* O, float* duals, void* workspace,
                                           size_t workspace_bytes, hipStream_t stream);

/* dustbin_block VJP: gradients for all L+1 rows, the dustbin token included.  O is optional as
 * for sinkhorn_attn_vjp: NULL, or the [bh][L+1][d] output sinkhorn_attn_dustbin_block_fwd wrote
 * for the same problem, inputs and duals. */
ska_status sinkhorn_attn_dustbin_block_vjp(const ska_problem* p, const void* Q, const void* K,
                                           const void* V, const float* duals, const void* dO,
                                           const void* O, void* dQ, void* dK, void* dV,
                                           ska_schedule schedule, void* workspace,
                                           size_t workspace_bytes, hipStream_t stream);

/* A posteriori bias certificate of the stopped base (technical summaries §2.4: a measurement of
 * the gradient remainder eta_R that the stop-gradient on the base drops, certified against a
 * tolerance tau, which selects the tail depth R; Key results: it reconstructs the full remainder
 * to numerical precision and selects R = 2 at tau = 1e-5).
 * Full backpropagation through all T + R steps from u = v = 0 is exactly the tail adjoint at
 * depth T + R with no stopped base (T' = 0: the initial v = 0 is a constant), so this entry runs
 * the forward and the one-reference VJP twice on the caller's workspace, at (T, R) and at
 * (0, T + R), and writes the remainder and full-gradient squared norms summed over all problems:
 *   sums[0] = ||dQ_full - dQ_R||^2,  sums[1] = ||dQ_full||^2,
 *   sums[2] = ||dK_full - dK_R||^2,  sums[3] = ||dK_full||^2
 * (dV has no remainder: V enters only the output).  eta_R = sqrt((sums[0] + sums[2]) /
 * (sums[1] + sums[3])).  `sums` is a device pointer to 4 doubles; the sums are taken in double in
 * a fixed order.  Forming eta_R from the four sums, and selecting the smallest certified R by
 * calling this entry point for R = 0, 1, 2, .. until eta_R <= tau, are left to the caller: two
 * scalar operations on the host after the sums are copied back, which the Python binding does
 * (tail_remainder, select_tail_depth).  Requires T + R <= 256 (and T >= 1 when R = 0); workspace from
 * ska_workspace_bytes(p, SKA_OP_TAIL_REMAINDER): O(bh L (T + R)) floats of duals and cotangent
 * vectors plus seven [bh][L][d] tensors.  Gradients are formed in the input dtype, so with bf16
 * inputs remainders below the bf16 rounding of the gradients (about 4e-3 relative) are not
 * resolved: certify with fp32 inputs.  An empty problem writes nothing. */
ska_status sinkhorn_attn_tail_remainder(const ska_problem* p, const void* Q, const void* K,
                                        const void* V, const void* dO, double* sums,
                                        void* workspace, size_t workspace_bytes,
                                        hipStream_t stream);

/* Projective contraction certificate of the Sinkhorn map's active blocks (technical summaries
 * §2.4: Hilbert's projective metric shows that strictly positive active blocks of the Sinkhorn
 * map are contractions; atlas.scime.ai, Builds on: Birkhoff-Hopf contraction).
 * The Lr tokens (L, or L + 1 for the dustbin_block entry point) are cut into nb = ceil(Lr / block)
 * blocks of `block` tokens (16, 32, 64 or 128; the last block ragged).  A block pair (row block
 * rb, column block cb = rb + o) is active when every pair in it lies on the support (|i - j| <=
 * W/2; every pair for the dustbin_block support), so its Gibbs kernel exp(S) is strictly
 * positive.  For each active pair the entry writes its projective diameter
 *   Delta = max over rows i, i' and columns j, j' of  S_ij + S_i'j' - S_ij' - S_i'j
 * (the largest log cross ratio of exp(S), S = q.k / (sqrt(d) epsilon) in fp32) and, if kappa is
 * not NULL, its Birkhoff-Hopf coefficient kappa = tanh(Delta / 4) < 1: a log-domain row or column
 * half-step restricted to the block shrinks the oscillation of a dual difference by at least
 * kappa, a full step by kappa^2.  Block pairs that are not active (or lie past either end) get
 * -1 in both outputs.  Layout of delta and kappa: fp32 [bh][nb][2 m + 1], entry (b, rb, o + m),
 * with m = min(floor(h / block), nb - 1), h the support half-width (ska_contraction_layout
 * returns nb and m).  If delta_max is not NULL it receives, per problem b, the largest Delta over
 * the active pairs, or -1 if there is none.  T and R do not enter (they must still be valid).
 * Only Q and K are read; no workspace.  An empty problem writes nothing. */
ska_status ska_contraction_layout(const ska_problem* p, ska_op op, int32_t block, int64_t* nb,
                                  int32_t* m);
ska_status sinkhorn_attn_contraction_certificate(const ska_problem* p, int32_t block,
                                                 const void* Q, const void* K, float* delta,
                                                 float* kappa, float* delta_max,
                                                 hipStream_t stream);
/* The same on the dustbin_block support: Q, K hold L + 1 rows, the dustbin token last. */
ska_status sinkhorn_attn_dustbin_block_contraction_certificate(const ska_problem* p,
                                                               int32_t block, const void* Q,
                                                               const void* K, float* delta,
                                                               float* kappa, float* delta_max,
                                                               hipStream_t stream);

/* Static string for a status code. */
const char* ska_status_string(ska_status s);

/* Detail of the last error returned on the calling thread ("" if none). */
const char* ska_last_error(void);

/* Kernel timing for measurement.  While enabled, the launches of the kernel family `kernel`
 * (0: forward Sinkhorn step, 1: forward output, 2: VJP passes, 3: the contraction certificate's
 * diameter kernel, without the per-problem maximum), from any thread of the process, are
 * bracketed by HIP events on their own stream: the T + R fused step launches of a forward, and
 * the four streaming passes of an R = 2 VJP, each under one bracket (the short gaps between
 * those back-to-back launches included); every other launch under its own.  ska_timing_read()
 * synchronises on those events and returns the summed milliseconds and the number of launches
 * covered since ska_timing_enable(1).
 * Launches create HIP event pairs as they need them (no device memory); disabling returns them
 * to a pool that the next enable reuses, so a region timed after an earlier enable creates none.
 * The pool lives until the process ends.  Each event pair leaves the GPU idle for a few
 * microseconds between launches: enable timing only around the launches to be measured. */
ska_status ska_timing_enable(int on);
ska_status ska_timing_read(int kernel, double* total_ms, int64_t* launches);

#ifdef __cplusplus
}
#endif

#endif /* SINKHORN_ATTN_H */
