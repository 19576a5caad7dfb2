// Streaming passes of the forward output and of the exact R = 2 tail VJP, one-reference-tile
// schedule (gfx950).
//
// The adjoint [abstract: dS = P22 * M, M formed from the tail's vector cotangents and the
// exp(u^(a) - u^(2)), exp(v^(b) - v^(2)) factors; technical summaries §2.2: orbit equation
// P^(a,b) = P^(2,2) exp(u^(a) - u^(2)) exp(v^(b) - v^(2))], with P22 = exp(S + u2 + v2),
// g_ij = dO_i . V_j and e^{du1} = exp(u1 - u2), e^{dv_b} = exp(v_b - v2), in four passes:
//
//   0 (owns queries)  forward output O_i = sum_j P22_ij V_j   [the reference plan applied to V]
//   1 (owns keys)     dV_j = sum_i P22_ij dO_i,  dv2_j = sum_i P22 g = V_j . dV_j
//   2 (owns queries)  du2_i = sum_j P22 (g - dv2_j), or given the forward's output O,
//                     dO_i . O_i - sum_j P22 dv2_j (no V window, no g);
//                     per-segment column sums sum_i P22 du2_i
//   3 (owns queries)  dv1_j = -e^{dv1_j} (column sums)  (finished for the window on arrival)
//                     du1_i = -e^{du1_i} sum_j P22 e^{dv1_j} dv1_j
//                     dQ_i  = s sum_j dS_ij k_j,  dS = Z1 - C_i Z2 with
//                             Z1 = P22 (g - D_j - A_i E_j - B_i F_j), Z2 = P22 G_j
//   4 (owns keys)     dK_j = s sum_i dS_ij q_i,  dS = P22 (g - D_j - A_i E_j - B_i F_j - C_i G_j)
// (A = du2, B = e^{du1}, C = du1 e^{du1}, D = dv2, E = e^{dv1}, F = dv1 e^{dv1}, G = e^{dv0}).
//
// Work decomposition as in the fused forward step: a workgroup of NW waves walks a segment of
// consecutive blocks of 16 NW owned tokens; the band window of the block (16 NW + 32 H16
// tokens) of the two window-side tensors lives in LDS rings, each block brings in only its 16 NW
// new rows (loaded one block ahead, together with the next block's owned operands and owned-side
// vectors; no load is waited on where it is issued), and the window-side vectors live in rings
// alongside.  Pass 2 keeps its 16 x (16 + 32 H16) reference-plan strip in registers (owned rows
// in lane registers, keys across lanes) so the column sums need du2, known only after the sweep;
// passes 0, 1, 3 and 4 put the window in lane registers and the owned tokens across lanes, so
// sums over the window stay in-lane and contractions over the window feed the matrix cores
// directly, the other operand read transposed from its LDS ring.  The owned-side dual enters the
// matrix-core accumulator, so each reference-plan entry costs one fma and one exponential.
// Interior blocks of a band that fills its halo class (h = 16 H16) run a straight-line path whose
// only masks are fixed per-lane patterns on the first and last tiles.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "ska_device.h"
#include "ska_internal.h"

namespace ska {

// Transposing LDS read (ds_read_b64_tr_b16): within each 16-lane row, lane i receives element
// i % 4 of the 8 bytes loaded by lane i / 4 + 4 e, as its element e.  With lane (g, n) loading
// ring row rb + 4 g + n / 4 at columns c0 + 4 (n % 4) .. + 3, lane (g, n) receives rows
// rb + 4 g + e (e = 0..3) of column c0 + n: one half of a bf16 MFMA A operand of the
// transposed ring rows.
typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ s16x4 tr_read(const bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 __attribute__((address_space(3)))*)(p));
}

// Four fp32 values as bf16 (high, low) parts, (h0, h1, h2, h3, l0, l1, l2, l3) with
// h = bf16(x) and l = bf16(x - h), both rounded to nearest: x = h + l + e, |e| <= 2^-18 |x|, so a
// product x y formed as hx hy + lx hy + hx ly on the bf16 matrix cores (fp32 accumulation) is
// within about 2^-16 of x y relative.
__device__ __forceinline__ bf16x8 split_bf16x4(const float (&x)[4]) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const bf16 h = (bf16)x[e];
    r[e] = h;
    r[4 + e] = (bf16)(x[e] - (float)h);
  }
  return r;
}

// z[tt][r] -> bf16 B operand (rows 4 g + r of tile tt of the pair)
__device__ __forceinline__ bf16x8 pack_z(const float (&z)[2][4]) {
  bf16x8 zb;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    zb[e] = (bf16)z[0][e];
    zb[e + 4] = (bf16)z[1][e];
  }
  return zb;
}

// Part of row `row` of a [., 64] tensor in the layout store_row writes (lane holds columns
// 16 b + 4 g + r, r = 0..3), kept as loaded until at() converts it.
template <typename T> struct RowPart;
template <> struct RowPart<bf16> {
  typedef __bf16 bf16x4 __attribute__((__vector_size__(8)));
  bf16x4 v[4];
  __device__ __forceinline__ void load(const bf16* row, int g) {
#pragma unroll
    for (int b = 0; b < 4; ++b) v[b] = *reinterpret_cast<const bf16x4*>(row + 16 * b + 4 * g);
  }
  __device__ __forceinline__ float at(int b, int r) const { return (float)v[b][r]; }
};
template <> struct RowPart<float> {
  f32x4 v[4];
  __device__ __forceinline__ void load(const float* row, int g) {
#pragma unroll
    for (int b = 0; b < 4; ++b) v[b] = *reinterpret_cast<const f32x4*>(row + 16 * b + 4 * g);
  }
  __device__ __forceinline__ float at(int b, int r) const { return v[b][r]; }
};

// Contractions over the 32 window rows of a tile pair (ring slots rt0, rt1):
//   acc[b][r] (lane (g, n)) += sum_rows Op[row][16 b + 4 g + r] * Z[row][n]
// with Op read transposed from the ring and z[tt][r] = Z[rt_tt + 4 g + r][n].
struct TrLane {   // per-lane part of the transposed-read address (bf16 rings)
  int off;
  __device__ TrLane(int g, int n) : off((4 * g + (n >> 2)) * Lds<bf16>::stride + 4 * (n & 3)) {}
};
__device__ __forceinline__ bf16x8 tr_operand(const bf16* ring, const TrLane& tl, int rt0, int rt1, int b) {
  const s16x4 lo = tr_read(ring + tl.off + rt0 * Lds<bf16>::stride + 16 * b);
  const s16x4 hi = tr_read(ring + tl.off + rt1 * Lds<bf16>::stride + 16 * b);
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}
__device__ __forceinline__ void contract_pair(f32x4 (&acc)[4], const bf16* ring, const TrLane& tl,
                                              int rt0, int rt1, const float (&z)[2][4], int, int) {
  const bf16x8 zb = pack_z(z);
#pragma unroll
  for (int b = 0; b < 4; ++b)
    acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(tr_operand(ring, tl, rt0, rt1, b), zb, acc[b], 0, 0, 0);
}
__device__ __forceinline__ void contract_pair2(f32x4 (&x)[4], f32x4 (&y)[4], const bf16* ring,
                                               const TrLane& tl, int rt0, int rt1,
                                               const float (&z1)[2][4], const float (&z2)[2][4], int,
                                               int) {
  const bf16x8 zb1 = pack_z(z1), zb2 = pack_z(z2);
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const bf16x8 av = tr_operand(ring, tl, rt0, rt1, b);
    x[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, zb1, x[b], 0, 0, 0);
    y[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, zb2, y[b], 0, 0, 0);
  }
}
__device__ __forceinline__ void contract_pair(f32x4 (&acc)[4], const float* ring, const TrLane&,
                                              int rt0, int rt1, const float (&z)[2][4], int g, int n) {
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = (tt == 0 ? rt0 : rt1) + 4 * g + r;
#pragma unroll
      for (int b = 0; b < 4; ++b)
        acc[b] = __builtin_amdgcn_mfma_f32_16x16x4f32(ring[row * Lds<float>::stride + 16 * b + n],
                                                      z[tt][r], acc[b], 0, 0, 0);
    }
}
__device__ __forceinline__ void contract_pair2(f32x4 (&x)[4], f32x4 (&y)[4], const float* ring,
                                               const TrLane&, int rt0, int rt1,
                                               const float (&z1)[2][4], const float (&z2)[2][4],
                                               int g, int n) {
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = (tt == 0 ? rt0 : rt1) + 4 * g + r;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const float av = ring[row * Lds<float>::stride + 16 * b + n];
        x[b] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, z1[tt][r], x[b], 0, 0, 0);
        y[b] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, z2[tt][r], y[b], 0, 0, 0);
      }
    }
}

// Contraction operands of a tile pair, fetched ahead of their use: bf16 holds the four
// transposed A operands; fp32 keeps the slots and reads the ring inside the contraction.
template <typename T> struct PairOps;
template <> struct PairOps<bf16> {
  bf16x8 v[4];
  __device__ __forceinline__ void fetch(const bf16* ring, const TrLane& tl, int rt0, int rt1) {
#pragma unroll
    for (int b = 0; b < 4; ++b) v[b] = tr_operand(ring, tl, rt0, rt1, b);
  }
  __device__ __forceinline__ void contract(f32x4 (&acc)[4], const bf16*, const TrLane&,
                                           const float (&z)[2][4], int, int) const {
    const bf16x8 zb = pack_z(z);
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v[b], zb, acc[b], 0, 0, 0);
  }
  __device__ __forceinline__ void contract2(f32x4 (&x)[4], f32x4 (&y)[4], const bf16*, const TrLane&,
                                            const float (&z1)[2][4], const float (&z2)[2][4], int,
                                            int) const {
    const bf16x8 zb1 = pack_z(z1), zb2 = pack_z(z2);
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      x[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v[b], zb1, x[b], 0, 0, 0);
      y[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v[b], zb2, y[b], 0, 0, 0);
    }
  }
};
template <> struct PairOps<float> {
  int rt0, rt1;
  __device__ __forceinline__ void fetch(const float*, const TrLane&, int r0, int r1) {
    rt0 = r0;
    rt1 = r1;
  }
  __device__ __forceinline__ void contract(f32x4 (&acc)[4], const float* ring, const TrLane& tl,
                                           const float (&z)[2][4], int g, int n) const {
    contract_pair(acc, ring, tl, rt0, rt1, z, g, n);
  }
  __device__ __forceinline__ void contract2(f32x4 (&x)[4], f32x4 (&y)[4], const float* ring,
                                            const TrLane& tl, const float (&z1)[2][4],
                                            const float (&z2)[2][4], int g, int n) const {
    contract_pair2(x, y, ring, tl, rt0, rt1, z1, z2, g, n);
  }
};

// Window-tile operand fragment at ring slot rt (rows rt + n, d-slice of lane group g): bf16 reads
// from a per-lane base plus a wave-uniform row offset; fp32 through lds_frag.
__device__ __forceinline__ void ring_frag(Frag<bf16>& f, const bf16* ring, const bf16* lane_base, int rt,
                                          int, int) {
  const f32x4* p = reinterpret_cast<const f32x4*>(lane_base + rt * Lds<bf16>::stride);
  f.a = __builtin_bit_cast(bf16x8, p[0]);
  f.b = __builtin_bit_cast(bf16x8, p[1]);
}
__device__ __forceinline__ void ring_frag(Frag<float>& f, const float* ring, const float*, int rt, int g,
                                          int n) {
  lds_frag(f, ring, rt + n, g);
}

template <int PASS, bool D4, int GEN, bool DELTA> struct VjpPass {
  static constexpr bool owns_keys = (PASS == 1 || PASS == 4 || PASS == 7);
  // pass 2 given the forward's output O: sum_j P22_ij g_ij = dO_i . O_i (delta_i), so the pass
  // forms du2_i = delta_i - sum_j P22_ij dv2_j from the owned dO and O rows, without g or the
  // window's V
  static constexpr bool delta = DELTA && PASS == 2;
  // owned rows in lane registers and window tokens across lanes (the passes that emit column
  // partials); the others hold the window in registers and the owned tokens across lanes
  static constexpr bool rows_in_regs = (PASS == 2 || PASS == 5);
  // pass 1 contracts the plan with the window's dO (dV) and takes dv = V . dV, so it needs no g
  static constexpr bool needs_g = (PASS != 0 && PASS != 1 && PASS != 5 && !delta);
  // writes dV: pass 1, and pass 7 at R = 0 (GEN 0 there), where no pass 1 runs
  static constexpr bool writes_dv = (PASS == 1) || (PASS == 7 && GEN == 0);
  static constexpr bool uses_ring_b = (PASS != 5 && !delta);
  static constexpr bool reads_part = (PASS == 3 || PASS == 5);
  static constexpr bool writes_part = (PASS == 2 || PASS == 5);
  // contracts the reference plan (or the score cotangent) with a window tensor, tile pair by
  // tile pair
  // (the direct-four passes 3 and 4 run at phase 0 only: two phases of their wider tile work
  // exceed the register file)
  static constexpr bool contracts = (PASS == 0 || PASS == 1 || ((PASS == 3 || PASS == 4) && !D4) ||
                                     PASS == 6 || PASS == 7);
  // the modifier field on the matrix cores: general depth passes 6 and 7, and the one-reference
  // passes 3 (D + A E + B F) and 4 (D + A E + B F + C G); one fp32 16x16x4 product per k-step of
  // 4 terms, except for bf16 inputs at R = 2, where it is one split-bf16 16x16x32 product added to
  // the g tile (SPLITMOD in the kernel)
  static constexpr bool modk = (PASS == 6 || PASS == 7) || ((PASS == 3 || PASS == 4) && !D4 && GEN < 0);
  // k-steps of the modifier contraction (general depth: 2 R terms, 4 per step)
  static constexpr int KS = GEN > 0 ? GEN : (modk && GEN < 0) ? 1 : 0;
  // window-side vectors kept in LDS rings (direct-four pass 2 also needs v1 for P21; the
  // one-reference pass 4 adds a vector of ones, the modifier's constant term on its window side)
  static constexpr int nvec = PASS <= 1 ? 1 : PASS == 2 ? (D4 ? 3 : 2) : PASS == 3 ? 5
                            : PASS == 4 ? (modk ? 5 : 4) : PASS == 5 ? 2 : 1 + 4 * KS;
  // owned-side values per lane (passes 2 and 5: per owned row of the lane's 4)
  static constexpr int nown = PASS <= 1 ? 1 : PASS == 2 ? 4 : PASS == 3 ? 3 : PASS == 4 ? 5
                            : PASS == 5 ? 8 : 1 + KS;
};

// D4: the direct-four schedule, each staircase plan P^(2,2), P^(2,1), P^(1,1), P^(1,0) from its own
// exponential [technical summaries §2.2: the comparison variant of the adjoint]; passes 0 and 1
// are the same for both schedules.  Its window- and owned-side vectors are the duals and
// cotangents themselves (v1, dv1, v0, u1, du1) instead of the orbit factors.
//
// GEN >= 0: a general tail depth R (a.R) with the vectors of tail_vecs(R) [technical summaries
// §2.1-§2.2: R differentiable tail steps, every staircase plan in the orbit of P^(R,R)]:
//   1 (owns keys)     dV_j = sum_i P dO_i,  dv^(R)_j = sum_i P g = V_j . dV_j   -> F_R (EV_R = 1)
//   2 (owns queries)  du^(R)_i = sum_j P (g - F_R) (given O: delta_i - sum_j P F_R);
//                     column partials sum_i P C_R
//   5 (owns queries)  level a = R-1 .. 1: F_a = -EV_a^2 (partials of level a), finished for the
//                     window on arrival; C_a = -EU_a^2 sum_j P F_a;  column partials sum_i P C_a
//                     for level a - 1
//   6 (owns queries)  dQ_i = s sum_j P M k_j,   7 (owns keys) dK_j = s sum_i P M q_i (and
//                     dV_j = sum_i P dO_i at R = 0), with M = g - sum_k alpha_k(i) beta_k(j)
//                     over the 2 R pairs (alpha, beta) = (EU_a, F_a), (C_a, EV_(a-1)),
//                     a = 1 .. R: a rank-2R product formed per tile on the matrix cores (fp32,
//                     GEN = ceil(2 R / 4) k-steps of 4).
template <typename T, int NT, int NW, int PASS, bool D4 = false, int GEN = -1, bool DELTA = false>
__global__ __launch_bounds__(NW * 64) void vjp_stream_kernel(VjpArgs a) {
  using P = VjpPass<PASS, D4, GEN, DELTA>;
  constexpr int H16 = (NT - 1) / 2;
  constexpr int BR = 16 * NW;                  // owned tokens per block
  constexpr int RING = BR + 32 * H16;          // block window
  constexpr int NTHR = NW * 64;
  constexpr int NV = P::nvec, NO = P::nown;
  constexpr int LS = Lds<T>::stride;
  __shared__ __attribute__((aligned(16))) T ringA[RING * LS];  // S window operand
  __shared__ __attribute__((aligned(16))) T ringB[RING * LS];  // g window operand
  __shared__ __attribute__((aligned(16))) float wv[NV][RING];  // window vectors
  __shared__ float pring[P::writes_part ? RING : 1];
  __shared__ float cpart[P::writes_part ? NW * RING : 1];
  // bf16 one-reference passes 3 and 4: the modifier's window-side factors of each window token,
  // split into high and low bf16 parts, (h0, h1, h2, h3, l0, l1, l2, l3)
  constexpr bool SPLITMOD = P::modk && GEN < 0 && std::is_same<T, bf16>::value;
  __shared__ __attribute__((aligned(16))) bf16x8 wmod[SPLITMOD ? RING : 1];

  const int lane = threadIdx.x & 63, g = lane >> 4, n = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // pairing phase of the wave: waves w and w + 4 of an 8-wave workgroup share a SIMD
  const bool phase = NW == 8 && ((wave >> 2) & 1) != 0;
  const int64_t head = blockIdx.x / a.nseg;
  const int seg = blockIdx.x % a.nseg;
  const int blk0 = seg * a.seg_len, blk1 = min(blk0 + a.seg_len, a.nblk);
  const int halo = 16 * H16;
  const int c_lo = BR * blk0 - halo;
  const int own_lo = BR * blk0, own_hi = BR * blk1;
  const int Lr = a.Lr, h = a.h;
  const float c2 = a.c2, inv_c2 = 1.f / a.c2;
  const int64_t tb = head * (int64_t)Lr * kD;
  const T* winA = static_cast<const T*>(P::owns_keys ? a.Q : a.K) + tb;
  const T* winB = static_cast<const T*>(P::owns_keys ? a.dO : a.V) + tb;
  const T* ownA = static_cast<const T*>(P::owns_keys ? a.K : a.Q) + tb;
  const T* ownB = static_cast<const T*>(P::owns_keys ? a.V : a.dO) + tb;
  const T* ownO = static_cast<const T*>(a.O) + tb;   // delta: the forward's output
  const int64_t vo = head * (int64_t)a.Lpad;
  auto vec = [&](int which) -> float* { return a.ws + which * a.vec_stride + vo; };
  const bool exact_h = (h == 16 * H16);
  const float* part_h = a.part + head * (int64_t)a.nseg * a.pstride;
  // workspace vector indices: the R = 2 layout, or the general-depth layout of tail_vecs(R)
  // (u, v, EU_1..R, EV_0..R, F_1..R, C_1..R)
  const int R = a.R, lev = a.level;
  constexpr bool G = GEN >= 0;
  const int ix_u = G ? 0 : (int)kU2, ix_v = G ? 1 : (int)kV2;
  const int ix_dv = G ? 2 + 3 * R : (int)kDV2;          // F_R = dv^(R)
  const int ix_du = G ? 2 + 4 * R : (int)kDU2;          // C_R = du^(R)
  auto ix_eu = [&](int q) { return 1 + q; };
  auto ix_ev = [&](int b) { return 2 + R + b; };
  auto ix_f = [&](int q) { return 2 + 2 * R + q; };
  auto ix_c = [&](int q) { return 2 + 3 * R + q; };
  // modifier pairs k = 0 .. 2R - 1: alpha (row side) and beta (column side); 0 past 2R
  auto alpha_at = [&](int k, int t) -> float {
    if (k >= 2 * R) return 0.f;
    return vec(k < R ? ix_eu(k + 1) : ix_c(k - R + 1))[t];
  };
  auto beta_at = [&](int k, int t) -> float {
    if (k >= 2 * R) return 0.f;
    return vec(k < R ? ix_f(k + 1) : ix_ev(k - R))[t];
  };

  // ---- window-side vectors of token j: raw loads and a 0/1 weight applied when stored ----
  struct VecIn {
    float v[NV];
    float w;               // token inside the sequence
    float p0, p1, w0, w1;  // passes 3, 5: column partials of the previous pass's segments, weights
    float e;               // pass 5: EV_a of the token
  };
  auto vec_raw = [&](int jc, VecIn& r) {
    if constexpr (PASS == 0) {
      r.v[0] = a.fv[vo + jc];
    } else if constexpr (PASS == 1) {
      r.v[0] = vec(ix_u)[jc];
    } else if constexpr (PASS == 2) {
      r.v[0] = vec(ix_v)[jc];
      r.v[1] = vec(ix_dv)[jc];
      if constexpr (D4) r.v[2 % NV] = vec(kV1)[jc];
    } else if constexpr (PASS == 5) {
      r.v[0] = vec(ix_v)[jc];
      r.v[1 % NV] = 0.f;             // F_a: from the partials when stored
      r.e = vec(ix_ev(lev))[jc];
    } else if constexpr (PASS == 6) {
      r.v[0] = vec(ix_v)[jc];
#pragma unroll
      for (int k = 0; k < 4 * P::KS; ++k) r.v[1 + k] = beta_at(k, jc);
    } else if constexpr (PASS == 7) {
      r.v[0] = vec(ix_u)[jc];
#pragma unroll
      for (int k = 0; k < 4 * P::KS; ++k) r.v[1 + k] = alpha_at(k, jc);
    } else if constexpr (PASS == 3) {
      r.v[0] = vec(kV2)[jc];
      r.v[1] = vec(kDV2)[jc];
      r.v[2] = vec(D4 ? kV1 : kEE)[jc];
      r.v[3] = 0.f;                  // F (dv1 when direct): from the dv1 partials when stored
      r.v[4] = vec(D4 ? kV0 : kEG)[jc];
    } else {
      r.v[0] = vec(kU2)[jc];
      r.v[1] = vec(kDU2)[jc];
      r.v[2] = vec(D4 ? kU1 : kEB)[jc];
      r.v[3] = vec(D4 ? kDU1 : kCC)[jc];
      if constexpr (NV > 4) r.v[4 % NV] = 1.f;
    }
  };
  // any token j (window of the first block): clamped loads, partials found by segment division
  auto vec_loads_any = [&](int j) -> VecIn {
    VecIn r;
    const int jc = min(max(j, 0), Lr - 1);
    vec_raw(jc, r);
    r.w = (j >= 0 && j < Lr) ? 1.f : 0.f;
    r.p0 = r.p1 = r.w0 = r.w1 = 0.f;
    if constexpr (P::reads_part) {
      const int S = BR * a.seg_len;
      const int k0 = max(0, floor_div(jc - halo, S)), k1 = min(a.nseg - 1, floor_div(jc + halo, S));
      float pp[2];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int k = k0 + q, c = jc - (S * k - halo);
        const bool ok = (k <= k1) & (c >= 0) & (c < a.pstride);
        const float x = part_h[(int64_t)min(k, a.nseg - 1) * a.pstride + min(max(c, 0), a.pstride - 1)];
        pp[q] = ok ? x : 0.f;   // an unused slot may hold anything
      }
      r.p0 = pp[0];
      r.p1 = pp[1];
      r.w0 = r.w1 = 1.f;
    }
    return r;
  };
  // token j = cb + RING + t entering with the next block (j > 0).  Inside a segment its first
  // dv1 partial is the segment's own, at offset j - c_lo of its row, and a second one comes from
  // the next segment once j - c_lo reaches S = BR seg_len (no division; the loads never wait).
  auto vec_loads_next = [&](int j) -> VecIn {
    VecIn r;
    const bool in = j < Lr;
    vec_raw(in ? j : Lr - 1, r);
    r.w = in ? 1.f : 0.f;
    r.p0 = r.p1 = r.w0 = r.w1 = 0.f;
    if constexpr (P::reads_part) {
      const int c0 = j - c_lo, c1 = c0 - BR * a.seg_len;
      const bool two = in & (c1 >= 0) & (seg + 1 < a.nseg);
      const int c0i = in ? c0 : 0;      // offset 0 of a segment row is always written
      r.p0 = part_h[(int64_t)seg * a.pstride + c0i];
      r.p1 = part_h[(int64_t)(two ? seg + 1 : seg) * a.pstride + (two ? c1 : c0i)];
      r.w0 = r.w;
      r.w1 = two ? 1.f : 0.f;
    }
    return r;
  };
  auto vec_store = [&](int j, int slot, const VecIn& in) {
#pragma unroll
    for (int k = 0; k < NV; ++k) wv[k][slot] = in.v[k] * in.w;
    if constexpr (SPLITMOD) {
      // pass 3: (D, E, F, 0); pass 4: (A, B, C, 1)
      float m[4];
      if constexpr (PASS == 3) {
        const float E = in.v[2] * in.w;
        m[0] = in.v[1] * in.w;
        m[1] = E;
        m[2] = -E * E * (in.p0 * in.w0 + in.p1 * in.w1);
        m[3] = 0.f;
      } else {
        m[0] = in.v[1] * in.w;
        m[1] = in.v[2] * in.w;
        m[2] = in.v[3] * in.w;
        m[3] = in.w;
      }
      wmod[slot] = split_bf16x4(m);
    }
    if constexpr (PASS == 3 && !D4) {
      const float E = in.v[2] * in.w;
      const float dv1 = -E * (in.p0 * in.w0 + in.p1 * in.w1);
      wv[3][slot] = dv1 * E;                         // F = dv1 e^{dv1}
      if (in.w != 0.f && j >= own_lo && j < own_hi) {
        vec(kDV1)[j] = dv1;
        vec(kFF)[j] = dv1 * E;
      }
    } else if constexpr (PASS == 3) {
      // direct: the partials already hold sum_i P21 du2
      const float dv1 = -(in.p0 * in.w0 + in.p1 * in.w1) * in.w;
      wv[3][slot] = dv1;
      if (in.w != 0.f && j >= own_lo && j < own_hi) vec(kDV1)[j] = dv1;
    } else if constexpr (PASS == 5) {
      // dv^(a) = -EV_a (partials), F_a = dv^(a) EV_a
      const float E = in.e * in.w;
      const float F = -E * E * (in.p0 * in.w0 + in.p1 * in.w1);
      wv[1][slot] = F;
      if (in.w != 0.f && j >= own_lo && j < own_hi) vec(ix_f(lev))[j] = F;
    }
  };

  // ---- owned-side values of the block rows o0 .. o0 + 15 (raw loads), and their prepared
  // form: own[0] (pass 2: own[0..3]) becomes the owned dual / c2 for the accumulator ----
  auto own_loads = [&](int o0, float (&o)[NO]) {
    if constexpr (P::rows_in_regs) {
      const int oc4 = min(o0 + 4 * g, a.Lpad - 4);
      const f32x4 u = load4(vec(ix_u) + oc4);
#pragma unroll
      for (int r = 0; r < 4; ++r) o[r] = u[r];
      if constexpr (PASS == 5) {
        const f32x4 e = load4(vec(ix_eu(lev)) + oc4);
#pragma unroll
        for (int r = 0; r < 4; ++r) o[4 + r] = e[r];
      }
    } else {
      const int oc = min(o0 + n, Lr - 1);
      if constexpr (PASS == 0) {
        o[0] = a.fu[vo + oc];
      } else if constexpr (PASS == 1) {
        o[0] = vec(ix_v)[oc];
      } else if constexpr (PASS == 6) {
        o[0] = vec(ix_u)[oc];
#pragma unroll
        for (int st = 0; st < P::KS; ++st) o[1 + st] = alpha_at(4 * st + g, oc);
      } else if constexpr (PASS == 7) {
        o[0] = vec(ix_v)[oc];
#pragma unroll
        for (int st = 0; st < P::KS; ++st) o[1 + st] = beta_at(4 * st + g, oc);
      } else if constexpr (PASS == 3) {
        o[0] = vec(kU2)[oc];
        o[1] = vec(kDU2)[oc];
        o[2] = vec(D4 ? kU1 : kEB)[oc];
      } else {
        o[0] = vec(kV2)[oc];
        o[1] = vec(kDV2)[oc];
        o[2] = vec(D4 ? kV1 : kEE)[oc];
        o[3] = vec(D4 ? kDV1 : kFF)[oc];
        o[4] = vec(D4 ? kV0 : kEG)[oc];
      }
    }
  };
  auto own_prep = [&](float (&o)[NO]) {
    if constexpr (D4) return;      // direct: plain duals, added to the exponents explicitly
    if constexpr (P::rows_in_regs) {
#pragma unroll
      for (int r = 0; r < 4; ++r) o[r] *= inv_c2;
    } else {
      o[0] *= inv_c2;
    }
    if constexpr (P::modk && GEN < 0 && !SPLITMOD) {
      // owned-side operand of the modifier product for lane group g (k-slot g):
      // pass 3: (1, A_i, B_i, 0) against the window's (D_j, E_j, F_j, G_j);
      // pass 4: (E_j, F_j, G_j, D_j) against the window's (A_i, B_i, C_i, 1)
      if constexpr (PASS == 3) {
        o[1 % NO] = (g == 0) ? 1.f : (g == 1) ? o[1 % NO] : (g == 2) ? o[2 % NO] : 0.f;
      } else {
        o[1 % NO] = (g == 0) ? o[2 % NO] : (g == 1) ? o[3 % NO] : (g == 2) ? o[4 % NO] : o[1 % NO];
      }
    }
  };

  // bf16 one-reference passes 3 and 4: the owned side of the modifier product, negated (the
  // product is added to the g tile) and split: lane group 0 gives (h0..h3, h0..h3) against the
  // window's (h0..h3, l0..l3), lane group 1 (l0..l3, 0..0), lane groups 2 and 3 zeros, so the
  // product sums hw ho + lw ho + hw lo over the four factors.
  // pass 3: (1, A_i, B_i, 0); pass 4: (E_j, F_j, G_j, D_j)
  auto mod_operand = [&](const float (&o)[NO]) -> bf16x8 {
    float m[4];
    if constexpr (PASS == 3) {
      m[0] = -1.f;
      m[1] = -o[1 % NO];
      m[2] = -o[2 % NO];
      m[3] = 0.f;
    } else {
      m[0] = -o[2 % NO];
      m[1] = -o[3 % NO];
      m[2] = -o[4 % NO];
      m[3] = -o[1 % NO];
    }
    const bf16x8 hl = split_bf16x4(m);
    bf16x8 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      r[e] = (g == 0) ? hl[e] : (g == 1) ? hl[4 + e] : (bf16)0.f;
      r[4 + e] = (g == 0) ? hl[e] : (bf16)0.f;
    }
    return r;
  };
  bf16x8 ownmod;

  // ---- prologue: the first block's window, vectors and owned operands ----
  {
    RowStage<T, RING, NTHR> ra, rb;
    ra.load(winA, c_lo, Lr);
    if constexpr (P::uses_ring_b) rb.load(winB, c_lo, Lr);
    ra.template store<RING>(ringA, c_lo);
    if constexpr (P::uses_ring_b) rb.template store<RING>(ringB, c_lo);
  }
  for (int c = threadIdx.x; c < RING; c += NTHR)
    vec_store(c_lo + c, (c_lo + c + 4 * RING) % RING, vec_loads_any(c_lo + c));
  if constexpr (P::writes_part) {
    for (int c = threadIdx.x; c < RING; c += NTHR) pring[c] = 0.f;
    for (int c = threadIdx.x; c < NW * RING; c += NTHR) cpart[c] = 0.f;
  }
  Frag<T> fA, fB;   // owned operands of the score and value-score products
  float own[NO];
  RowPart<T> vj;    // pass 1: V of the owned key, for dv2 = V . dV
  Frag<T> fO;       // delta: O of the owned query (fB holds its dO)
  {
    const int o = BR * blk0 + 16 * wave + n;
    load_frag(fA, ownA + (int64_t)o * kD, o < Lr, g);
    if (P::needs_g || P::delta) load_frag(fB, ownB + (int64_t)o * kD, o < Lr, g);
    if constexpr (P::delta) load_frag(fO, ownO + (int64_t)o * kD, o < Lr, g);
    if constexpr (PASS == 1) vj.load(ownB + (int64_t)min(o, Lr - 1) * kD, g);
    own_loads(BR * blk0 + 16 * wave, own);
    own_prep(own);
    if constexpr (SPLITMOD) ownmod = mod_operand(own);
  }
  __syncthreads();

  // per-lane parts of the LDS addresses
  const T* laneA = ringA + n * LS + 16 * g;
  const T* laneB = ringB + n * LS + 16 * g;
  const TrLane trl(g, n);

  // the block walk, with the pairing phase of this wave fixed for the whole walk
  auto walk = [&](auto phase_c) {
  for (int blk = blk0; blk < blk1; ++blk) {
    const int b0 = BR * blk;
    const int cb = b0 - halo;                  // block window [cb, cb + RING)
    const bool more = blk + 1 < blk1;
    const int s_cb = (cb + RING) % RING;       // ring slot of the window's first token
    auto slot_of = [&](int c) {                // ring slot of window token cb + c, 0 <= c < RING
      const int sl = s_cb + c;
      return (sl >= RING) ? sl - RING : sl;
    };
    // prefetch the next block: its BR new window rows, vectors, owned operands and values
    RowStage<T, BR, NTHR> na, nb;
    VecIn nv;
    Frag<T> fA_next, fB_next, fO_next;
    RowPart<T> vj_next;
    float own_next[NO];
    if (more) {
      if (cb + RING + BR <= Lr) {
        na.load_inside(winA, cb + RING);
        if constexpr (P::uses_ring_b) nb.load_inside(winB, cb + RING);
      } else {
        na.load(winA, cb + RING, Lr);
        if constexpr (P::uses_ring_b) nb.load(winB, cb + RING, Lr);
      }
      if ((int)threadIdx.x < BR) nv = vec_loads_next(cb + RING + (int)threadIdx.x);
      const int on = b0 + BR + 16 * wave + n;
      const bool next_in = (b0 + 2 * BR <= Lr) || (on < Lr);
      load_frag(fA_next, ownA + (int64_t)on * kD, next_in, g);
      if (P::needs_g || P::delta) load_frag(fB_next, ownB + (int64_t)on * kD, next_in, g);
      if constexpr (P::delta) load_frag(fO_next, ownO + (int64_t)on * kD, next_in, g);
      if constexpr (PASS == 1) vj_next.load(ownB + (int64_t)min(on, Lr - 1) * kD, g);
      own_loads(b0 + BR + 16 * wave, own_next);
    }

    const int o0 = b0 + 16 * wave;             // owned tokens o0 .. o0 + 15
    const int cw = o0 - halo;                  // window tiles cw + 16 t
    const int s_cw = slot_of(16 * wave);       // ring slot of tile 0
    auto tile_slot = [&](int t) {
      const int sl = s_cw + 16 * t;
      return (sl >= RING) ? sl - RING : sl;
    };
    const bool interior = exact_h & (cb >= 0) & (cb + RING <= Lr) & (b0 + BR <= Lr);
    // window vector k of the lane's 4 window tokens 4 g + r of the tile at slot rt
    // (indexed as 16-byte groups, so that the read is one ds_read_b128 at a constant offset per
    // vector: tile slots are multiples of 16)
    auto wvec4 = [&](int k, int rt) -> f32x4 {
      return reinterpret_cast<const f32x4*>(&wv[k][0])[(rt >> 2) + g];
    };

    // Score tile t with the owned dual in the accumulator: the exponent of P22 is
    // c2 * sc + (window dual).  Masks: I (interior) needs them only on tiles 0 and NT - 1, along
    // fixed lane patterns; otherwise per entry, and tiles off the band or the sequence are dead.
    auto body = [&](auto interior_c, auto phase_c) {
      constexpr bool I = decltype(interior_c)::value;
      // Pairing phase of the contractions over window-tile pairs: phase 0 pairs tiles (0, 1),
      // (2, 3), ..., phase 1 (0), (1, 2), (3, 4), ...  The two waves that share a SIMD take
      // opposite phases, so one issues its burst of contraction products while the other works
      // on its vector operations.
      constexpr int PH = decltype(phase_c)::value;
      auto zslot = [](int t) { return (t + PH) & 1; };
      auto pair_starts = [&](int t) { return zslot(t) == 0 || t == 0; };
      auto pair_ends = [&](int t) { return zslot(t) == 1 || t == NT - 1; };
      auto dead = [&](int t) -> bool {
        if constexpr (I) return false;
        const int j0 = cw + 16 * t;
        const int dlo = 16 * H16 - 16 * t - 15, dhi = 16 * H16 - 16 * t + 15;
        return (dlo > h) | (dhi < -h) | (j0 >= Lr) | (j0 + 15 < 0) | (o0 >= Lr);
      };
      // window in registers (rows 4 g + r of the tile), owned token o0 + n across lanes
      auto keep_w = [&](int t, int r) -> bool {
        if constexpr (I) return (t == 0) ? (4 * g + r >= n) : (t == NT - 1) ? (4 * g + r <= n) : true;
        const int w = cw + 16 * t + 4 * g + r, o = o0 + n;
        return (w >= 0) & (w < Lr) & (o < Lr) & (abs(w - o) <= h);
      };
      // owned rows o0 + 4 g + r in registers, window token cw + 16 t + n across lanes
      auto keep_o = [&](int t, int r) -> bool {
        if constexpr (I) return (t == 0) ? (4 * g + r <= n) : (t == NT - 1) ? (4 * g + r >= n) : true;
        const int i = o0 + 4 * g + r, j = cw + 16 * t + n;
        return (i < Lr) & (j >= 0) & (j < Lr) & (abs(i - j) <= h);
      };

      // Software pipeline over the strip (kDepth 2: window fragments two tiles ahead and
      // matrix-core products one tile ahead; 1: fragments one tile ahead; 0: none, where the
      // strip itself fills the registers), vector work on the current tile; a scheduling fence
      // per tile keeps the compiler from hoisting every tile's reads (and registers) up front.
#ifndef SKA_VJP_DEPTH
#define SKA_VJP_DEPTH 2
#endif
      constexpr int kDepth = SKA_VJP_DEPTH;
      Frag<T> fw[2], fwg[2];
      f32x4 sc[2], gv[2];
      // window vectors of the tile, read with its fragments (passes 2 and 5: two per lane;
      // passes 6 and 7: the window dual, then the lane's modifier operands, one per k-step)
      constexpr bool MODK = P::modk;
      // MODK: the window dual, the lane's modifier operands, and (pass 3) F and G for du1 and
      // the second dQ contraction
      constexpr int NWV = P::rows_in_regs ? 1 : MODK ? (PASS == 3 ? 4 : 2) : NV;
      f32x4 wb[2][NWV];
      f32x4 md[2];      // passes 6 and 7: modifier tile sum_k alpha_k beta_k, same layout as sc
      bf16x8 wm[2];     // bf16 passes 3 and 4: the window side of the split modifier product
      const f32x4 ci = D4 ? f32x4{0.f, 0.f, 0.f, 0.f}
                   : P::rows_in_regs ? f32x4{own[0], own[1 % NO], own[2 % NO], own[3 % NO]}
                                     : f32x4{own[0], own[0], own[0], own[0]};
      // (fragments of tile t + 2 are read before the vector work on tile t, its window vectors
      // after it: wb[t & 1] still holds tile t's until then)
      auto load_frags = [&](int t) {
        const int rt = tile_slot(t);
        ring_frag(fw[t & 1], ringA, laneA, rt, g, n);
        if constexpr (P::needs_g) ring_frag(fwg[t & 1], ringB, laneB, rt, g, n);
      };
      auto load_vecs = [&](int t) {
        const int rt = tile_slot(t);
        if constexpr (P::rows_in_regs) {
          wb[t & 1][0][0] = wv[0][rt + n];
          wb[t & 1][0][1] = wv[1][rt + n];
          if constexpr (D4) wb[t & 1][0][2] = wv[2 % NV][rt + n];
        } else if constexpr (MODK) {
          wb[t & 1][0] = wvec4(0, rt);
          if constexpr (SPLITMOD) {
            wm[t & 1] = wmod[rt + n];            // A operand: window token n, every lane group
          } else {
            // A operand of k-step st: lane (g, n) gives the tile's window token n, pair 4 st + g
#pragma unroll
            for (int st = 0; st < P::KS; ++st) wb[t & 1][1 % NWV][st] = wv[(1 + 4 * st + g) % NV][rt + n];
          }
          if constexpr (PASS == 3) {
            wb[t & 1][2 % NWV] = wvec4(3, rt);     // F
            wb[t & 1][3 % NWV] = wvec4(4, rt);     // G
          }
        } else {
#pragma unroll
          for (int k = 0; k < NWV; ++k) wb[t & 1][k] = wvec4(k, rt);
        }
      };
      // transposed contraction operands of the pair starting at tile t (fetched at its first
      // tile, used after its second).  A single-tile pair (the first tile at phase 1, the last
      // one where the count is odd) reads its own rows twice against a zero half.
      PairOps<T> opA, opB;
      auto pair_fetch = [&](int t) {
        const int r0 = tile_slot(t), r1 = (zslot(t) == 0 && t + 1 < NT) ? tile_slot(t + 1) : r0;
        if constexpr (PASS == 0 || P::writes_dv) opB.fetch(ringB, trl, r0, r1);
        if constexpr (PASS == 3 || PASS == 4 || PASS == 6 || PASS == 7) opA.fetch(ringA, trl, r0, r1);
      };
      auto mma = [&](int t) {
        if constexpr (P::rows_in_regs) {
          sc[t & 1] = dot_tile(fA, fw[t & 1], ci);
          if constexpr (P::needs_g) gv[t & 1] = dot_tile(fB, fwg[t & 1]);
        } else {
          sc[t & 1] = dot_tile(fw[t & 1], fA, ci);
          if constexpr (SPLITMOD) {
            // g - (modifier) in one accumulator
            gv[t & 1] = dot_tile(fwg[t & 1], fB,
                                 __builtin_amdgcn_mfma_f32_16x16x32_bf16(wm[t & 1], ownmod,
                                                                         f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0));
          } else if constexpr (PASS != 0) {
            gv[t & 1] = dot_tile(fwg[t & 1], fB);
          }
          if constexpr (MODK && !SPLITMOD) {
            // md[r] = sum_k (window token 4 g + r side)_k (owned token n side)_k
            f32x4 m = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int st = 0; st < P::KS; ++st)
              m = __builtin_amdgcn_mfma_f32_16x16x4f32(wb[t & 1][1 % NWV][st], own[(1 + st) % NO], m, 0, 0, 0);
            md[t & 1] = m;
          }
        }
      };
      auto pipeline = [&](auto&& valu) {
        if constexpr (kDepth == 2) {
          load_frags(0);
          load_vecs(0);
          mma(0);
          if (NT > 1) {
            load_frags(1);
            load_vecs(1);
          }
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            if (t + 1 < NT) mma(t + 1);
            if (t + 2 < NT) load_frags(t + 2);
            valu(t, sc[t & 1], gv[t & 1]);
            if (t + 2 < NT) load_vecs(t + 2);
            __builtin_amdgcn_sched_barrier(0);
          }
        } else if constexpr (kDepth == 1) {
          load_frags(0);
          load_vecs(0);
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            if (t + 1 < NT) {
              load_frags(t + 1);
              load_vecs(t + 1);
            }
            mma(t);
            valu(t, sc[t & 1], gv[t & 1]);
            __builtin_amdgcn_sched_barrier(0);
          }
        } else {
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            load_frags(t);
            load_vecs(t);
            mma(t);
            valu(t, sc[t & 1], gv[t & 1]);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      };

      if constexpr (PASS == 0) {
        // ---- O_i = sum_j P22_ij V_j (owned query i across lanes, window keys in registers) ----
        f32x4 Y[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) Y[b] = f32x4{0.f, 0.f, 0.f, 0.f};
        float z[2][4];
        pipeline([&](int t, const f32x4& s, const f32x4&) {
          const int tt = zslot(t);
          if (pair_starts(t)) pair_fetch(t);
          const f32x4 vw = wb[t & 1][0];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float p = fast_exp2(fmaf(s[r], c2, vw[r]));
            z[tt][r] = (keep_w(t, r) && !dead(t)) ? p : 0.f;
          }
          if (pair_ends(t)) {
            if (pair_starts(t)) {
#pragma unroll
              for (int r = 0; r < 4; ++r) z[1 - tt][r] = 0.f;
            }
            opB.contract(Y, ringB, trl, z, g, n);
          }
        });
        if (o0 + n < Lr) store_row(static_cast<T*>(a.out0) + tb + (int64_t)(o0 + n) * kD, Y, 1.f, g);
      } else if constexpr (PASS == 1) {
        // ---- dV_j = sum_i P22_ij dO_i and dv2_j = sum_i P22 g = V_j . dV_j (owned key j across
        // lanes, window queries in registers) ----
        f32x4 Y[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) Y[b] = f32x4{0.f, 0.f, 0.f, 0.f};
        float z[2][4];
        pipeline([&](int t, const f32x4& s, const f32x4&) {
          const int tt = zslot(t);
          if (pair_starts(t)) pair_fetch(t);
          const f32x4 uw = wb[t & 1][0];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float p = fast_exp2(fmaf(s[r], c2, uw[r]));
            z[tt][r] = (keep_w(t, r) && !dead(t)) ? p : 0.f;
          }
          if (pair_ends(t)) {
            if (pair_starts(t)) {
#pragma unroll
              for (int r = 0; r < 4; ++r) z[1 - tt][r] = 0.f;
            }
            opB.contract(Y, ringB, trl, z, g, n);
          }
        });
        float acc = 0.f;
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc = fmaf(vj.at(b, r), Y[b][r], acc);
        const float dv2 = lane_group_sum(acc);
        if (o0 + n < Lr) {
          if (g == 0) vec(ix_dv)[o0 + n] = dv2;
          store_row(static_cast<T*>(a.out1) + tb + (int64_t)(o0 + n) * kD, Y, 1.f, g);
        }
      } else if constexpr (PASS == 2) {
        // ---- du2_i = sum_j P22 (g - dv2_j); column sums of P22 du2 (owned rows in registers) ----
        f32x4 x[NT];
        float racc[4] = {0.f, 0.f, 0.f, 0.f};
        pipeline([&](int t, const f32x4& s, const f32x4& gg) {
          if (dead(t)) {
            x[t] = f32x4{0.f, 0.f, 0.f, 0.f};
            return;
          }
          const float v2j = wb[t & 1][0][0], dj = wb[t & 1][0][1];
          if constexpr (!D4) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float e = fast_exp2(fmaf(s[r], c2, v2j));
              const float p = keep_o(t, r) ? e : 0.f;
              x[t][r] = p;
              racc[r] = P::delta ? fmaf(p, -dj, racc[r]) : fmaf(p, gg[r] - dj, racc[r]);
            }
          } else {
            // direct: du2 from P22, the column sums from P21 = exp(S + u2 + v1)
            const float v1j = wb[t & 1][0][2];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float xs = fmaf(s[r], c2, own[r]);
              const bool keep = keep_o(t, r);
              const float p22 = fast_exp2(xs + v2j), p21 = fast_exp2(xs + v1j);
              x[t][r] = keep ? p21 : 0.f;
              racc[r] = keep ? (P::delta ? fmaf(p22, -dj, racc[r]) : fmaf(p22, gg[r] - dj, racc[r]))
                             : racc[r];
            }
          }
        });
        float du2[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) du2[r] = row16_sum(racc[r]);
        if constexpr (P::delta) {
          // delta of owned row n (fragments: row n, d-slice of lane group g), summed over the
          // lane groups, then moved to the rows_in_regs layout (rows 4 g + r)
          const float dn = lane_group_sum(frag_dot(fB, fO));
#pragma unroll
          for (int r = 0; r < 4; ++r) du2[r] += __shfl(dn, 4 * g + r);
        }
        if (n < 4) {
          const int i = o0 + 4 * g + n;
          const float di = (n == 0) ? du2[0] : (n == 1) ? du2[1] : (n == 2) ? du2[2] : du2[3];
          if (i < Lr) vec(ix_du)[i] = di;
        }
        float cp[NT + 3];
#pragma unroll
        for (int t = 0; t < NT; ++t)
          cp[t] = x[t][0] * du2[0] + x[t][1] * du2[1] + x[t][2] * du2[2] + x[t][3] * du2[3];
#pragma unroll
        for (int t = NT; t < NT + 3; ++t) cp[t] = 0.f;
        // lane group g of a reduced quad (tiles q..q+3) holds tile q + {0, 2, 1, 3}[g]
        const int gsel = (g == 1) ? 2 : (g == 2) ? 1 : g;
#pragma unroll
        for (int q = 0; q < NT; q += 4) {
          const float s4 = swap16_sum(swap32_sum(cp[q], cp[q + 1]), swap32_sum(cp[q + 2], cp[q + 3]));
          const int t = q + gsel;
          if (t < NT) cpart[wave * RING + 16 * wave + 16 * t + n] = s4;
        }
      } else if constexpr (PASS == 3) {
        // ---- du1, dQ (owned query i across lanes, window keys in registers) ----
        const float Ai = own[1 % NO], Bi = own[2 % NO];
        float acc = 0.f;
        f32x4 X[4], Y[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) X[b] = Y[b] = f32x4{0.f, 0.f, 0.f, 0.f};
        float z1[2][4], z2[2][4];
        pipeline([&](int t, const f32x4& s, const f32x4& gg) {
          const int tt = zslot(t);
          if (pair_starts(t)) pair_fetch(t);
          const bool live = !dead(t);
          if constexpr (!D4) {
            // md = D_j + A_i E_j + B_i F_j from the matrix cores
            const f32x4 vw = wb[t & 1][0], Fw = wb[t & 1][2 % NWV], Gw = wb[t & 1][3 % NWV],
                        mm = md[t & 1];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float e = fast_exp2(fmaf(s[r], c2, vw[r]));
              const float p = (keep_w(t, r) && live) ? e : 0.f;
              acc = fmaf(p, Fw[r], acc);
              z1[tt][r] = SPLITMOD ? p * gg[r] : p * (gg[r] - mm[r]);
              z2[tt][r] = p * Gw[r];
            }
          } else {
            const f32x4 vw = wb[t & 1][0], Dw = wb[t & 1][1 % NWV], Ew = wb[t & 1][2 % NWV],
                        Fw = wb[t & 1][3 % NWV], Gw = wb[t & 1][4 % NWV];
            // direct: Ai = du2, Bi = u1 of the owned query; window E = v1, F = dv1, G = v0
            const float u2i = own[0];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float xs = s[r] * c2;
              const float p22 = fast_exp2(xs + u2i + vw[r]), p21 = fast_exp2(xs + u2i + Ew[r]);
              const float p11 = fast_exp2(xs + Bi + Ew[r]), p10 = fast_exp2(xs + Bi + Gw[r]);
              const bool keep = keep_w(t, r) && live;
              acc = keep ? fmaf(p11, Fw[r], acc) : acc;
              z1[tt][r] = keep ? p22 * (gg[r] - Dw[r]) - p21 * Ai - p11 * Fw[r] : 0.f;
              z2[tt][r] = keep ? p10 : 0.f;
            }
          }
          if (pair_ends(t)) {
            if (pair_starts(t)) {
#pragma unroll
              for (int r = 0; r < 4; ++r) z1[1 - tt][r] = z2[1 - tt][r] = 0.f;
            }
            opA.contract2(X, Y, ringA, trl, z1, z2, g, n);
          }
        });
        // one-reference: du1 = -B sum P22 E F, coefficient of Z2 is C = du1 B;
        // direct: du1 = -sum P11 dv1, coefficient du1 (C = du1 e^{du1} is not needed)
        const float du1 = D4 ? -lane_group_sum(acc) : -Bi * lane_group_sum(acc);
        const float Ci = D4 ? du1 : du1 * Bi;
        if (o0 + n < Lr) {
          if (g == 0) {
            vec(kDU1)[o0 + n] = du1;
            if constexpr (!D4) vec(kCC)[o0 + n] = Ci;
          }
          f32x4 r4[4];
#pragma unroll
          for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int r = 0; r < 4; ++r) r4[b][r] = X[b][r] - Ci * Y[b][r];
          store_row(static_cast<T*>(a.out0) + tb + (int64_t)(o0 + n) * kD, r4, a.s, g);
        }
      } else if constexpr (PASS == 4) {
        // ---- dK (owned key j across lanes, window queries in registers) ----
        const float Dj = own[1 % NO], Ej = own[2 % NO], Fj = own[3 % NO], Gj = own[4 % NO];
        f32x4 X[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) X[b] = f32x4{0.f, 0.f, 0.f, 0.f};
        float z1[2][4];
        pipeline([&](int t, const f32x4& s, const f32x4& gg) {
          const int tt = zslot(t);
          if (pair_starts(t)) pair_fetch(t);
          const f32x4 uw = wb[t & 1][0];
          const bool live = !dead(t);
          if constexpr (!D4) {
            // md = D_j + A_i E_j + B_i F_j + C_i G_j from the matrix cores
            const f32x4 mm = md[t & 1];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float e = fast_exp2(fmaf(s[r], c2, uw[r]));
              const float p = (keep_w(t, r) && live) ? e : 0.f;
              z1[tt][r] = SPLITMOD ? p * gg[r] : p * (gg[r] - mm[r]);
            }
          } else {
            const f32x4 Aw = wb[t & 1][1 % NWV], Bw = wb[t & 1][2 % NWV], Cw = wb[t & 1][3 % NWV];
            // direct: owned D = dv2, E = v1, F = dv1, G = v0; window A = du2, B = u1, C = du1
            const float v2j = own[0];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float xs = s[r] * c2;
              const float p22 = fast_exp2(xs + uw[r] + v2j), p21 = fast_exp2(xs + uw[r] + Ej);
              const float p11 = fast_exp2(xs + Bw[r] + Ej), p10 = fast_exp2(xs + Bw[r] + Gj);
              const bool keep = keep_w(t, r) && live;
              z1[tt][r] = keep ? p22 * (gg[r] - Dj) - p21 * Aw[r] - p11 * Fj - p10 * Cw[r] : 0.f;
            }
          }
          if (pair_ends(t)) {
            if (pair_starts(t)) {
#pragma unroll
              for (int r = 0; r < 4; ++r) z1[1 - tt][r] = 0.f;
            }
            opA.contract(X, ringA, trl, z1, g, n);
          }
        });
        if (o0 + n < Lr) store_row(static_cast<T*>(a.out0) + tb + (int64_t)(o0 + n) * kD, X, a.s, g);
      } else if constexpr (PASS == 5) {
        // ---- level a: C_a = -EU_a^2 sum_j P F_a; column sums of P C_a (owned rows in
        // registers) ----
        f32x4 x[NT];
        float racc[4] = {0.f, 0.f, 0.f, 0.f};
        pipeline([&](int t, const f32x4& s, const f32x4&) {
          if (dead(t)) {
            x[t] = f32x4{0.f, 0.f, 0.f, 0.f};
            return;
          }
          const float v2j = wb[t & 1][0][0], fj = wb[t & 1][0][1];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float e = fast_exp2(fmaf(s[r], c2, v2j));
            const float p = keep_o(t, r) ? e : 0.f;
            x[t][r] = p;
            racc[r] = fmaf(p, fj, racc[r]);
          }
        });
        float ca[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) ca[r] = -own[4 + r] * own[4 + r] * row16_sum(racc[r]);
        if (n < 4) {
          const int i = o0 + 4 * g + n;
          const float ci_ = (n == 0) ? ca[0] : (n == 1) ? ca[1] : (n == 2) ? ca[2] : ca[3];
          if (i < Lr) vec(ix_c(lev))[i] = ci_;
        }
        if (lev > 1) {
          float cp[NT + 3];
#pragma unroll
          for (int t = 0; t < NT; ++t)
            cp[t] = x[t][0] * ca[0] + x[t][1] * ca[1] + x[t][2] * ca[2] + x[t][3] * ca[3];
#pragma unroll
          for (int t = NT; t < NT + 3; ++t) cp[t] = 0.f;
          const int gsel = (g == 1) ? 2 : (g == 2) ? 1 : g;
#pragma unroll
          for (int q = 0; q < NT; q += 4) {
            const float s4 = swap16_sum(swap32_sum(cp[q], cp[q + 1]), swap32_sum(cp[q + 2], cp[q + 3]));
            const int t = q + gsel;
            if (t < NT) cpart[wave * RING + 16 * wave + 16 * t + n] = s4;
          }
        }
      } else if constexpr (PASS == 6) {
        // ---- dQ with the general modifier (owned query i across lanes, window keys in
        // registers) ----
        f32x4 X[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) X[b] = f32x4{0.f, 0.f, 0.f, 0.f};
        float z[2][4];
        pipeline([&](int t, const f32x4& s, const f32x4& gg) {
          const int tt = zslot(t);
          if (pair_starts(t)) pair_fetch(t);
          const f32x4 vw = wb[t & 1][0], mm = md[t & 1];
          const bool live = !dead(t);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float e = fast_exp2(fmaf(s[r], c2, vw[r]));
            const float p = (keep_w(t, r) && live) ? e : 0.f;
            z[tt][r] = p * (gg[r] - mm[r]);
          }
          if (pair_ends(t)) {
            if (pair_starts(t)) {
#pragma unroll
              for (int r = 0; r < 4; ++r) z[1 - tt][r] = 0.f;
            }
            opA.contract(X, ringA, trl, z, g, n);
          }
        });
        if (o0 + n < Lr) store_row(static_cast<T*>(a.out0) + tb + (int64_t)(o0 + n) * kD, X, a.s, g);
      } else {
        // ---- dK with the general modifier, and dV at R = 0 (owned key j across lanes, window
        // queries in registers) ----
        constexpr bool DV = P::writes_dv;
        f32x4 X[4], Y[DV ? 4 : 1];
#pragma unroll
        for (int b = 0; b < 4; ++b) X[b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int b = 0; b < (DV ? 4 : 1); ++b) Y[b] = f32x4{0.f, 0.f, 0.f, 0.f};
        float z1[2][4], z2[2][4];
        pipeline([&](int t, const f32x4& s, const f32x4& gg) {
          const int tt = zslot(t);
          if (pair_starts(t)) pair_fetch(t);
          const f32x4 uw = wb[t & 1][0], mm = md[t & 1];
          const bool live = !dead(t);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float e = fast_exp2(fmaf(s[r], c2, uw[r]));
            const float p = (keep_w(t, r) && live) ? e : 0.f;
            z1[tt][r] = p * (gg[r] - mm[r]);
            z2[tt][r] = p;
          }
          if (pair_ends(t)) {
            if (pair_starts(t)) {
#pragma unroll
              for (int r = 0; r < 4; ++r) z1[1 - tt][r] = z2[1 - tt][r] = 0.f;
            }
            opA.contract(X, ringA, trl, z1, g, n);
            if constexpr (DV) opB.contract(Y, ringB, trl, z2, g, n);
          }
        });
        if (o0 + n < Lr) {
          store_row(static_cast<T*>(a.out0) + tb + (int64_t)(o0 + n) * kD, X, a.s, g);
          if constexpr (DV) store_row(static_cast<T*>(a.out1) + tb + (int64_t)(o0 + n) * kD, Y, 1.f, g);
        }
      }
    };
    if (interior) {
      body(std::true_type{}, phase_c);
    } else {
      body(std::false_type{}, std::integral_constant<int, 0>{});
    }

    __syncthreads();   // every wave is done with this block's window
    if constexpr (P::writes_part) {
      if (PASS == 2 || lev > 1) {
        // block column sums (fixed wave order) into the segment accumulator; columns [cb, cb + BR)
        // leave the window with this block and are written out
        float* out = (PASS == 5 ? a.part_out : a.part) + (head * (int64_t)a.nseg + seg) * a.pstride +
                     (cb - c_lo);
        for (int c = threadIdx.x; c < RING; c += NTHR) {
          float sacc = 0.f;
#pragma unroll
          for (int w = 0; w < NW; ++w) sacc += cpart[w * RING + c];
          const int slot = slot_of(c);
          if (!more) {
            out[c] = pring[slot] + sacc;
          } else if (c < BR) {
            out[c] = pring[slot] + sacc;
            pring[slot] = 0.f;
          } else {
            pring[slot] += sacc;
          }
        }
      }
    }
    if (more) {
      if ((int)threadIdx.x < BR) vec_store(cb + RING + (int)threadIdx.x, slot_of(threadIdx.x), nv);
      na.template store_slots<RING>(ringA, s_cb);
      if constexpr (P::uses_ring_b) nb.template store_slots<RING>(ringB, s_cb);
      fA = fA_next;
      fB = fB_next;
      if constexpr (P::delta) fO = fO_next;
      if constexpr (PASS == 1) vj = vj_next;
      own_prep(own_next);
#pragma unroll
      for (int k = 0; k < NO; ++k) own[k] = own_next[k];
      if constexpr (SPLITMOD) ownmod = mod_operand(own);
      __syncthreads();
    }
  }
  };
  if (P::contracts && phase) walk(std::integral_constant<int, 1>{});
  else walk(std::integral_constant<int, 0>{});
}

template <typename T, int NT, int NW>
static void launch_nt_general(int pass, const VjpArgs& a, hipStream_t st) {
  const dim3 grid((unsigned)(a.bh * (int64_t)a.nseg)), block(NW * 64);
  const int ks = (2 * a.R + 3) / 4;          // modifier k-steps of passes 6 and 7
  switch (pass) {
    case 1: vjp_stream_kernel<T, NT, NW, 1, false, 0><<<grid, block, 0, st>>>(a); break;
    case 2:
      if (a.O != nullptr) vjp_stream_kernel<T, NT, NW, 2, false, 0, true><<<grid, block, 0, st>>>(a);
      else vjp_stream_kernel<T, NT, NW, 2, false, 0><<<grid, block, 0, st>>>(a);
      break;
    case 5: vjp_stream_kernel<T, NT, NW, 5, false, 0><<<grid, block, 0, st>>>(a); break;
    case 6:
      if (ks == 0) vjp_stream_kernel<T, NT, NW, 6, false, 0><<<grid, block, 0, st>>>(a);
      else if (ks == 1) vjp_stream_kernel<T, NT, NW, 6, false, 1><<<grid, block, 0, st>>>(a);
      else vjp_stream_kernel<T, NT, NW, 6, false, 2><<<grid, block, 0, st>>>(a);
      break;
    default:
      if (ks == 0) vjp_stream_kernel<T, NT, NW, 7, false, 0><<<grid, block, 0, st>>>(a);
      else if (ks == 1) vjp_stream_kernel<T, NT, NW, 7, false, 1><<<grid, block, 0, st>>>(a);
      else vjp_stream_kernel<T, NT, NW, 7, false, 2><<<grid, block, 0, st>>>(a);
      break;
  }
}

template <typename T, int NT, int NW>
static void launch_nt(int pass, bool d4, const VjpArgs& a, hipStream_t st) {
  const dim3 grid((unsigned)(a.bh * (int64_t)a.nseg)), block(NW * 64);
  switch (pass) {
    case 0: vjp_stream_kernel<T, NT, NW, 0><<<grid, block, 0, st>>>(a); break;
    case 1: vjp_stream_kernel<T, NT, NW, 1><<<grid, block, 0, st>>>(a); break;
    case 2:
      if (a.O != nullptr) {
        if (d4) vjp_stream_kernel<T, NT, NW, 2, true, -1, true><<<grid, block, 0, st>>>(a);
        else vjp_stream_kernel<T, NT, NW, 2, false, -1, true><<<grid, block, 0, st>>>(a);
      } else {
        if (d4) vjp_stream_kernel<T, NT, NW, 2, true><<<grid, block, 0, st>>>(a);
        else vjp_stream_kernel<T, NT, NW, 2><<<grid, block, 0, st>>>(a);
      }
      break;
    case 3:
      if (d4) vjp_stream_kernel<T, NT, NW, 3, true><<<grid, block, 0, st>>>(a);
      else vjp_stream_kernel<T, NT, NW, 3><<<grid, block, 0, st>>>(a);
      break;
    default:
      if (d4) vjp_stream_kernel<T, NT, NW, 4, true><<<grid, block, 0, st>>>(a);
      else vjp_stream_kernel<T, NT, NW, 4><<<grid, block, 0, st>>>(a);
      break;
  }
}

hipError_t launch_vjp_stream_general(int elt, int nt, int nw, int pass, const VjpArgs& a,
                                     hipStream_t st) {
  if (a.R < 0 || a.R > kTailMaxR || (pass != 1 && pass != 2 && pass != 5 && pass != 6 && pass != 7))
    return hipErrorInvalidValue;
  if ((pass == 6 || pass == 7) && a.R > kStreamMaxR) return hipErrorInvalidValue;
  if ((pass == 1 || pass == 2) && a.R < 1) return hipErrorInvalidValue;
  if (pass == 5 && (a.level < 1 || a.level >= a.R)) return hipErrorInvalidValue;
  if (elt == 1) {
    if (nt == 5) launch_nt_general<bf16, 5, kBf16StreamWaves>(pass, a, st);
    else if (nt == 9) launch_nt_general<bf16, 9, kBf16StreamWaves>(pass, a, st);
    else launch_nt_general<bf16, 17, kBf16StreamWaves>(pass, a, st);
  } else {
    if (nt == 5) launch_nt_general<float, 5, 4>(pass, a, st);
    else launch_nt_general<float, 9, 4>(pass, a, st);
  }
  return hipGetLastError();
}

hipError_t launch_vjp_stream_pass(int elt, int nt, int nw, int pass, bool d4, const VjpArgs& a,
                                  hipStream_t st) {
  if (elt == 1) {
    if (nt == 5) launch_nt<bf16, 5, kBf16StreamWaves>(pass, d4, a, st);
    else if (nt == 9) launch_nt<bf16, 9, kBf16StreamWaves>(pass, d4, a, st);
    else launch_nt<bf16, 17, kBf16StreamWaves>(pass, d4, a, st);
  } else {
    if (nt == 5) launch_nt<float, 5, 4>(pass, d4, a, st);
    else launch_nt<float, 9, 4>(pass, d4, a, st);
  }
  return hipGetLastError();
}

}  // namespace ska
