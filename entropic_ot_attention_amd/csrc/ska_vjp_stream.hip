// Streaming passes of the forward output and of the exact R = 2 tail VJP, one-reference-tile
// schedule (gfx950).
//
// The adjoint [abstract: the R = 2 score cotangent is the reference plan tile times a modifier
// field of vector cotangents and dual differences; technical summaries §2.2: orbit equation
// P^(a,b) = P^(2,2) exp(u^(a) - u^(2)) exp(v^(b) - v^(2))], with P22 = exp(S + u2 + v2),
// g_ij = dO_i . V_j and e^{du1} = exp(u1 - u2), e^{dv_b} = exp(v_b - v2), in four passes:
//
//   0 (owns queries)  forward output O_i = sum_j P22_ij V_j   [spec output: plan x V]
//   1 (owns keys)     dv2_j = sum_i P22 g
//   2 (owns queries)  du2_i = sum_j P22 (g - dv2_j);  per-segment column sums sum_i P22 du2_i
//   3 (owns queries)  dv1_j = -e^{dv1_j} (column sums)  (finished for the window on arrival)
//                     du1_i = -e^{du1_i} sum_j P22 e^{dv1_j} dv1_j
//                     dQ_i  = s sum_j dS_ij k_j,  dS = Z1 - C_i Z2 with
//                             Z1 = P22 (g - D_j - A_i E_j - B_i F_j), Z2 = P22 G_j
//   4 (owns keys)     dK_j = s sum_i dS_ij q_i,  dS = P22 (g - D_j - A_i E_j - B_i F_j - C_i G_j)
//                     dV_j = sum_i P22_ij dO_i
// (A = du2, B = e^{du1}, C = du1 e^{du1}, D = dv2, E = e^{dv1}, F = dv1 e^{dv1}, G = e^{dv0}).
//
// Work decomposition as in the fused forward step: a workgroup of NW waves walks a segment of
// consecutive blocks of 16 NW owned tokens; the band window of the block (16 NW + 32 H16
// tokens) of the two window-side tensors lives in LDS rings, each block brings in only its 16 NW
// new rows (loaded one block ahead), and the window-side vectors live in rings alongside.
// Pass 2 keeps its 16 x (16 + 32 H16) reference-plan strip in registers (owned rows in lane
// registers, keys across lanes) so the column sums need du2, known only after the sweep; passes
// 1, 3 and 4 put the window in lane registers and the owned tokens across lanes, so sums over
// the window stay in-lane and contractions over the window feed the matrix cores directly, the
// other operand read transposed from its LDS ring.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "ska_device.h"
#include "ska_internal.h"

namespace ska {

// Transposing LDS read (ds_read_b64_tr_b16): within each 16-lane row, lane i receives element
// i % 4 of the 8 bytes loaded by lane i / 4 + 4 e, as its element e.  With lane (g, n) loading
// ring row rb + 4 g + n / 4 at columns c0 + 4 (n % 4) .. + 3, lane (g, n) receives rows
// rb + 4 g + e (e = 0..3) of column c0 + n: one half of a bf16 MFMA A operand of the
// transposed ring rows.
typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ s16x4 tr_read(const bf16* ring, int row, int col) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (s16x4 __attribute__((address_space(3)))*)(ring + row * Lds<bf16>::stride + col));
}
__device__ __forceinline__ bf16x8 tr_operand(const bf16* ring, int rb0, int rb1, int b, int g, int n) {
  const int r = 4 * g + (n >> 2), c = 16 * b + 4 * (n & 3);
  const s16x4 lo = tr_read(ring, rb0 + r, c), hi = tr_read(ring, rb1 + r, c);
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

// acc[b][r] (lane l) += sum over the 32 window rows of tiles (rb0, rb1) of
//   Op[row][16 b + 4 g + r] * Z[row][n]    (Op rows read transposed from the LDS ring)
// z[tt][r] holds Z for row rb_tt + 4 g + r at owned token n.
__device__ __forceinline__ bf16x8 pack_z(const float (&z)[2][4]) {
  bf16x8 zb;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    zb[e] = (bf16)z[0][e];
    zb[e + 4] = (bf16)z[1][e];
  }
  return zb;
}
__device__ __forceinline__ void contract_ring(f32x4 (&acc)[4], const bf16* ring, int rb0, int rb1,
                                              const float (&z)[2][4], int g, int n) {
  const bf16x8 zb = pack_z(z);
#pragma unroll
  for (int b = 0; b < 4; ++b)
    acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(tr_operand(ring, rb0, rb1, b, g, n), zb, acc[b], 0, 0, 0);
}
// Two contractions against the same ring rows (shares the transposed reads).
__device__ __forceinline__ void contract_ring2(f32x4 (&x)[4], f32x4 (&y)[4], const bf16* ring, int rb0,
                                               int rb1, const float (&z1)[2][4],
                                               const float (&z2)[2][4], int g, int n) {
  const bf16x8 zb1 = pack_z(z1), zb2 = pack_z(z2);
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const bf16x8 av = tr_operand(ring, rb0, rb1, b, g, n);
    x[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, zb1, x[b], 0, 0, 0);
    y[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, zb2, y[b], 0, 0, 0);
  }
}
__device__ __forceinline__ void contract_ring(f32x4 (&acc)[4], const float* ring, int rb0, int rb1,
                                              const float (&z)[2][4], int g, int n) {
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = (tt == 0 ? rb0 : rb1) + 4 * g + r;
#pragma unroll
      for (int b = 0; b < 4; ++b)
        acc[b] = __builtin_amdgcn_mfma_f32_16x16x4f32(ring[row * Lds<float>::stride + 16 * b + n],
                                                      z[tt][r], acc[b], 0, 0, 0);
    }
}

__device__ __forceinline__ void contract_ring2(f32x4 (&x)[4], f32x4 (&y)[4], const float* ring,
                                               int rb0, int rb1, const float (&z1)[2][4],
                                               const float (&z2)[2][4], int g, int n) {
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = (tt == 0 ? rb0 : rb1) + 4 * g + r;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const float av = ring[row * Lds<float>::stride + 16 * b + n];
        x[b] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, z1[tt][r], x[b], 0, 0, 0);
        y[b] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, z2[tt][r], y[b], 0, 0, 0);
      }
    }
}

template <int PASS> struct VjpPass {
  static constexpr bool owns_keys = (PASS == 1 || PASS == 4);
  // window-side vectors kept in LDS rings
  static constexpr int nvec = PASS <= 1 ? 1 : PASS == 2 ? 2 : PASS == 3 ? 5 : 4;
};

template <typename T, int NT, int NW, int PASS>
struct VjpSmem {
  static constexpr int kH16 = (NT - 1) / 2;
  static constexpr int kBR = 16 * NW;
  static constexpr int kRing = kBR + 32 * kH16;
};

template <typename T, int NT, int NW, int PASS>
__global__ __launch_bounds__(NW * 64) void vjp_stream_kernel(VjpArgs a) {
  using P = VjpPass<PASS>;
  constexpr int H16 = (NT - 1) / 2;
  constexpr int BR = 16 * NW;                  // owned tokens per block
  constexpr int RING = BR + 32 * H16;          // block window
  constexpr int NTHR = NW * 64;
  constexpr int NV = P::nvec;
  constexpr int NP = (NT + 1) / 2;             // tile pairs of a contraction
  __shared__ __attribute__((aligned(16))) T ringA[RING * Lds<T>::stride];  // S window operand
  __shared__ __attribute__((aligned(16))) T ringB[RING * Lds<T>::stride];  // g window operand
  __shared__ float wv[NV][RING];                                          // window vectors
  __shared__ float pring[PASS == 2 ? RING : 1];
  __shared__ float cpart[PASS == 2 ? NW * RING : 1];

  const int lane = threadIdx.x & 63, g = lane >> 4, n = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t head = blockIdx.x / a.nseg;
  const int seg = blockIdx.x % a.nseg;
  const int blk0 = seg * a.seg_len, blk1 = min(blk0 + a.seg_len, a.nblk);
  const int c_lo = BR * blk0 - 16 * H16;
  const int own_lo = BR * blk0, own_hi = BR * blk1;
  const int Lr = a.Lr, h = a.h;
  const int64_t tb = head * (int64_t)Lr * kD;
  const T* winA = static_cast<const T*>(P::owns_keys ? a.Q : a.K) + tb;
  const T* winB = static_cast<const T*>(P::owns_keys ? a.dO : a.V) + tb;
  const T* ownA = static_cast<const T*>(P::owns_keys ? a.K : a.Q) + tb;
  const T* ownB = static_cast<const T*>(P::owns_keys ? a.V : a.dO) + tb;
  const int64_t vo = head * (int64_t)a.Lpad;
  auto vec = [&](int which) -> float* { return a.ws + which * a.vec_stride + vo; };
  const bool exact_h = (h == 16 * H16);

  // window-side vector entry k of token j (0 outside the sequence)
  auto window_vec = [&](int k, int j) -> float {
    const int jc = min(max(j, 0), Lr - 1);
    float x;
    if (PASS == 0) x = a.fv[vo + jc];
    else if (PASS == 1) x = vec(kU2)[jc];
    else if (PASS == 2) x = (k == 0) ? vec(kV2)[jc] : vec(kDV2)[jc];
    else if (PASS == 3) {
      const int src[5] = {kV2, kDV2, kEE, kFF, kEG};
      x = vec(src[k])[jc];
    } else {
      const int src[4] = {kU2, kDU2, kEB, kCC};
      x = vec(src[k])[jc];
    }
    return (j >= 0 && j < Lr) ? x : 0.f;
  };
  // pass 3: finished dv1 of key j from the pass-2 segment column sums; the owner stores dv1, F
  const float* part_h = a.part + head * (int64_t)a.nseg * a.pstride;
  auto dv1_loads = [&](int j, float& p0, float& p1, float& e) {
    const int S = BR * a.seg_len, halo = 16 * H16;
    const int jc = min(max(j, 0), Lr - 1);
    const int k0 = max(0, floor_div(jc - halo, S)), k1 = min(a.nseg - 1, floor_div(jc + halo, S));
    float pp[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int k = k0 + q, c = jc - (S * k - halo);
      const bool ok = (k <= k1) & (c >= 0) & (c < a.pstride);
      const float x = part_h[(int64_t)min(k, a.nseg - 1) * a.pstride + min(max(c, 0), a.pstride - 1)];
      pp[q] = ok ? x : 0.f;
    }
    p0 = pp[0];
    p1 = pp[1];
    e = vec(kEE)[jc];
  };
  // loads of the NV window vectors of token j (pass 3 computes F from the dv1 partials)
  struct VecIn {
    float v[NV];
    float p0, p1;
  };
  auto vec_loads = [&](int j) -> VecIn {
    VecIn r;
#pragma unroll
    for (int k = 0; k < NV; ++k) r.v[k] = window_vec(k, j);
    r.p0 = r.p1 = 0.f;
    if (PASS == 3) {
      float e;
      dv1_loads(j, r.p0, r.p1, e);
    }
    return r;
  };
  auto vec_store = [&](int j, const VecIn& in) {
    const int slot = (j + 4 * RING) % RING;
#pragma unroll
    for (int k = 0; k < NV; ++k) wv[k][slot] = in.v[k];
    if (PASS == 3) {
      const bool ok = (j >= 0 && j < Lr);
      const float E = in.v[2];
      const float dv1 = ok ? -E * (in.p0 + in.p1) : 0.f;
      wv[3][slot] = dv1 * E;                         // F = dv1 e^{dv1}
      if (ok && j >= own_lo && j < own_hi) {
        vec(kDV1)[j] = dv1;
        vec(kFF)[j] = dv1 * E;
      }
    }
  };

  // ---- prologue: the first block's window, vectors and owned operands ----
  {
    RowStage<T, RING, NTHR> ra, rb;
    ra.load(winA, c_lo, Lr);
    rb.load(winB, c_lo, Lr);
    ra.template store<RING>(ringA, c_lo);
    rb.template store<RING>(ringB, c_lo);
  }
  for (int c = threadIdx.x; c < RING; c += NTHR) vec_store(c_lo + c, vec_loads(c_lo + c));
  if (PASS == 2) {
    for (int c = threadIdx.x; c < RING; c += NTHR) pring[c] = 0.f;
    for (int c = threadIdx.x; c < NW * RING; c += NTHR) cpart[c] = 0.f;
  }
  Frag<T> fA, fB;   // owned operands of the score and value-score products
  {
    const int o = BR * blk0 + 16 * wave + n;
    load_frag(fA, ownA + (int64_t)o * kD, o < Lr, g);
    if (PASS != 0) load_frag(fB, ownB + (int64_t)o * kD, o < Lr, g);
  }
  __syncthreads();

  for (int blk = blk0; blk < blk1; ++blk) {
    const int b0 = BR * blk;
    const int cb = b0 - 16 * H16;              // block window [cb, cb + RING)
    const bool more = blk + 1 < blk1;
    // prefetch the next block: its BR new window rows, vectors and owned operands
    RowStage<T, BR, NTHR> na, nb;
    VecIn nv;
    Frag<T> fA_next, fB_next;
    if (more) {
      na.load(winA, cb + RING, Lr);
      nb.load(winB, cb + RING, Lr);
      if ((int)threadIdx.x < BR) nv = vec_loads(cb + RING + (int)threadIdx.x);
      const int on = b0 + BR + 16 * wave + n;
      load_frag(fA_next, ownA + (int64_t)on * kD, on < Lr, g);
      if (PASS != 0) load_frag(fB_next, ownB + (int64_t)on * kD, on < Lr, g);
    }

    const int o0 = b0 + 16 * wave;             // owned tokens o0 .. o0 + 15
    const int cw = o0 - 16 * H16;              // window tiles cw + 16 t
    const bool interior = exact_h & (cb >= 0) & (cb + RING <= Lr) & (b0 + BR <= Lr);
    auto tile_row = [&](int t) -> int { return (cw + 16 * t + 4 * RING) % RING; };
    auto dead_tile = [&](int t) -> bool {
      const int j0 = cw + 16 * t;
      const int dlo = 16 * H16 - 16 * t - 15, dhi = 16 * H16 - 16 * t + 15;
      return (dlo > h) | (dhi < -h) | (j0 >= Lr) | (j0 + 15 < 0) | (o0 >= Lr);
    };
    // band/sequence mask of a window-in-registers entry (window token w = cw + 16t + 4g + r,
    // owned token o0 + n) and of an owned-in-registers entry (owned o0 + 4g + r, window
    // cw + 16t + n); on interior blocks only tiles 0 and NT - 1 are partial, along fixed lanes
    auto keep_w = [&](int t, int r) -> bool {
      if (interior) return (t == 0) ? (4 * g + r >= n) : (t == NT - 1) ? (4 * g + r <= n) : true;
      const int w = cw + 16 * t + 4 * g + r, o = o0 + n;
      return (w >= 0) & (w < Lr) & (o < Lr) & (abs(w - o) <= h);
    };
    auto keep_o = [&](int t, int r) -> bool {
      if (interior) return (t == 0) ? (4 * g + r <= n) : (t == NT - 1) ? (4 * g + r >= n) : true;
      const int i = o0 + 4 * g + r, j = cw + 16 * t + n;
      return (i < Lr) & (j >= 0) & (j < Lr) & (abs(i - j) <= h);
    };

    if (PASS == 0) {
      // ---- O_i = sum_j P22_ij V_j (owned query i across lanes, window keys in registers) ----
      const float u2o = a.fu[vo + min(o0 + n, Lr - 1)];
      f32x4 Y[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) Y[b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int pq = 0; pq < NP; ++pq) {
        float z[2][4];
        int rbs[2];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          const int t = 2 * pq + tt;
          rbs[tt] = (t < NT) ? tile_row(t) : tile_row(2 * pq);
#pragma unroll
          for (int r = 0; r < 4; ++r) z[tt][r] = 0.f;
          if (t >= NT || dead_tile(t)) continue;
          const int rr = rbs[tt];
          Frag<T> fw;
          lds_frag(fw, ringA, rr + n, g);
          const f32x4 sc = dot_tile(fw, fA);
#pragma unroll
          for (int r = 0; r < 4; ++r)
            z[tt][r] = keep_w(t, r) ? fast_exp2(fmaf(sc[r], a.c2, u2o + wv[0][rr + 4 * g + r])) : 0.f;
        }
        contract_ring(Y, ringB, rbs[0], rbs[1], z, g, n);
      }
      if (o0 + n < Lr) store_row(static_cast<T*>(a.out0) + tb + (int64_t)(o0 + n) * kD, Y, 1.f, g);
    } else if (PASS == 1) {
      // ---- dv2_j = sum_i P22 g (owned key j across lanes, window queries in registers) ----
      const float v2o = vec(kV2)[min(o0 + n, Lr - 1)];
      float acc = 0.f;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        if (dead_tile(t)) continue;
        const int rr = tile_row(t);
        Frag<T> fw, fwg;
        lds_frag(fw, ringA, rr + n, g);
        lds_frag(fwg, ringB, rr + n, g);
        const f32x4 sc = dot_tile(fw, fA);
        const f32x4 gv = dot_tile(fwg, fB);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float p = fast_exp2(fmaf(sc[r], a.c2, wv[0][rr + 4 * g + r] + v2o));
          acc = keep_w(t, r) ? fmaf(p, gv[r], acc) : acc;
        }
      }
      const float dv2 = lane_group_sum(acc);
      if (g == 0 && o0 + n < Lr) vec(kDV2)[o0 + n] = dv2;
    } else if (PASS == 2) {
      // ---- du2_i = sum_j P22 (g - dv2_j); column sums of P22 du2 (owned rows in registers) ----
      float u2o[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) u2o[r] = vec(kU2)[min(o0 + 4 * g + r, Lr - 1)];
      f32x4 x[NT];
      float racc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        if (dead_tile(t)) {
          x[t] = f32x4{0.f, 0.f, 0.f, 0.f};
          continue;
        }
        const int rr = tile_row(t);
        Frag<T> fw, fwg;
        lds_frag(fw, ringA, rr + n, g);
        lds_frag(fwg, ringB, rr + n, g);
        const f32x4 sc = dot_tile(fA, fw);
        const f32x4 gv = dot_tile(fB, fwg);
        const float v2j = wv[0][rr + n], dj = wv[1][rr + n];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float p = keep_o(t, r) ? fast_exp2(fmaf(sc[r], a.c2, u2o[r] + v2j)) : 0.f;
          x[t][r] = p;
          racc[r] = fmaf(p, gv[r] - dj, racc[r]);
        }
      }
      float du2[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) du2[r] = row16_sum(racc[r]);
      if (n < 4) {
        const int i = o0 + 4 * g + n;
        const float di = (n == 0) ? du2[0] : (n == 1) ? du2[1] : (n == 2) ? du2[2] : du2[3];
        if (i < Lr) vec(kDU2)[i] = di;
      }
      float cp[NT + 3];
#pragma unroll
      for (int t = 0; t < NT; ++t)
        cp[t] = x[t][0] * du2[0] + x[t][1] * du2[1] + x[t][2] * du2[2] + x[t][3] * du2[3];
#pragma unroll
      for (int t = NT; t < NT + 3; ++t) cp[t] = 0.f;
      const int gsel = (g == 1) ? 2 : (g == 2) ? 1 : g;
#pragma unroll
      for (int q = 0; q < NT; q += 4) {
        const float s4 = swap16_sum(swap32_sum(cp[q], cp[q + 1]), swap32_sum(cp[q + 2], cp[q + 3]));
        const int t = q + gsel;
        if (t < NT) cpart[wave * RING + 16 * wave + 16 * t + n] = s4;
      }
      __syncthreads();
      for (int c = threadIdx.x; c < RING; c += NTHR) {
        float sacc = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) sacc += cpart[w * RING + c];
        pring[(cb + c + 4 * RING) % RING] += sacc;
      }
    } else if (PASS == 3) {
      // ---- du1, dQ (owned query i across lanes, window keys in registers) ----
      const int oi = min(o0 + n, Lr - 1);
      const float u2o = vec(kU2)[oi], Ai = vec(kDU2)[oi], Bi = vec(kEB)[oi];
      float acc = 0.f;
      f32x4 X[4], Y[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) X[b] = Y[b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int pq = 0; pq < NP; ++pq) {
        float z1[2][4], z2[2][4];
        int rbs[2];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          const int t = 2 * pq + tt;
          rbs[tt] = (t < NT) ? tile_row(t) : tile_row(2 * pq);
#pragma unroll
          for (int r = 0; r < 4; ++r) z1[tt][r] = z2[tt][r] = 0.f;
          if (t >= NT || dead_tile(t)) continue;
          const int rr = rbs[tt];
          Frag<T> fw, fwg;
          lds_frag(fw, ringA, rr + n, g);
          lds_frag(fwg, ringB, rr + n, g);
          const f32x4 sc = dot_tile(fw, fA);
          const f32x4 gv = dot_tile(fwg, fB);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int k = rr + 4 * g + r;
            const float v2j = wv[0][k], Dj = wv[1][k], Ej = wv[2][k], Fj = wv[3][k], Gj = wv[4][k];
            const float p = keep_w(t, r) ? fast_exp2(fmaf(sc[r], a.c2, u2o + v2j)) : 0.f;
            acc = fmaf(p, Fj, acc);
            z1[tt][r] = p * (gv[r] - Dj - Ai * Ej - Bi * Fj);
            z2[tt][r] = p * Gj;
          }
        }
        contract_ring2(X, Y, ringA, rbs[0], rbs[1], z1, z2, g, n);
      }
      const float du1 = -Bi * lane_group_sum(acc);
      const float Ci = du1 * Bi;
      if (o0 + n < Lr) {
        if (g == 0) {
          vec(kDU1)[o0 + n] = du1;
          vec(kCC)[o0 + n] = Ci;
        }
        f32x4 r4[4];
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
          for (int r = 0; r < 4; ++r) r4[b][r] = X[b][r] - Ci * Y[b][r];
        store_row(static_cast<T*>(a.out0) + tb + (int64_t)(o0 + n) * kD, r4, a.s, g);
      }
    } else {
      // ---- dK, dV (owned key j across lanes, window queries in registers) ----
      const int oj = min(o0 + n, Lr - 1);
      const float v2o = vec(kV2)[oj], Dj = vec(kDV2)[oj], Ej = vec(kEE)[oj], Fj = vec(kFF)[oj],
                  Gj = vec(kEG)[oj];
      f32x4 X[4], Y[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) X[b] = Y[b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int pq = 0; pq < NP; ++pq) {
        float z1[2][4], z2[2][4];
        int rbs[2];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          const int t = 2 * pq + tt;
          rbs[tt] = (t < NT) ? tile_row(t) : tile_row(2 * pq);
#pragma unroll
          for (int r = 0; r < 4; ++r) z1[tt][r] = z2[tt][r] = 0.f;
          if (t >= NT || dead_tile(t)) continue;
          const int rr = rbs[tt];
          Frag<T> fw, fwg;
          lds_frag(fw, ringA, rr + n, g);
          lds_frag(fwg, ringB, rr + n, g);
          const f32x4 sc = dot_tile(fw, fA);
          const f32x4 gv = dot_tile(fwg, fB);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int k = rr + 4 * g + r;
            const float u2i = wv[0][k], Ai = wv[1][k], Bi = wv[2][k], Ci = wv[3][k];
            const float p = keep_w(t, r) ? fast_exp2(fmaf(sc[r], a.c2, u2i + v2o)) : 0.f;
            z1[tt][r] = p * (gv[r] - Dj - Ai * Ej - Bi * Fj - Ci * Gj);
            z2[tt][r] = p;
          }
        }
        contract_ring(X, ringA, rbs[0], rbs[1], z1, g, n);
        contract_ring(Y, ringB, rbs[0], rbs[1], z2, g, n);
      }
      if (o0 + n < Lr) {
        store_row(static_cast<T*>(a.out0) + tb + (int64_t)(o0 + n) * kD, X, a.s, g);
        store_row(static_cast<T*>(a.out1) + tb + (int64_t)(o0 + n) * kD, Y, 1.f, g);
      }
    }

    __syncthreads();   // every wave is done with this block's window
    if (more) {
      if (PASS == 2 && (int)threadIdx.x < BR) {
        // columns [cb, cb + BR) leave the window: write this segment's sums out
        const int j = cb + threadIdx.x, slot = (j + 4 * RING) % RING;
        a.part[(head * (int64_t)a.nseg + seg) * a.pstride + (j - c_lo)] = pring[slot];
        pring[slot] = 0.f;
      }
      if ((int)threadIdx.x < BR) vec_store(cb + RING + (int)threadIdx.x, nv);
      na.template store<RING>(ringA, cb + RING);
      nb.template store<RING>(ringB, cb + RING);
      fA = fA_next;
      fB = fB_next;
      __syncthreads();
    } else if (PASS == 2) {
      for (int c = threadIdx.x; c < RING; c += NTHR)
        a.part[(head * (int64_t)a.nseg + seg) * a.pstride + (cb + c - c_lo)] =
            pring[(cb + c + 4 * RING) % RING];
    }
  }
}

// Waves per workgroup of the streaming passes: bf16 uses 12 waves (192-token blocks) with two
// window rings of 192 + 32 H16 rows, fp32 4 waves; both up to the halo LDS holds.
int vjp_stream_waves(int elt, int h, int* nt) {
  const int h16 = (h + 15) / 16;
  const int H16 = (h16 <= 2) ? 2 : (h16 <= 4) ? 4 : (h16 <= 8) ? 8 : 0;
  if (H16 == 0) return 0;
  if (elt == 0 && H16 > 4) return 0;
  *nt = 1 + 2 * H16;
  return (elt == 1) ? 12 : 4;
}

void vjp_stream_segments(int64_t bh, int Lr, int nw, int nt, int* seg_len, int* nseg) {
  const int br = 16 * nw;
  const int64_t nblk = (Lr + br - 1) / br;
  const int64_t target = 256;   // one workgroup per CU
  int64_t sl = (bh * nblk + target - 1) / target;
  const int64_t min_sl = (16 * (nt - 1) + br - 1) / br;   // 2 * halo <= seg span
  if (sl < min_sl) sl = min_sl;
  if (sl < 1) sl = 1;
  if (sl > nblk) sl = nblk;
  *seg_len = (int)sl;
  *nseg = (int)((nblk + sl - 1) / sl);
}

template <typename T, int NT, int NW>
static void launch_nt(int pass, const VjpArgs& a, hipStream_t st) {
  const dim3 grid((unsigned)(a.bh * (int64_t)a.nseg)), block(NW * 64);
  switch (pass) {
    case 0: vjp_stream_kernel<T, NT, NW, 0><<<grid, block, 0, st>>>(a); break;
    case 1: vjp_stream_kernel<T, NT, NW, 1><<<grid, block, 0, st>>>(a); break;
    case 2: vjp_stream_kernel<T, NT, NW, 2><<<grid, block, 0, st>>>(a); break;
    case 3: vjp_stream_kernel<T, NT, NW, 3><<<grid, block, 0, st>>>(a); break;
    default: vjp_stream_kernel<T, NT, NW, 4><<<grid, block, 0, st>>>(a); break;
  }
}

hipError_t launch_vjp_stream_pass(int elt, int nt, int nw, int pass, const VjpArgs& a,
                                  hipStream_t st) {
  if (elt == 1 && nw == 12) {
    if (nt == 5) launch_nt<bf16, 5, 12>(pass, a, st);
    else if (nt == 9) launch_nt<bf16, 9, 12>(pass, a, st);
    else launch_nt<bf16, 17, 12>(pass, a, st);
  } else {
    if (nt == 5) launch_nt<float, 5, 4>(pass, a, st);
    else launch_nt<float, 9, 4>(pass, a, st);
  }
  return hipGetLastError();
}

}  // namespace ska
