// HIP kernels (gfx950) for banded balanced Sinkhorn attention: log-domain Sinkhorn half-steps,
// the reference-plan output, and the five passes of the exact R = 2 tail VJP.
//
// Method: arXiv 2605.08123 as summarised on gist.science (technical summaries §2.1-§2.3),
// the abstract listings, and atlas.scime.ai.  Scores live on the fixed band |i - j| <= h and are
// recomputed per 16x16 tile on the matrix cores in every pass; nothing of size L x W is stored.
//
// Work decomposition shared by every kernel.  A workgroup is 4 independent waves; wave w of
// block b owns the 16 tokens o0 = (4b + w) * 16 ... o0 + 15 and streams over the 16-token tiles
// of its band window [o0 - h, o0 + 15 + h].  One MFMA tile X[m][n] = <win_{w0+m}, own_{o0+n}> is
// computed with the window token rows as the A operand and the owned rows as the B operand, so
// lane l holds owned token n = l % 16 and, in its 4 result registers r, window tokens
// m = 4 (l / 16) + r.  Sums over the window therefore run inside each lane (plus one exchange
// across the 4 lane groups at the end), and a contraction over the window (P V, dS K, ...) can
// feed the result registers straight into a second MFMA as its B operand, with the window rows
// of the other tensor staged through LDS and read transposed as the A operand.
//
// Which side is owned decides what a pass can reduce without cross-workgroup traffic: a pass
// that owns queries reduces over keys (row sums, dQ, O); a pass that owns keys reduces over
// queries (column sums, dK, dV).  The score tile is symmetric in the two roles
// (S_ij = s q_i . k_j), so one kernel body serves both orientations with Q and K swapped.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "ska_device.h"
#include "ska_internal.h"

namespace ska {

// =============================================================================================
// Balanced Sinkhorn half-step: out_o = -log sum_{w in band(o)} exp(S(o, w) + in_w).
// Row update: own = Q, win = K, in = v, out = u.  Column update: own = K, win = Q, in = u, out = v.
// Vectors are in log2 units: x = log2(e) * (S + in), out = -log2 sum 2^x.
// [technical summaries §2.1: balanced Sinkhorn iteration on the fixed band; log-domain updates]
// =============================================================================================
template <typename T>
__global__ __launch_bounds__(256) void lse_kernel(const T* __restrict__ own, const T* __restrict__ win,
                                                  const float* __restrict__ vin,
                                                  float* __restrict__ vout, float* __restrict__ vsave,
                                                  int64_t save_stride, int Lr, int Lpad, int h,
                                                  float c2) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 4, n = lane & 15;
  const int64_t head = blockIdx.y;
  const int o0 = (blockIdx.x * kWaves + wave) * 16;
  if (o0 >= Lr) return;
  const T* ownh = own + head * Lr * kD;
  const T* winh = win + head * Lr * kD;
  const float* vinh = vin + head * Lpad;
  const int o = o0 + n;

  Frag<T> fo;
  load_frag(fo, ownh + (int64_t)o * kD, o < Lr, g);
  const int wlo = max(0, o0 - h), whi = min(Lr - 1, o0 + 15 + h);
  float m = -INFINITY, l = 0.f;
  for (int w0 = wlo & ~15; w0 <= whi; w0 += 16) {
    Frag<T> fw;
    load_frag(fw, winh + (int64_t)(w0 + n) * kD, w0 + n < Lr, g);
    const f32x4 acc = dot_tile(fw, fo);
    const f32x4 vv = load4(vinh + w0 + 4 * g);
    float x[4];
#pragma unroll
    for (int r = 0; r < 4; ++r)
      x[r] = in_band(w0 + 4 * g + r, o, h, Lr) ? fmaf(acc[r], c2, vv[r]) : -INFINITY;
    const float mt = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    const float mn = fmaxf(m, mt);
    if (mn != -INFINITY) {
      l = l * fast_exp2(m - mn) + fast_exp2(x[0] - mn) + fast_exp2(x[1] - mn) +
          fast_exp2(x[2] - mn) + fast_exp2(x[3] - mn);
      m = mn;
    }
  }
#pragma unroll
  for (int off = 16; off <= 32; off <<= 1) {
    const float m2 = __shfl_xor(m, off), l2 = __shfl_xor(l, off);
    const float mn = fmaxf(m, m2);
    if (mn != -INFINITY) {
      l = l * fast_exp2(m - mn) + l2 * fast_exp2(m2 - mn);
      m = mn;
    }
  }
  if (g == 0 && o < Lr) {
    const float r = (m == -INFINITY) ? 0.f : -(m + fast_log2(l));
    vout[head * Lpad + o] = r;
    if (vsave) vsave[head * save_stride + o] = r * kLn2;
  }
}

// =============================================================================================
// Output: O_i = sum_j P22_ij V_j, P22 = exp(S + u2 + v2) on the band (query-owned).
// [technical summaries §2.2: the reference plan P^(2,2); spec output plan x V]
// =============================================================================================
template <typename T>
__global__ __launch_bounds__(256) void out_kernel(const T* __restrict__ Q, const T* __restrict__ K,
                                                  const T* __restrict__ V, const float* __restrict__ u2,
                                                  const float* __restrict__ v2, T* __restrict__ O,
                                                  int Lr, int Lpad, int h, float c2) {
  __shared__ __attribute__((aligned(16))) T lds_all[kWaves * kChunk * Lds<T>::stride];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 4, n = lane & 15;
  const int64_t head = blockIdx.y;
  const int o0 = (blockIdx.x * kWaves + wave) * 16;
  if (o0 >= Lr) return;
  T* lds = lds_all + wave * kChunk * Lds<T>::stride;
  const T* Qh = Q + head * Lr * kD;
  const T* Kh = K + head * Lr * kD;
  const T* Vh = V + head * Lr * kD;
  const float* u2h = u2 + head * Lpad;
  const float* v2h = v2 + head * Lpad;
  const int o = o0 + n;

  Frag<T> fo;
  load_frag(fo, Qh + (int64_t)o * kD, o < Lr, g);
  const float uo = u2h[o];
  f32x4 acc[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int wlo = max(0, o0 - h), whi = min(Lr - 1, o0 + 15 + h);
  for (int c0 = wlo & ~(kChunk - 1); c0 <= whi; c0 += kChunk) {
    stage_rows(lds, Vh, c0, Lr, lane);
    float p[2][4];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int w0 = c0 + 16 * tt;
      if (tile_live(w0, o0, h, Lr)) {
        Frag<T> fw;
        load_frag(fw, Kh + (int64_t)(w0 + n) * kD, w0 + n < Lr, g);
        const f32x4 s = dot_tile(fw, fo);
        const f32x4 vv = load4(v2h + w0 + 4 * g);
#pragma unroll
        for (int r = 0; r < 4; ++r)
          p[tt][r] = in_band(w0 + 4 * g + r, o, h, Lr) ? fast_exp2(fmaf(s[r], c2, uo + vv[r])) : 0.f;
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) p[tt][r] = 0.f;
      }
    }
    __builtin_amdgcn_wave_barrier();
    contract(acc, lds, p, g, n);
    __builtin_amdgcn_wave_barrier();
  }
  if (o < Lr) store_row(O + head * Lr * kD + (int64_t)o * kD, acc, 1.f, g);
}

// =============================================================================================
// R = 2 tail VJP passes.  Notation: entry (i, j), i = query, j = key;
// P22 = exp(S + u2_i + v2_j), g_ij = dO_i . V_j; e^{du1} = exp(u1 - u2), e^{dv_b} = exp(v_b - v2).
//   A: owns keys.    dv2_j = sum_i P22 g;            dV_j = sum_i P22_ij dO_i
//   B: owns queries. du2_i = sum_j P22 (g - dv2_j)
//   C: owns keys.    dv1_j = -e^{dv1_j} sum_i P22 du2_i          (direct: -sum_i P21 du2_i)
//   D: owns queries. du1_i = -e^{du1_i} sum_j P22 e^{dv1_j} dv1_j (direct: -sum_j P11 dv1_j)
//                    dQ_i = s sum_j dS_ij k_j, with dS = Z1 - C_i Z2 split so du1_i can be
//                    finished after the sweep: one-ref Z1 = P22 (g - D_j - A_i E_j - B_i F_j),
//                    Z2 = P22 G_j, C_i = du1_i e^{du1_i}; direct Z1 = P22 (g - dv2_j) - P21 du2_i
//                    - P11 dv1_j, Z2 = P10, C_i = du1_i.
//   E: owns keys.    dK_j = s sum_i dS_ij q_i,  dS = P22 M (one-ref) or the four-plan sum.
// Modifier field (one reference tile): M_ij = g_ij - D_j - A_i E_j - B_i F_j - C_i G_j with
// A = du2, B = e^{du1}, C = du1 e^{du1}, D = dv2, E = e^{dv1}, F = dv1 e^{dv1}, G = e^{dv0}.
// [abstract: one reference plan tile times a modifier field of vector cotangents and dual
// differences; technical summaries §2.2: orbit equation and the four staircase plan factors]
// =============================================================================================
enum Pass : int { kPassA = 0, kPassB = 1, kPassC = 2, kPassD = 3, kPassE = 4 };

template <int PASS> struct PassTraits {
  static constexpr bool owns_keys = (PASS == kPassA || PASS == kPassC || PASS == kPassE);
  static constexpr bool needs_g = (PASS != kPassC);
  static constexpr bool contracts = (PASS == kPassA || PASS == kPassD || PASS == kPassE);
};

template <typename T, int PASS, bool DIRECT4>
__global__ __launch_bounds__(256) void vjp_kernel(const T* __restrict__ Q, const T* __restrict__ K,
                                                  const T* __restrict__ V, const T* __restrict__ dO,
                                                  T* __restrict__ out, float* __restrict__ ws, int Lr,
                                                  int Lpad, int h, float c2, float s,
                                                  int64_t vec_stride) {
  using PT = PassTraits<PASS>;
  __shared__ __attribute__((aligned(16))) T lds_all[PT::contracts ? kWaves * kChunk * Lds<T>::stride : 8];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 4, n = lane & 15;
  const int64_t head = blockIdx.y;
  const int o0 = (blockIdx.x * kWaves + wave) * 16;
  if (o0 >= Lr) return;
  T* lds = lds_all + (PT::contracts ? wave * kChunk * Lds<T>::stride : 0);
  const int64_t tb = head * Lr * kD;
  // score operands: owned side and window side; value-score operands likewise
  const T* own_s = (PT::owns_keys ? K : Q) + tb;
  const T* win_s = (PT::owns_keys ? Q : K) + tb;
  const T* own_g = (PT::owns_keys ? V : dO) + tb;
  const T* win_g = (PT::owns_keys ? dO : V) + tb;
  // second-contraction operand (staged): A -> dO, D -> K, E -> Q
  const T* win_c = (PASS == kPassA ? dO : (PASS == kPassD ? K : Q)) + tb;

  auto vec = [&](int which) -> float* { return ws + which * vec_stride + head * Lpad; };
  // query-indexed ("u side") and key-indexed ("v side") vectors
  const float* u2 = vec(kU2);
  const float* v2 = vec(kV2);
  const float* u1 = vec(kU1);
  const float* v1 = vec(kV1);
  const float* v0 = vec(kV0);
  const int o = o0 + n;

  Frag<T> fo, fog;
  load_frag(fo, own_s + (int64_t)o * kD, o < Lr, g);
  if (PT::needs_g) load_frag(fog, own_g + (int64_t)o * kD, o < Lr, g);

  // owned-token vector values
  float own_u2, own_v2, own_x0 = 0.f, own_x1 = 0.f, own_x2 = 0.f, own_x3 = 0.f, own_x4 = 0.f;
  if (PT::owns_keys) {
    own_v2 = v2[o];
    own_u2 = 0.f;
    if (PASS == kPassA) {
    } else if (PASS == kPassC) {
      own_x0 = DIRECT4 ? v1[o] : vec(kEE)[o];                   // v1 (direct) or E
    } else {                                                    // E
      own_x0 = vec(kDV2)[o];                                    // D
      own_x1 = DIRECT4 ? v1[o] : vec(kEE)[o];                   // v1 or E
      own_x2 = DIRECT4 ? vec(kDV1)[o] : vec(kFF)[o];            // dv1 or F
      own_x3 = DIRECT4 ? v0[o] : vec(kEG)[o];                   // v0 or G
    }
  } else {
    own_u2 = u2[o];
    own_v2 = 0.f;
    if (PASS == kPassD) {
      own_x0 = vec(kDU2)[o];                                    // A = du2
      own_x1 = DIRECT4 ? u1[o] : vec(kEB)[o];                   // u1 (direct) or B
    }
  }
  (void)own_x4;

  float red = 0.f;  // per-lane partial of the pass's window reduction
  f32x4 acc[4], acc2[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) acc[b] = acc2[b] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int wlo = max(0, o0 - h), whi = min(Lr - 1, o0 + 15 + h);
  for (int c0 = wlo & ~(kChunk - 1); c0 <= whi; c0 += kChunk) {
    if (PT::contracts) stage_rows(lds, win_c, c0, Lr, lane);
    float z1[2][4], z2[2][4];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int w0 = c0 + 16 * tt;
#pragma unroll
      for (int r = 0; r < 4; ++r) z1[tt][r] = z2[tt][r] = 0.f;
      if (!tile_live(w0, o0, h, Lr)) continue;
      Frag<T> fw;
      load_frag(fw, win_s + (int64_t)(w0 + n) * kD, w0 + n < Lr, g);
      const f32x4 sc = dot_tile(fw, fo);
      f32x4 gv = {0.f, 0.f, 0.f, 0.f};
      if (PT::needs_g) {
        Frag<T> fwg;
        load_frag(fwg, win_g + (int64_t)(w0 + n) * kD, w0 + n < Lr, g);
        gv = dot_tile(fwg, fog);
      }
      const int wb = w0 + 4 * g;
      // window-token vectors (4 consecutive tokens per lane)
      if (PT::owns_keys) {
        const f32x4 wu2 = load4(u2 + wb);
        f32x4 wa = {0.f, 0.f, 0.f, 0.f}, wbv = wa, wc = wa;
        if (PASS == kPassC) wa = load4(vec(kDU2) + wb);
        if (PASS == kPassE) {
          wa = load4(vec(kDU2) + wb);                               // A = du2
          wbv = DIRECT4 ? load4(u1 + wb) : load4(vec(kEB) + wb);    // u1 or B
          wc = DIRECT4 ? load4(vec(kDU1) + wb) : load4(vec(kCC) + wb);  // du1 or C
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if (!in_band(wb + r, o, h, Lr)) continue;
          const float x = fmaf(sc[r], c2, wu2[r]);           // log2(e) S + u2_i
          const float p22 = fast_exp2(x + own_v2);
          if (PASS == kPassA) {
            red = fmaf(p22, gv[r], red);
            z1[tt][r] = p22;
          } else if (PASS == kPassC) {
            if (DIRECT4) red = fmaf(fast_exp2(x + own_x0), wa[r], red);   // P21 du2
            else red = fmaf(p22, wa[r], red);
          } else {  // E
            float ds;
            if (DIRECT4) {
              const float xs = fmaf(sc[r], c2, 0.f);
              const float p21 = fast_exp2(x + own_x1);
              const float p11 = fast_exp2(xs + wbv[r] + own_x1);
              const float p10 = fast_exp2(xs + wbv[r] + own_x3);
              ds = p22 * (gv[r] - own_x0) - p21 * wa[r] - p11 * own_x2 - p10 * wc[r];
            } else {
              const float mfield = gv[r] - own_x0 - wa[r] * own_x1 - wbv[r] * own_x2 - wc[r] * own_x3;
              ds = p22 * mfield;
            }
            z1[tt][r] = ds;
          }
        }
      } else {
        const f32x4 wv2 = load4(v2 + wb);
        f32x4 wd = {0.f, 0.f, 0.f, 0.f}, we = wd, wf = wd, wg = wd;
        if (PASS == kPassB) wd = load4(vec(kDV2) + wb);
        if (PASS == kPassD) {
          wd = load4(vec(kDV2) + wb);                                   // D
          we = DIRECT4 ? load4(v1 + wb) : load4(vec(kEE) + wb);         // v1 or E
          wf = DIRECT4 ? load4(vec(kDV1) + wb) : load4(vec(kFF) + wb);  // dv1 or F
          wg = DIRECT4 ? load4(v0 + wb) : load4(vec(kEG) + wb);         // v0 or G
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if (!in_band(wb + r, o, h, Lr)) continue;
          const float xs = sc[r] * c2;
          const float p22 = fast_exp2(xs + own_u2 + wv2[r]);
          if (PASS == kPassB) {
            red = fmaf(p22, gv[r] - wd[r], red);
          } else {  // D
            if (DIRECT4) {
              const float p21 = fast_exp2(xs + own_u2 + we[r]);
              const float p11 = fast_exp2(xs + own_x1 + we[r]);
              const float p10 = fast_exp2(xs + own_x1 + wg[r]);
              red = fmaf(p11, wf[r], red);
              z1[tt][r] = p22 * (gv[r] - wd[r]) - p21 * own_x0 - p11 * wf[r];
              z2[tt][r] = p10;
            } else {
              red = fmaf(p22, wf[r], red);
              z1[tt][r] = p22 * (gv[r] - wd[r] - own_x0 * we[r] - own_x1 * wf[r]);
              z2[tt][r] = p22 * wg[r];
            }
          }
        }
      }
    }
    if (PT::contracts) {
      __builtin_amdgcn_wave_barrier();
      if (PASS == kPassD) contract2(acc, acc2, lds, z1, z2, g, n);
      else contract(acc, lds, z1, g, n);
      __builtin_amdgcn_wave_barrier();
    }
  }

  red = group_sum(red);
  const bool valid = o < Lr;
  const int64_t ob = head * Lpad + o;
  if (PASS == kPassA) {
    if (valid && g == 0) ws[kDV2 * vec_stride + ob] = red;
    if (valid) store_row(out + tb + (int64_t)o * kD, acc, 1.f, g);
  } else if (PASS == kPassB) {
    if (valid && g == 0) ws[kDU2 * vec_stride + ob] = red;
  } else if (PASS == kPassC) {
    const float dv1 = DIRECT4 ? -red : -own_x0 * red;
    if (valid && g == 0) {
      ws[kDV1 * vec_stride + ob] = dv1;
      ws[kFF * vec_stride + ob] = dv1 * ws[kEE * vec_stride + ob];
    }
  } else if (PASS == kPassD) {
    const float eb = ws[kEB * vec_stride + ob];
    const float du1 = DIRECT4 ? -red : -eb * red;
    const float cc = DIRECT4 ? du1 : du1 * eb;   // coefficient of Z2 in dS
    if (valid && g == 0) {
      ws[kDU1 * vec_stride + ob] = du1;
      ws[kCC * vec_stride + ob] = du1 * eb;
    }
    if (valid) {
      f32x4 r4[4];
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r) r4[b][r] = acc[b][r] - cc * acc2[b][r];
      store_row(out + tb + (int64_t)o * kD, r4, s, g);
    }
  } else {  // E
    if (valid) store_row(out + tb + (int64_t)o * kD, acc, s, g);
  }
}

// =============================================================================================
// small vector kernels
// =============================================================================================
__global__ void fill_kernel(float* __restrict__ p, int64_t n, float value) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = value;
}

// duals[head][0][t] = vec[head][t] * ln 2 for t < Lr (the stopped base v^(0) in natural units)
__global__ void save_dual_kernel(const float* __restrict__ vec, float* __restrict__ duals,
                                 int64_t dual_stride_head, int Lr, int Lpad) {
  const int64_t head = blockIdx.y;
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t < Lr) duals[head * dual_stride_head + t] = vec[head * Lpad + t] * kLn2;
}

// Prepare VJP vectors: duals (natural) -> log2 units, plus the orbit factors exp(u1 - u2),
// exp(v1 - v2), exp(v0 - v2).  Padding tokens get zeros.
__global__ void vjp_prep_kernel(const float* __restrict__ duals, float* __restrict__ ws, int Lr,
                                int Lpad, int64_t vec_stride) {
  const int64_t head = blockIdx.y;
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= Lpad) return;
  const int64_t ob = head * Lpad + t;
  float v0 = 0.f, u1 = 0.f, v1 = 0.f, u2 = 0.f, v2 = 0.f;
  if (t < Lr) {
    const float* dh = duals + head * 5 * (int64_t)Lr;
    v0 = dh[t];
    u1 = dh[Lr + t];
    v1 = dh[2 * (int64_t)Lr + t];
    u2 = dh[3 * (int64_t)Lr + t];
    v2 = dh[4 * (int64_t)Lr + t];
  }
  ws[kV0 * vec_stride + ob] = v0 * kLog2e;
  ws[kU1 * vec_stride + ob] = u1 * kLog2e;
  ws[kV1 * vec_stride + ob] = v1 * kLog2e;
  ws[kU2 * vec_stride + ob] = u2 * kLog2e;
  ws[kV2 * vec_stride + ob] = v2 * kLog2e;
  const bool ok = t < Lr;
  ws[kEB * vec_stride + ob] = ok ? expf(u1 - u2) : 0.f;
  ws[kEE * vec_stride + ob] = ok ? expf(v1 - v2) : 0.f;
  ws[kEG * vec_stride + ob] = ok ? expf(v0 - v2) : 0.f;
  for (int k = kDV2; k < kVjpVecs; ++k) ws[k * vec_stride + ob] = 0.f;
}

// =============================================================================================
// launchers
// =============================================================================================
static dim3 pass_grid(const Geometry& g) {
  return dim3((unsigned)((g.Lr + kOwnPerBlock - 1) / kOwnPerBlock), (unsigned)g.bh, 1);
}

hipError_t launch_fill(float* p, int64_t n, float value, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  fill_kernel<<<dim3((unsigned)blocks), dim3(256), 0, st>>>(p, n, value);
  return hipGetLastError();
}

hipError_t launch_save_duals(const float* vec_log2, float* duals, int64_t dual_stride_head,
                             const Geometry& g, hipStream_t st) {
  save_dual_kernel<<<dim3((unsigned)((g.Lr + 255) / 256), (unsigned)g.bh), dim3(256), 0, st>>>(
      vec_log2, duals, dual_stride_head, g.Lr, g.Lpad);
  return hipGetLastError();
}

hipError_t launch_lse(int elt, const void* own, const void* win, const float* vin, float* vout,
                      float* vsave, int64_t save_stride, const Geometry& g, hipStream_t st) {
  if (elt == 1)
    lse_kernel<bf16><<<pass_grid(g), dim3(256), 0, st>>>(
        (const bf16*)own, (const bf16*)win, vin, vout, vsave, save_stride, g.Lr, g.Lpad, g.h, g.c2);
  else
    lse_kernel<float><<<pass_grid(g), dim3(256), 0, st>>>(
        (const float*)own, (const float*)win, vin, vout, vsave, save_stride, g.Lr, g.Lpad, g.h, g.c2);
  return hipGetLastError();
}

hipError_t launch_out(int elt, const void* Q, const void* K, const void* V, const float* u2,
                      const float* v2, void* O, const Geometry& g, hipStream_t st) {
  if (elt == 1)
    out_kernel<bf16><<<pass_grid(g), dim3(256), 0, st>>>((const bf16*)Q, (const bf16*)K,
                                                          (const bf16*)V, u2, v2, (bf16*)O, g.Lr,
                                                          g.Lpad, g.h, g.c2);
  else
    out_kernel<float><<<pass_grid(g), dim3(256), 0, st>>>((const float*)Q, (const float*)K,
                                                           (const float*)V, u2, v2, (float*)O,
                                                           g.Lr, g.Lpad, g.h, g.c2);
  return hipGetLastError();
}

hipError_t launch_vjp_prep(const float* duals, float* ws, const Geometry& g, hipStream_t st) {
  const int64_t vs = g.bh * (int64_t)g.Lpad;
  vjp_prep_kernel<<<dim3((unsigned)((g.Lpad + 255) / 256), (unsigned)g.bh), dim3(256), 0, st>>>(
      duals, ws, g.Lr, g.Lpad, vs);
  return hipGetLastError();
}

template <typename T, int PASS, bool D4>
static void launch_pass_t(const void* Q, const void* K, const void* V, const void* dO, void* out,
                          float* ws, const Geometry& g, hipStream_t st) {
  const int64_t vs = g.bh * (int64_t)g.Lpad;
  vjp_kernel<T, PASS, D4><<<pass_grid(g), dim3(256), 0, st>>>(
      (const T*)Q, (const T*)K, (const T*)V, (const T*)dO, (T*)out, ws, g.Lr, g.Lpad, g.h, g.c2, g.s,
      vs);
}

template <typename T, bool D4>
static void launch_pass_d(int pass, const void* Q, const void* K, const void* V, const void* dO,
                          void* out, float* ws, const Geometry& g, hipStream_t st) {
  switch (pass) {
    case kPassA: launch_pass_t<T, kPassA, D4>(Q, K, V, dO, out, ws, g, st); break;
    case kPassB: launch_pass_t<T, kPassB, D4>(Q, K, V, dO, out, ws, g, st); break;
    case kPassC: launch_pass_t<T, kPassC, D4>(Q, K, V, dO, out, ws, g, st); break;
    case kPassD: launch_pass_t<T, kPassD, D4>(Q, K, V, dO, out, ws, g, st); break;
    default: launch_pass_t<T, kPassE, D4>(Q, K, V, dO, out, ws, g, st); break;
  }
}

hipError_t launch_vjp_pass(int elt, int pass, bool direct4, const void* Q, const void* K,
                           const void* V, const void* dO, void* out, float* ws, const Geometry& g,
                           hipStream_t st) {
  if (elt == 1) {
    if (direct4) launch_pass_d<bf16, true>(pass, Q, K, V, dO, out, ws, g, st);
    else launch_pass_d<bf16, false>(pass, Q, K, V, dO, out, ws, g, st);
  } else {
    if (direct4) launch_pass_d<float, true>(pass, Q, K, V, dO, out, ws, g, st);
    else launch_pass_d<float, false>(pass, Q, K, V, dO, out, ws, g, st);
  }
  return hipGetLastError();
}

}  // namespace ska
