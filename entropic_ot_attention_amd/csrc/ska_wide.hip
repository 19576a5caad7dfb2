// Wide-band engine (gfx950): bands too wide for the register-resident streaming kernels, up to
// the dense support of the dustbin-block variant [technical summaries §2.3: the dustbin token
// joins a support widened to every active pair; cost O(L max(W, L))].
//
// Decomposition.  One workgroup of 8 waves per 16-token row tile of one problem.  The row tile's
// window (its band: every token of a dense problem) is cut into 8 contiguous runs of 16-token
// tiles, one per wave, so a problem of a few thousand tokens still gives each SIMD two waves and
// the matrix cores a long independent MFMA stream per wave.  Per-wave partial results (row maxima
// and sums, vector cotangent sums, 16 x 64 contraction accumulators) are combined across the
// workgroup through LDS in fixed wave order, so results do not depend on timing.
//
// Forward step [technical summaries §2.1: log-domain row update, then column update, on the
// fixed support]: wide_step_kernel keeps the row tile's scores against its whole window in
// registers (up to 8 x 33 tiles per workgroup), so one score evaluation and one exponential per
// entry give the exact row update (workgroup max and sum) and the row tile's column sums of the
// row-normalised plan; wide_finish_kernel adds each column's partials in a fixed order and
// finishes the column update, exactly where a column's mass underflows.
//
// Output and VJP [output: the reference plan P^(2,2) applied to V; abstract and technical
// summaries §2.2: dS = P22 * M, M from the vector cotangents and the dual-difference factors]:
// wide_pass_kernel runs the output and five VJP passes, each owning the side it reduces over, so
// no pass needs partial sums across workgroups:
//   out (owns queries)  O_i = sum_j P22_ij V_j
//   A   (owns keys)     dV_j = sum_i P22_ij dO_i,  dv2_j = sum_i P22 g = V_j . dV_j
//   B   (owns queries)  du2_i = sum_j P22 (g - dv2_j)  (given O: dO_i . O_i - sum_j P22 dv2_j)
//   C   (owns keys)     dv1_j = -e^{dv1_j} sum_i P22 du2_i          (direct: -sum_i P21 du2_i)
//   D   (owns queries)  du1_i = -e^{du1_i} sum_j P22 E_j dv1_j      (direct: -sum_j P11 dv1_j)
//                       dQ_i = s sum_j dS_ij k_j with dS = Z1 - C_i Z2, so du1_i (known only at
//                       the end of the row) multiplies a second accumulator
//   E   (owns keys)     dK_j = s sum_i dS_ij q_i
// with P22 = exp(S + u2 + v2), g_ij = dO_i . V_j, A = du2, B = e^{u1 - u2}, C = du1 B, D = dv2,
// E = e^{v1 - v2}, F = dv1 E, G = e^{v0 - v2} (one reference tile), or each staircase plan from
// its own exponential (direct four).
//
// Tile layout: a score tile has the window tokens in lane registers (4 g + r) and the owned tokens
// across lanes (n) in the passes, so sums over the window stay in-lane and the contraction over
// the window takes the plan values straight from the result registers as its B operand, the
// window rows of the other tensor read transposed from LDS.  The fused step swaps the roles
// (owned rows in registers, window across lanes): its row sums stay in-lane and its column sums
// reduce over the four lane groups with lane swaps.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "ska_device.h"
#include "ska_internal.h"

namespace ska {

constexpr int kWideThreads = 64 * kWideWaves;

// Window of row tile rt: tiles t0 .. t0 + nt - 1; wave w takes tiles wt0 .. wt0 + wnt - 1.
struct WideTile {
  int o0, t0, nt, wt0, wnt;
};
__device__ __forceinline__ WideTile wide_tile(int rt, int Lr, int h, int wave) {
  WideTile w;
  w.o0 = 16 * rt;
  const int lo = max(0, w.o0 - h), hi = min(Lr - 1, w.o0 + 15 + h);
  w.t0 = lo >> 4;
  w.nt = (hi >> 4) - w.t0 + 1;
  w.wt0 = w.t0 + (w.nt * wave) / kWideWaves;
  w.wnt = w.t0 + (w.nt * (wave + 1)) / kWideWaves - w.wt0;
  return w;
}

// Workgroup -> (problem, row tile).  Workgroups are dispatched round-robin over the 8 XCDs
// (XCD = id mod 8); each XCD is given a contiguous run of the row tiles in (problem, tile) order,
// so the workgroups sharing an XCD's L2 mostly read the window tensors of one problem.  Ids past
// the last tile return at once.
__device__ __forceinline__ bool wide_work(int64_t nwork, int nrt, int64_t* head, int* rt) {
  const int64_t id = blockIdx.x, per = (nwork + 7) / 8;
  const int64_t w = (id % 8) * per + id / 8;
  if (w >= nwork) return false;
  *head = w / nrt;
  *rt = (int)(w % nrt);
  return true;
}

__device__ __forceinline__ float pick4(const float (&v)[4], int k) {
  return (k == 0) ? v[0] : (k == 1) ? v[1] : (k == 2) ? v[2] : v[3];
}

// 32 window rows of a [L][64] tensor held per lane between their global load and their LDS store
// (rows outside the sequence become zeros when stored).
template <typename T>
struct WaveStage {
  static constexpr int kCPR = 64 * (int)sizeof(T) / 16;   // 16-byte chunks per row
  static constexpr int kPer = 32 * kCPR / 64;
  uint4 x[kPer];
  __device__ __forceinline__ void load(const T* base, int r0, int Lr, int lane) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int c = i * 64 + lane, row = c / kCPR, col = (c % kCPR) * (16 / (int)sizeof(T));
      const int t = min(r0 + row, Lr - 1);
      x[i] = *reinterpret_cast<const uint4*>(base + (int64_t)t * kD + col);
    }
  }
  __device__ __forceinline__ void store(T* lds, int r0, int Lr, int lane) const {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int c = i * 64 + lane, row = c / kCPR, col = (c % kCPR) * (16 / (int)sizeof(T));
      const bool ok = r0 + row < Lr;
      *reinterpret_cast<uint4*>(lds + row * Lds<T>::stride + col) =
          uint4{ok ? x[i].x : 0u, ok ? x[i].y : 0u, ok ? x[i].z : 0u, ok ? x[i].w : 0u};
    }
  }
};

// fp32 inputs on the bf16 matrix cores.  Each value becomes three bf16 parts, x = h + m + l with
// h = bf16(x), m = bf16(x - h), l = bf16(x - h - m), all rounded to nearest (the two differences
// are exact in fp32), so |x - h - m - l| <= 2^-24 |x|; a row of 64 values is stored as the three
// planes (h, m, l), 192 bf16.  A dot product q . k is then the six bf16 products
// hq hk + hq mk + mq hk + hq lk + lq hk + mq mk with fp32 accumulation; the three dropped ones are
// below 2^-24 |q| |k| per term, so the score keeps fp32 accuracy at twelve bf16 16x16x32 products
// per tile instead of sixteen fp32 16x16x4 ones (a SIMD spends about 193 cycles on the former and
// 512 on the latter).
constexpr int kPlaneRow = 3 * kD;
__global__ __launch_bounds__(256) void split3_kernel(const float* __restrict__ x, bf16* __restrict__ out,
                                                     int64_t rows) {
  typedef __bf16 bf16x4v __attribute__((__vector_size__(8)));
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;   // 4 values of one row
  if (i >= rows * (kD / 4)) return;
  const int64_t row = i / (kD / 4);
  const int c = (int)(i % (kD / 4)) * 4;
  const f32x4 v = *reinterpret_cast<const f32x4*>(x + row * kD + c);
  bf16x4v hv, mv, lv;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const bf16 h = (bf16)v[e];
    const float r1 = v[e] - (float)h;
    const bf16 m = (bf16)r1;
    hv[e] = h;
    mv[e] = m;
    lv[e] = (bf16)(r1 - (float)m);
  }
  bf16* o = out + row * kPlaneRow + c;
  *reinterpret_cast<bf16x4v*>(o) = hv;
  *reinterpret_cast<bf16x4v*>(o + kD) = mv;
  *reinterpret_cast<bf16x4v*>(o + 2 * kD) = lv;
}

// q . k of a 16 x 16 tile from the three planes of each side (A: q, B: k), smallest terms first
__device__ __forceinline__ f32x4 dot_tile3(const Frag<bf16> (&q)[3], const Frag<bf16> (&k)[3], f32x4 acc) {
  acc = dot_tile(q[2], k[0], acc);
  acc = dot_tile(q[0], k[2], acc);
  acc = dot_tile(q[1], k[1], acc);
  acc = dot_tile(q[1], k[0], acc);
  acc = dot_tile(q[0], k[1], acc);
  return dot_tile(q[0], k[0], acc);
}

// 16 window rows of three-plane bf16 [L][192] held per lane between their global load and their
// LDS store (rows of kPlaneStage bf16; rows outside the sequence become zeros when stored)
constexpr int kPlaneStage = kPlaneRow + 8;
struct PlaneStage {
  static constexpr int kCPR = kPlaneRow * 2 / 16;          // 16-byte chunks per row: 24
  static constexpr int kPer = 16 * kCPR / 64;              // per lane: 6
  uint4 x[kPer];
  __device__ __forceinline__ void load(const bf16* base, int r0, int Lr, int lane) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int c = i * 64 + lane, row = c / kCPR, col = (c % kCPR) * 8;
      const int t = min(r0 + row, Lr - 1);
      x[i] = *reinterpret_cast<const uint4*>(base + (int64_t)t * kPlaneRow + col);
    }
  }
  __device__ __forceinline__ void store(bf16* lds, int r0, int Lr, int lane) const {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int c = i * 64 + lane, row = c / kCPR, col = (c % kCPR) * 8;
      const bool ok = r0 + row < Lr;
      *reinterpret_cast<uint4*>(lds + row * kPlaneStage + col) =
          uint4{ok ? x[i].x : 0u, ok ? x[i].y : 0u, ok ? x[i].z : 0u, ok ? x[i].w : 0u};
    }
  }
};

// =============================================================================================
// Fused step: row update of the row tile against its window, plus the tile's column partials.
// =============================================================================================
template <typename T, int KT, bool SHIFT>
__global__ __launch_bounds__(kWideThreads) void wide_step_kernel(WideArgs a) {
  __shared__ float red[2][kWideWaves][16];
  const int lane = threadIdx.x & 63, g = lane >> 4, n = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int64_t head;
  int rt;
  if (!wide_work(a.bh * a.nrt, a.nrt, &head, &rt)) return;
  const int Lr = a.Lr, h = a.h;
  const float c2 = a.c2;
  const WideTile wt = wide_tile(rt, Lr, h, wave);
  const int o0 = wt.o0;
  const int64_t tb = head * (int64_t)Lr * kD;
  const T* Qh = static_cast<const T*>(a.Q) + tb;
  const T* Kh = static_cast<const T*>(a.K) + tb;
  const int64_t vo = head * (int64_t)a.Lpad;
  const float* vin = a.v_in + vo;

  // Owned query rows o0 + n (A operand: result rows 4 g + r), window keys across lanes.  The
  // window keys reach the wave two tiles at a time through its own LDS buffer: coalesced row
  // loads (adjacent lanes, adjacent addresses) cost the vector L1 a quarter of the accesses of
  // per-lane fragment loads.  Loads are never conditional (rows clamped into the sequence, chunks
  // past the wave's run re-read its rows) and validity is applied to the results, so a load is
  // waited on only where its data is used and the next chunk stays in flight.
  // fp32 (S3): Q and K arrive as three bf16 planes each (split3_kernel), the window one tile per
  // chunk; bf16: the tensors themselves, two tiles per chunk.
  constexpr bool S3 = std::is_same<T, float>::value;
  constexpr int CT = S3 ? 1 : 2;           // tiles per staged chunk
  __shared__ __attribute__((aligned(16))) T kstage[S3 ? 1 : kWideWaves][S3 ? 4 : 32 * Lds<T>::stride];
  __shared__ __attribute__((aligned(16))) bf16 pstage[S3 ? kWideWaves : 1][S3 ? 16 * kPlaneStage : 8];
  T* sK = kstage[S3 ? 0 : wave];
  bf16* sP = pstage[S3 ? wave : 0];
  const bf16* Qp = static_cast<const bf16*>(a.Qs) + head * (int64_t)Lr * kPlaneRow;
  const bf16* Kp = static_cast<const bf16*>(a.Ks) + head * (int64_t)Lr * kPlaneRow;
  Frag<T> fq;
  Frag<bf16> fq3[3];
  if constexpr (S3) {
    const bf16* qrow = Qp + (int64_t)min(o0 + n, Lr - 1) * kPlaneRow;
#pragma unroll
    for (int p = 0; p < 3; ++p) load_frag_raw(fq3[p], qrow + p * kD, g);
  } else {
    load_frag_raw(fq, Qh + (int64_t)min(o0 + n, Lr - 1) * kD, g);
  }
  constexpr int NC = (KT + CT - 1) / CT;
  WaveStage<T> ns;
  PlaneStage ps;
  float vj[3][2];                          // v of key n of each tile of a chunk, chunk c in slot c % 3
  auto chunk_row0 = [&](int c) { return 16 * (wt.wt0 + min(CT * c, max(wt.wnt - 1, 0))); };
  auto load_vj = [&](int c) {
#pragma unroll
    for (int tt = 0; tt < CT; ++tt) vj[c % 3][tt] = vin[min(chunk_row0(c) + 16 * tt + n, Lr - 1)];
  };
  auto stage_load = [&](int c) {
    if constexpr (S3) ps.load(Kp, chunk_row0(c), Lr, lane);
    else ns.load(Kh, chunk_row0(c), Lr, lane);
  };
  auto stage_store = [&](int c) {
    if constexpr (S3) ps.store(sP, chunk_row0(c), Lr, lane);
    else ns.store(sK, chunk_row0(c), Lr, lane);
  };
  load_vj(0);
  stage_load(0);
  stage_store(0);
  if (NC > 1) {
    load_vj(1);
    stage_load(1);
  }
  __builtin_amdgcn_wave_barrier();

  // Strip of the wave: x[t][r] holds the plan entry 2^(log2(e) S + v_j - shift_i) of row
  // 4 g + r, key n of tile t (0 off the support).  SHIFT (every step after the first): the shift
  // is the previous step's row dual, which enters the matrix-core accumulator; after a column
  // update every column of the previous plan sums to one, so each entry is at most 1 and each
  // row sum lies in [1 / n, n] (n = window length): the exponentials are taken as the tiles
  // arrive, with no maximum pass.  The first step shifts by the exact row maximum instead.
  float x[KT][4];
  float up[4] = {0.f, 0.f, 0.f, 0.f};      // previous row duals of rows 4 g + r
  f32x4 ci = {0.f, 0.f, 0.f, 0.f};
  if constexpr (SHIFT) {
    const f32x4 u4 = load4(a.u_out + vo + min(o0 + 4 * g, a.Lpad - 4));
    const float inv_c2 = 1.f / c2;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      up[r] = u4[r];
      ci[r] = u4[r] * inv_c2;
    }
  }
  // rows 4 g + r: inside the sequence, and their band limits
  bool iv[4];
  int ilo[4], ihi[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int i = o0 + 4 * g + r;
    iv[r] = i < Lr;
    ilo[r] = i - h;
    ihi[r] = i + h;
  }
  float m[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
  float l[4] = {0.f, 0.f, 0.f, 0.f};
  // Every one of the KT tiles is computed (tiles past the wave's run, at most one per wave for a
  // dense support, are masked), so the strip is one branch-free block: the matrix-core chain of
  // tile t + 1 is issued ahead of the vector work on tile t and the two interleave within the
  // wave, instead of the two waves of a SIMD alternating between whole MFMA and VALU phases.
  auto mma = [&](int t) -> f32x4 {
    if constexpr (S3) {
      Frag<bf16> fk3[3];
      const bf16* krow = sP + n * kPlaneStage;
#pragma unroll
      for (int p = 0; p < 3; ++p) load_frag_raw(fk3[p], krow + p * kD, g);
      return dot_tile3(fq3, fk3, ci);
    } else {
      Frag<T> fk;
      lds_frag(fk, sK, 16 * (t & 1) + n, g);
      return dot_tile(fq, fk, ci);
    }
  };
  f32x4 sc[2];
  sc[0] = mma(0);
#pragma unroll
  for (int t = 0; t < KT; ++t) {
    if (t + 1 < KT) {
      if ((t + 1) % CT == 0) {
        // tile t + 1 opens chunk c + 1: into the buffer (whose reads by the earlier products were
        // issued before, and LDS accesses of a wave complete in order), and chunk c + 2 into
        // registers
        const int c1 = (t + 1) / CT;
        __builtin_amdgcn_wave_barrier();
        stage_store(c1);
        __builtin_amdgcn_wave_barrier();
        if (c1 + 1 < NC) {
          load_vj(c1 + 1);
          stage_load(c1 + 1);
        }
      }
      sc[(t + 1) & 1] = mma(t + 1);
    }
    const f32x4 s = sc[t & 1];
    const float vjt = vj[(t / CT) % 3][t % CT];
    const int j = 16 * (wt.wt0 + t) + n;
    const bool jv = (j < Lr) & (t < wt.wnt);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float xv = fmaf(s[r], c2, vjt);
      const bool ok = jv & iv[r] & (j >= ilo[r]) & (j <= ihi[r]);
      if constexpr (SHIFT) {
        x[t][r] = ok ? fast_exp2(xv) : 0.f;
        l[r] += x[t][r];
      } else {
        x[t][r] = ok ? xv : -INFINITY;
        m[r] = fmaxf(m[r], x[t][r]);
      }
    }
  }

  float M[4] = {0.f, 0.f, 0.f, 0.f};
  if constexpr (!SHIFT) {
    // exact row maximum over the workgroup, then the exponentials
#pragma unroll
    for (int r = 0; r < 4; ++r) m[r] = row16_max(m[r]);
    if (n < 4) red[0][wave][4 * g + n] = pick4(m, n);
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float mm = red[0][0][4 * g + r];
#pragma unroll
      for (int w = 1; w < kWideWaves; ++w) mm = fmaxf(mm, red[0][w][4 * g + r]);
      M[r] = (mm > -INFINITY) ? mm : 0.f;   // a row with no support entries
    }
#pragma unroll
    for (int t = 0; t < KT; ++t) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = fast_exp2(x[t][r] - M[r]);   // 0 off the support and past the run
        x[t][r] = p;
        l[r] += p;
      }
    }
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) l[r] = row16_sum(l[r]);
  if (n < 4) red[1][wave][4 * g + n] = pick4(l, n);
  __syncthreads();
  float rinv[4], uu[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float ll = red[1][0][4 * g + r];
#pragma unroll
    for (int w = 1; w < kWideWaves; ++w) ll += red[1][w][4 * g + r];
    const bool live = ll > 0.f;
    // new row dual: shift - log2(row sum of the shifted plan)
    uu[r] = live ? (SHIFT ? up[r] - fast_log2(ll) : -(M[r] + fast_log2(ll))) : 0.f;
    rinv[r] = live ? __builtin_amdgcn_rcpf(ll) : 0.f;
  }

  // column partials of the row-normalised plan: in-lane over the 4 rows, then over the 4 lane
  // groups; a reduced quad of tiles q .. q + 3 leaves tile q + {0, 2, 1, 3}[g] in lane group g
  float* prow = a.part + ((int64_t)head * a.nrt + rt) * a.pw + 16 * (wt.wt0 - wt.t0);
  const int gsel = (g == 1) ? 2 : (g == 2) ? 1 : g;
#pragma unroll
  for (int q = 0; q < KT; q += 4) {
    if (q < wt.wnt) {
      float c[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int t = q + k;
        c[k] = (t < KT) ? fmaf(x[t][3], rinv[3], fmaf(x[t][2], rinv[2], fmaf(x[t][1], rinv[1], x[t][0] * rinv[0])))
                        : 0.f;
      }
      const float s4 = swap16_sum(swap32_sum(c[0], c[1]), swap32_sum(c[2], c[3]));
      const int t = q + gsel;
      if (t < wt.wnt) prow[16 * t + n] = s4;
    }
  }

  if (wave == 0 && n < 4) {
    const int i = o0 + 4 * g + n;
    if (i < Lr) {
      const float ui = pick4(uu, n);
      a.u_out[vo + i] = ui;
      if (a.save_u) a.save_u[head * a.save_stride + i] = ui * kLn2;
    }
  }
  // the column duals this step started from, for the owned tokens (saved duals)
  if (a.save_v && wave == 1 && lane < 16 && o0 + lane < Lr)
    a.save_v[head * a.save_stride + o0 + lane] = vin[o0 + lane] * kLn2;
}

// =============================================================================================
// Column finish: v_j <- v_j - log2(sum of the row tiles' partials, added in a fixed order); exact
// log-sum-exp over the column's support where the summed mass underflows.
// =============================================================================================
template <typename T>
__global__ __launch_bounds__(256) void wide_finish_kernel(WideArgs a) {
  // 64 columns per workgroup; thread group q (of 4) adds a contiguous quarter of each column's
  // row tiles, the quarters are then added in order
  __shared__ float quarter[4][64];
  const int c = threadIdx.x & 63, q = threadIdx.x >> 6;
  const int64_t head = blockIdx.y;
  const int j = blockIdx.x * 64 + c;
  const int h = a.h, jc = min(j, a.Lr - 1);
  // row tiles with a row in the band of key j
  const int rlo = max(0, floor_div(jc - h, 16)), rhi = min(a.nrt - 1, (jc + h) / 16);
  const int nr = rhi - rlo + 1, r0 = rlo + (nr * q) / 4, r1 = rlo + (nr * (q + 1)) / 4;
  const float* ph = a.part + head * (int64_t)a.nrt * a.pw;
  float s = 0.f;
#pragma unroll 8
  for (int rt = r0; rt < r1; ++rt) s += ph[(int64_t)rt * a.pw + jc - 16 * (max(0, 16 * rt - h) >> 4)];
  quarter[q][c] = s;
  __syncthreads();
  if (q != 0 || j >= a.Lr) return;
  s = ((quarter[0][c] + quarter[1][c]) + quarter[2][c]) + quarter[3][c];
  const int64_t vo = head * (int64_t)a.Lpad;
  float v;
  if (s >= 0x1p-60f) {
    v = a.v_in[vo + j] - fast_log2(s);
  } else {
    const int64_t tb = head * (int64_t)a.Lr * kD;
    v = exact_column<T>(j, a.u_out + vo, static_cast<const T*>(a.Q) + tb,
                        static_cast<const T*>(a.K) + tb, a.Lr, h, a.c2);
  }
  a.v_out[vo + j] = v;
  if (a.save_v) a.save_v[head * a.save_stride + j] = v * kLn2;
}

// =============================================================================================
// Output and VJP passes.
// =============================================================================================
enum WidePass : int { kWOut = 0, kWA, kWB, kWC, kWD, kWE };

// A forms dV = P22^T dO and takes dv2_j = sum_i P22 g = V_j . dV_j, without g; B given the
// forward's output (DELTA) takes sum_j P22_ij g_ij = dO_i . O_i, without g or V's window.
template <int P, bool DELTA = false> struct WideTraits {
  static constexpr bool delta = DELTA && P == kWB;
  static constexpr bool owns_keys = (P == kWA || P == kWC || P == kWE);
  static constexpr bool needs_g = ((P == kWB) && !delta) || P == kWD || P == kWE;
  static constexpr int nstage = (P == kWC || delta) ? 1 : 2;   // window tensors staged per wave
  // staged tensor the contraction reads: 0 = the score operand, 1 = the second tensor, -1 none
  static constexpr int csrc = (P == kWOut || P == kWA) ? 1 : (P == kWD || P == kWE) ? 0 : -1;
  static constexpr int nacc = (P == kWD) ? 2 : (csrc >= 0) ? 1 : 0;   // 16 x 64 accumulators
  static constexpr bool has_red = (P != kWOut && P != kWA && P != kWE);
};

template <typename T, int P, bool DELTA>
struct WideSmem {
  using TR = WideTraits<P, DELTA>;
  static constexpr int kStageElems = 32 * Lds<T>::stride;   // one staged tensor of one wave
  static constexpr int kStageBytes = kWideWaves * TR::nstage * kStageElems * (int)sizeof(T);
  static constexpr int kRedFloats = (TR::nacc * 16 + 1) * 64;   // one wave's partials
  static constexpr int kRedBytes = kWideWaves * kRedFloats * 4;
  static constexpr int kBytes = kStageBytes > kRedBytes ? kStageBytes : kRedBytes;
};

template <typename T, int P, bool D4, bool DELTA = false>
__global__ __launch_bounds__(kWideThreads, (WideTraits<P, DELTA>::delta ? 4 : 1))
void wide_pass_kernel(WideArgs a) {
  using TR = WideTraits<P, DELTA>;
  using SM = WideSmem<T, P, DELTA>;
  __shared__ __attribute__((aligned(16))) unsigned char smem[SM::kBytes];
  const int lane = threadIdx.x & 63, g = lane >> 4, n = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int64_t head;
  int rt;
  if (!wide_work(a.bh * a.nrt, a.nrt, &head, &rt)) return;
  const int Lr = a.Lr, h = a.h;
  const float c2 = a.c2;
  const WideTile wt = wide_tile(rt, Lr, h, wave);
  const int o0 = wt.o0, o = o0 + n;
  const int64_t tb = head * (int64_t)Lr * kD;
  const T* Qp = static_cast<const T*>(a.Q) + tb;
  const T* Kp = static_cast<const T*>(a.K) + tb;
  const T* Vp = static_cast<const T*>(a.V) + tb;
  const T* dOp = static_cast<const T*>(a.dO) + tb;
  const T* own_s = TR::owns_keys ? Kp : Qp;
  const T* own_g = TR::owns_keys ? Vp : dOp;
  const T* winA = TR::owns_keys ? Qp : Kp;                         // score operand
  const T* winB = (P == kWOut) ? Vp : (TR::owns_keys ? dOp : Vp);   // value-score / value operand
  const int64_t vo = head * (int64_t)a.Lpad;
  auto vec = [&](int which) -> const float* { return a.ws + which * a.vec_stride + vo; };

  T* sA = reinterpret_cast<T*>(smem) + wave * TR::nstage * SM::kStageElems;
  T* sB = sA + SM::kStageElems;

  // (loads are never conditional: rows clamped into the sequence, results masked where used)
  Frag<T> fo, fog, foo;
  const int oc = min(o, Lr - 1);
  load_frag_raw(fo, own_s + (int64_t)oc * kD, g);
  if (TR::needs_g || TR::delta) load_frag_raw(fog, own_g + (int64_t)oc * kD, g);
  if constexpr (TR::delta) load_frag_raw(foo, static_cast<const T*>(a.O) + tb + (int64_t)oc * kD, g);

  // owned-token vectors (o < Lpad always; padding entries are zero)
  float own_u2 = 0.f, own_v2 = 0.f, ox0 = 0.f, ox1 = 0.f, ox2 = 0.f, ox3 = 0.f;
  if constexpr (P == kWOut) {
    own_u2 = a.fu[vo + o];
  } else if constexpr (TR::owns_keys) {
    own_v2 = vec(kV2)[o];
    if constexpr (P == kWC) {
      ox0 = D4 ? vec(kV1)[o] : vec(kEE)[o];                 // v1 (direct) or E
    } else if constexpr (P == kWE) {
      ox0 = vec(kDV2)[o];                                   // D
      ox1 = D4 ? vec(kV1)[o] : vec(kEE)[o];                 // v1 or E
      ox2 = D4 ? vec(kDV1)[o] : vec(kFF)[o];                // dv1 or F
      ox3 = D4 ? vec(kV0)[o] : vec(kEG)[o];                 // v0 or G
    }
  } else {
    own_u2 = vec(kU2)[o];
    if constexpr (P == kWD) {
      ox0 = vec(kDU2)[o];                                   // A = du2
      ox1 = D4 ? vec(kU1)[o] : vec(kEB)[o];                 // u1 (direct) or B
    }
  }
  const float* fv = (P == kWOut) ? a.fv + vo : nullptr;

  float red = 0.f;
  f32x4 acc[4], acc2[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) acc[b] = acc2[b] = f32x4{0.f, 0.f, 0.f, 0.f};

  // window-side vectors of a tile: 4 consecutive tokens per lane (clamped into the padding)
  constexpr int NWV = (P == kWOut || P == kWA) ? 1 : (P == kWB || P == kWC) ? 2 : (P == kWD) ? 5 : 4;
  auto load_vecs = [&](int wb, f32x4 (&v)[NWV]) {
    const int wc = min(wb, a.Lpad - 4);
    if constexpr (P == kWOut) {
      v[0] = load4(fv + wc);
    } else if constexpr (TR::owns_keys) {
      v[0] = load4(vec(kU2) + wc);
      if constexpr (P == kWC) v[1 % NWV] = load4(vec(kDU2) + wc);
      if constexpr (P == kWE) {
        v[1 % NWV] = load4(vec(kDU2) + wc);                          // A = du2
        v[2 % NWV] = load4(vec(D4 ? kU1 : kEB) + wc);                // u1 or B
        v[3 % NWV] = load4(vec(D4 ? kDU1 : kCC) + wc);               // du1 or C
      }
    } else {
      v[0] = load4(vec(kV2) + wc);
      if constexpr (P == kWB) v[1 % NWV] = load4(vec(kDV2) + wc);
      if constexpr (P == kWD) {
        v[1 % NWV] = load4(vec(kDV2) + wc);                          // D
        v[2 % NWV] = load4(vec(D4 ? kV1 : kEE) + wc);                // v1 or E
        v[3 % NWV] = load4(vec(D4 ? kDV1 : kFF) + wc);               // dv1 or F
        v[4 % NWV] = load4(vec(D4 ? kV0 : kEG) + wc);                // v0 or G
      }
    }
  };

  WaveStage<T> na, nb;
  const int nch = (wt.wnt + 1) >> 1;     // chunks of two tiles
  int w0 = 16 * wt.wt0;
  na.load(winA, w0, Lr, lane);
  if (TR::nstage == 2) nb.load(winB, w0, Lr, lane);
  na.store(sA, w0, Lr, lane);
  if (TR::nstage == 2) nb.store(sB, w0, Lr, lane);
  __builtin_amdgcn_wave_barrier();
  for (int c = 0; c < nch; ++c, w0 += 32) {
    // this chunk's window vectors, then the next chunk's rows (issued unconditionally, past the
    // run they read rows clamped into the sequence): waiting for the vectors leaves the rows in
    // flight
    f32x4 wvv[2][NWV];
    load_vecs(w0 + 4 * g, wvv[0]);
    load_vecs(w0 + 16 + 4 * g, wvv[1]);
    na.load(winA, w0 + 32, Lr, lane);
    if (TR::nstage == 2) nb.load(winB, w0 + 32, Lr, lane);
    float z1[2][4], z2[2][4];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
      for (int r = 0; r < 4; ++r) z1[tt][r] = z2[tt][r] = 0.f;
      if (2 * c + tt >= wt.wnt) continue;
      const int wb = w0 + 16 * tt + 4 * g;          // this lane's window tokens wb + r
      const f32x4 (&wv)[NWV] = wvv[tt];
      Frag<T> fw;
      lds_frag(fw, sA, 16 * tt + n, g);
      const f32x4 sc = dot_tile(fw, fo);
      f32x4 gv = {0.f, 0.f, 0.f, 0.f};
      if constexpr (TR::needs_g) {
        Frag<T> fwg;
        lds_frag(fwg, sB, 16 * tt + n, g);
        gv = dot_tile(fwg, fog);
      }
      if constexpr (P == kWOut) {
        const f32x4 wv2 = wv[0];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float p = fast_exp2(fmaf(sc[r], c2, own_u2 + wv2[r]));
          z1[tt][r] = in_band(wb + r, o, h, Lr) ? p : 0.f;
        }
      } else if constexpr (TR::owns_keys) {
        const f32x4 wu2 = wv[0], wa = wv[1 % NWV], wbv = wv[2 % NWV], wc = wv[3 % NWV];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const bool keep = in_band(wb + r, o, h, Lr);
          const float xq = fmaf(sc[r], c2, wu2[r]);                 // log2(e) S + u2_i
          const float p22 = fast_exp2(xq + own_v2);
          if constexpr (P == kWA) {
            z1[tt][r] = keep ? p22 : 0.f;
          } else if constexpr (P == kWC) {
            const float pw = D4 ? fast_exp2(xq + ox0) : p22;        // P21 (direct) or P22
            red = keep ? fmaf(pw, wa[r], red) : red;
          } else {  // E
            float ds;
            if constexpr (D4) {
              const float xs = sc[r] * c2;
              const float p21 = fast_exp2(xq + ox1);
              const float p11 = fast_exp2(xs + wbv[r] + ox1);
              const float p10 = fast_exp2(xs + wbv[r] + ox3);
              ds = p22 * (gv[r] - ox0) - p21 * wa[r] - p11 * ox2 - p10 * wc[r];
            } else {
              ds = p22 * (gv[r] - ox0 - wa[r] * ox1 - wbv[r] * ox2 - wc[r] * ox3);
            }
            z1[tt][r] = keep ? ds : 0.f;
          }
        }
      } else {
        const f32x4 wv2 = wv[0], wd = wv[1 % NWV], we = wv[2 % NWV], wf = wv[3 % NWV], wg = wv[4 % NWV];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const bool keep = in_band(wb + r, o, h, Lr);
          const float xs = sc[r] * c2;
          const float p22 = fast_exp2(xs + own_u2 + wv2[r]);
          if constexpr (P == kWB) {
            red = keep ? fmaf(p22, TR::delta ? -wd[r] : gv[r] - wd[r], red) : red;
          } else {  // D
            if constexpr (D4) {
              const float p21 = fast_exp2(xs + own_u2 + we[r]);
              const float p11 = fast_exp2(xs + ox1 + we[r]);
              const float p10 = fast_exp2(xs + ox1 + wg[r]);
              red = keep ? fmaf(p11, wf[r], red) : red;
              z1[tt][r] = keep ? p22 * (gv[r] - wd[r]) - p21 * ox0 - p11 * wf[r] : 0.f;
              z2[tt][r] = keep ? p10 : 0.f;
            } else {
              red = keep ? fmaf(p22, wf[r], red) : red;
              z1[tt][r] = keep ? p22 * (gv[r] - wd[r] - ox0 * we[r] - ox1 * wf[r]) : 0.f;
              z2[tt][r] = keep ? p22 * wg[r] : 0.f;
            }
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);   // one tile's operands live at a time
    }
    if constexpr (TR::csrc >= 0) {
      const T* src = (TR::csrc == 0) ? sA : sB;
      if constexpr (P == kWD) contract2(acc, acc2, src, z1, z2, g, n);
      else contract(acc, src, z1, g, n);
    }
    __builtin_amdgcn_wave_barrier();
    na.store(sA, w0 + 32, Lr, lane);
    if (TR::nstage == 2) nb.store(sB, w0 + 32, Lr, lane);
    __builtin_amdgcn_wave_barrier();
  }

  // ---- combine the waves' partials (fixed order) in wave 0 ----
  if constexpr (TR::has_red) red = group_sum(red);
  __syncthreads();                      // every wave is done with its staging area
  float* rbuf = reinterpret_cast<float*>(smem);
  if (wave != 0) {
    float* mine = rbuf + wave * SM::kRedFloats;
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if constexpr (TR::nacc >= 1) mine[(4 * b + r) * 64 + lane] = acc[b][r];
        if constexpr (TR::nacc >= 2) mine[(16 + 4 * b + r) * 64 + lane] = acc2[b][r];
      }
    if constexpr (TR::has_red) mine[TR::nacc * 16 * 64 + lane] = red;
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll 1
  for (int w = 1; w < kWideWaves; ++w) {
    const float* theirs = rbuf + w * SM::kRedFloats;
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if constexpr (TR::nacc >= 1) acc[b][r] += theirs[(4 * b + r) * 64 + lane];
        if constexpr (TR::nacc >= 2) acc2[b][r] += theirs[(16 + 4 * b + r) * 64 + lane];
      }
    if constexpr (TR::has_red) red += theirs[TR::nacc * 16 * 64 + lane];
  }

  if constexpr (TR::delta) red += group_sum(frag_dot(fog, foo));   // + dO_o . O_o
  const bool valid = o < Lr;
  if (!valid) return;
  float* ws = a.ws;
  const int64_t ob = vo + o;
  T* out_row = static_cast<T*>(a.out0) + tb + (int64_t)o * kD;
  if constexpr (P == kWOut) {
    store_row(out_row, acc, 1.f, g);
  } else if constexpr (P == kWA) {
    // dv2 = V . dV over the lane's columns 16 b + 4 g + r, summed over the lane groups
    float vd = 0.f;
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) vd = fmaf((float)Vp[(int64_t)o * kD + 16 * b + 4 * g + r], acc[b][r], vd);
    vd = group_sum(vd);
    if (g == 0) ws[kDV2 * a.vec_stride + ob] = vd;
    store_row(out_row, acc, 1.f, g);
  } else if constexpr (P == kWB) {
    if (g == 0) ws[kDU2 * a.vec_stride + ob] = red;
  } else if constexpr (P == kWC) {
    const float dv1 = D4 ? -red : -ox0 * red;
    if (g == 0) {
      ws[kDV1 * a.vec_stride + ob] = dv1;
      ws[kFF * a.vec_stride + ob] = dv1 * ws[kEE * a.vec_stride + ob];
    }
  } else if constexpr (P == kWD) {
    const float eb = ws[kEB * a.vec_stride + ob];
    const float du1 = D4 ? -red : -eb * red;
    const float cc = D4 ? du1 : du1 * eb;            // coefficient of Z2 in dS
    if (g == 0) {
      ws[kDU1 * a.vec_stride + ob] = du1;
      ws[kCC * a.vec_stride + ob] = du1 * eb;
    }
    f32x4 r4[4];
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) r4[b][r] = acc[b][r] - cc * acc2[b][r];
    store_row(out_row, r4, a.s, g);
  } else {  // E
    store_row(out_row, acc, a.s, g);
  }
}

// =============================================================================================
// General tail depth R: the exact one-reference-tile adjoint through an R-step tail.
// [technical summaries §2.1: R differentiable tail steps from the stopped base state; §2.2 and
// abstract: every staircase plan is the reference tile P = P^(R,R) times row and column factors]
// With EU_a = exp(u^(a) - u^(R)), EV_b = exp(v^(b) - v^(R)), the vector cotangents are reductions
// of the reference tile, level by level (F_a = dv^(a) EV_a, C_a = du^(a) EU_a):
//   A (owns keys)     dv^(R)_j = sum_i P g                          F_R = dv^(R);  dV = P^T dO
//   B (owns queries)  du^(R)_i = sum_j P (g - F_R(j))               C_R = du^(R)
//   for a = R-1 .. 1:
//   C (owns keys)     dv^(a)_j = -EV_a(j) sum_i P C_{a+1}(i)        F_a = dv^(a) EV_a
//   D (owns queries)  du^(a)_i = -EU_a(i) sum_j P F_a(j)            C_a = du^(a) EU_a
//   Q (owns queries)  dQ_i = s sum_j P M k_j,  E (owns keys) dK_j = s sum_i P M q_i, with the
//                     modifier M = g - sum_a [EU_a(i) F_a(j) + C_a(i) EV_{a-1}(j)] (2 R terms).
// (R = 2 gives A = du2, B, C, D, E, F, G of the two-level passes.)
// =============================================================================================
struct TailVec {
  int R;
  __device__ int u() const { return 0; }
  __device__ int v() const { return 1; }
  __device__ int eu(int a) const { return 2 + (a - 1); }        // a = 1..R
  __device__ int ev(int b) const { return 2 + R + b; }          // b = 0..R
  __device__ int f(int a) const { return 3 + 2 * R + (a - 1); }
  __device__ int c(int a) const { return 3 + 3 * R + (a - 1); }
};

// duals (natural units, [bh][n_duals(R)][Lr]: v0, u1, v1, .., uR, vR, or u0, v0 for R = 0) -> the
// tail vectors
__global__ void tail_prep_kernel(const float* __restrict__ duals, float* __restrict__ ws, int R,
                                 int Lr, int Lpad, int64_t vec_stride) {
  const int64_t head = blockIdx.y;
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= Lpad) return;
  const TailVec tv{R};
  const int64_t ob = head * Lpad + t;
  auto at = [&](int k) -> float& { return ws[k * vec_stride + ob]; };
  const bool ok = t < Lr;
  const int nd = (R == 0) ? 2 : 2 * R + 1;   // n_duals(R)
  const float* dh = duals + head * nd * (int64_t)Lr;
  auto dual = [&](int slot) { return ok ? dh[(int64_t)slot * Lr + t] : 0.f; };
  const float uR = dual(nd - 2), vR = dual(nd - 1);
  at(tv.u()) = uR * kLog2e;
  at(tv.v()) = vR * kLog2e;
  for (int a = 1; a <= R; ++a) {
    at(tv.eu(a)) = ok ? expf(dual(2 * a - 1) - uR) : 0.f;
    at(tv.f(a)) = 0.f;
    at(tv.c(a)) = 0.f;
  }
  if (R == 0) return;   // no levels: the modifier is g itself
  for (int b = 0; b <= R; ++b) at(tv.ev(b)) = ok ? expf(dual(2 * b) - vR) : 0.f;
}

enum TailPass : int { kTA = 0, kTB, kTC, kTD, kTQ, kTE };

// A forms dV = P^T dO and takes dv^(R)_j = sum_i P g = V_j . dV_j, without g.
template <int GP> struct TailTraits {
  static constexpr bool owns_keys = (GP == kTA || GP == kTC || GP == kTE);
  static constexpr bool needs_g = (GP != kTA && GP != kTC && GP != kTD);
  static constexpr int nstage = (needs_g || GP == kTA) ? 2 : 1;
  // staged tensor the contraction reads: 0 = the score operand, 1 = the second tensor, -1 none
  static constexpr int csrc = (GP == kTA) ? 1 : (GP == kTQ || GP == kTE) ? 0 : -1;
  static constexpr bool has_red = (GP == kTB || GP == kTC || GP == kTD);
};

// RT: the tail depth for the dQ and dK passes (0..4 at compile time: their 2 RT modifier terms
// and owned factors stay in registers, none at depth 0, where M = g); RT = -1: any depth, the
// modifier accumulated level by level with its factors read per tile; 0 for the level passes,
// which take R and the level at run time.
template <typename T, int GP, int RT>
__global__ __launch_bounds__(kWideThreads) void tail_pass_kernel(WideArgs a) {
  using TR = TailTraits<GP>;
  constexpr int kStageElems = 32 * Lds<T>::stride;
  constexpr int kStageBytes = kWideWaves * TR::nstage * kStageElems * (int)sizeof(T);
  constexpr int kRedFloats = ((TR::csrc >= 0 ? 16 : 0) + 1) * 64;
  constexpr int kRedBytes = kWideWaves * kRedFloats * 4;
  __shared__ __attribute__((aligned(16))) unsigned char smem[kStageBytes > kRedBytes ? kStageBytes : kRedBytes];
  constexpr int NM = (GP == kTQ || GP == kTE) && RT > 0 ? RT : 0;   // register-held modifier levels
  constexpr bool kLoopM = (GP == kTQ || GP == kTE) && RT < 0;        // modifier levels at run time
  const int lane = threadIdx.x & 63, g = lane >> 4, n = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int64_t head;
  int rt;
  if (!wide_work(a.bh * a.nrt, a.nrt, &head, &rt)) return;
  const int Lr = a.Lr, h = a.h;
  const float c2 = a.c2;
  const TailVec tv{a.R};
  const int lev = a.level;
  const WideTile wt = wide_tile(rt, Lr, h, wave);
  const int o0 = wt.o0, o = o0 + n;
  const int64_t tb = head * (int64_t)Lr * kD;
  const T* Qp = static_cast<const T*>(a.Q) + tb;
  const T* Kp = static_cast<const T*>(a.K) + tb;
  const T* Vp = static_cast<const T*>(a.V) + tb;
  const T* dOp = static_cast<const T*>(a.dO) + tb;
  const T* own_s = TR::owns_keys ? Kp : Qp;
  const T* own_g = TR::owns_keys ? Vp : dOp;
  const T* winA = TR::owns_keys ? Qp : Kp;
  const T* winB = TR::owns_keys ? dOp : Vp;
  const int64_t vo = head * (int64_t)a.Lpad;
  auto vec = [&](int which) -> float* { return a.ws + which * a.vec_stride + vo; };

  T* sA = reinterpret_cast<T*>(smem) + wave * TR::nstage * kStageElems;
  T* sB = sA + kStageElems;
  Frag<T> fo, fog;
  const int oc = min(o, Lr - 1);
  load_frag_raw(fo, own_s + (int64_t)oc * kD, g);
  if constexpr (TR::needs_g) load_frag_raw(fog, own_g + (int64_t)oc * kD, g);

  // owned-token values: its dual of the reference tile, and the modifier factors
  const float own_d = vec(TR::owns_keys ? tv.v() : tv.u())[o];
  float own_x[NM > 0 ? NM : 1], own_y[NM > 0 ? NM : 1];
#pragma unroll
  for (int k = 0; k < NM; ++k) {
    if constexpr (GP == kTQ) {
      own_x[k] = vec(tv.eu(k + 1))[o];          // EU_a(i)
      own_y[k] = vec(tv.c(k + 1))[o];           // C_a(i)
    } else {
      own_x[k] = vec(tv.f(k + 1))[o];           // F_a(j)
      own_y[k] = vec(tv.ev(k))[o];              // EV_{a-1}(j)
    }
  }
  // window vector of the level passes
  const int wsel = (GP == kTB) ? tv.f(a.R) : (GP == kTC) ? tv.c(lev + 1) : (GP == kTD) ? tv.f(lev) : 0;

  float red = 0.f;
  f32x4 acc[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};

  WaveStage<T> na, nb;
  const int nch = (wt.wnt + 1) >> 1;
  int w0 = 16 * wt.wt0;
  na.load(winA, w0, Lr, lane);
  if (TR::nstage == 2) nb.load(winB, w0, Lr, lane);
  na.store(sA, w0, Lr, lane);
  if (TR::nstage == 2) nb.store(sB, w0, Lr, lane);
  __builtin_amdgcn_wave_barrier();
  for (int c = 0; c < nch; ++c, w0 += 32) {
    na.load(winA, w0 + 32, Lr, lane);
    if (TR::nstage == 2) nb.load(winB, w0 + 32, Lr, lane);
    float z[2][4];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
      for (int r = 0; r < 4; ++r) z[tt][r] = 0.f;
      if (2 * c + tt >= wt.wnt) continue;
      const int wb = w0 + 16 * tt + 4 * g;        // this lane's window tokens wb + r
      const int wc = min(wb, a.Lpad - 4);
      Frag<T> fw;
      lds_frag(fw, sA, 16 * tt + n, g);
      const f32x4 sc = dot_tile(fw, fo);
      f32x4 gv = {0.f, 0.f, 0.f, 0.f};
      if constexpr (TR::needs_g) {
        Frag<T> fwg;
        lds_frag(fwg, sB, 16 * tt + n, g);
        gv = dot_tile(fwg, fog);
      }
      const f32x4 wd = load4(vec(TR::owns_keys ? tv.u() : tv.v()) + wc);
      f32x4 wsv = {0.f, 0.f, 0.f, 0.f};
      if constexpr (GP == kTB || GP == kTC || GP == kTD) wsv = load4(vec(wsel) + wc);
      f32x4 wx[NM > 0 ? NM : 1], wy[NM > 0 ? NM : 1];
#pragma unroll
      for (int k = 0; k < NM; ++k) {
        if constexpr (GP == kTQ) {
          wx[k] = load4(vec(tv.f(k + 1)) + wc);   // F_a(j)
          wy[k] = load4(vec(tv.ev(k)) + wc);      // EV_{a-1}(j)
        } else {
          wx[k] = load4(vec(tv.eu(k + 1)) + wc);  // EU_a(i)
          wy[k] = load4(vec(tv.c(k + 1)) + wc);   // C_a(i)
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool keep = in_band(wb + r, o, h, Lr);
        const float p = fast_exp2(fmaf(sc[r], c2, own_d + wd[r]));
        if constexpr (GP == kTA) {
          z[tt][r] = keep ? p : 0.f;
        } else if constexpr (GP == kTB) {
          red = keep ? fmaf(p, gv[r] - wsv[r], red) : red;
        } else if constexpr (GP == kTC || GP == kTD) {
          red = keep ? fmaf(p, wsv[r], red) : red;
        } else {
          float m = gv[r];
#pragma unroll
          for (int k = 0; k < NM; ++k) {
            if constexpr (GP == kTQ) m -= own_x[k] * wx[k][r] + own_y[k] * wy[k][r];
            else m -= wx[k][r] * own_x[k] + wy[k][r] * own_y[k];
          }
          z[tt][r] = keep ? p * m : 0.f;     // (kLoopM: the modifier is applied below)
        }
      }
      if constexpr (kLoopM) {
        // z = p g so far: subtract p sum_a [EU_a(i) F_a(j) + C_a(i) EV_{a-1}(j)], level by level
        f32x4 msub = {0.f, 0.f, 0.f, 0.f};
        for (int lv = 1; lv <= a.R; ++lv) {
          if constexpr (GP == kTQ) {
            const float ox = vec(tv.eu(lv))[o], oy = vec(tv.c(lv))[o];
            const f32x4 fx = load4(vec(tv.f(lv)) + wc), fy = load4(vec(tv.ev(lv - 1)) + wc);
#pragma unroll
            for (int r = 0; r < 4; ++r) msub[r] += ox * fx[r] + oy * fy[r];
          } else {
            const float ox = vec(tv.f(lv))[o], oy = vec(tv.ev(lv - 1))[o];
            const f32x4 fx = load4(vec(tv.eu(lv)) + wc), fy = load4(vec(tv.c(lv)) + wc);
#pragma unroll
            for (int r = 0; r < 4; ++r) msub[r] += fx[r] * ox + fy[r] * oy;
          }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const bool keep = in_band(wb + r, o, h, Lr);
          const float p = fast_exp2(fmaf(sc[r], c2, own_d + wd[r]));
          z[tt][r] = keep ? p * (gv[r] - msub[r]) : 0.f;
        }
      }
      __builtin_amdgcn_sched_barrier(0);   // one tile's operands live at a time
    }
    if constexpr (TR::csrc >= 0) contract(acc, (TR::csrc == 0) ? sA : sB, z, g, n);
    __builtin_amdgcn_wave_barrier();
    na.store(sA, w0 + 32, Lr, lane);
    if (TR::nstage == 2) nb.store(sB, w0 + 32, Lr, lane);
    __builtin_amdgcn_wave_barrier();
  }

  // ---- combine the waves' partials (fixed order) in wave 0 ----
  if constexpr (TR::has_red) red = group_sum(red);
  __syncthreads();
  float* rbuf = reinterpret_cast<float*>(smem);
  constexpr int NA = (TR::csrc >= 0) ? 16 : 0;
  if (wave != 0) {
    float* mine = rbuf + wave * kRedFloats;
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if constexpr (NA > 0) mine[(4 * b + r) * 64 + lane] = acc[b][r];
    if constexpr (TR::has_red) mine[NA * 64 + lane] = red;
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll 1
  for (int w = 1; w < kWideWaves; ++w) {
    const float* theirs = rbuf + w * kRedFloats;
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if constexpr (NA > 0) acc[b][r] += theirs[(4 * b + r) * 64 + lane];
    if constexpr (TR::has_red) red += theirs[NA * 64 + lane];
  }
  if (o >= Lr) return;
  T* out_row = static_cast<T*>(a.out0) + tb + (int64_t)o * kD;
  if constexpr (GP == kTA) {
    // dv^(R) = V . dV over the lane's columns 16 b + 4 g + r, summed over the lane groups (the
    // four lanes of a key share its validity)
    float vd = 0.f;
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) vd = fmaf((float)Vp[(int64_t)o * kD + 16 * b + 4 * g + r], acc[b][r], vd);
    vd = group_sum(vd);
    if (g == 0 && a.R > 0) vec(tv.f(a.R))[o] = vd;          // dv^(R) (EV_R = 1)
    store_row(out_row, acc, 1.f, g);                        // dV
  } else if constexpr (GP == kTB) {
    if (g == 0) vec(tv.c(a.R))[o] = red;                    // du^(R) (EU_R = 1)
  } else if constexpr (GP == kTC) {
    const float e = vec(tv.ev(lev))[o];
    if (g == 0) vec(tv.f(lev))[o] = -e * e * red;           // dv^(a) = -EV_a red, F_a = dv^(a) EV_a
  } else if constexpr (GP == kTD) {
    const float e = vec(tv.eu(lev))[o];
    if (g == 0) vec(tv.c(lev))[o] = -e * e * red;           // du^(a) = -EU_a red, C_a = du^(a) EU_a
  } else {
    store_row(out_row, acc, a.s, g);                        // dQ or dK
  }
}

// =============================================================================================
// launchers
// =============================================================================================
static dim3 wide_grid(const WideArgs& a) {
  const int64_t nwork = a.bh * (int64_t)a.nrt;
  return dim3((unsigned)(8 * ((nwork + 7) / 8)), 1, 1);
}

template <typename T, bool SHIFT>
static void wide_step_t(int kt, const WideArgs& a, hipStream_t st) {
  const dim3 grid = wide_grid(a), block(kWideThreads);
  switch (kt) {
    case 4: wide_step_kernel<T, 4, SHIFT><<<grid, block, 0, st>>>(a); break;
    case 8: wide_step_kernel<T, 8, SHIFT><<<grid, block, 0, st>>>(a); break;
    case 12: wide_step_kernel<T, 12, SHIFT><<<grid, block, 0, st>>>(a); break;
    case 16: wide_step_kernel<T, 16, SHIFT><<<grid, block, 0, st>>>(a); break;
    case 24: wide_step_kernel<T, 24, SHIFT><<<grid, block, 0, st>>>(a); break;
    default: wide_step_kernel<T, 33, SHIFT><<<grid, block, 0, st>>>(a); break;
  }
}

hipError_t launch_wide_step(int elt, int kt, bool first, const WideArgs& a, hipStream_t st) {
  if (kt != 4 && kt != 8 && kt != 12 && kt != 16 && kt != 24 && kt != 33) return hipErrorInvalidValue;
  if (elt == 1) {
    if (first) wide_step_t<bf16, false>(kt, a, st);
    else wide_step_t<bf16, true>(kt, a, st);
  } else {
    if (first) wide_step_t<float, false>(kt, a, st);
    else wide_step_t<float, true>(kt, a, st);
  }
  return hipGetLastError();
}

hipError_t launch_split3(const float* x, void* out, int64_t rows, hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  const int64_t n = rows * (kD / 4);
  split3_kernel<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(x, static_cast<bf16*>(out), rows);
  return hipGetLastError();
}

hipError_t launch_wide_finish(int elt, const WideArgs& a, hipStream_t st) {
  const dim3 grid((unsigned)((a.Lr + 63) / 64), (unsigned)a.bh);
  if (elt == 1) wide_finish_kernel<bf16><<<grid, dim3(256), 0, st>>>(a);
  else wide_finish_kernel<float><<<grid, dim3(256), 0, st>>>(a);
  return hipGetLastError();
}

template <typename T, bool D4>
static void wide_pass_t(int pass, const WideArgs& a, hipStream_t st) {
  const dim3 grid = wide_grid(a), block(kWideThreads);
  switch (pass) {
    case kWOut: wide_pass_kernel<T, kWOut, false><<<grid, block, 0, st>>>(a); break;
    case kWA: wide_pass_kernel<T, kWA, false><<<grid, block, 0, st>>>(a); break;
    case kWB:
      if (a.O != nullptr) wide_pass_kernel<T, kWB, false, true><<<grid, block, 0, st>>>(a);
      else wide_pass_kernel<T, kWB, false><<<grid, block, 0, st>>>(a);
      break;
    case kWC: wide_pass_kernel<T, kWC, D4><<<grid, block, 0, st>>>(a); break;
    case kWD: wide_pass_kernel<T, kWD, D4><<<grid, block, 0, st>>>(a); break;
    default: wide_pass_kernel<T, kWE, D4><<<grid, block, 0, st>>>(a); break;
  }
}

hipError_t launch_tail_prep(const float* duals, float* ws, int R, const Geometry& g, hipStream_t st) {
  const int64_t vs = g.bh * (int64_t)g.Lpad;
  tail_prep_kernel<<<dim3((unsigned)((g.Lpad + 255) / 256), (unsigned)g.bh), dim3(256), 0, st>>>(
      duals, ws, R, g.Lr, g.Lpad, vs);
  return hipGetLastError();
}

template <typename T, int GP>
static void tail_pass_r(const WideArgs& a, hipStream_t st) {
  const dim3 grid = wide_grid(a), block(kWideThreads);
  switch (a.R) {
    case 0: tail_pass_kernel<T, GP, 0><<<grid, block, 0, st>>>(a); break;    // M = g
    case 1: tail_pass_kernel<T, GP, 1><<<grid, block, 0, st>>>(a); break;
    case 2: tail_pass_kernel<T, GP, 2><<<grid, block, 0, st>>>(a); break;
    case 3: tail_pass_kernel<T, GP, 3><<<grid, block, 0, st>>>(a); break;
    case 4: tail_pass_kernel<T, GP, 4><<<grid, block, 0, st>>>(a); break;
    default: tail_pass_kernel<T, GP, -1><<<grid, block, 0, st>>>(a); break;
  }
}

template <typename T>
static void tail_pass_t(int pass, const WideArgs& a, hipStream_t st) {
  const dim3 grid = wide_grid(a), block(kWideThreads);
  switch (pass) {
    case kTA: tail_pass_kernel<T, kTA, 0><<<grid, block, 0, st>>>(a); break;
    case kTB: tail_pass_kernel<T, kTB, 0><<<grid, block, 0, st>>>(a); break;
    case kTC: tail_pass_kernel<T, kTC, 0><<<grid, block, 0, st>>>(a); break;
    case kTD: tail_pass_kernel<T, kTD, 0><<<grid, block, 0, st>>>(a); break;
    case kTQ: tail_pass_r<T, kTQ>(a, st); break;
    default: tail_pass_r<T, kTE>(a, st); break;
  }
}

hipError_t launch_tail_pass(int elt, int pass, const WideArgs& a, hipStream_t st) {
  if (pass < kTA || pass > kTE || a.R < 0 || a.R > kTailMaxR) return hipErrorInvalidValue;
  if (a.R == 0 && (pass == kTB || pass == kTC || pass == kTD)) return hipErrorInvalidValue;
  if ((pass == kTC || pass == kTD) && (a.level < 1 || a.level >= a.R)) return hipErrorInvalidValue;
  if (elt == 1) tail_pass_t<bf16>(pass, a, st);
  else tail_pass_t<float>(pass, a, st);
  return hipGetLastError();
}

hipError_t launch_wide_pass(int elt, int pass, bool d4, const WideArgs& a, hipStream_t st) {
  if (pass < kWOut || pass > kWE) return hipErrorInvalidValue;
  if (elt == 1) {
    if (d4) wide_pass_t<bf16, true>(pass, a, st);
    else wide_pass_t<bf16, false>(pass, a, st);
  } else {
    if (d4) wide_pass_t<float, true>(pass, a, st);
    else wide_pass_t<float, false>(pass, a, st);
  }
  return hipGetLastError();
}

}  // namespace ska
