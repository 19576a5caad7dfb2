// Fused balanced Sinkhorn step for bands that fit in registers (gfx950).
//
// One launch performs one full Sinkhorn step of the stopped base or of the tail
// [technical summaries §2.1: T-step balanced Sinkhorn on the fixed band, then the R-step tail]:
//
//   1. finish the previous column update for the block's key window:
//        v_j <- v_j - log sum_i exp(S_ij + u_i + v_j)      (column sums from the previous launch)
//   2. row update for the 64 owned queries:  u_i = -log sum_j exp(S_ij + v_j)   (exact max shift)
//   3. column sums of the new plan exp(S + u + v) restricted to the owned rows, written as one
//      partial row per block; the next launch (or the finishing kernel) completes step 1.
//
// Each band entry costs one score recompute on the matrix cores and one exponential per full
// step.  The 16 x (16 + 32 ceil(h/16)) score strip of each wave stays in registers: lane l holds
// key column n = l % 16 of every 16-key tile and query rows 4 (l / 16) + r, so the row
// log-sum-exp reduces in-lane over tiles and then across the 16-lane DPP row, and the column sum
// of a tile reduces in-lane over 4 rows and then over lane groups and waves through LDS in a fixed
// order (no atomics, bitwise reproducible).  K's window for the block is staged in LDS once and
// shared by the four waves.
//
// Column sums can underflow only when a column's mass under the current plan falls below
// 2^-100 (scores spanning more than ~70 nats inside one band); such a column is finished by an
// exact log-sum-exp over its band instead, so the result never depends on that threshold beyond
// rounding.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "ska_device.h"
#include "ska_internal.h"

namespace ska {

template <int C>
__device__ __forceinline__ float dpp_row(float x) {
  return __builtin_amdgcn_update_dpp(0.f, x, C, 0xf, 0xf, false);
}
// all-reduce over the 16 lanes of a DPP row (row_ror 8, 4, 2, 1)
__device__ __forceinline__ float row16_max(float x) {
  x = fmaxf(x, dpp_row<0x128>(x));
  x = fmaxf(x, dpp_row<0x124>(x));
  x = fmaxf(x, dpp_row<0x122>(x));
  x = fmaxf(x, dpp_row<0x121>(x));
  return x;
}
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp_row<0x128>(x);
  x += dpp_row<0x124>(x);
  x += dpp_row<0x122>(x);
  x += dpp_row<0x121>(x);
  return x;
}

__device__ __forceinline__ int floor_div(int a, int b) { return (a >= 0) ? a / b : -((-a + b - 1) / b); }

// Map a launch-order block id to a logical (problem, row-block) index so that each of the 8
// XCDs (which receive block ids round-robin) works on a contiguous run of row blocks: the key
// windows of neighbouring blocks then overlap inside one XCD's L2.
__device__ __forceinline__ int64_t xcd_logical_block(int64_t bid, int64_t nblocks) {
  const int64_t q = nblocks / 8, rem = nblocks % 8;
  const int64_t x = bid % 8, k = bid / 8;
  return x * q + (x < rem ? x : rem) + k;
}

__device__ __forceinline__ float dot64(const bf16* a, const bf16* b) {
  float s = 0.f;
  for (int d = 0; d < kD; ++d) s = fmaf((float)a[d], (float)b[d], s);
  return s;
}
__device__ __forceinline__ float dot64(const float* a, const float* b) {
  float s = 0.f;
  for (int d = 0; d < kD; ++d) s = fmaf(a[d], b[d], s);
  return s;
}

// Exact column update (log2 units): -log2 sum_i 2^(c2 q_i.k_j + u_i) over the band of key j.
// Used where a column's summed mass underflows; the same arithmetic runs in every block that
// needs column j, so all of them agree bitwise.
template <typename T>
__device__ float exact_column(int j, const float* u_h, const T* Qh, const T* Kh, int Lr, int h,
                              float c2) {
  float m = -INFINITY;
  const int i0 = max(0, j - h), i1 = min(Lr - 1, j + h);
  for (int i = i0; i <= i1; ++i)
    m = fmaxf(m, fmaf(dot64(Qh + (int64_t)i * kD, Kh + (int64_t)j * kD), c2, u_h[i]));
  if (!(m > -INFINITY)) return m == m ? 0.f : m;   // NaN propagates
  float l = 0.f;
  for (int i = i0; i <= i1; ++i)
    l += fast_exp2(fmaf(dot64(Qh + (int64_t)i * kD, Kh + (int64_t)j * kD), c2, u_h[i]) - m);
  return -(m + fast_log2(l));
}

// Blocks whose key window holds column j: windows are [64 b - 16 H16, 64 b + 64 + 16 H16).
__device__ __forceinline__ int first_block_of(int j, int H16) {
  return max(0, floor_div(j - 16 * H16 - 63, 64));
}

// Finished column dual (log2 units) of key j given the previous dual and the per-block column
// sums of exp(S + u + v_prev), summed in ascending block order.
template <typename T, int NB>
__device__ float finish_column(int j, const float* vprev_h, const float* part_h, const float* u_h,
                               const T* Qh, const T* Kh, int Lr, int h, int H16, int nblk,
                               int pstride, float c2) {
  const int lo = first_block_of(j, H16);
  const int hi = min(nblk - 1, floor_div(j + 16 * H16, 64));
  float p[NB];
#pragma unroll
  for (int q = 0; q < NB; ++q) {
    const int b = lo + q, c = j - (b * 64 - 16 * H16);
    const bool ok = (b <= hi) & (c >= 0) & (c < pstride);
    const int bc = min(b, nblk - 1), cc = min(max(c, 0), pstride - 1);
    const float x = part_h[(int64_t)bc * pstride + cc];
    p[q] = ok ? x : 0.f;
  }
  const float vp = vprev_h[j];
  float s = 0.f;
#pragma unroll
  for (int q = 0; q < NB; ++q) s += p[q];
  if (s >= 0x1p-100f) return vp - fast_log2(s);
  return exact_column<T>(j, u_h, Qh, Kh, Lr, h, c2);
}

// B-operand fragment of key row `row` of the staged window (LDS), d-slice of lane group g.
__device__ __forceinline__ void lds_frag(Frag<bf16>& f, const bf16* kw, int row, int g) {
  const uint4* p = reinterpret_cast<const uint4*>(kw + row * Lds<bf16>::stride + 16 * g);
  f.a = __builtin_bit_cast(bf16x8, p[0]);
  f.b = __builtin_bit_cast(bf16x8, p[1]);
}
__device__ __forceinline__ void lds_frag(Frag<float>& f, const float* kw, int row, int g) {
  const f32x4* p = reinterpret_cast<const f32x4*>(kw + row * Lds<float>::stride + 16 * g);
#pragma unroll
  for (int i = 0; i < 4; ++i) f.v[i] = p[i];
}

// Stage ROWS key rows starting at token r0 (zeros outside [0, Lr)) into LDS, whole workgroup
// of 256 threads: every thread issues all of its 16-byte loads before its first LDS store, so the
// loads overlap instead of each paying the full memory latency.
template <int ROWS>
__device__ __forceinline__ void stage_block(bf16* lds, const bf16* base, int r0, int Lr) {
  constexpr int kPer = ROWS * 8 / 256;
  static_assert(ROWS * 8 % 256 == 0, "rows must fill the workgroup");
  uint4 buf[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int c = i * 256 + threadIdx.x, row = c >> 3, col = (c & 7) * 8, t = r0 + row;
    const int tc = min(max(t, 0), Lr - 1);          // always a valid row; zeroed below if outside
    const uint4 x = *reinterpret_cast<const uint4*>(base + (int64_t)tc * kD + col);
    const bool ok = (t >= 0) & (t < Lr);
    buf[i] = uint4{ok ? x.x : 0u, ok ? x.y : 0u, ok ? x.z : 0u, ok ? x.w : 0u};
  }
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int c = i * 256 + threadIdx.x, row = c >> 3, col = (c & 7) * 8;
    *reinterpret_cast<uint4*>(lds + row * Lds<bf16>::stride + col) = buf[i];
  }
}
template <int ROWS>
__device__ __forceinline__ void stage_block(float* lds, const float* base, int r0, int Lr) {
  constexpr int kPer = ROWS * 16 / 256;
  static_assert(ROWS * 16 % 256 == 0, "rows must fill the workgroup");
  f32x4 buf[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int c = i * 256 + threadIdx.x, row = c >> 4, col = (c & 15) * 4, t = r0 + row;
    const int tc = min(max(t, 0), Lr - 1);
    const f32x4 x = *reinterpret_cast<const f32x4*>(base + (int64_t)tc * kD + col);
    const bool ok = (t >= 0) & (t < Lr);
    buf[i] = f32x4{ok ? x[0] : 0.f, ok ? x[1] : 0.f, ok ? x[2] : 0.f, ok ? x[3] : 0.f};
  }
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int c = i * 256 + threadIdx.x, row = c >> 4, col = (c & 15) * 4;
    *reinterpret_cast<f32x4*>(lds + row * Lds<float>::stride + col) = buf[i];
  }
}

template <typename T, int NT>
struct StepSmem {
  static constexpr int kRows = 64 + 16 * (NT - 1);           // block key window (64 + 32 H16)
  static constexpr int kKwinBytes = kRows * Lds<T>::stride * (int)sizeof(T);
  static constexpr int kPartBytes = 16 * 16 * NT * 4;        // [wave][group][16 NT] floats
  static constexpr int kBytes = kKwinBytes > kPartBytes ? kKwinBytes : kPartBytes;
};

template <typename T, int NT>
__global__ __launch_bounds__(256) void sinkhorn_step_kernel(StepArgs a) {
  constexpr int H16 = (NT - 1) / 2;
  constexpr int kRows = StepSmem<T, NT>::kRows;
  __shared__ __attribute__((aligned(16))) char smem[StepSmem<T, NT>::kBytes];
  __shared__ float vwin[kRows];
  T* kw = reinterpret_cast<T*>(smem);
  float* cpart = reinterpret_cast<float*>(smem);

  const int lane = threadIdx.x & 63, g = lane >> 4, n = lane & 15;
  // the wave index is uniform across the wave: keep it scalar so tile tests branch on SGPRs
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t lb = xcd_logical_block(blockIdx.x, (int64_t)gridDim.x);
  const int64_t head = lb / a.nblk;
  const int blk = (int)(lb % a.nblk);
  const int b0 = blk * 64;
  const int cb = b0 - 16 * H16;                 // first key of the block window
  const int Lr = a.Lr, h = a.h;
  const T* Qh = static_cast<const T*>(a.Q) + head * (int64_t)Lr * kD;
  const T* Kh = static_cast<const T*>(a.K) + head * (int64_t)Lr * kD;
  const int64_t vo = head * (int64_t)a.Lpad;

  // 1. stage keys, finish the previous column update for the window.  All global loads of the
  //    block are in flight together: the key rows first, then the column partials.
  constexpr int kNB = kRows / 64 + 1;   // blocks whose windows can hold one column
  stage_block<kRows>(kw, Kh, cb, Lr);
#pragma unroll
  for (int pass = 0; pass < (kRows + 255) / 256; ++pass) {
    const int c = pass * 256 + (int)threadIdx.x;
    if (c < kRows) {
      const int j = cb + c;
      float v = 0.f;
      if (j >= 0 && j < Lr) {
        v = a.part_prev ? finish_column<T, kNB>(j, a.v_prev + vo,
                                                 a.part_prev + head * (int64_t)a.nblk * a.pstride,
                                                 a.u_prev + vo, Qh, Kh, Lr, h, H16, a.nblk,
                                                 a.pstride, a.c2)
                        : a.v_prev[vo + j];
        if (j >= b0 && j < b0 + 64) {
          a.v_next[vo + j] = v;
          if (a.save_v) a.save_v[head * a.save_v_stride + j] = v * kLn2;
        }
      }
      vwin[c] = v;
    }
  }
  __syncthreads();

  // 2. score strip in registers, exact row log-sum-exp
  const int o0 = b0 + 16 * wave;       // owned rows o0 .. o0 + 15 (rows 4g + r in this lane)
  const int cw = o0 - 16 * H16;        // first key of the wave window; LDS row offset 16 * wave
  Frag<T> fq;
  load_frag(fq, Qh + (int64_t)(o0 + n) * kD, o0 + n < Lr, g);
  // Tile t covers keys cw + 16t .. cw + 16t + 15; over its entries i - j spans
  // [16 H16 - 16 t - 15, 16 H16 - 16 t + 15].  Wave-uniform classes: "dead" tiles (no entry on the
  // band or inside the sequence) skip the MFMA; "clean" tiles (every entry valid) skip the masks.
  const bool rows_in = (o0 + 15 < Lr);
  float x[NT][4];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int j0 = cw + 16 * t;
    const int dlo = 16 * H16 - 16 * t - 15, dhi = 16 * H16 - 16 * t + 15;
    const bool dead = (dlo > h) | (dhi < -h) | (j0 >= Lr) | (j0 + 15 < 0) | (o0 >= Lr);
    if (dead) {
#pragma unroll
      for (int r = 0; r < 4; ++r) x[t][r] = -INFINITY;
      continue;
    }
    Frag<T> fk;
    lds_frag(fk, kw, 16 * wave + 16 * t + n, g);
    const f32x4 sc = dot_tile(fq, fk);
    const float vj = vwin[16 * wave + 16 * t + n];
    const bool clean = rows_in & (j0 >= 0) & (j0 + 15 < Lr) & (dhi <= h) & (dlo >= -h);
    if (clean) {
#pragma unroll
      for (int r = 0; r < 4; ++r) x[t][r] = fmaf(sc[r], a.c2, vj);
    } else {
      const int j = j0 + n;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = o0 + 4 * g + r;
        const bool ok = (i < Lr) & (j >= 0) & (j < Lr) & (abs(i - j) <= h);
        x[t][r] = ok ? fmaf(sc[r], a.c2, vj) : -INFINITY;
      }
    }
  }
  float m[4], l[4], rinv[4], u[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float mm = x[0][r];
#pragma unroll
    for (int t = 1; t < NT; ++t) mm = fmaxf(mm, x[t][r]);
    m[r] = row16_max(mm);
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float ms = (m[r] == -INFINITY) ? 0.f : m[r];
    float ll = 0.f;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      x[t][r] = fast_exp2(x[t][r] - ms);
      ll += x[t][r];
    }
    l[r] = row16_sum(ll);
    const bool empty = (m[r] == -INFINITY);
    u[r] = empty ? 0.f : -(m[r] + fast_log2(l[r]));
    rinv[r] = empty ? 0.f : __builtin_amdgcn_rcpf(l[r]);
  }
  if (n < 4) {
    const int i = o0 + 4 * g + n;
    const float ui = (n == 0) ? u[0] : (n == 1) ? u[1] : (n == 2) ? u[2] : u[3];
    if (i < Lr) {
      a.u_out[vo + i] = ui;
      if (a.save_u) a.save_u[head * a.save_u_stride + i] = ui * kLn2;
    }
  }

  // 3. column sums of the new plan over the owned rows
  float cp[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t)
    cp[t] = x[t][0] * rinv[0] + x[t][1] * rinv[1] + x[t][2] * rinv[2] + x[t][3] * rinv[3];
  __syncthreads();                     // every wave is done with the staged keys
#pragma unroll
  for (int t = 0; t < NT; ++t) cpart[(wave * 4 + g) * (16 * NT) + 16 * t + n] = cp[t];
  __syncthreads();
  float* pout = a.part_out + (head * (int64_t)a.nblk + blk) * a.pstride;
  for (int c = threadIdx.x; c < a.pstride; c += blockDim.x) {
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int cc = c - 16 * w;
      if (cc >= 0 && cc < 16 * NT) {
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) s += cpart[(w * 4 + gg) * (16 * NT) + cc];
      }
    }
    pout[c] = s;
  }
}

// Finish the last column update of the forward for every token; also writes the saved dual.
template <typename T>
__global__ __launch_bounds__(256) void finish_columns_kernel(StepArgs a) {
  const int64_t head = blockIdx.y;
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= a.Lr) return;
  const int H16 = (a.pstride - 64) / 32;
  const T* Qh = static_cast<const T*>(a.Q) + head * (int64_t)a.Lr * kD;
  const T* Kh = static_cast<const T*>(a.K) + head * (int64_t)a.Lr * kD;
  const int64_t vo = head * (int64_t)a.Lpad;
  const float v = finish_column<T, 8>(j, a.v_prev + vo, a.part_prev + head * (int64_t)a.nblk * a.pstride,
                                      a.u_prev + vo, Qh, Kh, a.Lr, a.h, H16, a.nblk, a.pstride, a.c2);
  a.v_next[vo + j] = v;
  if (a.save_v) a.save_v[head * a.save_v_stride + j] = v * kLn2;
}

int fused_tiles_for(int h) {
  const int nt = 1 + 2 * ((h + 15) / 16);
  if (nt <= 5) return 5;
  if (nt <= 9) return 9;
  if (nt <= 17) return 17;
  if (nt <= 25) return 25;
  return 0;
}

template <typename T, int NT>
static void launch_step_t(const StepArgs& a, hipStream_t st) {
  const unsigned blocks = (unsigned)(a.bh * (int64_t)a.nblk);
  sinkhorn_step_kernel<T, NT><<<dim3(blocks), dim3(256), 0, st>>>(a);
}

hipError_t launch_fused_step(int elt, int nt, const StepArgs& a, hipStream_t st) {
  if (elt == 1) {
    switch (nt) {
      case 5: launch_step_t<bf16, 5>(a, st); break;
      case 9: launch_step_t<bf16, 9>(a, st); break;
      case 17: launch_step_t<bf16, 17>(a, st); break;
      default: launch_step_t<bf16, 25>(a, st); break;
    }
  } else {
    switch (nt) {
      case 5: launch_step_t<float, 5>(a, st); break;
      case 9: launch_step_t<float, 9>(a, st); break;
      case 17: launch_step_t<float, 17>(a, st); break;
      default: launch_step_t<float, 25>(a, st); break;
    }
  }
  return hipGetLastError();
}

hipError_t launch_finish_columns(int elt, const StepArgs& a, hipStream_t st) {
  dim3 grid((unsigned)((a.Lr + 255) / 256), (unsigned)a.bh);
  if (elt == 1) finish_columns_kernel<bf16><<<grid, dim3(256), 0, st>>>(a);
  else finish_columns_kernel<float><<<grid, dim3(256), 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace ska
