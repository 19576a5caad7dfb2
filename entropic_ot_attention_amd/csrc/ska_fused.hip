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

// Finished column dual (log2 units) of key j given the previous dual and the per-block column
// sums of exp(S + u + v_prev).  Exact fallback: -log2 sum_i 2^(c2 q_i.k_j + u_i) over the band.
template <typename T>
__device__ float finish_column(int j, const float* vprev_h, const float* part_h, const float* u_h,
                               const T* Qh, const T* Kh, int Lr, int h, int H16, int nblk,
                               int pstride, float c2) {
  float s = 0.f;
  const int lo = max(0, floor_div(j - 16 * H16 - 63, 64));
  const int hi = min(nblk - 1, floor_div(j + 16 * H16, 64));
  for (int b = lo; b <= hi; ++b) {
    const int c = j - (b * 64 - 16 * H16);
    if (c >= 0 && c < pstride) s += part_h[(int64_t)b * pstride + c];
  }
  if (s >= 0x1p-100f) return vprev_h[j] - fast_log2(s);
  // exact column log-sum-exp (rare path; same arithmetic in every block that needs column j)
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

// Stage `rows` key rows starting at token r0 (zeros outside [0, Lr)) into LDS, whole workgroup.
__device__ __forceinline__ void stage_block(bf16* lds, const bf16* base, int r0, int rows, int Lr) {
  for (int c = threadIdx.x; c < rows * 8; c += blockDim.x) {
    const int row = c >> 3, col = (c & 7) * 8, t = r0 + row;
    uint4 x = {0u, 0u, 0u, 0u};
    if (t >= 0 && t < Lr) x = *reinterpret_cast<const uint4*>(base + (int64_t)t * kD + col);
    *reinterpret_cast<uint4*>(lds + row * Lds<bf16>::stride + col) = x;
  }
}
__device__ __forceinline__ void stage_block(float* lds, const float* base, int r0, int rows, int Lr) {
  for (int c = threadIdx.x; c < rows * 16; c += blockDim.x) {
    const int row = c >> 4, col = (c & 15) * 4, t = r0 + row;
    f32x4 x = {0.f, 0.f, 0.f, 0.f};
    if (t >= 0 && t < Lr) x = *reinterpret_cast<const f32x4*>(base + (int64_t)t * kD + col);
    *reinterpret_cast<f32x4*>(lds + row * Lds<float>::stride + col) = x;
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

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 4, n = lane & 15;
  const int64_t lb = xcd_logical_block(blockIdx.x, (int64_t)gridDim.x);
  const int64_t head = lb / a.nblk;
  const int blk = (int)(lb % a.nblk);
  const int b0 = blk * 64;
  const int cb = b0 - 16 * H16;                 // first key of the block window
  const int Lr = a.Lr, h = a.h;
  const T* Qh = static_cast<const T*>(a.Q) + head * (int64_t)Lr * kD;
  const T* Kh = static_cast<const T*>(a.K) + head * (int64_t)Lr * kD;
  const int64_t vo = head * (int64_t)a.Lpad;

  // 1. stage keys, finish the previous column update for the window
  stage_block(kw, Kh, cb, kRows, Lr);
  for (int c = threadIdx.x; c < kRows; c += blockDim.x) {
    const int j = cb + c;
    float v = 0.f;
    if (j >= 0 && j < Lr) {
      v = a.part_prev ? finish_column<T>(j, a.v_prev + vo, a.part_prev + head * (int64_t)a.nblk * a.pstride,
                                         a.u_prev + vo, Qh, Kh, Lr, h, H16, a.nblk, a.pstride, a.c2)
                      : a.v_prev[vo + j];
      if (j >= b0 && j < b0 + 64) {
        a.v_next[vo + j] = v;
        if (a.save_v) a.save_v[head * a.save_v_stride + j] = v * kLn2;
      }
    }
    vwin[c] = v;
  }
  __syncthreads();

  // 2. score strip in registers, exact row log-sum-exp
  const int o0 = b0 + 16 * wave;       // owned rows o0 .. o0 + 15 (rows 4g + r in this lane)
  const int cw = o0 - 16 * H16;        // first key of the wave window; LDS row offset 16 * wave
  Frag<T> fq;
  load_frag(fq, Qh + (int64_t)(o0 + n) * kD, o0 + n < Lr, g);
  float x[NT][4];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    Frag<T> fk;
    lds_frag(fk, kw, 16 * wave + 16 * t + n, g);
    const f32x4 s = dot_tile(fq, fk);
    const int j = cw + 16 * t + n;
    const float vj = vwin[16 * wave + 16 * t + n];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = o0 + 4 * g + r;
      const bool ok = i < Lr && j >= 0 && j < Lr && abs(i - j) <= h;
      x[t][r] = ok ? fmaf(s[r], a.c2, vj) : -INFINITY;
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
  const float v = finish_column<T>(j, a.v_prev + vo, a.part_prev + head * (int64_t)a.nblk * a.pstride,
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
