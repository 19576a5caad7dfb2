// HIP kernels (gfx950) for banded balanced Sinkhorn attention: the separate row and column
// log-domain half-steps for windows wider than the wide fused step holds in registers, and the
// small vector kernels (fill, dual save, VJP vector preparation).
//
// Half-step decomposition: a workgroup is 4 independent waves; wave w of block b owns the 16
// tokens o0 = (4b + w) * 16 ... o0 + 15 and streams over the 16-token tiles of its band window
// [o0 - h, o0 + 15 + h] with an online maximum and sum.  One MFMA tile
// X[m][n] = <win_{w0+m}, own_{o0+n}> has the window rows as the A operand and the owned rows as
// the B operand, so lane l holds owned token n = l % 16 and, in its 4 result registers r, window
// tokens m = 4 (l / 16) + r: the sums over the window run inside each lane plus one exchange
// across the 4 lane groups at the end.  The score tile is symmetric in the two roles
// (S_ij = s q_i . k_j), so the column half-step is the row half-step with Q and K swapped.

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
// Squared-norm reductions of the tail-remainder certificate: sum (a - b)^2 and sum a^2 over n
// elements, in double, in a fixed order (per-block tree, then one block over the block sums).
// =============================================================================================
constexpr int kSqBlocks = kSqPartials;

template <typename T>
__global__ __launch_bounds__(256) void sqdiff_partial_kernel(const T* __restrict__ a, const T* __restrict__ b,
                                                             int64_t n, double* __restrict__ part) {
  __shared__ double sd[256], sa[256];
  double d2 = 0.0, a2 = 0.0;
  for (int64_t i = blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const double x = (double)(float)a[i], y = (double)(float)b[i];
    d2 += (x - y) * (x - y);
    a2 += x * x;
  }
  sd[threadIdx.x] = d2;
  sa[threadIdx.x] = a2;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if ((int)threadIdx.x < off) {
      sd[threadIdx.x] += sd[threadIdx.x + off];
      sa[threadIdx.x] += sa[threadIdx.x + off];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    part[2 * blockIdx.x] = sd[0];
    part[2 * blockIdx.x + 1] = sa[0];
  }
}

__global__ __launch_bounds__(256) void sum_pairs_kernel(const double* __restrict__ part, int nblk,
                                                        double* __restrict__ out) {
  __shared__ double sd[256], sa[256];
  sd[threadIdx.x] = ((int)threadIdx.x < nblk) ? part[2 * threadIdx.x] : 0.0;
  sa[threadIdx.x] = ((int)threadIdx.x < nblk) ? part[2 * threadIdx.x + 1] : 0.0;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if ((int)threadIdx.x < off) {
      sd[threadIdx.x] += sd[threadIdx.x + off];
      sa[threadIdx.x] += sa[threadIdx.x + off];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    out[0] = sd[0];
    out[1] = sa[0];
  }
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

hipError_t launch_sq_diff(int elt, const void* a, const void* b, int64_t n, double* part,
                          double* out2, hipStream_t st) {
  if (elt == 1)
    sqdiff_partial_kernel<bf16><<<dim3(kSqBlocks), dim3(256), 0, st>>>((const bf16*)a, (const bf16*)b, n, part);
  else
    sqdiff_partial_kernel<float><<<dim3(kSqBlocks), dim3(256), 0, st>>>((const float*)a, (const float*)b, n, part);
  sum_pairs_kernel<<<dim3(1), dim3(256), 0, st>>>(part, kSqBlocks, out2);
  return hipGetLastError();
}

hipError_t launch_vjp_prep(const float* duals, float* ws, const Geometry& g, hipStream_t st) {
  const int64_t vs = g.bh * (int64_t)g.Lpad;
  vjp_prep_kernel<<<dim3((unsigned)((g.Lpad + 255) / 256), (unsigned)g.bh), dim3(256), 0, st>>>(
      duals, ws, g.Lr, g.Lpad, vs);
  return hipGetLastError();
}

}  // namespace ska
