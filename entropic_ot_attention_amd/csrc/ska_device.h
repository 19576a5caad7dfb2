// Device-side helpers shared by the HIP kernels of libsinkhorn_attn.so (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "ska_internal.h"

namespace ska {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((__vector_size__(16)));
typedef float f32x4 __attribute__((__vector_size__(16)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kChunk = 32;  // window rows staged per LDS round (two 16-row tiles)

template <typename T> struct Lds;
template <> struct Lds<bf16> { static constexpr int stride = 72; };   // 64 + 8 pad elements
template <> struct Lds<float> { static constexpr int stride = 68; };  // 64 + 4 pad elements

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// ---------------------------------------------------------------------------------------------
// Operand fragments of the score contraction over d = 64.
// bf16: v_mfma_f32_16x16x32_bf16 twice; lane group g = l/16 supplies d in [16g, 16g+16),
//       split as k-slots 8g..8g+7 of the first MFMA (d = 16g + e) and of the second
//       (d = 16g + 8 + e).  The same permutation on both operands leaves the dot product intact.
// fp32: v_mfma_f32_16x16x4_f32 sixteen times; MFMA s takes d = 16g + s in k-slot g.
// ---------------------------------------------------------------------------------------------
template <typename T> struct Frag;
template <> struct Frag<bf16> { bf16x8 a, b; };
template <> struct Frag<float> { f32x4 v[4]; };

__device__ __forceinline__ void load_frag(Frag<bf16>& f, const bf16* row, bool ok, int g) {
  if (ok) {
    const uint4* p = reinterpret_cast<const uint4*>(row + 16 * g);
    uint4 x = p[0], y = p[1];
    f.a = __builtin_bit_cast(bf16x8, x);
    f.b = __builtin_bit_cast(bf16x8, y);
  } else {
    uint4 z = {0u, 0u, 0u, 0u};
    f.a = __builtin_bit_cast(bf16x8, z);
    f.b = __builtin_bit_cast(bf16x8, z);
  }
}

__device__ __forceinline__ void load_frag(Frag<float>& f, const float* row, bool ok, int g) {
  if (ok) {
    const f32x4* p = reinterpret_cast<const f32x4*>(row + 16 * g);
#pragma unroll
    for (int i = 0; i < 4; ++i) f.v[i] = p[i];
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) f.v[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
}

// The same without a validity test: the caller passes a readable row and masks the results.
__device__ __forceinline__ void load_frag_raw(Frag<bf16>& f, const bf16* row, int g) {
  const uint4* p = reinterpret_cast<const uint4*>(row + 16 * g);
  f.a = __builtin_bit_cast(bf16x8, p[0]);
  f.b = __builtin_bit_cast(bf16x8, p[1]);
}
__device__ __forceinline__ void load_frag_raw(Frag<float>& f, const float* row, int g) {
  const f32x4* p = reinterpret_cast<const f32x4*>(row + 16 * g);
#pragma unroll
  for (int i = 0; i < 4; ++i) f.v[i] = p[i];
}

// Fragment loads with the lane groups' d-slices interleaved along the row (fp32: MFMA (i, e)
// takes d = 16 i + 4 g + e; bf16: the two MFMAs take d = 8 g + e and d = 32 + 8 g + e), so the
// four lane groups of a row read one contiguous piece of it per load instruction instead of four
// pieces of separate cache lines.  The sum over d is unchanged when both operands of a
// contraction use this layout (and only then).
__device__ __forceinline__ void load_frag_il(Frag<bf16>& f, const bf16* row, int g) {
  f.a = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(row + 8 * g));
  f.b = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(row + 32 + 8 * g));
}
__device__ __forceinline__ void load_frag_il(Frag<float>& f, const float* row, int g) {
#pragma unroll
  for (int i = 0; i < 4; ++i) f.v[i] = *reinterpret_cast<const f32x4*>(row + 16 * i + 4 * g);
}

// Partial dot product of two rows held as fragments in the same layout (this lane's d-slice).
__device__ __forceinline__ float frag_dot(const Frag<bf16>& x, const Frag<bf16>& y) {
  float acc = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    acc = fmaf((float)x.a[e], (float)y.a[e], acc);
    acc = fmaf((float)x.b[e], (float)y.b[e], acc);
  }
  return acc;
}
__device__ __forceinline__ float frag_dot(const Frag<float>& x, const Frag<float>& y) {
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) acc = fmaf(x.v[i][e], y.v[i][e], acc);
  return acc;
}

// init + w.o over d = 64 for a 16 x 16 tile (init enters the matrix-core accumulator)
__device__ __forceinline__ f32x4 dot_tile(const Frag<bf16>& w, const Frag<bf16>& o,
                                          f32x4 init = f32x4{0.f, 0.f, 0.f, 0.f}) {
  f32x4 acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w.a, o.a, init, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w.b, o.b, acc, 0, 0, 0);
  return acc;
}

__device__ __forceinline__ f32x4 dot_tile(const Frag<float>& w, const Frag<float>& o,
                                          f32x4 init = f32x4{0.f, 0.f, 0.f, 0.f}) {
  f32x4 acc = init;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(w.v[i][j], o.v[i][j], acc, 0, 0, 0);
  return acc;
}

// ---------------------------------------------------------------------------------------------
// LDS staging of 32 window rows x 64 columns of the second contraction's operand, per wave.
// Rows outside [0, Lr) are written as zeros.
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ void stage_rows(bf16* lds, const bf16* base, int r0, int Lr, int lane) {
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int c = it * 64 + lane;
    const int row = c >> 3, col = (c & 7) * 8;
    const int t = r0 + row;
    uint4 x = {0u, 0u, 0u, 0u};
    if (t >= 0 && t < Lr) x = *reinterpret_cast<const uint4*>(base + (int64_t)t * kD + col);
    *reinterpret_cast<uint4*>(lds + row * Lds<bf16>::stride + col) = x;
  }
}

__device__ __forceinline__ void stage_rows(float* lds, const float* base, int r0, int Lr, int lane) {
#pragma unroll
  for (int it = 0; it < 8; ++it) {
    const int c = it * 64 + lane;
    const int row = c >> 4, col = (c & 15) * 4;
    const int t = r0 + row;
    f32x4 x = {0.f, 0.f, 0.f, 0.f};
    if (t >= 0 && t < Lr) x = *reinterpret_cast<const f32x4*>(base + (int64_t)t * kD + col);
    *reinterpret_cast<f32x4*>(lds + row * Lds<float>::stride + col) = x;
  }
}

// acc[b][r] (lane l) += sum over the 32 staged rows k of  Op[k][16b + 4g + r] * Z[k][n],
// where Z[16tt + 4g' + r'] at lane (g', n) is z[tt][r'].  The result layout is
// acc[b][r] <-> (column 16b + 4g + r of the operand, owned token n = l % 16).
__device__ __forceinline__ void contract(f32x4 (&acc)[4], const bf16* lds, const float (&z)[2][4],
                                         int g, int n) {
  bf16x8 zb;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    zb[e] = (bf16)z[0][e];
    zb[e + 4] = (bf16)z[1][e];
  }
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    bf16x8 a;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int row = (e < 4) ? (4 * g + e) : (16 + 4 * g + e - 4);
      a[e] = lds[row * Lds<bf16>::stride + 16 * b + n];
    }
    acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, zb, acc[b], 0, 0, 0);
  }
}

__device__ __forceinline__ void contract(f32x4 (&acc)[4], const float* lds, const float (&z)[2][4],
                                         int g, int n) {
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 16 * tt + 4 * g + r;
#pragma unroll
      for (int b = 0; b < 4; ++b)
        acc[b] = __builtin_amdgcn_mfma_f32_16x16x4f32(lds[row * Lds<float>::stride + 16 * b + n],
                                                      z[tt][r], acc[b], 0, 0, 0);
    }
}

// Two contractions against the same staged operand (shares the LDS reads).
__device__ __forceinline__ void contract2(f32x4 (&x)[4], f32x4 (&y)[4], const bf16* lds,
                                          const float (&z1)[2][4], const float (&z2)[2][4], int g,
                                          int n) {
  bf16x8 b1, b2;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    b1[e] = (bf16)z1[0][e];
    b1[e + 4] = (bf16)z1[1][e];
    b2[e] = (bf16)z2[0][e];
    b2[e + 4] = (bf16)z2[1][e];
  }
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    bf16x8 a;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int row = (e < 4) ? (4 * g + e) : (16 + 4 * g + e - 4);
      a[e] = lds[row * Lds<bf16>::stride + 16 * b + n];
    }
    x[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b1, x[b], 0, 0, 0);
    y[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b2, y[b], 0, 0, 0);
  }
}

__device__ __forceinline__ void contract2(f32x4 (&x)[4], f32x4 (&y)[4], const float* lds,
                                          const float (&z1)[2][4], const float (&z2)[2][4], int g,
                                          int n) {
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 16 * tt + 4 * g + r;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const float a = lds[row * Lds<float>::stride + 16 * b + n];
        x[b] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, z1[tt][r], x[b], 0, 0, 0);
        y[b] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, z2[tt][r], y[b], 0, 0, 0);
      }
    }
}

// Store acc (scaled) as row `o` of out: lane holds columns 16b + 4g + r, r = 0..3.
__device__ __forceinline__ void store_row(bf16* out_row, const f32x4 (&acc)[4], float scale, int g) {
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    typedef __bf16 bf16x4 __attribute__((__vector_size__(8)));
    bf16x4 v;
#pragma unroll
    for (int r = 0; r < 4; ++r) v[r] = (bf16)(acc[b][r] * scale);
    *reinterpret_cast<bf16x4*>(out_row + 16 * b + 4 * g) = v;
  }
}

__device__ __forceinline__ void store_row(float* out_row, const f32x4 (&acc)[4], float scale, int g) {
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    f32x4 v;
#pragma unroll
    for (int r = 0; r < 4; ++r) v[r] = acc[b][r] * scale;
    *reinterpret_cast<f32x4*>(out_row + 16 * b + 4 * g) = v;
  }
}

// Sum of a per-lane value over the 4 lane groups holding the same owned token.
__device__ __forceinline__ float group_sum(float x) {
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}

// Does the 16-row window tile starting at w0 meet the band of owned tokens [o0, o0 + 16)?
__device__ __forceinline__ bool tile_live(int w0, int o0, int h, int Lr) {
  return w0 < Lr && w0 <= o0 + 15 + h && w0 + 15 >= o0 - h;
}

__device__ __forceinline__ bool in_band(int w, int o, int h, int Lr) {
  return w < Lr && o < Lr && abs(w - o) <= h;
}

__device__ __forceinline__ f32x4 load4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }


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

// gfx950 lane swaps.  swap32(a, b): low 32 lanes get a[l] + a[l + 32], high 32 lanes get
// b[l - 32] + b[l]; swap16(a, b): lane rows (16 lanes) 0,1,2,3 get a.r0 + a.r1, b.r0 + b.r1,
// a.r2 + a.r3, b.r2 + b.r3.
__device__ __forceinline__ float swap32_sum(float a, float b) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float swap16_sum(float a, float b) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
// Sum over the four lane groups (lanes n, n + 16, n + 32, n + 48), result in every lane.
__device__ __forceinline__ float lane_group_sum(float x) {
  return swap16_sum(swap32_sum(x, x), swap32_sum(x, x));
}
// Maximum over the 64 lanes of a wave, result in every lane: DPP within each 16-lane row, then
// the two lane swaps across rows.
__device__ __forceinline__ float wave_max(float x) {
  x = row16_max(x);
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
  const auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(q[0]), __uint_as_float(q[1]));
}

__device__ __forceinline__ int floor_div(int a, int b) { return (a >= 0) ? a / b : -((-a + b - 1) / b); }

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

// MFMA operand fragment of row `row` of a row-major LDS array (d-slice of lane group g).
__device__ __forceinline__ void lds_frag(Frag<bf16>& f, const bf16* rows, int row, int g) {
  const uint4* p = reinterpret_cast<const uint4*>(rows + row * Lds<bf16>::stride + 16 * g);
  f.a = __builtin_bit_cast(bf16x8, p[0]);
  f.b = __builtin_bit_cast(bf16x8, p[1]);
}
__device__ __forceinline__ void lds_frag(Frag<float>& f, const float* rows, int row, int g) {
  const f32x4* p = reinterpret_cast<const f32x4*>(rows + row * Lds<float>::stride + 16 * g);
#pragma unroll
  for (int i = 0; i < 4; ++i) f.v[i] = p[i];
}

// ROWS token rows of a [L][64] tensor, starting at token r0 (zeros outside [0, Lr)), held in
// registers of a workgroup of NTHR threads between their global load and their store into an
// LDS ring (token t at ring row t mod RING).  All loads are issued before the first store.
template <typename T, int ROWS, int NTHR>
struct RowStage {
  static constexpr int kChunksPerRow = 64 * (int)sizeof(T) / 16;
  static constexpr int kPer = (ROWS * kChunksPerRow + NTHR - 1) / NTHR;
  uint4 x[kPer];
  __device__ __forceinline__ void load(const T* base, int r0, int Lr) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int c = i * NTHR + (int)threadIdx.x;
      const int row = c / kChunksPerRow, col = (c % kChunksPerRow) * (16 / (int)sizeof(T));
      const int t = r0 + row;
      const int tc = min(max(t, 0), Lr - 1);
      const uint4 v = *reinterpret_cast<const uint4*>(base + (int64_t)tc * kD + col);
      const bool ok = (t >= 0) & (t < Lr) & (row < ROWS);
      x[i] = uint4{ok ? v.x : 0u, ok ? v.y : 0u, ok ? v.z : 0u, ok ? v.w : 0u};
    }
  }
  // the same when every row lies inside the sequence: no clamping or selection, and the
  // per-thread offset from the (wave-uniform) first row is loop-invariant
  __device__ __forceinline__ void load_inside(const T* base, int r0) {
    const T* rb = base + (int64_t)r0 * kD;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int c = i * NTHR + (int)threadIdx.x;
      const int row = c / kChunksPerRow, col = (c % kChunksPerRow) * (16 / (int)sizeof(T));
      if (ROWS * kChunksPerRow % NTHR == 0 || row < ROWS)
        x[i] = *reinterpret_cast<const uint4*>(rb + (unsigned)(row * kD + col));
    }
  }
  // store into ring slots slot0, slot0 + 1, .. (slot0 a wave-uniform multiple of 16), wrapping
  // at RING
  template <int RING>
  __device__ __forceinline__ void store_slots(T* ring, int slot0) const {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int c = i * NTHR + (int)threadIdx.x;
      const int row = c / kChunksPerRow, col = (c % kChunksPerRow) * (16 / (int)sizeof(T));
      if (ROWS * kChunksPerRow % NTHR == 0 || row < ROWS) {
        int rr = slot0 + row;
        if (RING % 64 != 0 || ROWS > 64 || rr >= RING) rr = (rr >= RING) ? rr - RING : rr;
        *reinterpret_cast<uint4*>(ring + rr * Lds<T>::stride + col) = x[i];
      }
    }
  }
  template <int RING>
  __device__ __forceinline__ void store(T* ring, int r0) const {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int c = i * NTHR + (int)threadIdx.x;
      const int row = c / kChunksPerRow, col = (c % kChunksPerRow) * (16 / (int)sizeof(T));
      if (ROWS * kChunksPerRow % NTHR == 0 || row < ROWS) {
        const int rr = (r0 + row + 4 * RING) % RING;
        *reinterpret_cast<uint4*>(ring + rr * Lds<T>::stride + col) = x[i];
      }
    }
  }
};

}  // namespace ska
