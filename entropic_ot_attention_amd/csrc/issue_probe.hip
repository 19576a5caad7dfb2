// Issue cost of the instruction classes the kernels are built from, on one SIMD of gfx950, in shader
// cycles.  Each wave runs a fixed loop of one class (independent operations, so nothing waits on
// a result) and times it with s_memtime; a SIMD's cost per instruction is the slowest wave's loop
// time over the instructions all of the SIMD's waves issued.  The split rows run matrix-core
// products in some waves and vector instructions in others on the same SIMDs: if the two
// overlapped, the slowest wave would take as long as the slower class alone.
//
// Used to derive the VALU and issue rooflines of the fused step and the streaming passes.  Every
// store is in bounds (one slot per wave of the grid) and every loop has a fixed trip count.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <vector>

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kIters = 1024;
constexpr int kBlocks = 256;          // one workgroup per CU
constexpr int kMaxWaves = 16;

// NM bf16 16x16x32 products, NF fp32 16x16x4 products, NV fmas and NE exponentials (each with one
// multiply that keeps its argument bounded) per iteration.  SPLIT: waves below `split` issue the
// products, the others the vector instructions.
template <int NM, int NF, int NV, int NE, bool SPLIT>
__global__ __launch_bounds__(1024) void probe_kernel(float* out, unsigned long long* cycles, float seed,
                                                     int split) {
  const int wave = threadIdx.x >> 6;
  const bool mat = !SPLIT || wave < split;
  const bool vec = !SPLIT || wave >= split;
  f32x4 acc[8], facc[4];
  for (int i = 0; i < 8; ++i) acc[i] = f32x4{seed, 0.f, 0.f, 0.f};
  for (int i = 0; i < 4; ++i) facc[i] = f32x4{seed, 0.f, 0.f, 0.f};
  bf16x8 a, b;
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(seed * (float)(e + 1));
    b[e] = (__bf16)(seed * 0.5f);
  }
  const float fa = seed * 0.25f, fb = seed * 0.125f;
  float v[32];
  for (int i = 0; i < 32; ++i) v[i] = seed + (float)threadIdx.x * 1e-3f + (float)i;
  const float c = 0.999f, d = 1e-4f;
  __syncthreads();
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < kIters; ++it) {
    if (mat) {
#pragma unroll
      for (int i = 0; i < NM; ++i) acc[i % 8] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[i % 8], 0, 0, 0);
#pragma unroll
      for (int i = 0; i < NF; ++i) facc[i % 4] = __builtin_amdgcn_mfma_f32_16x16x4f32(fa, fb, facc[i % 4], 0, 0, 0);
    }
    if (vec) {
#pragma unroll
      for (int i = 0; i < NV; ++i) v[i % 32] = fmaf(v[i % 32], c, d);
#pragma unroll
      for (int i = 0; i < NE; ++i) v[i % 32] = __builtin_amdgcn_exp2f(v[i % 32] * -0.01f);
    }
  }
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  float s = 0.f;
  for (int i = 0; i < 8; ++i) s += acc[i][0] + acc[i][1] + acc[i][2] + acc[i][3];
  for (int i = 0; i < 4; ++i) s += facc[i][0];
  for (int i = 0; i < 32; ++i) s += v[i];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
  if ((threadIdx.x & 63) == 0) cycles[blockIdx.x * kMaxWaves + wave] = t1 - t0;
}

// Slowest wave's loop, in cycles per iteration, over every workgroup; the first launch warms up.
template <int NM, int NF, int NV, int NE, bool SPLIT>
double run(float* out, unsigned long long* cycles, int waves, int split) {
  for (int rep = 0; rep < 2; ++rep)
    probe_kernel<NM, NF, NV, NE, SPLIT><<<kBlocks, 64 * waves>>>(out, cycles, 1.0f, split);
  if (hipDeviceSynchronize() != hipSuccess) return -1.0;
  std::vector<unsigned long long> h(kBlocks * kMaxWaves);
  if (hipMemcpy(h.data(), cycles, h.size() * sizeof(unsigned long long), hipMemcpyDeviceToHost) != hipSuccess)
    return -1.0;
  std::vector<double> per;
  for (int b = 0; b < kBlocks; ++b)
    for (int w = 0; w < waves; ++w) per.push_back((double)h[b * kMaxWaves + w] / kIters);
  std::sort(per.begin(), per.end());
  return per[per.size() * 9 / 10];   // 90th percentile: the slow wave of a typical SIMD
}

// instr_per_simd <= 0: a mixed loop, reported by its total only
void row(const char* what, int per_simd, double cyc, double instr_per_simd) {
  if (instr_per_simd > 0)
    std::printf("| %s | %d | %.1f | %.2f |\n", what, per_simd, cyc, cyc / instr_per_simd);
  else
    std::printf("| %s | %d | %.1f | - |\n", what, per_simd, cyc);
}

}  // namespace

int main() {
  float* out = nullptr;
  unsigned long long* cycles = nullptr;
  if (hipMalloc(&out, kBlocks * 1024 * sizeof(float)) != hipSuccess) return 1;
  if (hipMalloc(&cycles, kBlocks * kMaxWaves * sizeof(unsigned long long)) != hipSuccess) return 1;
  std::printf("| loop per wave and iteration | waves per SIMD | cycles per iteration (slow wave) | "
              "cycles per instruction per SIMD |\n|---|---:|---:|---:|\n");
  for (int w = 1; w <= 4; ++w) {
    row("32 fp32 fma", w, run<0, 0, 32, 0, false>(out, cycles, 4 * w, 0), 32.0 * w);
    row("16 exp + 16 mul (per exp and mul)", w,
        run<0, 0, 0, 16, false>(out, cycles, 4 * w, 0), 16.0 * w);
    row("8 bf16 16x16x32", w, run<8, 0, 0, 0, false>(out, cycles, 4 * w, 0), 8.0 * w);
    row("4 fp32 16x16x4", w, run<0, 4, 0, 0, false>(out, cycles, 4 * w, 0), 4.0 * w);
  }
  // one wave of products and one of vector instructions on each SIMD
  row("split: one wave 8 bf16 16x16x32, the other 32 fma", 2, run<8, 0, 32, 0, true>(out, cycles, 8, 4), 0.0);
  row("split: one wave 8 bf16 16x16x32, the other 16 exp + 16 mul", 2,
      run<8, 0, 0, 16, true>(out, cycles, 8, 4), 0.0);
  row("both waves: 8 bf16 16x16x32 + 32 fma", 2, run<8, 0, 32, 0, false>(out, cycles, 8, 0), 0.0);
  (void)hipFree(out);
  (void)hipFree(cycles);
  return 0;
}
