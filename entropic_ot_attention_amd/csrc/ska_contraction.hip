// Projective contraction certificate of the Sinkhorn map's active blocks (gfx950)
// [technical summaries §2.4: Hilbert's projective metric shows that strictly positive active
// blocks of the Sinkhorn map are contractions; atlas.scime.ai, Builds on: Birkhoff-Hopf
// contraction].
//
// The tokens are cut into blocks of B (16, 32, 64 or 128; the last one ragged).  A block pair
// (row block rb, column block cb = rb + o) is active when every pair in it lies on the support,
// so its Gibbs kernel exp(S) is strictly positive.  Its projective diameter is the largest log
// cross ratio, which for a Gibbs kernel is a sum of scores:
//   Delta = max over row pairs (i, i') of  max_j (S_ij - S_i'j) - min_j (S_ij - S_i'j),
// and its Birkhoff-Hopf coefficient is kappa = tanh(Delta / 4): a log-domain half-step on the
// block shrinks the oscillation of a dual difference by at least that factor, a full step by
// kappa^2.
//
// One wave per block pair.  The score block is formed on the matrix cores (16 x 16 tiles over
// d = 64, as in every other kernel here) into the wave's LDS slice, rows padded by one float so
// the row-pair loop reads distinct banks; then each lane takes row partners i' of a row i shared
// by the wave (one LDS broadcast per column) and the wave's maximum is the diameter.
// Scores are fp32 (bf16 inputs: exact products, fp32 sums), as in the forward.

#include "ska_device.h"
#include "ska_internal.h"

namespace ska {

template <int B> struct ContractionShape {
  static constexpr int waves = (B <= 64) ? 4 : 1;      // LDS: waves * B * (B + 1) floats
  static constexpr int stride = B + 1;
};

template <typename T, int B>
__global__ __launch_bounds__(ContractionShape<B>::waves * 64) void contraction_kernel(
    ContractionArgs a) {
  using CS = ContractionShape<B>;
  constexpr int kT = B / 16;
  __shared__ float lds[CS::waves * B * CS::stride];
  const int lane = threadIdx.x & 63, g = lane >> 4, n = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int noff = 2 * a.m + 1;
  const int64_t q = (int64_t)blockIdx.x * CS::waves + wave;    // block pair of this problem
  const int64_t head = blockIdx.y;
  if (q >= (int64_t)a.nb * noff) return;
  const int rb = (int)(q / noff), o = (int)(q % noff) - a.m, cb = rb + o;
  const int64_t out = head * (int64_t)a.nb * noff + q;
  const int r0 = rb * B, c0 = cb * B;
  const int r1 = min(r0 + B, a.Lr), c1 = min(c0 + B, a.Lr);
  const bool exists = cb >= 0 && cb < a.nb;
  if (!exists || max(r1 - 1 - c0, c1 - 1 - r0) > a.h) {
    // no such block, or a pair off the support: no strictly positive kernel, no certificate
    if (lane == 0) {
      a.delta[out] = -1.f;
      if (a.kappa) a.kappa[out] = -1.f;
    }
    return;
  }
  const int nr = r1 - r0, nc = c1 - c0;
  const T* Qh = static_cast<const T*>(a.Q) + head * (int64_t)a.Lr * kD;
  const T* Kh = static_cast<const T*>(a.K) + head * (int64_t)a.Lr * kD;
  float* S = lds + wave * B * CS::stride;

  // score block S[i][j] = s q_(r0+i) . k_(c0+j); rows and columns past the sequence read its last
  // token (finite values, never used)
#pragma unroll 1
  for (int ti = 0; ti < kT; ++ti) {
    Frag<T> fq;
    load_frag_raw(fq, Qh + (int64_t)min(r0 + 16 * ti + n, a.Lr - 1) * kD, g);
#pragma unroll 1
    for (int tj = 0; tj < kT; ++tj) {
      Frag<T> fk;
      load_frag_raw(fk, Kh + (int64_t)min(c0 + 16 * tj + n, a.Lr - 1) * kD, g);
      const f32x4 acc = dot_tile(fq, fk);          // acc[r] = q_(16 ti + 4 g + r) . k_(16 tj + n)
#pragma unroll
      for (int r = 0; r < 4; ++r) S[(16 * ti + 4 * g + r) * CS::stride + 16 * tj + n] = acc[r] * a.s;
    }
  }
  __builtin_amdgcn_wave_barrier();

  // Delta = max over row pairs of the oscillation of the row difference
  float best = 0.f;
#pragma unroll 1
  for (int i = 0; i + 1 < nr; ++i) {
    const float* Si = S + i * CS::stride;
#pragma unroll 1
    for (int ip = i + 1 + lane; ip < nr; ip += 64) {
      const float* Sp = S + ip * CS::stride;
      float mx = -INFINITY, mn = INFINITY;
#pragma unroll 4
      for (int j = 0; j < nc; ++j) {
        const float dlt = Si[j] - Sp[j];
        mx = fmaxf(mx, dlt);
        mn = fminf(mn, dlt);
      }
      best = fmaxf(best, mx - mn);
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) best = fmaxf(best, __shfl_xor(best, off, 64));
  if (lane == 0) {
    a.delta[out] = best;
    if (a.kappa) a.kappa[out] = tanhf(0.25f * best);
    // Delta >= 0, so its bit pattern orders like the value (the initial -1 is negative)
    if (a.delta_max) atomicMax(reinterpret_cast<int*>(a.delta_max) + head, __float_as_int(best));
  }
}

template <typename T, int B>
static void launch_contraction_b(const ContractionArgs& a, hipStream_t st) {
  using CS = ContractionShape<B>;
  const int64_t pairs = (int64_t)a.nb * (2 * a.m + 1);
  const dim3 grid((unsigned)((pairs + CS::waves - 1) / CS::waves), (unsigned)a.bh);
  contraction_kernel<T, B><<<grid, dim3(CS::waves * 64), 0, st>>>(a);
}

template <typename T>
static hipError_t launch_contraction_t(const ContractionArgs& a, hipStream_t st) {
  switch (a.B) {
    case 16: launch_contraction_b<T, 16>(a, st); break;
    case 32: launch_contraction_b<T, 32>(a, st); break;
    case 64: launch_contraction_b<T, 64>(a, st); break;
    case 128: launch_contraction_b<T, 128>(a, st); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_contraction(int elt, const ContractionArgs& a, hipStream_t st) {
  const int64_t pairs = (int64_t)a.nb * (2 * a.m + 1);
  if (a.bh < 1 || a.bh > 65535 || a.nb < 1 || a.m < 0 || pairs > (int64_t(1) << 31))
    return hipErrorInvalidValue;
  return elt == 1 ? launch_contraction_t<bf16>(a, st) : launch_contraction_t<float>(a, st);
}

}  // namespace ska
