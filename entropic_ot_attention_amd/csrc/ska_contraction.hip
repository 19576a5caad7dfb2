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
// One wave per row block and run of up to kOffsetRun column-block offsets: the wave keeps its
// query fragments, loads the next column block's key fragments while it scans the current one,
// and forms each score block on the matrix cores (16 x 16 tiles over d = 64, as in every other
// kernel here) into its LDS slice.  Every unordered row pair is one (row i, cyclic offset delta)
// item with i' = (i + delta) mod nr and 1 <= delta <= nr / 2 (for even nr the pairs at
// delta = nr / 2 come twice, which a maximum ignores); the items are spread over the 64 lanes,
// each scanning both rows four columns at a time with 3-input max and min.  Columns past a
// ragged last block read the last token's key, so they repeat the last column and change no
// oscillation.  The wave maximum (DPP and lane swaps) is the diameter; a second kernel takes the
// maximum per problem.
// Scores are fp32 (bf16 inputs: exact products, fp32 sums), as in the forward.

#include "ska_device.h"
#include "ska_internal.h"

namespace ska {

constexpr int kOffsetRun = 24;

template <int B> struct ContractionShape {
  static constexpr int waves = (B <= 64) ? 4 : 1;      // LDS: waves * B * (B + 4) floats
  static constexpr int stride = B + 4;                 // rows 16-byte aligned, banks staggered
  static constexpr int log2b = (B == 16) ? 4 : (B == 32) ? 5 : (B == 64) ? 6 : 7;
  static constexpr int kT = B / 16;
};

// oscillation maximum over the row-pair items of one score block, this lane's share
template <int B>
__device__ __forceinline__ float scan_pairs(const float* S, int nr, int lane) {
  using CS = ContractionShape<B>;
  float best = 0.f;
  auto scan = [&](int i, int ip) {
    const f32x4* Si = reinterpret_cast<const f32x4*>(S + i * CS::stride);
    const f32x4* Sp = reinterpret_cast<const f32x4*>(S + ip * CS::stride);
    float mx = -INFINITY, mn = INFINITY;
#pragma unroll 8
    for (int j = 0; j < B / 4; ++j) {
      const f32x4 x = Si[j], y = Sp[j];
      const float d0 = x[0] - y[0], d1 = x[1] - y[1], d2 = x[2] - y[2], d3 = x[3] - y[3];
      mx = fmaxf(mx, fmaxf(d0, d1));
      mn = fminf(mn, fminf(d0, d1));
      mx = fmaxf(mx, fmaxf(d2, d3));
      mn = fminf(mn, fminf(d2, d3));
    }
    best = fmaxf(best, mx - mn);
  };
  if (nr == B) {
#pragma unroll 1
    for (int t = lane; t < B * (B / 2); t += 64) {
      const int i = t & (B - 1);
      scan(i, (i + 1 + (t >> CS::log2b)) & (B - 1));
    }
  } else {
    const int items = nr * (nr >> 1);
#pragma unroll 1
    for (int t = lane; t < items; t += 64) {
      const int i = t % nr;
      int ip = i + 1 + t / nr;
      ip -= (ip >= nr) ? nr : 0;
      scan(i, ip);
    }
  }
  return best;
}

template <typename T, int B>
__global__ __launch_bounds__(ContractionShape<B>::waves * 64) void contraction_kernel(
    ContractionArgs a) {
  using CS = ContractionShape<B>;
  __shared__ float lds[CS::waves * B * CS::stride];
  const int lane = threadIdx.x & 63, g = lane >> 4, n = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int noff = 2 * a.m + 1;
  const int nrun = (noff + kOffsetRun - 1) / kOffsetRun;
  const int64_t q = (int64_t)blockIdx.x * CS::waves + wave;    // (row block, offset run)
  const int64_t head = blockIdx.y;
  if (q >= (int64_t)a.nb * nrun) return;
  const int rb = (int)(q / nrun);
  const int k0 = (int)(q % nrun) * kOffsetRun, k1 = min(k0 + kOffsetRun, noff);
  const int r0 = rb * B, r1 = min(r0 + B, a.Lr), nr = r1 - r0;
  const T* Qh = static_cast<const T*>(a.Q) + head * (int64_t)a.Lr * kD;
  const T* Kh = static_cast<const T*>(a.K) + head * (int64_t)a.Lr * kD;
  float* S = lds + wave * B * CS::stride;
  float* drow = a.delta + (head * a.nb + rb) * (int64_t)noff;
  float* krow = a.kappa ? a.kappa + (head * a.nb + rb) * (int64_t)noff : nullptr;
  // a column block is scanned when it exists and every pair with the row block is on the support
  auto active = [&](int k) {
    const int cb = rb + k - a.m;
    if (cb < 0 || cb >= a.nb) return false;
    const int c0 = cb * B, c1 = min(c0 + B, a.Lr);
    return max(r1 - 1 - c0, c1 - 1 - r0) <= a.h;
  };
  // rows and columns past the sequence read its last token (finite values: repeated columns,
  // rows never scanned)
  auto qrow = [&](int ti) { return Qh + (int64_t)min(r0 + 16 * ti + n, a.Lr - 1) * kD; };
  auto krow_ptr = [&](int k, int tj) {
    return Kh + (int64_t)min((rb + k - a.m) * B + 16 * tj + n, a.Lr - 1) * kD;
  };

  Frag<T> fq0;
  load_frag_raw(fq0, qrow(0), g);
  // next active offset at or after k (k1 if none)
  auto next_active = [&](int k) {
    while (k < k1 && !active(k)) {
      if (lane == 0) {
        drow[k] = -1.f;
        if (krow) krow[k] = -1.f;
      }
      ++k;
    }
    return k;
  };
  int k = next_active(k0);
  Frag<T> fk;
  if (k < k1) load_frag_raw(fk, krow_ptr(k, 0), g);
#pragma unroll 1
  while (k < k1) {
    // score block of offset k into LDS; the first key tile is already in registers
#pragma unroll 1
    for (int ti = 0; ti < CS::kT; ++ti) {
      Frag<T> fq = fq0;
      if (ti > 0) load_frag_raw(fq, qrow(ti), g);
#pragma unroll 1
      for (int tj = 0; tj < CS::kT; ++tj) {
        Frag<T> fkt = fk;
        if (ti + tj > 0) load_frag_raw(fkt, krow_ptr(k, tj), g);
        const f32x4 acc = dot_tile(fq, fkt);       // acc[r] = q_(16 ti + 4 g + r) . k_(16 tj + n)
#pragma unroll
        for (int r = 0; r < 4; ++r) S[(16 * ti + 4 * g + r) * CS::stride + 16 * tj + n] = acc[r] * a.s;
      }
    }
    const int kn = next_active(k + 1);
    if (kn < k1) load_frag_raw(fk, krow_ptr(kn, 0), g);   // in flight during the scan
    __builtin_amdgcn_wave_barrier();
    const float best = wave_max(scan_pairs<B>(S, nr, lane));
    if (lane == 0) {
      drow[k] = best;
      if (krow) krow[k] = tanhf(0.25f * best);
    }
    __builtin_amdgcn_wave_barrier();
    k = kn;
  }
}

// delta_max[b] = max over the problem's block pairs (-1 entries included, so -1 if none is
// active).  Each workgroup reduces a chunk of kMaxChunk entries and folds its maximum into
// delta_max (set to -1 beforehand) with one atomic maximum on the bit pattern, which orders like
// the value for -1 and non-negative floats; a maximum does not depend on the order.
constexpr int kMaxChunk = 8192;

__global__ __launch_bounds__(256) void block_max_kernel(const float* __restrict__ delta,
                                                        float* __restrict__ delta_max, int64_t n) {
  __shared__ float red[256];
  const float* d = delta + blockIdx.y * n;
  const int64_t k0 = (int64_t)blockIdx.x * kMaxChunk;
  const int64_t k1 = min(k0 + kMaxChunk, n);
  float x = -1.f;
  for (int64_t k = k0 + threadIdx.x; k < k1; k += 256) x = fmaxf(x, d[k]);
  red[threadIdx.x] = x;
  __syncthreads();
#pragma unroll
  for (int w = 128; w >= 1; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + w]);
    __syncthreads();
  }
  if (threadIdx.x == 0) atomicMax(reinterpret_cast<int*>(delta_max) + blockIdx.y, __float_as_int(red[0]));
}

template <typename T, int B>
static void launch_contraction_b(const ContractionArgs& a, hipStream_t st) {
  using CS = ContractionShape<B>;
  const int64_t runs = (int64_t)a.nb * ((2 * a.m + 1 + kOffsetRun - 1) / kOffsetRun);
  const dim3 grid((unsigned)((runs + CS::waves - 1) / CS::waves), (unsigned)a.bh);
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

static bool contraction_shape_ok(const ContractionArgs& a) {
  const int64_t pairs = (int64_t)a.nb * (2 * a.m + 1);
  return a.bh >= 1 && a.bh <= 65535 && a.nb >= 1 && a.m >= 0 && pairs < (int64_t(1) << 31);
}

hipError_t launch_contraction(int elt, const ContractionArgs& a, hipStream_t st) {
  if (!contraction_shape_ok(a)) return hipErrorInvalidValue;
  return elt == 1 ? launch_contraction_t<bf16>(a, st) : launch_contraction_t<float>(a, st);
}

hipError_t launch_contraction_max(const ContractionArgs& a, hipStream_t st) {
  if (!contraction_shape_ok(a) || !a.delta_max) return hipErrorInvalidValue;
  const int64_t pairs = (int64_t)a.nb * (2 * a.m + 1);
  const hipError_t e = launch_fill(a.delta_max, a.bh, -1.f, st);
  if (e != hipSuccess) return e;
  block_max_kernel<<<dim3((unsigned)((pairs + kMaxChunk - 1) / kMaxChunk), (unsigned)a.bh), dim3(256), 0,
                     st>>>(a.delta, a.delta_max, pairs);
  return hipGetLastError();
}

}  // namespace ska
