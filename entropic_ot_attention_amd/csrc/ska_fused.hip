// Fused balanced Sinkhorn step for bands that fit in registers (gfx950).
//
// One launch performs one full Sinkhorn step of the stopped base or of the tail
// [technical summaries §2.1: T-step balanced Sinkhorn on the fixed band, then the R-step tail]:
//
//   1. finish the previous column update for the block's key window:
//        v_j <- v_j - log sum_i exp(S_ij + u_i + v_j)      (column sums from the previous launch)
//   2. row update for the 64 owned queries:  u_i = -log sum_j exp(S_ij + v_j)
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
// After the first step the row log-sum-exp is shifted by the previous step's row dual, which
// enters the matrix-core accumulator, instead of by the row maximum.  Each shifted term is then
// an entry of the previous plan after its column normalisation, hence at most 1, and each row
// sum lies in [1 / (2h + 1), 2h + 1]: the max pass disappears with no loss of range.  The first
// step (from u = 0) subtracts the exact row maximum.
//
// Column sums can underflow only when a column's mass under the current plan falls below
// 2^-60 (scores spanning more than ~40 nats inside one band); such a column is finished by an
// exact log-sum-exp over its band instead, so the result never depends on that threshold beyond
// rounding.  (A plan entry lost to underflow is below 2^-118.)

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "ska_device.h"
#include "ska_internal.h"

namespace ska {

// Finished column dual (log2 units) of key j from the previous dual and the column sums of
// exp(S + u + v_prev) that the previous launch left per segment.  Segment k of a problem covers
// columns [S k - 16 H16, S (k + 1) + 16 H16) with S = 64 seg_len, so at most two segments hold a
// partial for j (seg_len >= H16 / 2); they are added in ascending segment order.
// Loads of the column finish for key j: the (at most two) segment partials and the previous dual.
// The column sum is p0 w0 + p1 w1 with weights 0 or 1 (partials are finite), applied where the
// values are used, so that issuing the loads never waits on them.
struct ColIn {
  float p0, p1, vp, w0, w1;
};
__device__ __forceinline__ ColIn column_loads(int j, const float* vprev_h, const float* part_h,
                                              const StepArgs& a) {
  const int S = 64 * a.seg_len, halo = 16 * a.H16;
  const int jc = min(max(j, 0), a.Lr - 1);
  const int k0 = max(0, floor_div(jc - halo, S));
  const int k1 = min(a.nseg - 1, floor_div(jc + halo, S));
  float p[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int k = k0 + q, c = jc - (S * k - halo);
    const bool ok = (k <= k1) & (c >= 0) & (c < a.pstride);
    const int kc = min(k, a.nseg - 1), cc = min(max(c, 0), a.pstride - 1);
    const float x = part_h[(int64_t)kc * a.pstride + cc];
    p[q] = ok ? x : 0.f;     // an unused slot may hold anything, even non-finite values
  }
  return ColIn{p[0], p[1], vprev_h[jc], 1.f, 1.f};
}

// Finished column dual (log2 units) of key j from the previous dual and the column sums of
// exp(S + u + v_prev) that the previous launch left per segment.  Segment k of a problem covers
// columns [S k - 16 H16, S (k + 1) + 16 H16) with S = 64 seg_len, so at most two segments hold a
// partial for j (seg_len >= H16 / 2); they are added in ascending segment order.
template <typename T>
__device__ __forceinline__ float column_combine(int j, const ColIn& in, const float* u_h, const T* Qh,
                                                const T* Kh, const StepArgs& a) {
  const float s = in.p0 * in.w0 + in.p1 * in.w1;
  if (s >= 0x1p-60f) return in.vp - fast_log2(s);
  return exact_column<T>(j, u_h, Qh, Kh, a.Lr, a.h, a.c2);
}

template <typename T>
__device__ float finish_column(int j, const float* vprev_h, const float* part_h, const float* u_h,
                               const T* Qh, const T* Kh, const StepArgs& a) {
  return column_combine<T>(j, column_loads(j, vprev_h, part_h, a), u_h, Qh, Kh, a);
}

template <typename T, int NT>
struct StepSmem {
  static constexpr int kH16 = (NT - 1) / 2;
  static constexpr int kRing = 64 + 32 * kH16;               // block key window = ring rows
  static constexpr int kRingBytes = kRing * Lds<T>::stride * (int)sizeof(T);
};

// One full Sinkhorn step for one segment of consecutive 64-row blocks of one problem.  SHIFT:
// the row log-sum-exp is shifted by the previous step's row duals (every launch after the first);
// otherwise by the exact row maximum.  REV: the segment is walked from its last block down;
// consecutive launches alternate direction, so each starts on the keys and queries the previous
// one touched last (still in the last-level cache when a launch reads a little more than it
// holds).
template <typename T, int NT, bool SHIFT, bool REV>
__global__ __launch_bounds__(256) void sinkhorn_step_kernel(StepArgs a) {
  constexpr int H16 = (NT - 1) / 2;
  constexpr int RING = StepSmem<T, NT>::kRing;
  constexpr int LS = Lds<T>::stride;
  static_assert(H16 % 2 == 0, "ring rows must be a multiple of 64");
  __shared__ __attribute__((aligned(16))) T kring[RING * LS];
  __shared__ float vring[RING];            // finished column duals, by key mod RING
  __shared__ float pring[RING];            // this segment's column sums, by key mod RING
  __shared__ float cpart[kWaves * RING];   // [wave][RING] block column sums

  const int lane = threadIdx.x & 63, g = lane >> 4, n = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t head = blockIdx.x / a.nseg;
  const int seg = blockIdx.x % a.nseg;
  const int blk0 = seg * a.seg_len, blk1 = min(blk0 + a.seg_len, a.nblk);
  const int c_lo = 64 * blk0 - 16 * H16;    // first column this segment touches
  const int own_lo = 64 * blk0, own_hi = 64 * blk1;
  const int Lr = a.Lr, h = a.h;
  const float c2 = a.c2, inv_c2 = 1.f / a.c2;
  const T* Qh = static_cast<const T*>(a.Q) + head * (int64_t)Lr * kD;
  const T* Kh = static_cast<const T*>(a.K) + head * (int64_t)Lr * kD;
  const int64_t vo = head * (int64_t)a.Lpad;
  const float* u_prev_h = a.u_prev + vo;
  const float* part_prev_h = a.part_prev ? a.part_prev + head * (int64_t)a.nseg * a.pstride : nullptr;
  float* part_out_h = a.part_out + (head * (int64_t)a.nseg + seg) * a.pstride;

  // finished column dual of key j (log2 units) from its loads, and its owner-side copies
  auto finish_value = [&](int j, const ColIn& in) -> float {
    if (j < 0 || j >= Lr) return 0.f;
    return part_prev_h ? column_combine<T>(j, in, u_prev_h, Qh, Kh, a) : in.vp;
  };
  auto store_owned_v = [&](int j, float v) {
    if (j >= own_lo && j < own_hi && j < Lr) {
      a.v_next[vo + j] = v;
      if (a.save_v) a.save_v[head * a.save_v_stride + j] = v * kLn2;
    }
  };
  auto finish_from = [&](int j, const ColIn& in) -> float {
    const float v = finish_value(j, in);
    store_owned_v(j, v);
    return v;
  };
  // the first step (no column partials yet) starts from v = 0 and reads no column duals
  auto loads_for = [&](int j) -> ColIn {
    if (part_prev_h) return column_loads(j, a.v_prev + vo, part_prev_h, a);
    return ColIn{0.f, 0.f, 0.f, 0.f, 0.f};
  };
  // previous row duals of rows o, .., o + 3 (log2 units); the dual buffers are padded to Lpad,
  // a multiple of 64, and hold 0 past Lr
  auto shift_rows = [&](int o) -> f32x4 {
    if constexpr (SHIFT) return load4(u_prev_h + o);
    return f32x4{0.f, 0.f, 0.f, 0.f};
  };

  const bool exact_h = (h == 16 * H16);
  // per-lane offsets of the lane's query row (from a block's first row) and row-shift group
  const int q_lane = (16 * wave + n) * kD, u_lane = 16 * wave + 4 * g;
  // per-wave column sums live at columns [16 wave, 16 wave + 16 NT) of a RING-wide row; the
  // other columns stay zero so the block sum below needs no coverage tests
  for (int c = threadIdx.x; c < kWaves * RING; c += 256) cpart[c] = 0.f;

  // prologue: the first block's whole window, query fragment and row shifts
  const int blkF = REV ? blk1 - 1 : blk0;     // first block walked
  const int cF = 64 * blkF - 16 * H16;
  Frag<T> fq;
  load_frag(fq, Qh + (int64_t)(64 * blkF + 16 * wave + n) * kD, 64 * blkF + 16 * wave + n < Lr, g);
  // row shifts / c2 for the matrix-core accumulator, carried from block to block
  auto shift_acc = [&](f32x4 us) {
    return f32x4{us[0] * inv_c2, us[1] * inv_c2, us[2] * inv_c2, us[3] * inv_c2};
  };
  f32x4 shc = shift_acc(shift_rows(64 * blkF + 16 * wave + 4 * g));
  {
    RowStage<T, RING, 256> first;
    first.load(Kh, cF, Lr);
    first.template store<RING>(kring, cF);
  }
  for (int c = threadIdx.x; c < RING; c += 256) {
    const int j = cF + c;
    vring[(j + 4 * RING) % RING] = finish_from(j, loads_for(j));
    pring[c] = 0.f;
  }
  __syncthreads();

  // Graded wave priority.  Each SIMD runs waves of three workgroups, and a workgroup passes its
  // block barriers only when all four of its waves arrive.  A wave issues its block's prefetch
  // loads at the top priority (so they leave early), starts the strip at priority 0 and raises
  // it as it gets through the strip (1 and 2 at about 5/17 and 11/17 of the tiles, 3 once the
  // strip is done), so the SIMD favours the waves closest to their barrier: whole workgroups
  // spend less time waiting there (about 9% off each launch at h = 128).
  constexpr int kPrio1 = (5 * NT) / 17, kPrio2 = (11 * NT) / 17;
  for (int it = 0; it < blk1 - blk0; ++it) {
    __builtin_amdgcn_s_setprio(3);
    const int blk = REV ? blk1 - 1 - it : blk0 + it;
    const int b0 = 64 * blk;
    const int cb = b0 - 16 * H16;             // block window [cb, cb + RING)
    const bool more = it + 1 < blk1 - blk0;
    const int b0n = REV ? b0 - 64 : b0 + 64;  // rows of the next block walked
    // keys entering the window with the next block, and (window offset of) the keys leaving it
    // with this one; both take the same ring slots
    const int enter0 = REV ? cb - 64 : cb + RING;
    const int leave_c = REV ? RING - 64 : 0;
    // ring slot of the window's first key (a multiple of 16; the 64 keys [cb, cb + 64) occupy
    // consecutive slots unless the ring is not a multiple of 64 keys past it)
    const int s_cb = (cb + RING) % RING;
    // the wave that finishes the columns leaving with this block rotates, so that extra work
    // spreads over the four SIMDs
    const int dw = blk & 3;
    // prefetch the 64 key rows the next block adds: [enter0, enter0 + 64)
    // (and the next block's query fragment, row shifts and new column loads), all in flight
    // during compute
    RowStage<T, 64, 256> nr;
    ColIn nc{0.f, 0.f, 0.f, 0.f, 0.f};
    Frag<T> fq_next;
    f32x4 ush_next;
    if (more) {
      if (enter0 >= 0 && enter0 + 64 <= Lr) nr.load_inside(Kh, enter0);
      else nr.load(Kh, enter0, Lr);
      if (b0n >= 0 && b0n + 64 <= Lr) {
        // every row of the next block lies inside the sequence: a block base plus the lane's
        // fixed offset, with no validity test
        load_frag_raw(fq_next, Qh + (int64_t)b0n * kD + q_lane, g);
        if constexpr (SHIFT) ush_next = load4(u_prev_h + b0n + u_lane);
        else ush_next = f32x4{0.f, 0.f, 0.f, 0.f};
      } else {
        const int on = b0n + 16 * wave + n;
        load_frag(fq_next, Qh + (int64_t)on * kD, on < Lr, g);
        ush_next = shift_rows(b0n + u_lane);
      }
      if (wave == dw) {
        // Keys j = enter0 + lane enter with the next block.  Inside a segment their column
        // partials sit at fixed offsets (no divisions): the segment's own row at j - c_lo, and,
        // walking up, the next segment's row once j - c_lo reaches S = 64 seg_len, or, walking
        // down, the previous segment's row while j - c_lo < 2 halo.  Partials are summed in
        // ascending segment order, as column_loads does.
        const int j = enter0 + lane;
        // walking down, the first blocks of a problem take keys j < 0 into the window: their
        // (unused) dual is read at a clamped index, inside the problem's vector
        const float vp = part_prev_h ? a.v_prev[vo + min(max(j, 0), Lr - 1)] : 0.f;
        if (part_prev_h) {
          const int S = 64 * a.seg_len, c0 = j - c_lo;
          const float* own_row = part_prev_h + (int64_t)seg * a.pstride;
          if constexpr (!REV) {
            const int c1 = c0 - S;
            const bool two = (c1 >= 0) & (seg + 1 < a.nseg);
            const float p0 = own_row[c0];
            const float p1 = part_prev_h[(int64_t)(two ? seg + 1 : seg) * a.pstride + (two ? c1 : c0)];
            nc = ColIn{p0, p1, vp, 1.f, two ? 1.f : 0.f};
          } else {
            const bool low = (seg > 0) & (c0 < 32 * H16);
            const float p0 = part_prev_h[(int64_t)(low ? seg - 1 : seg) * a.pstride + (low ? c0 + S : c0)];
            const float p1 = own_row[c0];
            nc = ColIn{p0, p1, vp, 1.f, low ? 1.f : 0.f};
          }
        } else {
          nc = ColIn{0.f, 0.f, vp, 0.f, 0.f};
        }
      }
    }

    __builtin_amdgcn_s_setprio(0);
    // score strip in registers (wave rows o0 .. o0 + 15), row shift in the accumulator:
    // x = c2 (ush / c2 + q.k) + v_j  ~  log2(e) S + v_j + u_prev  on the band, -inf elsewhere
    const int o0 = b0 + 16 * wave;
    const int cw = o0 - 16 * H16;
    const bool rows_in = (o0 + 15 < Lr);
    // Interior blocks of a band whose half-width fills its halo class (h = 16 H16): every tile is
    // on the band and inside the sequence; only the first and last tiles cross the band edge,
    // along a fixed per-lane pattern (i - j <= h  <=>  4g + r <= n on tile 0, i - j >= -h  <=>
    // 4g + r >= n on tile NT - 1).  No per-tile tests.
    const bool interior = exact_h & (cb >= 0) & (cb + RING <= Lr) & (b0 + 64 <= Lr);
    const int row0 = (cw + 4 * RING) % RING;
    // Interior blocks of a shifted step take the exponentials (and row sums) as the tiles arrive,
    // which overlaps them with the key-fragment reads and the matrix-core work of later tiles;
    // their x then holds 2^x (0 off the band).
    const bool exp_in_strip = SHIFT && interior;
    auto strip = [&](f32x4 (&x)[NT], float (&ll)[4]) {
      if (interior) {
        // per-lane bases plus a wave-uniform row offset per tile: one address add per read
        const T* klane = kring + n * LS + 16 * g;
        const float* vlane = vring + n;
        auto tile_row = [&](int t) { return (row0 + 16 * t < RING) ? row0 + 16 * t : row0 + 16 * t - RING; };
        auto kfrag = [&](Frag<T>& f, int rt) {
          const f32x4* p = reinterpret_cast<const f32x4*>(klane + rt * LS);
          if constexpr (sizeof(T) == 2) {
            f.a = __builtin_bit_cast(bf16x8, p[0]);
            f.b = __builtin_bit_cast(bf16x8, p[1]);
          } else {
            lds_frag(f, kring, rt + n, g);
          }
        };
        // key fragments and column duals KA tiles ahead of the matrix cores (an LDS read takes
        // longer than the work on one tile; reads complete in order, so a dual read just before
        // its use would also wait for the fragments issued ahead of it)
        constexpr int KA = 2;
        Frag<T> fk[KA + 1];
        float vj[KA + 1];
#pragma unroll
        for (int t = 0; t < KA && t < NT; ++t) {
          kfrag(fk[t], tile_row(t));
          vj[t] = vlane[tile_row(t)];
        }
        // the matrix-core products run one tile ahead of the vector work on them
        x[0] = dot_tile(fq, fk[0], shc);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          if (t + 1 < NT) x[t + 1] = dot_tile(fq, fk[(t + 1) % (KA + 1)], shc);
          if (t + KA < NT) {
            kfrag(fk[(t + KA) % (KA + 1)], tile_row(t + KA));
            vj[(t + KA) % (KA + 1)] = vlane[tile_row(t + KA)];
          }
          if (t == kPrio1 && t > 0) __builtin_amdgcn_s_setprio(1);
          if (t == kPrio2) __builtin_amdgcn_s_setprio(2);
          const float vjt = vj[t % (KA + 1)];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float xv = fmaf(x[t][r], c2, vjt);
            bool keep = true;
            if (t == 0) keep = (4 * g + r <= n);
            if (t == NT - 1) keep = (4 * g + r >= n);
            if constexpr (SHIFT) {
              xv = keep ? fast_exp2(xv) : 0.f;
              ll[r] += xv;
            } else {
              xv = keep ? xv : -INFINITY;
            }
            x[t][r] = xv;
          }
        }
      } else {
        // Tile t covers keys cw + 16t .. cw + 16t + 15; over its entries i - j spans
        // [16 H16 - 16 t - 15, 16 H16 - 16 t + 15].  Wave-uniform classes: "dead" tiles (no entry
        // on the band or inside the sequence) skip the MFMA; "clean" tiles skip the masks.
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const int j0 = cw + 16 * t;
          const int dlo = 16 * H16 - 16 * t - 15, dhi = 16 * H16 - 16 * t + 15;
          const bool dead = (dlo > h) | (dhi < -h) | (j0 >= Lr) | (j0 + 15 < 0) | (o0 >= Lr);
          if (dead) {
            x[t] = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
            continue;
          }
          const int rt = (row0 + 16 * t) % RING;
          Frag<T> fk;
          lds_frag(fk, kring, rt + n, g);
          const float vjt = vring[rt + n];
          x[t] = dot_tile(fq, fk, shc);
          const bool clean = rows_in & (j0 >= 0) & (j0 + 15 < Lr) & (dhi <= h) & (dlo >= -h);
          if (clean) {
#pragma unroll
            for (int r = 0; r < 4; ++r) x[t][r] = fmaf(x[t][r], c2, vjt);
          } else {
            const int j = j0 + n;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int i = o0 + 4 * g + r;
              const bool ok = (i < Lr) & (j >= 0) & (j < Lr) & (abs(i - j) <= h);
              x[t][r] = ok ? fmaf(x[t][r], c2, vjt) : -INFINITY;
            }
          }
        }
      }
    };

    // column sums of the new plan over the wave's 16 rows: in-lane over the 4 rows, then over the
    // four lane groups (lanes n, n + 16, n + 32, n + 48 hold the same key).  gfx950 lane swaps
    // reduce four tiles at once: v_permlane32_swap(cp_a, cp_b) leaves a's and b's half sums in the
    // low and high 32 lanes, v_permlane16_swap of two such pairs leaves the full sums of tiles
    // a, c, b, d in lane groups 0..3; each lane then stores one tile's sum for its key.
    // Lane group g of a reduced quad (tiles q, q+1, q+2, q+3) holds tile q + {0, 2, 1, 3}[g].
    const int gsel = (g == 1) ? 2 : (g == 2) ? 1 : g;
    // cp[t]: this lane's key of tile t summed over its 4 rows of the new plan
    auto emit_columns = [&](float (&cp)[NT]) {
#pragma unroll
      for (int q = 0; q + 4 <= NT; q += 4) {
        const float s4 = swap16_sum(swap32_sum(cp[q], cp[q + 1]), swap32_sum(cp[q + 2], cp[q + 3]));
        cpart[wave * RING + 16 * wave + 16 * (q + gsel) + n] = s4;
      }
      // the tile left over after the quads: one sum over the lane groups, stored by group 0
      static_assert(NT % 4 == 1, "every tile class leaves one tile after the quads");
      const float s1 = lane_group_sum(cp[NT - 1]);
      if (g == 0) cpart[wave * RING + 16 * wave + 16 * (NT - 1) + n] = s1;
    };

    // Row log-sum-exp.  With SHIFT the previous row duals are already in x, and then 2^x is an
    // entry of the previous plan after its column normalisation (x = log2 P_prev - log2 colsum),
    // so every term is at most 1 and every row sum lies in [1 / (2h + 1), 2h + 1]: no max pass
    // is needed.  Without SHIFT (the first step, from u = 0) the exact row maximum is subtracted.
    // u = -log2 sum_j 2^(c2 S_ij + v_j) either way.
    float u[4];
    float cp[NT];
    {
      f32x4 x[NT];
      float ll[4] = {0.f, 0.f, 0.f, 0.f};
      strip(x, ll);
      __builtin_amdgcn_s_setprio(3);
      float mx[4] = {0.f, 0.f, 0.f, 0.f};
      if constexpr (!SHIFT) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float mm = x[0][r];
#pragma unroll
          for (int t = 1; t < NT; ++t) mm = fmaxf(mm, x[t][r]);
          mm = row16_max(mm);
          mx[r] = (mm == -INFINITY) ? 0.f : mm;     // empty rows (past the sequence) stay 0
#pragma unroll
          for (int t = 0; t < NT; ++t) x[t][r] -= mx[r];
        }
      }
      if (!exp_in_strip) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            x[t][r] = fast_exp2(x[t][r]);
            ll[r] += x[t][r];
          }
      }
      float rinv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) ll[r] = row16_sum(ll[r]);
      if (interior) {
        // every row has band entries
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float lg = SHIFT ? fast_log2(ll[r]) : mx[r] + fast_log2(ll[r]);
          u[r] = fmaf(shc[r], c2, -lg);
          rinv[r] = __builtin_amdgcn_rcpf(ll[r]);
        }
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          // no terms: rows past the sequence
          const bool empty = (ll[r] == 0.f);
          const float lg = SHIFT ? fast_log2(ll[r]) : mx[r] + fast_log2(ll[r]);
          u[r] = empty ? 0.f : fmaf(shc[r], c2, -lg);
          rinv[r] = empty ? 0.f : __builtin_amdgcn_rcpf(ll[r]);
        }
      }
#pragma unroll
      for (int t = 0; t < NT; ++t)
        cp[t] = x[t][0] * rinv[0] + x[t][1] * rinv[1] + x[t][2] * rinv[2] + x[t][3] * rinv[3];
    }
    emit_columns(cp);
    // Global stores of the block are issued after its end-of-block wait for the prefetched
    // registers: loads and stores share one counter, so a store issued earlier would be waited
    // for there as well.
    // row dual (lanes n < 4 of each group), for every row of the block: rows past the sequence
    // (empty, u = 0) keep the padding of the row-dual buffer at 0 for the next step's shifts
    const int st_i = (n < 4) ? o0 + 4 * g + n : a.Lpad;
    const float st_u = (n == 0) ? u[0] : (n == 1) ? u[1] : (n == 2) ? u[2] : u[3];
    int st_pj = -1, st_vj = Lr;                           // column partial / finished column dual
    float st_pv = 0.f, st_vv = 0.f;
    __syncthreads();
    // Block column sums (fixed wave order) into the segment accumulator.  The 64 columns at
    // window offset leave_c leave the window with this block: wave dw writes their sums out and
    // their slots take the next block's new keys [enter0, enter0 + 64) (every wave is past its
    // reads of kring and vring for this block).
    auto slot_of = [&](int c) {
      const int sl = s_cb + c;
      return (sl >= RING) ? sl - RING : sl;
    };
    auto block_sum = [&](int c) {
      return ((cpart[c] + cpart[RING + c]) + cpart[2 * RING + c]) + cpart[3 * RING + c];
    };
    for (int k = (int)threadIdx.x; k < RING - 64; k += 256) {
      const int c = REV ? k : k + 64;                     // the columns that stay
      const float sacc = block_sum(c);
      const int slot = slot_of(c);
      if (more) pring[slot] += sacc;
      else part_out_h[cb + c - c_lo] = pring[slot] + sacc;
    }
    if (wave == dw) {
      const int c = leave_c + lane, slot = slot_of(c);
      st_pj = cb + c - c_lo;
      st_pv = pring[slot] + block_sum(c);
      if (more) {
        pring[slot] = 0.f;
        st_vj = enter0 + lane;
        st_vv = finish_value(st_vj, nc);
        vring[slot] = st_vv;
      }
    }
    if (more) {
      nr.template store_slots<RING>(kring, slot_of(leave_c));
      fq = fq_next;
      shc = shift_acc(ush_next);
      __syncthreads();
    }
    if (st_i < a.Lpad) {
      a.u_out[vo + st_i] = st_u;
      if (a.save_u && st_i < Lr) a.save_u[head * a.save_u_stride + st_i] = st_u * kLn2;
    }
    if (st_pj >= 0) part_out_h[st_pj] = st_pv;
    store_owned_v(st_vj, st_vv);
  }
}

// Finish the last column update of the forward for every token; also writes the saved dual.
// The padding [Lr, Lpad) of the finished column duals is written as 0, so an output pass that
// loads whole vector groups of them reads defined values there.
template <typename T>
__global__ __launch_bounds__(256) void finish_columns_kernel(StepArgs a) {
  const int64_t head = blockIdx.y;
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= a.Lpad) return;
  if (j >= a.Lr) {
    a.v_next[head * (int64_t)a.Lpad + j] = 0.f;
    return;
  }
  const T* Qh = static_cast<const T*>(a.Q) + head * (int64_t)a.Lr * kD;
  const T* Kh = static_cast<const T*>(a.K) + head * (int64_t)a.Lr * kD;
  const int64_t vo = head * (int64_t)a.Lpad;
  const float v = finish_column<T>(j, a.v_prev + vo, a.part_prev + head * (int64_t)a.nseg * a.pstride,
                                   a.u_prev + vo, Qh, Kh, a);
  a.v_next[vo + j] = v;
  if (a.save_v) a.save_v[head * a.save_v_stride + j] = v * kLn2;
}

template <typename T, int NT>
static void launch_step_t(const StepArgs& a, bool rev, hipStream_t st) {
  const unsigned blocks = (unsigned)(a.bh * (int64_t)a.nseg);
  // the first step (no column partials yet, u = 0) has no previous plan to shift by
  if (!a.part_prev) sinkhorn_step_kernel<T, NT, false, false><<<dim3(blocks), dim3(256), 0, st>>>(a);
  else if (rev) sinkhorn_step_kernel<T, NT, true, true><<<dim3(blocks), dim3(256), 0, st>>>(a);
  else sinkhorn_step_kernel<T, NT, true, false><<<dim3(blocks), dim3(256), 0, st>>>(a);
}

hipError_t launch_fused_step(int elt, int nt, const StepArgs& a, bool rev, hipStream_t st) {
  if (elt == 1) {
    switch (nt) {
      case 5: launch_step_t<bf16, 5>(a, rev, st); break;
      case 9: launch_step_t<bf16, 9>(a, rev, st); break;
      case 17: launch_step_t<bf16, 17>(a, rev, st); break;
      default: launch_step_t<bf16, 25>(a, rev, st); break;
    }
  } else {
    switch (nt) {
      case 5: launch_step_t<float, 5>(a, rev, st); break;
      case 9: launch_step_t<float, 9>(a, rev, st); break;
      case 17: launch_step_t<float, 17>(a, rev, st); break;
      default: launch_step_t<float, 25>(a, rev, st); break;
    }
  }
  return hipGetLastError();
}

hipError_t launch_finish_columns(int elt, const StepArgs& a, hipStream_t st) {
  dim3 grid((unsigned)((a.Lpad + 255) / 256), (unsigned)a.bh);
  if (elt == 1) finish_columns_kernel<bf16><<<grid, dim3(256), 0, st>>>(a);
  else finish_columns_kernel<float><<<grid, dim3(256), 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace ska
