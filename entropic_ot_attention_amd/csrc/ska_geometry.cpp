// Launch geometry of libsinkhorn_attn.so: which kernel family and tile class a problem takes, and
// how its blocks are cut into workgroup segments.  Host code only, shared by workspace sizing and
// launch sequencing (ska_capi.cpp).

#include "ska_internal.h"

namespace ska {

// Register-resident tile class of the fused step (16-key tiles per wave, 1 + 2 H16 with H16 even),
// or 0 when the band is too wide for it.
int fused_tiles_for(int h) {
  const int h16 = (h + 15) / 16;     // halo tiles; classes use an even count
  if (h16 <= 2) return 5;
  if (h16 <= 4) return 9;
  if (h16 <= 8) return 17;
  if (h16 <= 12) return 25;
  return 0;
}

// Segments: enough workgroups to fill the GPU about once (256 CUs x 3 resident workgroups),
// and at least H16 / 2 blocks each so a column's partials come from at most two segments.
void fused_segments(int64_t bh, int Lr, int nt, int* seg_len, int* nseg) {
  const int64_t nblk = (Lr + 63) / 64;
  const int64_t target = 768;
  int64_t sl = (bh * nblk + target - 1) / target;
  const int64_t min_sl = ((nt - 1) / 2 + 1) / 2;
  if (sl < min_sl) sl = min_sl;
  if (sl < 1) sl = 1;
  if (sl > nblk) sl = nblk;
  *seg_len = (int)sl;
  *nseg = (int)((nblk + sl - 1) / sl);
}

// Waves per workgroup of the streaming passes: bf16 uses kBf16StreamWaves (128-token blocks, two
// waves per SIMD with room for the pipelined strips' registers) with two window rings of
// 128 + 32 H16 rows, fp32 4 waves; both up to the halo LDS holds (one workgroup per CU).
int vjp_stream_waves(int elt, int h, int* nt) {
  const int h16 = (h + 15) / 16;
  const int H16 = (h16 <= 2) ? 2 : (h16 <= 4) ? 4 : (h16 <= 8) ? 8 : 0;
  if (H16 == 0) return 0;
  if (elt == 0 && H16 > 4) return 0;
  *nt = 1 + 2 * H16;
  return (elt == 1) ? kBf16StreamWaves : 4;
}

// Segments of the streaming passes: one workgroup per CU, each segment spanning at least twice
// the halo so a column's partials come from at most two segments.
void vjp_stream_segments(int64_t bh, int Lr, int nw, int nt, int* seg_len, int* nseg) {
  const int br = 16 * nw;
  const int64_t nblk = (Lr + br - 1) / br;
  const int64_t target = 256;   // one workgroup per CU
  int64_t sl = (bh * nblk + target - 1) / target;
  const int64_t min_sl = (16 * (nt - 1) + br - 1) / br;   // 2 * halo <= seg span
  if (sl < min_sl) sl = min_sl;
  if (sl < 1) sl = 1;
  if (sl > nblk) sl = nblk;
  *seg_len = (int)sl;
  *nseg = (int)((nblk + sl - 1) / sl);
}

// Register tiles per wave of the wide fused step (its window of at most kWideWaves x 33 tiles stays
// in registers), or 0 when the window is wider than that.
int wide_step_tiles(int Lr, int h) {
  const int per_wave = (wide_window_tiles(Lr, h) + kWideWaves - 1) / kWideWaves;
  for (int kt : {4, 8, 12, 16, 24, 33})
    if (per_wave <= kt) return kt;
  return 0;
}

}  // namespace ska
