// Online-softmax and epilogue building blocks shared by the fused attention kernels.
#pragma once

#include "fa_device.hpp"

namespace fa {

// ------------------------------------------------------------------------------------
// Online softmax over one key tile (shared by the 16-bit and fp32 variants).
//   s[SB]   scores of the tile (S^T blocks of 32 keys), replaced by P in place
//   o[OB]   output accumulator, rescaled by alpha
//   mc, l   running max (pre-multiplied by c) and this lane's partial row sum
//   nvalid  number of valid keys in the tile (keys >= nvalid are masked to -inf)
//   SKIP    skip the O multiply when every alpha of the wave is 1 (a wave-uniform
//           branch); false keeps the tile body branch-free for instruction scheduling
// ------------------------------------------------------------------------------------
template <int SB, int OB, bool MASK, bool SKIP = true>
__device__ __forceinline__ void softmax_tile(f32x16 (&s)[SB], f32x16 (&o)[OB], float &mc, float &l,
                                             float c, int nvalid, int h) {
  if constexpr (MASK) {
#pragma unroll
    for (int t = 0; t < SB; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        int key = 32 * t + 8 * (r >> 2) + 4 * h + (r & 3);
        if (key >= nvalid) s[t][r] = -INFINITY;
      }
  }
  float mx = s[0][0];
#pragma unroll
  for (int t = 0; t < SB; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[t][r]);
  mx = pair_max(mx);                       // full row max over the tile's keys
  const float mc_new = fmaxf(mc, mx * c);  // running max in base-2 units
  // a row that has seen only masked keys keeps alpha = 0 and P = 0 (no inf - inf)
  const float alpha = (mc == -INFINITY) ? 0.f : ex2(mc - mc_new);
  const float sub = (mc_new == -INFINITY) ? 0.f : mc_new;
  float rs = 0.f;
#pragma unroll
  for (int t = 0; t < SB; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float p = ex2(fmaf(s[t][r], c, -sub));
      s[t][r] = p;
      rs += p;
    }
  l = fmaf(l, alpha, rs);
  mc = mc_new;
  // O = alpha O.  When no row of the wave raised its max, every alpha is exactly 1 and
  // the multiply is the identity: skip it (the result is bitwise the same).
  if (!SKIP || __builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0) {
#pragma unroll
    for (int e = 0; e < OB; ++e)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[e][r] *= alpha;
  }
}

// P (fp32, in the S^T register layout) -> binary16 operands of the P V product:
// step u takes S block u/2, registers 8(u%2) .. +7, i.e. keys 16u + 8x + 4h + s in
// slot 4x + s
template <int SB>
__device__ __forceinline__ void pack_p(const f32x16 (&s)[SB], u32x4 (&pf)[2 * SB]) {
#pragma unroll
  for (int u = 0; u < 2 * SB; ++u) {
    const int t = u >> 1, rb = (u & 1) * 8;
    pf[u] = u32x4{pack_f16(s[t][rb + 0], s[t][rb + 1]), pack_f16(s[t][rb + 2], s[t][rb + 3]),
                  pack_f16(s[t][rb + 4], s[t][rb + 5]), pack_f16(s[t][rb + 6], s[t][rb + 7])};
  }
}
// Epilogue: O / lnorm and LSE = (mc + log2 l) ln 2 for the lane's query row.  lnorm is
// the row sum O is normalised by: l itself, or the sum of P as rounded for the P V
// product, which makes the weights applied to V sum to exactly one.
template <int OB>
__device__ __forceinline__ void store_rows(f32x16 (&o)[OB], float mc, float l, float lnorm,
                                           float *orow, float *lse, int h, bool valid) {
  const float lt = pair_sum(l);  // both halves of the row hold partial sums
  const float inv = 1.0f / pair_sum(lnorm);
  if (!valid) return;
#pragma unroll
  for (int e = 0; e < OB; ++e)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      f32x4 v = {o[e][4 * g] * inv, o[e][4 * g + 1] * inv, o[e][4 * g + 2] * inv,
                 o[e][4 * g + 3] * inv};
      *reinterpret_cast<f32x4 *>(orow + 32 * e + 8 * g + 4 * h) = v;
    }
  if (h == 0) *lse = (mc + lg2(lt)) * kLn2;
}

// Epilogue through LDS for a wave's 32 query rows.  Written straight from the matrix-core
// layout, one store instruction covers 32 B of each of 32 rows, and those partial lines
// reach memory separately (up to 2.5x the bytes of O at d = 256).  Here the wave first
// writes O / lnorm to its own LDS region (wave_lds, 32 x D / NHALF floats, no other
// wave touches it), then reads it back row-contiguous so that every store instruction
// writes whole rows of O (whole 128-byte lines).  NHALF > 1 stages the columns in
// parts when the region holds only part of a row.  nvalid = rows of this wave that
// exist (rows >= nvalid are not written).  Within one wave LDS accesses complete in
// order, so no barrier is needed between the write, the read and the next part.
// WITH_LSE = false writes no LSE: the backward pass stores its gradients this way, with
// lnorm choosing the factor.
template <int D, int NHALF, bool WITH_LSE = true>
__device__ __forceinline__ void store_rows_lds(f32x16 (&o)[D / 32], float mc, float l,
                                               float lnorm, char *wave_lds, float *orow0,
                                               float *lse0, int lane, int nvalid) {
  constexpr int OB = D / 32;
  constexpr int EPH = OB / NHALF;        // 32-column blocks per part
  constexpr int CH = EPH * 8;            // 16-byte chunks of a row per part
  constexpr int RPI = 64 / CH;           // rows per read-back instruction
  static_assert(CH % 16 == 0 && 64 % CH == 0, "row parts of 16..64 chunks");
  const int h = lane >> 5, l32 = lane & 31;
  const float lt = pair_sum(l);  // both halves of the row hold partial sums
  const float inv = 1.0f / pair_sum(lnorm);
  if (WITH_LSE && h == 0 && l32 < nvalid) lse0[l32] = (mc + lg2(lt)) * kLn2;
  // chunk c of row r sits at chunk c ^ (r % 16) of the row: the 8 rows a write phase
  // covers land on distinct banks, and a read of whole rows is a permutation
#pragma unroll
  for (int k = 0; k < NHALF; ++k) {
#pragma unroll
    for (int e = k * EPH; e < (k + 1) * EPH; ++e)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int c = 8 * (e - k * EPH) + 2 * g + h;  // columns 32e + 8g + 4h .. +3
        f32x4 v = {o[e][4 * g] * inv, o[e][4 * g + 1] * inv, o[e][4 * g + 2] * inv,
                   o[e][4 * g + 3] * inv};
        *reinterpret_cast<f32x4 *>(wave_lds + (l32 * CH + (c ^ (l32 & 15))) * 16) = v;
      }
#pragma unroll
    for (int i = 0; i < 32 / RPI; ++i) {
      const int r = i * RPI + lane / CH, c = lane % CH;
      const f32x4 v =
          *reinterpret_cast<const f32x4 *>(wave_lds + (r * CH + (c ^ (r & 15))) * 16);
      if (r < nvalid)
        *reinterpret_cast<f32x4 *>(orow0 + int64_t(r) * D + k * (CH * 4) + c * 4) = v;
    }
  }
}

}  // namespace fa
