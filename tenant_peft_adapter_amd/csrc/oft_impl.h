// Device code of OFT's input transform in a pass of its own (Scute paper, arXiv
// 2611.01089, §4.1 route three, and the appendix "Propositions A2-A4"): each
// OFT row is multiplied by its tenant's block-diagonal R before the shared
// GEMM, which then sees the rotated row.  The pass reads and writes
// [rows, d_in] once plus each tenant's d_in / b blocks of b x b.
//
// Work-group = one OFT tile of the plan (rows of one tenant, so each R
// block is read once per tile) x a.bpw consecutive blocks shared out among
// its waves (a wave's blocks run one after another, each a round trip of
// loads).  A
// block is an MFMA product with K = b: D = Rᵀ · x_blockᵀ, so each lane ends
// with 4·(b/16) consecutive columns of one row.  R blocks are stored
// transposed ([c][t] = R[t][c]).  The rotated row p (plan order) is written
// to x_rot[p].
#pragma once

#include "internal.h"

namespace tpa {
namespace oft_impl {

// Work-group part `bg` (a.bpw consecutive blocks, a.bpw / NW per wave for
// a work-group of NW waves; a.bpw a multiple of NW) of OFT tile t.
template <typename T, int MB, int BS, int NW>
__device__ __forceinline__ void oft_part(const OftArgs& a, int t, int bg, int wave, int lane) {
  constexpr int NB = BS / 16;
  const int bpw = a.bpw;
  const int i16 = lane & 15, g = lane >> 4;
  // Header and row words load side by side.
  const int4 tile = *reinterpret_cast<const int4*>(a.oft_tiles + 4 * t);
  int rw[MB];
#pragma unroll
  for (int m = 0; m < MB; ++m) rw[m] = a.oft_rows_w[(size_t)t * 16 * MB + 16 * m + i16];
  if (tile.z < 0) return;
  const int p0 = tile.x;
  const SlotDev& sd = a.slots[tile.z];
  if (sd.oft_block != BS) return;
  const T* Rt = static_cast<const T*>(sd.Rt);
  const T* X = static_cast<const T*>(a.x);
  T* XR = static_cast<T*>(a.x_rot);
  const int nblocks = a.d_in / BS;

  const T* xp[MB];
  bool xv[MB];
#pragma unroll
  for (int m = 0; m < MB; ++m) {
    xv[m] = rw[m] >= 0;
    xp[m] = X + (size_t)(xv[m] ? (rw[m] & 0xFFFF) : 0) * a.d_in + 8 * g;
  }

  for (int j = 0; j < bpw / NW; ++j) {
    const int kb = bg * bpw + NW * j + wave;
    if (kb >= nblocks) break;
    f32x4 acc[NB][MB];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int m = 0; m < MB; ++m) acc[b][m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k0 = 0; k0 < BS; k0 += 32) {
      const bool kok = k0 + 8 * g < BS;
      typename Frag<T>::V af[NB], bf[MB];
#pragma unroll
      for (int b = 0; b < NB; ++b)
        af[b] = kok ? load_frag<T>(Rt + ((size_t)kb * BS + perm_col<NB>(i16, b)) * BS + k0 + 8 * g)
                    : zero_frag<T>();
#pragma unroll
      for (int m = 0; m < MB; ++m)
        bf[m] = (kok && xv[m]) ? load_frag<T>(xp[m] + kb * BS + k0) : zero_frag<T>();
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int m = 0; m < MB; ++m) acc[b][m] = mma(acc[b][m], af[b], bf[m]);
    }
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      if (!xv[m]) continue;
      T* dst = XR + (size_t)(p0 + 16 * m + i16) * a.d_in + kb * BS + 4 * NB * g;
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int q = 0; q < 4; ++q) dst[4 * b + q] = to_t<T>(acc[b][m][q]);
    }
  }
}

}  // namespace oft_impl
}  // namespace tpa
