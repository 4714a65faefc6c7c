// Device code of the shrink (included by the kernels that run it).
//
// Scute paper (arXiv 2611.01089), §2 "The LoRA schedule": the shrink computes
// V = x A per segment of rows of one adapter; §4.1 route two, first GEMM:
// for rows whose adapter's term sits on the shared factors (VeRA), U = (x A)
// ⊙ d over tiles of rows whatever their adapter, so the shared A is read once
// per tile rather than once per tenant.
#pragma once

#include "internal.h"

namespace tpa {
namespace shrink_impl {

// One wave per work item (plan tile, 16·NCB factor columns, k range):
// factor rows and the tile's x rows stream straight into MFMA registers
// (up to 8 k steps of loads issued together), no LDS and no barriers, so
// the whole GPU takes part even when one tile (VeRA's shared factor) holds
// most of the work.  Each item writes its fp32 partial [split][n][kmax] by
// plan position; the reduce pass below adds the splits in split order.
// With NCB = 4 an item reads its x rows once for 64 factor columns instead
// of once per 16 (blocks past the factor's rank load nothing); each block's
// products are the same MFMA steps in the same k order, so the partials
// are the same bits.

template <typename T, int MB, int NCB = 1>
__device__ __forceinline__ void shrink_item(const ShrinkArgs& a, int item, int lane) {
  typedef typename Frag<T>::V Vt;
  // k steps whose loads are issued together (fp32 fragments are twice as
  // wide, and wide items load four factor fragments a step, so fewer fit)
  constexpr int U = sizeof(T) == 4 ? (MB == 1 ? 4 : 2) : (MB == 1 ? (NCB == 1 ? 8 : 4) : 4);
  const int ks = item % a.split;
  int rest = item / a.split;
  const int own_items = a.own_tiles * a.own_nblk;
  const int* tile;
  const int* trow;  // the tile's row words
  int cb, want;
  const int i16 = lane & 15, g = lane >> 4;
  if (rest < own_items) {
    cb = rest % a.own_nblk;
    const int t = rest / a.own_nblk;
    tile = a.tiles + 4 * t;
    trow = a.tile_rows_w + (size_t)t * 16 * MB;
    want = CLS_OWNED;
  } else {
    rest -= own_items;
    const int t = rest / a.sh_nblk;
    if (t >= a.sh_ntiles) return;
    cb = rest % a.sh_nblk;
    tile = a.sh_tiles + 4 * t;
    trow = a.sh_rows_w + (size_t)t * 16 * MB;
    want = CLS_SHARED;
  }
  // Header and row words load side by side (row words of a padding entry
  // are never used).
  const int4 tl = *reinterpret_cast<const int4*>(tile);
  int rw[MB];
#pragma unroll
  for (int m = 0; m < MB; ++m) rw[m] = trow[16 * m + i16];
  const int kind = tl.z;
  if (kind != want) return;  // past the real tiles of that kind
  const int p0 = tl.x;
  const T* F;
  int N;
  if (kind == CLS_OWNED) {
    const SlotDev& sd = a.slots[tl.w];
    F = static_cast<const T*>(sd.A);
    N = sd.rank;
  } else {
    F = static_cast<const T*>(a.vera_At);
    N = a.r_v;
  }
  const int c0 = 16 * NCB * cb;
  if (c0 >= N) return;
  const int kbeg = ks * a.kc;
  const int kend = min(a.d_in, kbeg + a.kc);
  const T* X = static_cast<const T*>(a.x);

  const T* xp[MB];
  bool xv[MB];
#pragma unroll
  for (int m = 0; m < MB; ++m) {
    xv[m] = rw[m] >= 0;
    xp[m] = X + (size_t)(xv[m] ? (rw[m] & 0xFFFF) : 0) * a.d_in + 8 * g;
  }
  // Column blocks of this item within the factor's rank (a multiple of 16).
  const T* fp[NCB];
  bool fv[NCB];
#pragma unroll
  for (int j = 0; j < NCB; ++j) {
    fv[j] = c0 + 16 * j < N;
    fp[j] = F + (size_t)(fv[j] ? c0 + 16 * j + i16 : 0) * a.d_in + 8 * g;
  }

  f32x4 acc[NCB][MB];
#pragma unroll
  for (int j = 0; j < NCB; ++j)
#pragma unroll
    for (int m = 0; m < MB; ++m) acc[j][m] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int k = kbeg; k < kend; k += 32 * U) {
    Vt ff[U][NCB], xf[U][MB];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kk = k + 32 * u;
      const bool ok = kk < kend;
#pragma unroll
      for (int j = 0; j < NCB; ++j) ff[u][j] = (ok && fv[j]) ? load_frag<T>(fp[j] + kk) : zero_frag<T>();
#pragma unroll
      for (int m = 0; m < MB; ++m) xf[u][m] = (ok && xv[m]) ? load_frag<T>(xp[m] + kk) : zero_frag<T>();
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (k + 32 * u >= kend) break;
#pragma unroll
      for (int j = 0; j < NCB; ++j) {
        if (!fv[j]) continue;
#pragma unroll
        for (int m = 0; m < MB; ++m) acc[j][m] = mma(acc[j][m], ff[u][j], xf[u][m]);
      }
    }
  }
  // Lane holds V[p0 + 16m + i16][c0 + 16j + 4g + v], v = 0..3.
#pragma unroll
  for (int j = 0; j < NCB; ++j) {
    if (!fv[j]) continue;
    const int col = c0 + 16 * j + 4 * g;
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      const int p = p0 + 16 * m + i16;
      if (xv[m]) *reinterpret_cast<f32x4*>(a.part + ((size_t)ks * a.n + p) * a.kmax + col) = acc[j][m];
    }
  }
}

// Reduce pass: V[p][c] = Σ_s part[s][p][c] in split order (times d'[c] for
// a shared-term row), stored in the layer type; one thread per 4 columns of
// one plan position, only for columns below the row's rank.  A shared-term
// row's partials may come from another projection of the group
// (part_shared): x·A_vᵀ is the same for every projection that reads the
// same input with the same A_v, only d' differs.
template <typename T>
__device__ __forceinline__ void shrink_reduce_item(const ShrinkArgs& a, int idx) {
  const int q4 = a.kmax / 4;
  if (idx >= a.n * q4) return;
  const int p = idx / q4;
  const int col = 4 * (idx % q4);
  const SlotDev& sd = a.slots[a.pinfo[p] >> 16];
  const int cls = sd.cls;
  if (cls != CLS_OWNED && cls != CLS_SHARED) return;
  const int N = cls == CLS_OWNED ? sd.rank : a.r_v;
  if (col >= N) return;
  // Splits added in order; their loads go out 8 at a time.
  const bool borrowed = cls == CLS_SHARED && a.part_shared;
  const int ld = borrowed ? a.kmax_shared : a.kmax;
  const float* src = (borrowed ? a.part_shared : a.part) + (size_t)p * ld + col;
  const size_t stride = (size_t)a.n * ld;
  f32x4 v = f32x4{0.f, 0.f, 0.f, 0.f};
  int s = 0;
  for (; s + 8 <= a.split; s += 8) {
    f32x4 t[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) t[u] = gload<f32x4>(src + (size_t)(s + u) * stride);
#pragma unroll
    for (int u = 0; u < 8; ++u) v += t[u];
  }
  for (; s < a.split; ++s) v += gload<f32x4>(src + (size_t)s * stride);
  if (cls == CLS_SHARED) v = v * gload<f32x4>(sd.d + col);
  T* dst = static_cast<T*>(a.v) + (size_t)p * a.kmax + col;
#pragma unroll
  for (int q = 0; q < 4; ++q) dst[q] = to_t<T>(v[q]);
}

// Whole-k shrink: one work-group of Q waves per work item of slice si
// (plan tile, 16 factor columns).  Wave w runs the w-th k range of kc with
// the split items' loop (waves past the split add nothing), leaves its fp32
// sum in LDS, and wave 0 adds the Q sums in wave order: the same additions
// as the reduce pass over the splits.  Shared-term rows are then scaled by
// d' and written for this slice and, from the first slice, for every slice
// that borrows its x·A_vᵀ (each with its own d').  Every early return
// depends only on the item, so the work-group takes it together and the
// barrier is met by all of its waves.
// The item reaches the launch's slices through sh_of(j) (the ShrinkArgs of
// slice j, j < count): the launch before the GEMM and the decode GEMM's
// side work-groups both run it.
template <typename T, int Q, typename ShOf>
__device__ __forceinline__ void shrink_whole_item(ShOf sh_of, int count, int si, int item, int wave, int lane,
                                                  f32x4* red) {
  typedef typename Frag<T>::V Vt;
  constexpr int U = 8;
  const ShrinkArgs& a = sh_of(si);
  const int own_items = a.own_tiles * a.own_nblk;
  const int i16 = lane & 15, g = lane >> 4;
  const int* tile;
  const int* trow;
  int cb, want;
  int rest = item;
  if (rest < own_items) {
    cb = rest % a.own_nblk;
    const int tt = rest / a.own_nblk;
    tile = a.tiles + 4 * tt;
    trow = a.tile_rows_w + (size_t)tt * 16;
    want = CLS_OWNED;
  } else {
    rest -= own_items;
    const int tt = rest / a.sh_nblk;
    if (tt >= a.sh_ntiles) return;
    cb = rest % a.sh_nblk;
    tile = a.sh_tiles + 4 * tt;
    trow = a.sh_rows_w + (size_t)tt * 16;
    want = CLS_SHARED;
  }
  const int4 tl = *reinterpret_cast<const int4*>(tile);
  const int rw = trow[i16];
  if (tl.z != want) return;
  const T* F;
  int N;
  if (want == CLS_OWNED) {
    const SlotDev& sd = a.slots[tl.w];
    F = static_cast<const T*>(sd.A);
    N = sd.rank;
  } else {
    F = static_cast<const T*>(a.vera_At);
    N = a.r_v;
  }
  const int c0 = 16 * cb;
  if (c0 >= N) return;
  const int kbeg = wave * a.kc;
  const int kend = wave < a.split ? min(a.d_in, kbeg + a.kc) : kbeg;
  const bool xv = rw >= 0;
  const T* xp = static_cast<const T*>(a.x) + (size_t)(xv ? (rw & 0xFFFF) : 0) * a.d_in + 8 * g;
  const T* fp = F + (size_t)(c0 + i16) * a.d_in + 8 * g;
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int k = kbeg; k < kend; k += 32 * U) {
    Vt ff[U], xf[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kk = k + 32 * u;
      const bool ok = kk < kend;
      ff[u] = ok ? load_frag<T>(fp + kk) : zero_frag<T>();
      xf[u] = (ok && xv) ? load_frag<T>(xp + kk) : zero_frag<T>();
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (k + 32 * u >= kend) break;
      acc = mma(acc, ff[u], xf[u]);
    }
  }
  red[wave * 64 + lane] = acc;
  lds_barrier();
  if (wave != 0 || !xv) return;
  // Lane holds columns c0 + 4g .. + 3 of plan position p0 + i16.
  f32x4 v = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int w = 0; w < Q; ++w) v += red[w * 64 + lane];
  const int col = c0 + 4 * g;
  if (col >= N) return;
  const int p = tl.x + i16;
  const int slot = (int)((unsigned)rw >> 16);
  for (int j = 0; j < count; ++j) {
    const ShrinkArgs& b = sh_of(j);
    const bool mine = j == si;
    if (!mine && !(want == CLS_SHARED && si == 0 && b.borrows)) continue;
    f32x4 o = v;
    if (want == CLS_SHARED) o = v * gload<f32x4>(b.slots[slot].d + col);
    T* dst = static_cast<T*>(b.v) + (size_t)p * b.kmax + col;
#pragma unroll
    for (int q = 0; q < 4; ++q) dst[q] = to_t<T>(o[q]);
  }
}

template <typename T, int Q>
__device__ __forceinline__ void shrink_whole(const Slices<PreSlice>& t, int si, int item, int wave, int lane,
                                             f32x4* red) {
  shrink_whole_item<T, Q>([&](int j) -> const ShrinkArgs& { return t.s[j].sh; }, t.count, si, item, wave, lane, red);
}

}  // namespace shrink_impl
}  // namespace tpa
