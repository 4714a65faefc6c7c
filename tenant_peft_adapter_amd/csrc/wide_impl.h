// The k loop of the 128 x 128 direct-load prefill GEMM (h = x W over one
// tile of 128 rows by 128 output columns and one k range), shared by the
// plain kernel (gemm.hip) and the one with the expand in its epilogue
// (fused.hip).
//
// A work-group has 12 waves in three roles.
//   * Waves 8..11 are producers.  Producer p moves rows 64 p .. 64 p + 63 of
//     the tile's 256 (x rows 0..127, then W rows) of each 64-element k slice
//     straight from global memory into a ring of S LDS buffers (8 direct
//     loads of 16 bytes per lane per slice), waits for them to land and
//     meets the others at barriers; they never multiply.  A load that
//     cannot issue because the CU's memory queue is full stalls only them.
//   * Waves 0..3 (group 0) and 4..7 (group 1) multiply.  Wave 4 h + w
//     computes the same 64 x 64 block of the output as wave w, over k half
//     h (elements 32 h .. 32 h + 31) of every slice.
//   * The groups run one phase apart: a phase is either reading one k step's
//     fragments from LDS (8 reads) or the 16 MFMAs on them, and a barrier
//     separates phases, so on each SIMD (one wave of each group) one wave
//     reads while the other multiplies.
// After the loop the groups swap half of their sums through LDS, so that
// each compute wave finishes two of its block's four 16-row blocks: h =
// (sum over the slices' first halves) + (sum over the second halves), in
// that order, whatever the launch.
//
// Ring: slice st sits in buffer st % S.  The producers issue slice it + S - 1
// at the start of group 0's read phase of slice it; the barrier before that
// phase follows every read of slice it - 1 (its buffer).  Before the barrier
// that precedes group 0's reads of slice it + 1 the producers wait until
// that slice has landed (the loads issued after it are those of at most
// S - 2 later slices: s_waitcnt counts them in order).
#pragma once
#include "internal.h"

namespace tpa {
namespace wide_impl {

constexpr int WAVES = 12;
constexpr int THREADS = 64 * WAVES;
constexpr int STAGE = 256 * 128;  // one k slice: 128 x rows and 128 W rows of 128 bytes
constexpr int LI = 8;             // direct loads per producer per slice

struct Role {
  int wave, lane, i16, g;
  bool prod;
  int pw;                // producer index (producers)
  int grp, wr, wc;       // group and 64 x 64 block (compute waves)
};

__device__ __forceinline__ Role role() {
  Role r;
  r.lane = (int)threadIdx.x & 63;
  r.wave = (int)threadIdx.x >> 6;
  r.i16 = r.lane & 15;
  r.g = r.lane >> 4;
  r.prod = r.wave >= 8;
  r.pw = r.wave - 8;
  r.grp = r.prod ? 0 : r.wave >> 2;
  r.wr = r.wave & 1;
  r.wc = (r.wave >> 1) & 1;
  return r;
}

// Tile row (0..255: x rows, then W rows) that a producer lane loads with
// instruction j, and the element offset of its 16-byte chunk within the
// slice (chunks of a row are stored permuted, c ^ swz(row), so that the
// fragment reads hit distinct bank groups).
__device__ __forceinline__ int producer_row(const Role& r, int j) { return 64 * r.pw + 8 * j + (r.lane >> 3); }
__device__ __forceinline__ int producer_chunk_elems(const Role& r, int row) {
  const int lc = r.lane & 7;
  return 8 * (row < 128 ? (lc ^ swz<2>(row)) : (lc ^ swz<4>(row - 128)));
}

__device__ __forceinline__ void phase_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

// Runs the k loop over nst slices.  src: a producer's 8 row pointers at the
// start of the k range, chunk offset included (unused by the others).  acc:
// a compute wave's 16 accumulators, added to.  Every wave of the work-group
// must call it with the same nst.  On return every load has landed and
// every read of the ring is done.
template <typename T, int S>
__device__ __forceinline__ void k_loop(const Role& ro, const T* const (&src)[LI], int nst, unsigned char* smem,
                                       f32x4 (&acc)[4][4]) {
  typedef typename Frag<T>::V Vt;
  auto issue = [&](int st) {
    if (!ro.prod || st >= nst) return;
    unsigned char* buf = smem + (size_t)(st % S) * STAGE;
#pragma unroll
    for (int j = 0; j < LI; ++j)
      __builtin_amdgcn_global_load_lds((const void*)(src[j] + 64 * st),
                                       (__attribute__((address_space(3))) void*)(buf + (size_t)(64 * ro.pw + 8 * j) * 128),
                                       16, 0, 0);
  };
  auto landed = [&](int st) {
    if (!ro.prod) return;
    const int younger = min(S - 2, nst - 1 - st);
    if (younger >= 3)
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(3 * LI));
    else if (younger == 2)
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * LI));
    else if (younger == 1)
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(LI));
    else
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  };
  int arow[4], brow[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) arow[b] = 64 * ro.wc + perm_col<4>(ro.i16, b);  // W rows (output columns)
#pragma unroll
  // x rows; group 1 takes its row blocks in the order 2, 3, 0, 1, so that
  // each group's first two accumulator blocks are the ones it finishes.
  for (int m = 0; m < 4; ++m) brow[m] = 64 * ro.wr + 16 * ((m + 2 * ro.grp) & 3) + ro.i16;
  const int q = 4 * ro.grp + ro.g;
  Vt af[4], bf[4];
  auto R = [&](int st) {
    const unsigned char* buf = smem + (size_t)(st % S) * STAGE;
#pragma unroll
    for (int b = 0; b < 4; ++b)
      af[b] = *reinterpret_cast<const Vt*>(buf + 128 * 128 + arow[b] * 128 + 16 * (q ^ swz<4>(arow[b])));
#pragma unroll
    for (int m = 0; m < 4; ++m) bf[m] = *reinterpret_cast<const Vt*>(buf + brow[m] * 128 + 16 * (q ^ swz<2>(brow[m])));
    __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  };
  auto M = [&]() {
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int m = 0; m < 4; ++m) acc[b][m] = mma(acc[b][m], af[b], bf[m]);
  };

#pragma unroll
  for (int st = 0; st < S - 1; ++st) issue(st);
  if (nst > 0) landed(0);
  phase_barrier();
  // Every wave runs the same body; group 1 enters it one barrier later (and
  // group 0 and the producers leave through one more), which puts the groups
  // one phase apart.  Producers issue and wait, compute waves read and
  // multiply.
  if (ro.grp == 1) phase_barrier();
  for (int it = 0; it < nst; ++it) {
    issue(it + S - 1);
    if (!ro.prod) R(it);
    phase_barrier();
    if (!ro.prod) M();
    if (it + 1 < nst) landed(it + 1);
    phase_barrier();
  }
  if (ro.grp == 0) phase_barrier();  // the same number of barriers for every wave
}

// The two groups' sums combined through the ring's LDS, which k_loop
// leaves free.  A compute wave finishes row blocks 2 grp and 2 grp + 1 of
// its 64 x 64 block, which are its accumulator blocks acc[.][0] and
// acc[.][1] (k_loop's row order); it sends acc[.][2] and acc[.][3] (the
// other group's two blocks) and adds the other group's sums for its own:
// h = group 0's sum + group 1's (IEEE addition commutes, so both groups form
// the same value).  Every wave of the work-group calls it.
__device__ __forceinline__ void exchange(const Role& ro, unsigned char* smem, f32x4 (&acc)[4][4]) {
  f32x4* red = reinterpret_cast<f32x4*>(smem);
  const int blk = ro.wave & 3;
  if (!ro.prod) {
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int mm = 0; mm < 2; ++mm) red[((size_t)(ro.grp * 4 + blk) * 8 + b * 2 + mm) * 64 + ro.lane] = acc[b][2 + mm];
  }
  __syncthreads();
  if (!ro.prod) {
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int mm = 0; mm < 2; ++mm)
        acc[b][mm] = acc[b][mm] + red[((size_t)((1 - ro.grp) * 4 + blk) * 8 + b * 2 + mm) * 64 + ro.lane];
  }
}

}  // namespace wide_impl
}  // namespace tpa
