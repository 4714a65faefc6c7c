// The launch that precedes the base GEMM: the shrink (V = x A' for owned-
// term tiles, U = (x A_v) ⊙ d' for shared-term tiles) and OFT's rotation of
// its rows (x_rot = x R) in one grid.  Both only read x and the row plan,
// and neither needs the other, so one launch runs them side by side.
//
// Scute paper (arXiv 2611.01089): §2 "The LoRA schedule" (shrink per
// segment), §4.1 route two (shared-factor term over row tiles) and route
// three (input transform in a pass of its own before the shared GEMM).
//
// Grid: first the shrink's work-groups (4 independent waves each, one item
// per wave; or, in whole-k mode, one item per work-group of 16 waves that
// also adds the k ranges' sums), then OFT's (one OFT tile x 16 blocks per
// work-group).
#include "oft_impl.h"
#include "shrink_impl.h"

namespace tpa {

namespace {

constexpr int THREADS = 256;

template <typename T, int MB, int BS, int NCB>
__global__ __launch_bounds__(THREADS) void pre_kernel(Slices<PreSlice> t) {
  const int si = slice_of(t, (int)blockIdx.x);
  const PreSlice& ps = t.s[si];
  const int local = (int)blockIdx.x - t.first[si];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (local < ps.n_shrink_wg) {
    shrink_impl::shrink_item<T, MB, NCB>(ps.sh, local * (THREADS / 64) + wave, lane);
    return;
  }
  if (BS != 0) {
    const int o = local - ps.n_shrink_wg;
    oft_impl::oft_part<T, MB, (BS == 0 ? 16 : BS), THREADS / 64>(ps.of, o / ps.oft_bg, o % ps.oft_bg, wave, lane);
  }
}

// Whole-k mode (16-row tiles): one work-group of PRE_WHOLE_WAVES waves per
// shrink item, then OFT's work-groups (one block per wave).  The launch's
// first work-group also clears the arrival counters of the fused GEMM that
// follows it on the stream.
template <typename T, int BS>
__global__ __launch_bounds__(64 * PRE_WHOLE_WAVES) void pre_whole_kernel(Slices<PreSlice> t) {
  __shared__ f32x4 red[PRE_WHOLE_WAVES * 64];
  if (blockIdx.x == 0) {
    for (int j = 0; j < t.count; ++j) {
      int32_t* z = t.s[j].zero;
      if (!z) continue;
      for (int i = (int)threadIdx.x; i < t.s[j].zero_n; i += 64 * PRE_WHOLE_WAVES) z[i] = 0;
    }
  }
  const int si = slice_of(t, (int)blockIdx.x);
  const PreSlice& ps = t.s[si];
  const int local = (int)blockIdx.x - t.first[si];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (local < ps.n_shrink_wg) {
    shrink_impl::shrink_whole<T, PRE_WHOLE_WAVES>(t, si, local, wave, lane, red);
    return;
  }
  if (BS != 0) {
    const int o = local - ps.n_shrink_wg;
    oft_impl::oft_part<T, 1, (BS == 0 ? 16 : BS), PRE_WHOLE_WAVES>(ps.of, o / ps.oft_bg, o % ps.oft_bg, wave, lane);
  }
}

template <typename T>
hipError_t pre_whole_bs(int bs, const Slices<PreSlice>& t, hipStream_t s) {
  const dim3 grid((unsigned)t.first[t.count]);
  if (grid.x == 0) return hipSuccess;
  const dim3 block(64 * PRE_WHOLE_WAVES);
  switch (bs) {
    case 0: hipLaunchKernelGGL((pre_whole_kernel<T, 0>), grid, block, 0, s, t); break;
    case 16: hipLaunchKernelGGL((pre_whole_kernel<T, 16>), grid, block, 0, s, t); break;
    case 32: hipLaunchKernelGGL((pre_whole_kernel<T, 32>), grid, block, 0, s, t); break;
    case 64: hipLaunchKernelGGL((pre_whole_kernel<T, 64>), grid, block, 0, s, t); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T, int MB, int NCB>
hipError_t pre_bs(int bs, const Slices<PreSlice>& t, hipStream_t s) {
  const dim3 grid((unsigned)t.first[t.count]);
  if (grid.x == 0) return hipSuccess;
  switch (bs) {
    case 0: hipLaunchKernelGGL((pre_kernel<T, MB, 0, NCB>), grid, dim3(THREADS), 0, s, t); break;
    case 16: hipLaunchKernelGGL((pre_kernel<T, MB, 16, NCB>), grid, dim3(THREADS), 0, s, t); break;
    case 32: hipLaunchKernelGGL((pre_kernel<T, MB, 32, NCB>), grid, dim3(THREADS), 0, s, t); break;
    case 64: hipLaunchKernelGGL((pre_kernel<T, MB, 64, NCB>), grid, dim3(THREADS), 0, s, t); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T>
hipError_t pre_tm(int tile_rows, int bs, int ncb, const Slices<PreSlice>& t, hipStream_t s) {
  if (ncb == 4) {
    if constexpr (sizeof(T) == 2) {
      if (tile_rows == 16) return pre_bs<T, 1, 4>(bs, t, s);
    }
    return hipErrorInvalidValue;
  }
  if (ncb != 1) return hipErrorInvalidValue;
  if (tile_rows == 16) return pre_bs<T, 1, 1>(bs, t, s);
  if (tile_rows == 64) return pre_bs<T, 4, 1>(bs, t, s);
  return hipErrorInvalidValue;
}

template <typename T>
__global__ __launch_bounds__(THREADS) void shrink_reduce_kernel(ShrinkArgs a) {
  shrink_impl::shrink_reduce_item<T>(a, (int)(blockIdx.x * THREADS + threadIdx.x));
}

}  // namespace

PreSlice make_pre_slice(const ShrinkArgs* sh, const OftArgs* of, bool whole) {
  PreSlice ps{};
  ps.oft_bg = 1;
  if (sh) {
    ps.sh = *sh;
    const long tiles_x_blocks = (long)sh->own_tiles * sh->own_nblk + (long)sh->sh_ntiles * sh->sh_nblk;
    if (whole) {
      ps.n_shrink_wg = (int)tiles_x_blocks;
    } else {
      const long items = tiles_x_blocks * sh->split;
      ps.n_shrink_wg = (int)((items + THREADS / 64 - 1) / (THREADS / 64));
    }
  }
  if (of) {
    ps.of = *of;
    // Blocks per work-group: a multiple of its waves (4 in the split launch,
    // PRE_WHOLE_WAVES, one per wave, in the whole-k one).
    if (whole || ps.of.bpw < THREADS / 64 || ps.of.bpw % (THREADS / 64)) ps.of.bpw = whole ? PRE_WHOLE_WAVES : 16;
    ps.oft_bg = (of->d_in / of->block + ps.of.bpw - 1) / ps.of.bpw;
    ps.n_oft_wg = of->max_tiles * ps.oft_bg;
  }
  return ps;
}

hipError_t launch_pre(int dtype, int tile_rows, int bs, const PreSlice* slices, int count, hipStream_t s,
                      bool whole, int ncb) {
  if (count < 1 || count > MAX_SLICES) return hipErrorInvalidValue;
  if (whole && ncb != 1) return hipErrorInvalidValue;
  if (whole) {
    if (tile_rows != 16 || (dtype != 1 && dtype != 2)) return hipErrorInvalidValue;
    for (int i = 0; i < count; ++i)
      if (slices[i].n_shrink_wg > 0 &&
          (slices[i].sh.split > PRE_WHOLE_WAVES || (long)slices[i].sh.split * slices[i].sh.kc < slices[i].sh.d_in))
        return hipErrorInvalidValue;
  }
  Slices<PreSlice> t{};
  t.count = count;
  t.first[0] = 0;
  for (int i = 0; i < count; ++i) {
    t.s[i] = slices[i];
    t.first[i + 1] = t.first[i] + slices[i].n_shrink_wg + slices[i].n_oft_wg;
  }
  for (int i = count; i < MAX_SLICES; ++i) t.first[i + 1] = t.first[count];
  if (whole) return dtype == 1 ? pre_whole_bs<f16>(bs, t, s) : pre_whole_bs<bf16>(bs, t, s);
  switch (dtype) {
    case 0: return pre_tm<float>(tile_rows, bs, ncb, t, s);
    case 1: return pre_tm<f16>(tile_rows, bs, ncb, t, s);
    case 2: return pre_tm<bf16>(tile_rows, bs, ncb, t, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_shrink_reduce(int dtype, const ShrinkArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)(((long)a.n * (a.kmax / 4) + THREADS - 1) / THREADS));
  switch (dtype) {
    case 0: hipLaunchKernelGGL(shrink_reduce_kernel<float>, grid, dim3(THREADS), 0, s, a); break;
    case 1: hipLaunchKernelGGL(shrink_reduce_kernel<f16>, grid, dim3(THREADS), 0, s, a); break;
    case 2: hipLaunchKernelGGL(shrink_reduce_kernel<bf16>, grid, dim3(THREADS), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace tpa
