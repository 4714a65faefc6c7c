// The dense contractions of the layer on gfx950 MFMA:
//   * the shared base GEMM h = (xR) W over the whole batch (Scute paper,
//     arXiv 2611.01089, §2 "The LoRA schedule": one GEMM for every tenant;
//     §3.2: OFT rows enter it already rotated, so it stays one GEMM), and
//   * the shrink: V = x A' per owned-term tile (§2, Punica's segmented
//     shrink) and, for VeRA rows, U = (x A_v) ⊙ d' over tiles of rows
//     whatever their tenant (§4.1, route two, first GEMM).
//
// Two kernels:
//   gemm_skinny  -- n <= 64 rows (decode).  The layer is bound by reading W
//     once from HBM.  Each work-group owns 16·NB output columns and one k
//     range (split-K); its 4 waves take interleaved 32-wide k steps, so the
//     group reads whole 128-element runs of each weight row, and operands go
//     straight from memory into MFMA registers.  The 4 wave partials are
//     summed in LDS in a fixed order and written as fp32 split partials;
//     the expand sums the splits in a fixed order, so results do not depend
//     on scheduling.
//   gemm_tiled   -- larger n (prefill).  128x128 output tiles, 128-byte k
//     slices staged through double-buffered LDS, 2x2 waves of 64x64.
// The shrink uses the skinny structure over the plan's tiles.
#include "internal.h"

namespace tpa {

namespace {

constexpr int THREADS = 256;

// Sum the four waves' accumulators of a skinny work-group into wave 0, in
// the fixed order (w0 + w2) + (w1 + w3).  red holds 2 x (NB*MB*4) x 64.
template <int NB, int MB>
__device__ __forceinline__ void reduce_waves(f32x4 (&acc)[NB][MB], float* red, int wave, int lane) {
  constexpr int E = NB * MB * 4;
  auto at = [&](int half, int b, int m, int q) -> float& {
    return red[(half * E + (b * MB + m) * 4 + q) * 64 + lane];
  };
  if (wave >= 2) {
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int m = 0; m < MB; ++m)
#pragma unroll
        for (int q = 0; q < 4; ++q) at(wave - 2, b, m, q) = acc[b][m][q];
  }
  __syncthreads();
  if (wave < 2) {
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int m = 0; m < MB; ++m)
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[b][m][q] += at(wave, b, m, q);
  }
  __syncthreads();
  if (wave == 1) {
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int m = 0; m < MB; ++m)
#pragma unroll
        for (int q = 0; q < 4; ++q) at(0, b, m, q) = acc[b][m][q];
  }
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int m = 0; m < MB; ++m)
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[b][m][q] += at(0, b, m, q);
  }
}

// Main loop shared by the skinny GEMM and the shrink: acc[b][m] +=
// W-rows(b) · X-rows(m) over k in [kbeg, kend), waves interleaved by 32.
template <typename T, int MB, int NB>
__device__ __forceinline__ void skinny_loop(f32x4 (&acc)[NB][MB], const T* const* wp, const bool* wv,
                                            const T* const* xp, const bool* xv, int kbeg, int kend,
                                            int wave) {
  typedef typename Frag<T>::V V;
  constexpr int U = 4;
  for (int k = kbeg + 32 * wave; k < kend; k += 128 * U) {
    V wf[U][NB], xf[U][MB];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kk = k + 128 * u;
      const bool ok = kk < kend;
#pragma unroll
      for (int b = 0; b < NB; ++b) wf[u][b] = (ok && wv[b]) ? load_frag<T>(wp[b] + kk) : zero_frag<T>();
#pragma unroll
      for (int m = 0; m < MB; ++m) xf[u][m] = (ok && xv[m]) ? load_frag<T>(xp[m] + kk) : zero_frag<T>();
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int m = 0; m < MB; ++m) acc[b][m] = mma(acc[b][m], wf[u][b], xf[u][m]);
  }
}

template <typename T, int MB, int NB>
__global__ __launch_bounds__(THREADS) void gemm_skinny_kernel(BaseGemmArgs a) {
  __shared__ float red[2 * NB * MB * 4 * 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i16 = lane & 15, g = lane >> 4;
  const int col0 = blockIdx.x * (16 * NB);
  const int ks = blockIdx.y;
  const int kbeg = ks * a.kc;
  const int kend = min(a.d_in, kbeg + a.kc);
  const T* X = static_cast<const T*>(a.x);
  const T* XR = static_cast<const T*>(a.x_rot);
  const T* W = static_cast<const T*>(a.W);

  const T* xp[MB];
  bool xv[MB];
#pragma unroll
  for (int m = 0; m < MB; ++m) {
    const int r = 16 * m + i16;
    xv[m] = r < a.n;
    const int rp = (xv[m] && a.rot_pos) ? a.rot_pos[r] : -1;
    const T* base = rp >= 0 ? XR + (size_t)rp * a.d_in : X + (size_t)(xv[m] ? r : 0) * a.d_in;
    xp[m] = base + 8 * g;
  }
  const T* wp[NB];
  bool wv[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int c = col0 + perm_col<NB>(i16, b);
    wv[b] = true;
    wp[b] = W + (size_t)c * a.d_in + 8 * g;
  }
  f32x4 acc[NB][MB];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int m = 0; m < MB; ++m) acc[b][m] = f32x4{0.f, 0.f, 0.f, 0.f};

  skinny_loop<T, MB, NB>(acc, wp, wv, xp, xv, kbeg, kend, wave);
  reduce_waves<NB, MB>(acc, red, wave, lane);
  if (wave != 0) return;
#pragma unroll
  for (int m = 0; m < MB; ++m) {
    const int row = 16 * m + i16;
    if (row >= a.n) continue;
    float* dst = a.part + ((size_t)ks * a.n + row) * a.d_out + col0 + 4 * NB * g;
#pragma unroll
    for (int b = 0; b < NB; ++b) *reinterpret_cast<f32x4*>(dst + 4 * b) = acc[b][m];
  }
}

// --------------------------------------------------------------- tiled ----

template <typename T>
__device__ __forceinline__ typename Frag<T>::V lds_frag(const T* p) {
  return *reinterpret_cast<const typename Frag<T>::V*>(p);
}
template <>
__device__ __forceinline__ f32x8 lds_frag<float>(const float* p) {
  f32x4 lo = *reinterpret_cast<const f32x4*>(p);
  f32x4 hi = *reinterpret_cast<const f32x4*>(p + 4);
  return f32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

template <typename T>
__device__ __forceinline__ void store_run16(T* dst, const float* v);
template <>
__device__ __forceinline__ void store_run16<float>(float* dst, const float* v) {
#pragma unroll
  for (int q = 0; q < 4; ++q)
    *reinterpret_cast<f32x4*>(dst + 4 * q) = f32x4{v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]};
}
template <typename T>
__device__ __forceinline__ void store_run16(T* dst, const float* v) {
  typename Frag<T>::V lo, hi;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    lo[j] = to_t<T>(v[j]);
    hi[j] = to_t<T>(v[8 + j]);
  }
  *reinterpret_cast<typename Frag<T>::V*>(dst) = lo;
  *reinterpret_cast<typename Frag<T>::V*>(dst + 8) = hi;
}

template <typename T>
__global__ __launch_bounds__(THREADS) void gemm_tiled_kernel(BaseGemmArgs a) {
  constexpr int BM = 128, BN = 128;
  constexpr int EPC = 16 / sizeof(T);        // elements per 16-byte chunk
  constexpr int BK = 128 / sizeof(T);        // 128-byte k slice
  constexpr int LDK = BK + EPC;              // padded row, in elements
  __shared__ __attribute__((aligned(16))) T lds[2][(BM + BN) * LDK];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int i16 = lane & 15, g = lane >> 4;
  const int wr = wave & 1, wc = wave >> 1;
  const int row0 = blockIdx.y * BM, col0 = blockIdx.x * BN;
  const int ks = blockIdx.z;
  const int kbeg = ks * a.kc;
  const int kend = min(a.d_in, kbeg + a.kc);
  const int nk = (kend - kbeg) / BK;
  const T* X = static_cast<const T*>(a.x);
  const T* XR = static_cast<const T*>(a.x_rot);
  const T* W = static_cast<const T*>(a.W);

  // Loader: 256 rows (128 of x, 128 of W) x 8 chunks; thread -> chunk
  // (tid & 7) of rows (tid >> 3) + 32 j.
  const int chunk = tid & 7;
  const T* src[8];
  bool sv[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int r = (tid >> 3) + 32 * j;
    if (r < BM) {
      const int i = row0 + r;
      sv[j] = i < a.n;
      const int rp = (sv[j] && a.rot_pos) ? a.rot_pos[i] : -1;
      const T* base = rp >= 0 ? XR + (size_t)rp * a.d_in : X + (size_t)(sv[j] ? i : 0) * a.d_in;
      src[j] = base + kbeg + chunk * EPC;
    } else {
      sv[j] = true;
      src[j] = W + (size_t)(col0 + r - BM) * a.d_in + kbeg + chunk * EPC;
    }
  }
  uint4 regs[8];
  auto gload = [&](int kt) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      regs[j] = sv[j] ? *reinterpret_cast<const uint4*>(src[j] + kt * BK) : make_uint4(0, 0, 0, 0);
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int r = (tid >> 3) + 32 * j;
      *reinterpret_cast<uint4*>(&lds[buf][r * LDK + chunk * EPC]) = regs[j];
    }
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int m = 0; m < 4; ++m) acc[b][m] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (nk > 0) {
    gload(0);
    lstore(0);
  }
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
    const T* L = lds[buf];
#pragma unroll
    for (int kk = 0; kk < BK; kk += 32) {
      typename Frag<T>::V af[4], bf[4];
#pragma unroll
      for (int b = 0; b < 4; ++b)
        af[b] = lds_frag<T>(L + (BM + 64 * wc + perm_col<4>(i16, b)) * LDK + kk + 8 * g);
#pragma unroll
      for (int m = 0; m < 4; ++m) bf[m] = lds_frag<T>(L + (64 * wr + 16 * m + i16) * LDK + kk + 8 * g);
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int m = 0; m < 4; ++m) acc[b][m] = mma(acc[b][m], af[b], bf[m]);
    }
    if (kt + 1 < nk) lstore(buf ^ 1);
    __syncthreads();
  }

  // Lane holds, for row block m, 16 consecutive output columns.
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int row = row0 + 64 * wr + 16 * m + i16;
    if (row >= a.n) continue;
    const int col = col0 + 64 * wc + 16 * g;
    float v[16];
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int q = 0; q < 4; ++q) v[4 * b + q] = acc[b][m][q];
    if (a.split == 1) {
      store_run16<T>(static_cast<T*>(a.out) + (size_t)row * a.d_out + col, v);
    } else {
      store_run16<float>(a.part + ((size_t)ks * a.n + row) * a.d_out + col, v);
    }
  }
}

// -------------------------------------------------------------- shrink ----

template <typename T, int MB>
__global__ __launch_bounds__(THREADS) void shrink_kernel(ShrinkArgs a) {
  constexpr int NB = 4;
  __shared__ float red[2 * NB * MB * 4 * 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i16 = lane & 15, g = lane >> 4;
  const int t = blockIdx.x / a.nblk;
  const int nb = blockIdx.x % a.nblk;
  if (t >= a.counts[CNT_NTILES]) return;
  const int* tile = a.tiles + 4 * t;
  const int kind = tile[2];
  if (kind == CLS_NONE) return;
  const int p0 = tile[0], p1 = tile[1];
  const T* Bm;
  int N;
  if (kind == CLS_OWNED) {
    const SlotDev& sd = a.slots[tile[3]];
    Bm = static_cast<const T*>(sd.A);
    N = sd.rank;
  } else {
    Bm = static_cast<const T*>(a.vera_At);
    N = a.r_v;
  }
  const int col0 = nb * 64;
  if (col0 >= N) return;
  const int ks = blockIdx.y;
  const int kbeg = ks * a.kc;
  const int kend = min(a.d_in, kbeg + a.kc);
  const T* X = static_cast<const T*>(a.x);

  const T* xp[MB];
  bool xv[MB];
#pragma unroll
  for (int m = 0; m < MB; ++m) {
    const int p = p0 + 16 * m + i16;
    xv[m] = p < p1;
    xp[m] = X + (size_t)(xv[m] ? a.perm[p] : 0) * a.d_in + 8 * g;
  }
  const T* wp[NB];
  bool wv[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int c = col0 + perm_col<NB>(i16, b);
    wv[b] = c < N;
    wp[b] = Bm + (size_t)(wv[b] ? c : 0) * a.d_in + 8 * g;
  }
  f32x4 acc[NB][MB];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int m = 0; m < MB; ++m) acc[b][m] = f32x4{0.f, 0.f, 0.f, 0.f};

  skinny_loop<T, MB, NB>(acc, wp, wv, xp, xv, kbeg, kend, wave);
  reduce_waves<NB, MB>(acc, red, wave, lane);
  if (wave != 0) return;
#pragma unroll
  for (int m = 0; m < MB; ++m) {
    const int p = p0 + 16 * m + i16;
    if (p >= p1) continue;
    const float* dv = nullptr;
    if (kind == CLS_SHARED) dv = a.slots[a.row_slot[a.perm[p]]].d;
    float* dst = a.part + ((size_t)ks * a.n + p) * a.kmax;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int col = col0 + 4 * NB * g + 4 * b;
      if (col >= N) continue;
      f32x4 v = acc[b][m];
      if (dv) {
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(dv + col);
        v = v * d4;
      }
      *reinterpret_cast<f32x4*>(dst + col) = v;
    }
  }
}

template <typename T>
hipError_t skinny_dispatch(int nb, const BaseGemmArgs& a, hipStream_t s) {
  const int mb = (a.n + 15) / 16;
  dim3 grid(a.d_out / (16 * nb), a.split);
#define TPA_SK(MBV, NBV)                                                                        \
  if (mb == MBV && nb == NBV) {                                                                \
    hipLaunchKernelGGL((gemm_skinny_kernel<T, MBV, NBV>), grid, dim3(THREADS), 0, s, a);        \
    return hipGetLastError();                                                                  \
  }
  TPA_SK(1, 1) TPA_SK(2, 1) TPA_SK(3, 1) TPA_SK(4, 1)
  TPA_SK(1, 2) TPA_SK(2, 2) TPA_SK(3, 2) TPA_SK(4, 2)
  TPA_SK(1, 4) TPA_SK(2, 4) TPA_SK(3, 4) TPA_SK(4, 4)
#undef TPA_SK
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_gemm_skinny(int dtype, int nb, const BaseGemmArgs& a, hipStream_t s) {
  if (a.n <= 0 || a.n > 64) return hipErrorInvalidValue;
  switch (dtype) {
    case 0: return skinny_dispatch<float>(nb, a, s);
    case 1: return skinny_dispatch<f16>(nb, a, s);
    case 2: return skinny_dispatch<bf16>(nb, a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gemm_tiled(int dtype, const BaseGemmArgs& a, hipStream_t s) {
  dim3 grid(a.d_out / 128, (a.n + 127) / 128, a.split);
  switch (dtype) {
    case 0: hipLaunchKernelGGL(gemm_tiled_kernel<float>, grid, dim3(THREADS), 0, s, a); break;
    case 1: hipLaunchKernelGGL(gemm_tiled_kernel<f16>, grid, dim3(THREADS), 0, s, a); break;
    case 2: hipLaunchKernelGGL(gemm_tiled_kernel<bf16>, grid, dim3(THREADS), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_shrink(int dtype, int tile_rows, const ShrinkArgs& a, hipStream_t s) {
  dim3 grid(a.max_tiles * a.nblk, a.split);
#define TPA_SH(TT, MBV) hipLaunchKernelGGL((shrink_kernel<TT, MBV>), grid, dim3(THREADS), 0, s, a)
  if (tile_rows == 16) {
    switch (dtype) {
      case 0: TPA_SH(float, 1); break;
      case 1: TPA_SH(f16, 1); break;
      case 2: TPA_SH(bf16, 1); break;
      default: return hipErrorInvalidValue;
    }
  } else if (tile_rows == 64) {
    switch (dtype) {
      case 0: TPA_SH(float, 4); break;
      case 1: TPA_SH(f16, 4); break;
      case 2: TPA_SH(bf16, 4); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    return hipErrorInvalidValue;
  }
#undef TPA_SH
  return hipGetLastError();
}

}  // namespace tpa
