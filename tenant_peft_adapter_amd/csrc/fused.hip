// Prefill base GEMM with the expand in its epilogue.
//
// Scute paper (arXiv 2611.01089): §2 "The LoRA schedule" (one tile of rows
// belongs to one adapter, so it reads one adapter's factors), §4.1 route one
// and §5.2 (the output scale s, and the shift b, applied as each tile
// finishes), route two's second GEMM (U · B_v over row tiles whatever their
// tenant, times each row's e).  Instead of writing h and reading it back in
// a pass of its own, the work-group that computes a block of h finishes it:
//
//   out[row] = h[row] ⊙ s + b + V[p] B'ᵀ        (tile on owned factors)
//   out[row] = h[row] ⊙ s + b + (U[p] B_vᵀ) ⊙ e  (tile on the shared pair)
//
// The GEMM runs over the plan's tiles rather than the batch order: row slot
// 16·t + j of the GEMM is row j of plan tile t (a short tile's unused slots
// and the padding tiles compute nothing that is stored), so each 16-row MFMA
// block of a work-group is one plan tile and its term is one MFMA product
// with that tile's factor, as in the expand kernel.  Everything else -- the
// 128 x 128 tile, its k loop (wide_impl.h: producer waves streaming 64-element
// k slices into S LDS buffers by direct loads, two groups of multiplying
// waves taking the halves of each slice one phase apart, then each of those
// waves finishing two 16-row blocks with both groups' sums), the swizzle -- is
// the direct-load prefill GEMM's.  k is never split here (h of a row
// is complete in one work-group), and V / U must be final before the launch.
#include "internal.h"
#include "wide_impl.h"

namespace tpa {

namespace {

template <typename T, int S>
__global__ __launch_bounds__(wide_impl::THREADS) void gemm_fused_kernel(FusedArgs f) {
  typedef typename Frag<T>::V Vt;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const BaseGemmArgs& a = f.g;
  const ExpandArgs& e = f.e;
  const wide_impl::Role ro = wide_impl::role();
  const int i16 = ro.i16, g = ro.g;
  const int col_tiles = f.col_tiles;
  // Row-major tile order: consecutive work-groups go to different XCDs, so
  // the trailing row tiles (past the plan's real tiles when the tile bound
  // is loose) are spread over every XCD instead of idling the last ones.
  const int t = (int)blockIdx.x;
  const int rt = t / col_tiles, ct = t % col_tiles;
  const int row0 = rt * 128, col0 = ct * 128;  // row0: row slot (16 per plan tile)
  // Real tiles come first in the plan's list: a work-group whose first
  // tile is padding has nothing to do (the same for all its threads).
  const int t_first = row0 >> 4;
  if (t_first >= f.list_tiles || e.tiles[4 * t_first + 2] < 0) return;
  const int nst = a.d_in / 64;

  // Producer loads: tile rows 0..127 are row slots (x rows gathered through
  // the plan's row words), 128..255 W rows.
  const T* src[wide_impl::LI] = {};
  if (ro.prod) {
    const T* X = static_cast<const T*>(a.x);
    const T* XR = static_cast<const T*>(a.x_rot);
    const T* W = static_cast<const T*>(a.W);
#pragma unroll
    for (int j = 0; j < wide_impl::LI; ++j) {
      const int r = wide_impl::producer_row(ro, j);
      const T* base;
      if (r < 128) {
        const int q = row0 + r, tq = q >> 4;
        int row = -1;
        if (tq < f.list_tiles && e.tiles[4 * tq + 2] >= 0) {
          const int w = e.tile_rows_w[q];
          row = w >= 0 ? (w & 0xFFFF) : -1;
        }
        base = X;  // unused slots read row 0; their results are not stored
        if (row >= 0) {
          base = X + (size_t)row * a.d_in;
          if (a.rot_pos) {
            const int rp = a.rot_pos[row];
            if (rp >= 0) base = XR + (size_t)rp * a.d_in;
          }
        }
      } else {
        base = W + (size_t)(col0 + r - 128) * a.d_in;
      }
      src[j] = base + wide_impl::producer_chunk_elems(ro, r);
    }
  }

  // The epilogue's metadata, loaded now by the waves that store, so that its
  // chain of dependent loads (tile header -> slot record -> vector pointers)
  // is in flight while the GEMM runs: per row block 2 grp + mm of the wave's
  // 64 x 64 block, the plan tile, the lane's row word, the term's rank and
  // factor, and the row's s, b and e.
  int ekind[2], erow[2], ep0[2], eK[2];
  const T* eBt[2];
  const float* esp[2];
  const float* ebq[2];
  const float* eep[2];
#pragma unroll
  for (int mm = 0; mm < 2; ++mm) {
    ekind[mm] = -1;
    erow[mm] = -1;
    ep0[mm] = 0;
    eK[mm] = 0;
    eBt[mm] = nullptr;
    esp[mm] = nullptr;
    ebq[mm] = nullptr;
    eep[mm] = nullptr;
  }
  if (!ro.prod) {
#pragma unroll
    for (int mm = 0; mm < 2; ++mm) {
      const int tq = (row0 + 64 * ro.wr + 16 * (2 * ro.grp + mm)) >> 4;
      int4 tl = make_int4(0, 0, -1, -1);
      if (tq < f.list_tiles) tl = *reinterpret_cast<const int4*>(e.tiles + 4 * tq);
      ekind[mm] = tl.z;
      ep0[mm] = tl.x;
      const int w = tl.z >= 0 ? e.tile_rows_w[tq * 16 + i16] : -1;
      erow[mm] = w >= 0 ? (w & 0xFFFF) : -1;
      const SlotDev* rsd = e.slots + (tl.z == CLS_OWNED ? tl.w : (w >= 0 ? (w >> 16) : 0));
      if (w >= 0) {
        if (e.apply_scale) {
          esp[mm] = gload<const float*>(&rsd->s);
          ebq[mm] = gload<const float*>(&rsd->b);
        }
        if (tl.z == CLS_SHARED) eep[mm] = gload<const float*>(&rsd->e);
      }
      if (tl.z == CLS_OWNED) {
        eK[mm] = e.slots[tl.w].rank;
        eBt[mm] = static_cast<const T*>(e.slots[tl.w].Bt);
      } else if (tl.z == CLS_SHARED) {
        eK[mm] = e.r_v;
        eBt[mm] = static_cast<const T*>(e.vera_Bt);
      }
    }
  }

  f32x4 acc[4][4];
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int m = 0; m < 4; ++m) acc[b][m] = f32x4{0.f, 0.f, 0.f, 0.f};
  wide_impl::k_loop<T, S>(ro, src, nst, smem, acc);
  wide_impl::exchange(ro, smem, acc);
  if (ro.prod) return;

  // Epilogue: row block 2 grp + mm of this wave's block is one plan tile;
  // the lane holds 16 consecutive output columns of row slot i16 of it.
  const T* V = static_cast<const T*>(e.v);
  T* out = static_cast<T*>(e.out);
  const int n0 = col0 + 64 * ro.wc;
  const int col = n0 + 16 * g;
#pragma unroll
  for (int mm = 0; mm < 2; ++mm) {
    if (ekind[mm] < 0) continue;  // padding tile: the same for the whole wave
    const int row = erow[mm];
    const float* sp = esp[mm];
    const float* bq = ebq[mm];
    const float* ep = eep[mm];
    const int K = eK[mm];
    const T* Bt = eBt[mm];
    f32x4 tac[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) tac[b] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (K > 0) {
      const T* bp[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) bp[b] = Bt + (size_t)(n0 + perm_col<4>(i16, b)) * K + 8 * g;
      const T* vp = V + (size_t)(row >= 0 ? ep0[mm] + i16 : 0) * e.kmax + 8 * g;
      for (int k = 0; k < K; k += 32) {
        const bool ok = k + 8 * g < K;
        Vt af[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) af[b] = ok ? load_frag<T>(bp[b] + k) : zero_frag<T>();
        const Vt bf = (ok && row >= 0) ? load_frag<T>(vp + k) : zero_frag<T>();
#pragma unroll
        for (int b = 0; b < 4; ++b) tac[b] = mma(tac[b], af[b], bf);
      }
    }
    if (row < 0) continue;
    float v[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x4 s4 = sp ? gload<f32x4>(sp + col + 4 * q) : f32x4{1.f, 1.f, 1.f, 1.f};
      const f32x4 b4 = bq ? gload<f32x4>(bq + col + 4 * q) : f32x4{0.f, 0.f, 0.f, 0.f};
      const f32x4 e4 = ep ? gload<f32x4>(ep + col + 4 * q) : f32x4{1.f, 1.f, 1.f, 1.f};
      const f32x4 h4 = acc[q][mm];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        // h stays fp32 here (a separate expand reads it back rounded to the
        // layer type): only the output is rounded.
        const float h = h4[j];
        float r = h * s4[j] + b4[j];
        if (K > 0) r += tac[q][j] * e4[j];
        v[4 * q + j] = r;
      }
    }
    store_run16<T>(out + (size_t)row * a.d_out + col, v);
  }
}

}  // namespace

hipError_t launch_gemm_fused(int dtype, int stages, const FusedArgs& f, hipStream_t s) {
  const BaseGemmArgs& a = f.g;
  if (a.n <= 0 || a.d_out % 128 || a.d_in % 64 || f.col_tiles != a.d_out / 128 || f.row_tiles <= 0 ||
      f.list_tiles <= 0 || (long)f.row_tiles * 8 > (long)f.list_tiles + 7 || !f.e.apply_scale)
    return hipErrorInvalidValue;
  if (stages < 2 || stages > 5 || (dtype != 1 && dtype != 2)) return hipErrorInvalidValue;
  const dim3 grid((unsigned)(f.row_tiles * f.col_tiles));
  const dim3 block(wide_impl::THREADS);
  const size_t lds = (size_t)stages * wide_impl::STAGE;
#define TPA_FUSED(SV)                                                                  \
  if (stages == SV) {                                                                  \
    if (dtype == 1)                                                                    \
      hipLaunchKernelGGL((gemm_fused_kernel<f16, SV>), grid, block, lds, s, f);        \
    else                                                                               \
      hipLaunchKernelGGL((gemm_fused_kernel<bf16, SV>), grid, block, lds, s, f);       \
  }
  TPA_FUSED(2) TPA_FUSED(3) TPA_FUSED(4) TPA_FUSED(5)
#undef TPA_FUSED
  return hipGetLastError();
}

}  // namespace tpa
