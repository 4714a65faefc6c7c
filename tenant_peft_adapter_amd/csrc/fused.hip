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
// 128 x 128 tile of 4 waves (64 x 64 each), 64-element k slices streamed
// into S LDS buffers by direct loads, the swizzle, the XCD-aware tile order
// -- is the direct-load prefill GEMM's.  k is never split here (h of a row
// is complete in one work-group), and V / U must be final before the launch.
#include "internal.h"

namespace tpa {

namespace {

template <typename T, int S>
__global__ __launch_bounds__(256) void gemm_fused_kernel(FusedArgs f) {
  typedef typename Frag<T>::V Vt;
  constexpr int STAGE = 256 * 128;
  constexpr int LI = 8;  // loads per wave per slice
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const BaseGemmArgs& a = f.g;
  const ExpandArgs& e = f.e;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i16 = lane & 15, g = lane >> 4;
  const int wr = wave & 1, wc = wave >> 1;
  const int row_tiles = f.row_tiles, col_tiles = f.col_tiles;
  const int ntile = row_tiles * col_tiles;
  // Row-major tile order: consecutive work-groups go to different XCDs, so
  // the trailing row tiles (past the plan's real tiles when the tile bound
  // is loose) are spread over every XCD instead of idling the last ones.
  const int t = (int)blockIdx.x;
  (void)ntile;
  const int rt = t / col_tiles, ct = t % col_tiles;
  const int row0 = rt * 128, col0 = ct * 128;  // row0: row slot (16 per plan tile)
  // Real tiles come first in the plan's list: a work-group whose first
  // tile is padding has nothing to do (the same for all its threads).
  const int t_first = row0 >> 4;
  if (t_first >= f.list_tiles || e.tiles[4 * t_first + 2] < 0) return;
  const int nst = a.d_in / 64;
  const T* X = static_cast<const T*>(a.x);
  const T* XR = static_cast<const T*>(a.x_rot);
  const T* W = static_cast<const T*>(a.W);

  // Loads: instruction j < 4 takes row slots 32·wave + 8j .. +8 of the tile
  // (x rows gathered through the plan's row words), j >= 4 W rows.
  const int lr = lane >> 3, lc = lane & 7;
  const T* src[LI];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = 32 * wave + 8 * j + lr;
    const int q = row0 + r, tq = q >> 4;
    int row = -1;
    if (tq < f.list_tiles && e.tiles[4 * tq + 2] >= 0) {
      const int w = e.tile_rows_w[q];
      row = w >= 0 ? (w & 0xFFFF) : -1;
    }
    const T* base = X;  // unused slots read row 0; their results are not stored
    if (row >= 0) {
      base = X + (size_t)row * a.d_in;
      if (a.rot_pos) {
        const int rp = a.rot_pos[row];
        if (rp >= 0) base = XR + (size_t)rp * a.d_in;
      }
    }
    src[j] = base + 8 * (lc ^ swz<2>(r));
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = 32 * wave + 8 * j + lr;
    src[4 + j] = W + (size_t)(col0 + r) * a.d_in + 8 * (lc ^ swz<4>(r));
  }
  auto issue = [&](int st) {
    unsigned char* buf = smem + (size_t)(st % S) * STAGE;
#pragma unroll
    for (int j = 0; j < LI; ++j)
      __builtin_amdgcn_global_load_lds(
          (const void*)(src[j] + 64 * st),
          (__attribute__((address_space(3))) void*)(buf + (j < 4 ? 0 : 128 * 128) + (size_t)(32 * wave + 8 * (j & 3)) * 128),
          16, 0, 0);
  };

  // The epilogue's metadata, loaded now so that its chain of dependent
  // loads (tile header -> slot record -> vector pointers) is in flight while
  // the GEMM runs: per row block m of this wave, the plan tile, the lane's
  // row word, the term's rank and factor, and the row's s, b and e.
  int ekind[4], erow[4], ep0[4], eK[4];
  const T* eBt[4];
  const float* esp[4];
  const float* ebq[4];
  const float* eep[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int tq = (row0 + 64 * wr + 16 * m) >> 4;
    int4 tl = make_int4(0, 0, -1, -1);
    if (tq < f.list_tiles) tl = *reinterpret_cast<const int4*>(e.tiles + 4 * tq);
    ekind[m] = tl.z;
    ep0[m] = tl.x;
    const int w = tl.z >= 0 ? e.tile_rows_w[tq * 16 + i16] : -1;
    erow[m] = w >= 0 ? (w & 0xFFFF) : -1;
    const SlotDev* rsd = e.slots + (tl.z == CLS_OWNED ? tl.w : (w >= 0 ? (w >> 16) : 0));
    esp[m] = nullptr;
    ebq[m] = nullptr;
    eep[m] = nullptr;
    if (w >= 0) {
      if (e.apply_scale) {
        esp[m] = gload<const float*>(&rsd->s);
        ebq[m] = gload<const float*>(&rsd->b);
      }
      if (tl.z == CLS_SHARED) eep[m] = gload<const float*>(&rsd->e);
    }
    eK[m] = 0;
    eBt[m] = nullptr;
    if (tl.z == CLS_OWNED) {
      eK[m] = e.slots[tl.w].rank;
      eBt[m] = static_cast<const T*>(e.slots[tl.w].Bt);
    } else if (tl.z == CLS_SHARED) {
      eK[m] = e.r_v;
      eBt[m] = static_cast<const T*>(e.vera_Bt);
    }
  }

  int arow[4], brow[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) arow[b] = 64 * wc + perm_col<4>(i16, b);
#pragma unroll
  for (int m = 0; m < 4; ++m) brow[m] = 64 * wr + 16 * m + i16;
  f32x4 acc[4][4];
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int m = 0; m < 4; ++m) acc[b][m] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int st = 0; st < S - 1; ++st)
    if (st < nst) issue(st);
  for (int it = 0; it < nst; ++it) {
    const int younger = min(S - 2, nst - 1 - it);
    __builtin_amdgcn_sched_barrier(0);
    if (S >= 4 && younger == 2)
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * LI));
    else if (younger == 1)
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(LI));
    else
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    if (it + S - 1 < nst) issue(it + S - 1);
    const unsigned char* buf = smem + (size_t)(it % S) * STAGE;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int q = 4 * kk + g;
      Vt af[4], bf[4];
#pragma unroll
      for (int b = 0; b < 4; ++b)
        af[b] = *reinterpret_cast<const Vt*>(buf + 128 * 128 + arow[b] * 128 + 16 * (q ^ swz<4>(arow[b])));
#pragma unroll
      for (int m = 0; m < 4; ++m)
        bf[m] = *reinterpret_cast<const Vt*>(buf + brow[m] * 128 + 16 * (q ^ swz<2>(brow[m])));
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int m = 0; m < 4; ++m) acc[b][m] = mma(acc[b][m], af[b], bf[m]);
    }
  }

  // Epilogue: row block m of this wave is plan tile tq; the lane holds 16
  // consecutive output columns of row slot i16 of it.
  const T* V = static_cast<const T*>(e.v);
  T* out = static_cast<T*>(e.out);
  const int n0 = col0 + 64 * wc;
  const int col = n0 + 16 * g;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    if (ekind[m] < 0) continue;  // padding tile: the same for the whole wave
    const int row = erow[m];
    const float* sp = esp[m];
    const float* bq = ebq[m];
    const float* ep = eep[m];
    const int K = eK[m];
    const T* Bt = eBt[m];
    f32x4 tac[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) tac[b] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (K > 0) {
      const T* bp[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) bp[b] = Bt + (size_t)(n0 + perm_col<4>(i16, b)) * K + 8 * g;
      const T* vp = V + (size_t)(row >= 0 ? ep0[m] + i16 : 0) * e.kmax + 8 * g;
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
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        // h stays fp32 here (a separate expand reads it back rounded to the
        // layer type): only the output is rounded.
        const float h = acc[q][m][j];
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
  const size_t lds = (size_t)stages * 256 * 128;
#define TPA_FUSED(SV)                                                                       \
  if (stages == SV) {                                                                       \
    if (dtype == 1)                                                                         \
      hipLaunchKernelGGL((gemm_fused_kernel<f16, SV>), grid, dim3(256), lds, s, f);         \
    else                                                                                    \
      hipLaunchKernelGGL((gemm_fused_kernel<bf16, SV>), grid, dim3(256), lds, s, f);        \
  }
  TPA_FUSED(2) TPA_FUSED(3) TPA_FUSED(4) TPA_FUSED(5)
#undef TPA_FUSED
  return hipGetLastError();
}

}  // namespace tpa
