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
//     once from HBM.  Each work-group owns 64·NB output columns and one k
//     range (split-K): x for that range sits in LDS, W streams straight
//     from memory into MFMA registers; partial sums are combined in a fixed
//     order (k-groups in LDS, splits in the expand), so results do not
//     depend on scheduling.
//   gemm_tiled   -- larger n (prefill).  128x128 output tiles, 128-byte k
//     slices staged through double-buffered LDS, 2x2 waves of 64x64.
#include <algorithm>

#include "internal.h"
#include "shrink_impl.h"
#include "wide_impl.h"

namespace tpa {

namespace {

constexpr int THREADS = 256;


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

// Decode base GEMM (n <= 64 rows).  Work-group = 4·G waves; its tile is
// BN = 64·NB output columns (wave slice w % 4 owns 16·NB of them) by one k
// range of kc (split-K).  The work-group's x rows for that range are staged
// in LDS once (rows >= n zero), so each x byte serves BN columns; k-group
// w / 4 streams its share of the range of W straight into MFMA registers,
// U k steps of loads issued together, with x fragments read from LDS.  The
// k-groups are added in LDS in group order and the sum is the split's fp32
// partial [split][n][d_out]; the expand adds the splits in split order.
//
// Work-groups past the GEMM's own (when `side` is given) do another job: the
// shrink's split reduction (one thread per 4 columns of one plan position),
// which the previous launch made ready; placed after the GEMM's work-groups
// they take CUs the GEMM leaves free and are hidden under it.
template <typename T, int MB, int NB, int G>
__global__ __launch_bounds__(256 * G) void gemm_skinny_kernel(Slices<GemmSlice> t) {
  typedef typename Frag<T>::V Vt;
  constexpr int EPC = 16 / sizeof(T);  // elements per 16-byte chunk
  constexpr int U = sizeof(T) == 4 ? 2 : 8 / NB;  // k steps per register stage
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  T* xs = reinterpret_cast<T*>(smem);
  const int si = slice_of(t, (int)blockIdx.x);
  const BaseGemmArgs& a = t.s[si].g;
  const int local = (int)blockIdx.x - t.first[si];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col_tiles = a.d_out / (64 * NB);
  const int n_gemm = col_tiles * a.split;
  if (local >= n_gemm) {
    shrink_impl::shrink_reduce_item<T>(t.s[si].side, (local - n_gemm) * (256 * G) + tid);
    return;
  }
  const int gid = local;
  const int slice = wave & 3, grp = wave >> 2;
  const int i16 = lane & 15, g = lane >> 4;
  const int col0 = (gid % col_tiles) * (64 * NB) + slice * (16 * NB);
  const int ks = gid / col_tiles;
  const int kbeg = ks * a.kc;
  const int klen = min(a.d_in - kbeg, a.kc);  // a multiple of 32
  const int ldx = a.kc + EPC;                 // LDS row stride in elements
  const T* X = static_cast<const T*>(a.x);
  const T* XR = static_cast<const T*>(a.x_rot);
  const T* W = static_cast<const T*>(a.W);

  // 1. Stage the x rows of this k range.
  const int cpr = klen / EPC;
  for (int i = tid; i < 16 * MB * cpr; i += 256 * G) {
    const int r = i / cpr, c = (i % cpr) * EPC;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (r < a.n) {
      const int rp = a.rot_pos ? a.rot_pos[r] : -1;
      const T* src = rp >= 0 ? XR + (size_t)rp * a.d_in : X + (size_t)r * a.d_in;
      v = *reinterpret_cast<const uint4*>(src + kbeg + c);
    }
    *reinterpret_cast<uint4*>(xs + r * ldx + c) = v;
  }
  __syncthreads();

  // 2. This k-group's k steps [s_lo, s_hi) of 32.
  const int steps = klen / 32;
  const int per = (steps + G - 1) / G;
  const int s_lo = min(steps, grp * per), s_hi = min(steps, s_lo + per);
  const T* wp[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) wp[b] = W + (size_t)(col0 + perm_col<NB>(i16, b)) * a.d_in + kbeg + 8 * g;
  const T* xl = xs + i16 * ldx + 8 * g;
  f32x4 acc[NB][MB];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int m = 0; m < MB; ++m) acc[b][m] = f32x4{0.f, 0.f, 0.f, 0.f};
  // Two register stages of U k steps: the loads of batch i + 1 are in
  // flight while batch i is multiplied.  Scheduling barriers keep the
  // compiler from interleaving (and so serializing) loads and MFMAs.
  Vt wa[U][NB], wb[U][NB];
  auto load = [&](Vt(&w)[U][NB], int s0) {
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int b = 0; b < NB; ++b) w[u][b] = load_frag<T>(wp[b] + 32 * (s0 + u));
  };
  auto comp = [&](Vt(&w)[U][NB], int s0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      Vt xf[MB];
#pragma unroll
      for (int m = 0; m < MB; ++m) xf[m] = lds_frag<T>(xl + 16 * m * ldx + 32 * (s0 + u));
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int m = 0; m < MB; ++m) acc[b][m] = mma(acc[b][m], w[u][b], xf[m]);
    }
  };
  const int nfull = (s_hi - s_lo) / U;
  int st = s_lo;
  if (nfull > 0) load(wa, st);
  int i = 0;
  for (; i + 2 <= nfull; i += 2) {
    load(wb, st + U);
    __builtin_amdgcn_sched_barrier(0);
    comp(wa, st);
    __builtin_amdgcn_sched_barrier(0);
    if (i + 2 < nfull) load(wa, st + 2 * U);
    __builtin_amdgcn_sched_barrier(0);
    comp(wb, st + U);
    __builtin_amdgcn_sched_barrier(0);
    st += 2 * U;
  }
  if (i < nfull) {
    comp(wa, st);
    st += U;
  }
  for (; st < s_hi; ++st) {
    Vt wf[NB], xf[MB];
#pragma unroll
    for (int b = 0; b < NB; ++b) wf[b] = load_frag<T>(wp[b] + 32 * st);
#pragma unroll
    for (int m = 0; m < MB; ++m) xf[m] = lds_frag<T>(xl + 16 * m * ldx + 32 * st);
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int m = 0; m < MB; ++m) acc[b][m] = mma(acc[b][m], wf[b], xf[m]);
  }

  // 3. Add the k-groups in group order (group 0 keeps the sum).
  if (G > 1) {
    f32x4* red = reinterpret_cast<f32x4*>(smem);
    __syncthreads();  // every wave is done with the staged x
    for (int q = 1; q < G; ++q) {
      if (grp == q) {
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int m = 0; m < MB; ++m) red[((slice * NB + b) * MB + m) * 64 + lane] = acc[b][m];
      }
      __syncthreads();
      if (grp == 0) {
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int m = 0; m < MB; ++m) acc[b][m] += red[((slice * NB + b) * MB + m) * 64 + lane];
      }
      __syncthreads();
    }
    if (grp != 0) return;
  }
  // Lane holds columns col0 + 4·NB·g + [0, 4·NB) of row 16m + i16.
#pragma unroll
  for (int m = 0; m < MB; ++m) {
    const int row = 16 * m + i16;
    if (row >= a.n) continue;
    float* dst = a.part + ((size_t)ks * a.n + row) * a.d_out + col0 + 4 * NB * g;
#pragma unroll
    for (int b = 0; b < NB; ++b) *reinterpret_cast<f32x4*>(dst + 4 * b) = acc[b][m];
  }
}

// ------------------------------------------------------------- stream ----
//
// Decode base GEMM (n <= 64 rows, f16/bf16) fed by gfx950's direct global-
// to-LDS loads.  Work-group = G k-groups of 4 waves; its tile is 64·NB output
// columns (wave w of a group owns 16·NB) by one k range of kc (split-K),
// which the groups share out by 64-element slices (group g takes the g-th
// run of ceil(slices / G)).  Each group walks its run: each slice of W
// (64·NB rows x 128 B) and of x (16·MB rows x 128 B) is loaded straight into
// one of the group's S LDS buffers, 8 rows x 128 B (whole cache lines) per
// wave instruction, with no registers held while the loads are in flight;
// S - 1 slices are in flight while one is multiplied.  Per slice, each wave
// waits for its own loads (vmcnt), then the work-group meets at a barrier
// (every wave runs the same number of iterations); the loads write LDS
// directly, so no fence is needed.  The groups' sums are added in LDS in
// group order and the total is the split's fp32 partial [split][n][d_out];
// k-groups keep as many bytes in flight per CU as separate work-groups would
// while halving the partials written and read back.  Work-groups past the
// GEMM's own run the shrink's split reduction, as in gemm_skinny_kernel.
//
// Within a 128-byte LDS row the eight 16-byte chunks are permuted (swz in
// common.h) so that the fragment reads hit distinct bank groups.

// Fused epilogue of the streamed decode GEMM: the expand (Scute paper,
// §2 "The LoRA schedule": the expand reads h, adds V B and writes the
// tile; §4.1 route one and §5.2: s applied as the tile finishes; route two:
// the shared factor's term over rows of any tenant, times e) run by the
// work-group that completes a column tile, while h is still on chip.
//
// With k split, each work-group writes its split's fp32 sum, makes it
// visible at device scope (release fence) and counts itself in on the
// tile's counter; the one that brings the count to the split count
// (acquire fence) finishes the tile.  Nobody waits on anybody: the others
// have nothing left to do.  The finishing work-group builds tables in LDS
// (each row's plan position, class and s / b / e; each term tile's rows,
// rank and factor; the MFMA k steps over all term tiles), parks its own
// split in LDS, and then every thread takes runs of 4 columns of one row:
// the splits added in split order (its own from LDS), times s, plus b,
// exactly as the expand adds them, back into LDS with e beside it.  Group 0
// computes the term in the GEMM's register layout: for each k step of a
// tile, a = the factor's rows at the wave's output columns (B' or B_v,
// stored [d_out][K]), b = V (or U) of those of the wave's rows that lie in
// the tile, zero for the others, so a row collects its own tile's products
// in k order and exact zeros from every other tile (the expand's sums), and
// y = (h ⊙ s + b) + term ⊙ e is written once.
struct EpiLds {
  int wsum, rpos, rs, rb, re, tinfo, tbt, steps, end;
};
// Bytes of the rings the epilogue uses: the k-groups' sums, then h and e
// (16·MB rows of 64·NB + 4 floats each).
__host__ __device__ constexpr size_t epi_ring_bytes(int mb, int nb, int g) {
  return (size_t)(g - 1) * 4 * nb * mb * 1024 + (size_t)2 * 16 * mb * (64 * nb + 4) * 4;
}
__host__ __device__ inline EpiLds epi_lds_layout(int nrows, int max_tiles, int steps) {
  EpiLds o;
  o.wsum = 16;  // after the arrival flag; one word per wave (at most 16)
  o.rpos = 80;
  o.rs = o.rpos + ((4 * nrows + 15) & ~15);
  o.rb = o.rs + 8 * nrows;
  o.re = o.rb + 8 * nrows;
  o.tinfo = (o.re + 8 * nrows + 15) & ~15;
  o.tbt = o.tinfo + 16 * max_tiles;
  o.steps = o.tbt + 8 * max_tiles;
  o.end = o.steps + 4 * steps;
  return o;
}

// ring: the work-group's LDS rings (free once the k loop is done); its
// first red_bytes hold the k-groups' sums until group 0 has added them.
// tab: the tables, after the rings.
template <typename T, int MB, int NB, int G>
__device__ __forceinline__ void stream_epilogue(const GemmSlice& sl, const f32x4 (&acc)[NB][MB], int ks,
                                                int col_tile, int col0, unsigned char* ring, unsigned char* tab,
                                                int grp, int wave, int lane) {
  typedef typename Frag<T>::V Vt;
  typedef T T4 __attribute__((ext_vector_type(4)));
  constexpr int NT = 256 * G;
  constexpr int UE = 4;                      // k steps whose loads are issued together
  constexpr int PITCH = 64 * NB + 4;         // floats per LDS row of h (padded against bank conflicts)
  constexpr int UNITS = 16 * MB * 16 * NB;   // runs of 4 columns in the tile
  constexpr int UPT = (UNITS + NT - 1) / NT; // per thread
  // splits whose loads are issued together: 16 loads of 16 bytes per thread
  constexpr int SPB = UPT >= 16 ? 1 : (16 / UPT > 8 ? 8 : 16 / UPT);
  const BaseGemmArgs& a = sl.g;
  const ExpandArgs& e = sl.e;
  const int tid = (int)threadIdx.x;
  const int i16 = lane & 15, g = lane >> 4;
  const int n = a.n;
  int* flag = reinterpret_cast<int*>(tab);
  float* hs = reinterpret_cast<float*>(ring + (size_t)(G - 1) * 4 * NB * MB * 1024);  // [16·MB][PITCH]
  float* es = hs + 16 * MB * PITCH;                                                    // [16·MB][PITCH]

  // 1. Split sum out, arrival in.
  if (a.split > 1) {
    if (grp == 0) {
#pragma unroll
      for (int m = 0; m < MB; ++m) {
        const int row = 16 * m + i16;
        if (row >= n) continue;
        float* dst = a.part + ((size_t)ks * n + row) * a.d_out + col0 + 16 * NB * wave + 4 * NB * g;
#pragma unroll
        for (int b = 0; b < NB; ++b) *reinterpret_cast<f32x4*>(dst + 4 * b) = acc[b][m];
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __syncthreads();
    if (tid == 0)
      *flag = __hip_atomic_fetch_add(sl.cnt + col_tile, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT) ==
              a.split - 1;
    __syncthreads();
    if (!*flag) return;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }

  // 2. Tables in LDS, and this split's sum parked beside them.
  const EpiLds o = epi_lds_layout(16 * MB, e.max_tiles, 0);
  int* wsum = reinterpret_cast<int*>(tab + o.wsum);
  int* rpos = reinterpret_cast<int*>(tab + o.rpos);
  const float** rs = reinterpret_cast<const float**>(tab + o.rs);
  const float** rb = reinterpret_cast<const float**>(tab + o.rb);
  const float** re = reinterpret_cast<const float**>(tab + o.re);
  int4* tinfo = reinterpret_cast<int4*>(tab + o.tinfo);
  const void** tbt = reinterpret_cast<const void**>(tab + o.tbt);
  int* steps = reinterpret_cast<int*>(tab + o.steps);
  for (int p = tid; p < n; p += NT) {
    const int w = gload<int>(sl.pinfo + p);
    const int row = w & 0xFFFF;
    const SlotDev* sd = e.slots + ((unsigned)w >> 16);
    rpos[row] = p | (gload<int>(&sd->cls) << 16);
    rs[row] = gload<const float*>(&sd->s);
    rb[row] = gload<const float*>(&sd->b);
    re[row] = gload<const float*>(&sd->e);
  }
  int nst = 0;
  if (tid < e.max_tiles) {
    const int4 hd = *reinterpret_cast<const int4*>(e.tiles + 4 * tid);
    int K = 0;
    const void* bt = nullptr;
    if (hd.z == CLS_OWNED) {
      K = gload<int>(&e.slots[hd.w].rank);
      bt = gload<const void*>(&e.slots[hd.w].Bt);
    } else if (hd.z == CLS_SHARED) {
      K = e.r_v;
      bt = e.vera_Bt;
    }
    tinfo[tid] = make_int4(hd.x, hd.y, K, 0);
    tbt[tid] = bt;
    nst = (K + 31) / 32;
  }
  if (grp == 0) {
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
      for (int b = 0; b < NB; ++b)
        *reinterpret_cast<f32x4*>(hs + (16 * m + i16) * PITCH + 16 * NB * wave + 4 * NB * g + 4 * b) = acc[b][m];
  }
  const int incl = (int)wave_incl_scan((uint32_t)nst);
  if (lane == 63) wsum[tid >> 6] = incl;
  lds_barrier();
  int off = incl - nst, total = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    const int sw = wsum[w];
    if (w < (tid >> 6)) off += sw;
    total += sw;
  }
  for (int j = 0; j < nst; ++j) steps[off + j] = (tid << 8) | j;

  // 3. Every thread: runs of 4 columns, h = the splits in split order, then
  //    h ⊙ s + b into hs and e (1 for rows without a shared term) into es.
  f32x4 hv[UPT], sv[UPT], bv[UPT], ev[UPT];
#pragma unroll
  for (int u = 0; u < UPT; ++u) {
    const int unit = tid + u * NT;
    const int row = unit / (16 * NB), c4 = unit % (16 * NB);
    hv[u] = f32x4{0.f, 0.f, 0.f, 0.f};
    sv[u] = f32x4{1.f, 1.f, 1.f, 1.f};
    bv[u] = f32x4{0.f, 0.f, 0.f, 0.f};
    ev[u] = f32x4{1.f, 1.f, 1.f, 1.f};
    if (unit < UNITS && row < n) {
      const int colg = col0 + 4 * c4;
      const float* sp = rs[row];
      const float* bq = rb[row];
      const float* ep = re[row];
      if (sp) sv[u] = gload<f32x4>(sp + colg);
      if (bq) bv[u] = gload<f32x4>(bq + colg);
      if ((rpos[row] >> 16) == CLS_SHARED && ep) ev[u] = gload<f32x4>(ep + colg);
    }
  }
  for (int s0 = 0; s0 < a.split; s0 += SPB) {
    f32x4 ld[SPB][UPT];
#pragma unroll
    for (int q = 0; q < SPB; ++q)
#pragma unroll
      for (int u = 0; u < UPT; ++u) {
        const int unit = tid + u * NT;
        const int row = unit / (16 * NB), c4 = unit % (16 * NB);
        const int sp = s0 + q;
        ld[q][u] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (unit < UNITS && row < n && sp < a.split) {
          if (sp == ks)
            ld[q][u] = *reinterpret_cast<const f32x4*>(hs + row * PITCH + 4 * c4);
          else
            ld[q][u] = gload<f32x4>(a.part + ((size_t)sp * n + row) * a.d_out + col0 + 4 * c4);
        }
      }
#pragma unroll
    for (int q = 0; q < SPB; ++q) {
      if (s0 + q >= a.split) break;
#pragma unroll
      for (int u = 0; u < UPT; ++u) hv[u] += ld[q][u];
    }
  }
  lds_barrier();  // every read of the parked split is done
#pragma unroll
  for (int u = 0; u < UPT; ++u) {
    const int unit = tid + u * NT;
    if (unit >= UNITS) continue;
    const int row = unit / (16 * NB), c4 = unit % (16 * NB);
    f32x4 y;
#pragma unroll
    for (int j = 0; j < 4; ++j) y[j] = hv[u][j] * sv[u][j] + bv[u][j];
    *reinterpret_cast<f32x4*>(hs + row * PITCH + 4 * c4) = y;
    *reinterpret_cast<f32x4*>(es + row * PITCH + 4 * c4) = ev[u];
  }
  lds_barrier();
  if (grp != 0) return;

  // 4. Group 0: the term over every k step of every term tile, in the
  //    GEMM's layout (lane: columns colw .. colw + 4·NB of rows 16m + i16).
  int pos[MB];
#pragma unroll
  for (int m = 0; m < MB; ++m) {
    const int row = 16 * m + i16;
    pos[m] = row < n ? (rpos[row] & 0xFFFF) : -1;
  }
  f32x4 tacc[NB][MB];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int m = 0; m < MB; ++m) tacc[b][m] = f32x4{0.f, 0.f, 0.f, 0.f};
  const T* V = static_cast<const T*>(e.v);
  int acol[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) acol[b] = col0 + 16 * NB * wave + perm_col<NB>(i16, b);
  for (int j0 = 0; j0 < total; j0 += UE) {
    Vt af[UE][NB], bf[UE][MB];
#pragma unroll
    for (int u = 0; u < UE; ++u) {
      const int j = j0 + u;
      int4 ti = make_int4(0, 0, 0, 0);
      const T* bt = nullptr;
      int kk = 0;
      if (j < total) {
        const int sw = steps[j];
        ti = tinfo[sw >> 8];
        bt = static_cast<const T*>(tbt[sw >> 8]);
        kk = 32 * (sw & 255) + 8 * g;
      }
      const bool ok = kk < ti.z;
#pragma unroll
      for (int b = 0; b < NB; ++b) af[u][b] = ok ? load_frag<T>(bt + (size_t)acol[b] * ti.z + kk) : zero_frag<T>();
#pragma unroll
      for (int m = 0; m < MB; ++m)
        bf[u][m] = (ok && pos[m] >= ti.x && pos[m] < ti.y) ? load_frag<T>(V + (size_t)pos[m] * e.kmax + kk)
                                                            : zero_frag<T>();
    }
#pragma unroll
    for (int u = 0; u < UE; ++u) {
      if (j0 + u >= total) break;
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int m = 0; m < MB; ++m) tacc[b][m] = mma(tacc[b][m], af[u][b], bf[u][m]);
    }
  }

  // 5. y = (h ⊙ s + b) + term ⊙ e, written once.
  T* out = static_cast<T*>(e.out);
  const int cl = 16 * NB * wave + 4 * NB * g;  // column within the tile
#pragma unroll
  for (int m = 0; m < MB; ++m) {
    const int row = 16 * m + i16;
    if (row >= n) continue;
    T* dst = out + (size_t)row * e.d_out + col0 + cl;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const f32x4 hsb = *reinterpret_cast<const f32x4*>(hs + row * PITCH + cl + 4 * b);
      const f32x4 e4 = *reinterpret_cast<const f32x4*>(es + row * PITCH + cl + 4 * b);
      f32x4 y;
#pragma unroll
      for (int j = 0; j < 4; ++j) y[j] = hsb[j] + tacc[b][m][j] * e4[j];
      *reinterpret_cast<T4*>(dst + 4 * b) = T4{to_t<T>(y[0]), to_t<T>(y[1]), to_t<T>(y[2]), to_t<T>(y[3])};
    }
  }
}

template <int NB>
constexpr int log2_nb() {
  return NB == 1 ? 0 : NB == 2 ? 1 : 2;
}

template <int MB, int NB>
constexpr size_t stream_stage_bytes() {
  return (size_t)(64 * NB + 16 * MB) * 128;
}

template <typename T, int MB, int NB, int G, int S, bool EPI>
__global__ __launch_bounds__(256 * G) void gemm_stream_kernel(Slices<GemmSlice> t) {
  typedef typename Frag<T>::V Vt;
  constexpr int WROWS = 64 * NB;             // W rows (output columns) per work-group
  constexpr int W_INSTR = WROWS / 32;        // W loads per wave per slice (8 rows each)
  constexpr int X_INSTR = 2 * MB;            // x loads per slice, whole group
  constexpr int XJ = (X_INSTR + 3) / 4;      // x loads per slice a wave may issue
  constexpr int SHW = 2 + log2_nb<NB>();     // swz shift of the W rows
  constexpr int STAGE = (int)stream_stage_bytes<MB, NB>();
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int si = slice_of(t, (int)blockIdx.x);
  const BaseGemmArgs& a = t.s[si].g;
  const int local = (int)blockIdx.x - t.first[si];
  const int tid = threadIdx.x, lane = tid & 63;
  const int grp = tid >> 8, wave = (tid >> 6) & 3;
  const int col_tiles = a.d_out / WROWS;
  const int n_gemm = col_tiles * a.split;
  if (local >= n_gemm) {
    if (t.s[si].side_whole)
      shrink_impl::shrink_whole_item<T, 4 * G>([&](int j) -> const ShrinkArgs& { return t.s[j].side; }, t.count, si,
                                               local - n_gemm, tid >> 6, lane, reinterpret_cast<f32x4*>(smem));
    else
      shrink_impl::shrink_reduce_item<T>(t.s[si].side, (local - n_gemm) * 256 * G + tid);
    return;
  }
  const int col0 = (local % col_tiles) * WROWS;
  const int ks = local / col_tiles;
  const int ns = max(0, min(a.d_in - ks * a.kc, a.kc)) / 64;  // slices of the range
  const int per = (ns + G - 1) / G;                              // iterations, every wave
  const int s_lo = min(ns, grp * per);
  const int nst = min(ns, s_lo + per) - s_lo;                    // this group's slices
  const int kbeg = ks * a.kc + 64 * s_lo;
  const T* W = static_cast<const T*>(a.W);
  const T* X = static_cast<const T*>(a.x);
  const T* XR = static_cast<const T*>(a.x_rot);
  unsigned char* ring = smem + (size_t)grp * S * STAGE;

  // Global source of each of this lane's loads (the same for every slice
  // but for the k offset): lane = 8 · (row within the instruction) + LDS chunk.
  const int lr = lane >> 3, lc = lane & 7;
  const T* wsrc[W_INSTR];
#pragma unroll
  for (int j = 0; j < W_INSTR; ++j) {
    const int r = (wave * W_INSTR + j) * 8 + lr;
    wsrc[j] = W + (size_t)(col0 + r) * a.d_in + kbeg + 8 * (lc ^ swz<SHW>(r));
  }
  const T* xsrc[XJ];
  bool xmine[XJ];
#pragma unroll
  for (int j = 0; j < XJ; ++j) {
    const int ji = wave * XJ + j;  // x instruction index
    xmine[j] = ji < X_INSTR;
    const int rr = (xmine[j] ? ji : 0) * 8 + lr;  // row of the x tile
    const T* base = X;                             // rows >= n read row 0, unused
    if (rr < a.n) {
      base = X + (size_t)rr * a.d_in;
      if (a.rot_pos) {
        const int rp = a.rot_pos[rr];
        if (rp >= 0) base = XR + (size_t)rp * a.d_in;
      }
    }
    xsrc[j] = base + kbeg + 8 * (lc ^ swz<2>(rr));
  }
  auto issue = [&](int st) {
    unsigned char* buf = ring + (size_t)(st % S) * STAGE;
#pragma unroll
    for (int j = 0; j < W_INSTR; ++j)
      __builtin_amdgcn_global_load_lds(
          (const void*)(wsrc[j] + 64 * st),
          (__attribute__((address_space(3))) void*)(buf + (size_t)(wave * W_INSTR + j) * 1024), 16, 0, 0);
#pragma unroll
    for (int j = 0; j < XJ; ++j)
      if (xmine[j])
        __builtin_amdgcn_global_load_lds(
            (const void*)(xsrc[j] + 64 * st),
            (__attribute__((address_space(3))) void*)(buf + (size_t)WROWS * 128 + (size_t)(wave * XJ + j) * 1024),
            16, 0, 0);
  };

  // LDS rows of this lane's fragments.
  const int i16 = lane & 15, g = lane >> 4;
  int arow[NB], brow[MB];
#pragma unroll
  for (int b = 0; b < NB; ++b) arow[b] = wave * 16 * NB + perm_col<NB>(i16, b);
#pragma unroll
  for (int m = 0; m < MB; ++m) brow[m] = 16 * m + i16;

  f32x4 acc[NB][MB];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int m = 0; m < MB; ++m) acc[b][m] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int st = 0; st < S - 1; ++st)
    if (st < nst) issue(st);
  for (int it = 0; it < per; ++it) {
    // This wave's loads of slice `it` are done once no more than (slices
    // issued after it) x W_INSTR are outstanding (a wave issues at least
    // W_INSTR per slice; loads complete in order); every wave's, after the
    // barrier.  A group past its run only meets the barrier.
    const int younger = min(S - 2, nst - 1 - it);
    __builtin_amdgcn_sched_barrier(0);
    if (younger >= 1)
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(W_INSTR));
    else
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    if (it >= nst) continue;
    if (it + S - 1 < nst) issue(it + S - 1);
    const unsigned char* buf = ring + (size_t)(it % S) * STAGE;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int q = 4 * kk + g;  // 16-byte chunk of the row: k = 8q .. 8q + 7
      Vt af[NB], bf[MB];
#pragma unroll
      for (int b = 0; b < NB; ++b)
        af[b] = *reinterpret_cast<const Vt*>(buf + arow[b] * 128 + 16 * (q ^ swz<SHW>(arow[b])));
#pragma unroll
      for (int m = 0; m < MB; ++m)
        bf[m] = *reinterpret_cast<const Vt*>(buf + WROWS * 128 + brow[m] * 128 + 16 * (q ^ swz<2>(brow[m])));
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int m = 0; m < MB; ++m) acc[b][m] = mma(acc[b][m], af[b], bf[m]);
    }
  }

  if (G > 1) {
    // Groups 1.. leave their sums in LDS (over the rings, now idle); group 0
    // adds them in group order.
    f32x4* red = reinterpret_cast<f32x4*>(smem);
    __syncthreads();
    if (grp > 0) {
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int m = 0; m < MB; ++m) red[(((grp - 1) * 4 + wave) * NB * MB + b * MB + m) * 64 + lane] = acc[b][m];
    }
    __syncthreads();
    if (!EPI && grp > 0) return;  // with the fused epilogue every wave stays for its barriers
    if (grp == 0) {
#pragma unroll
      for (int q = 1; q < G; ++q)
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int m = 0; m < MB; ++m)
            acc[b][m] += red[(((q - 1) * 4 + wave) * NB * MB + b * MB + m) * 64 + lane];
    }
  }
  if constexpr (EPI) {
    static_assert(epi_ring_bytes(MB, NB, G) <= (size_t)G * S * STAGE,
                  "the epilogue's h and e fit in the rings beside the k-groups' sums");
    stream_epilogue<T, MB, NB, G>(t.s[si], acc, ks, local % col_tiles, col0, smem, smem + (size_t)G * S * STAGE,
                                  grp, wave, lane);
    return;
  }

  // The lane holds columns col0 + 16·NB·wave + 4·NB·g + [0, 4·NB) of row
  // 16m + i16: fp32 partials when k is split, else h in the layer type.
#pragma unroll
  for (int m = 0; m < MB; ++m) {
    const int row = 16 * m + i16;
    if (row >= a.n) continue;
    const size_t col = (size_t)col0 + 16 * NB * wave + 4 * NB * g;
    if (a.split == 1 && !a.h_fp32) {
      typedef T T4 __attribute__((ext_vector_type(4)));
      T* dst = static_cast<T*>(a.out) + (size_t)row * a.d_out + col;
#pragma unroll
      for (int b = 0; b < NB; ++b)
        *reinterpret_cast<T4*>(dst + 4 * b) =
            T4{to_t<T>(acc[b][m][0]), to_t<T>(acc[b][m][1]), to_t<T>(acc[b][m][2]), to_t<T>(acc[b][m][3])};
    } else {
      float* dst = a.part + ((size_t)ks * a.n + row) * a.d_out + col;
#pragma unroll
      for (int b = 0; b < NB; ++b) *reinterpret_cast<f32x4*>(dst + 4 * b) = acc[b][m];
    }
  }
}

// --------------------------------------------------------------- tiled ----

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
    if (a.split == 1 && !a.h_fp32) {
      store_run16<T>(static_cast<T*>(a.out) + (size_t)row * a.d_out + col, v);
    } else {
      store_run16<float>(a.part + ((size_t)ks * a.n + row) * a.d_out + col, v);
    }
  }
}

// ---------------------------------------------------------------- wide ----
//
// Base GEMM for n > 64 rows, f16/bf16, where MFMA throughput rather than the
// single read of W sets the time.  Work-group = one tile of 128 rows of x by
// 128 output columns by one k range, 12 waves: the k loop of wide_impl.h
// (4 producer waves stream each 64-element slice of the tile's x and W rows
// into a ring of S 32 KB LDS buffers by direct loads; two groups of 4 waves,
// each wave 64 x 64 as 4 x 4 MFMA tiles, take the two 32-element halves of
// every slice one phase apart), then each of those waves stores two 16-row
// blocks of its 64 x 64 block.  One work-group per CU
// (12 waves and 128 KB of LDS at S = 4).  Tiles are handed to work-groups so
// that each XCD (work-group i runs on XCD i % 8) takes a contiguous run of
// the tile order below: the slices of x and W its CUs read together stay in
// its L2.  Work-groups past the tiles (first split only) run the shrink's
// split reduction, which needs nothing from the GEMM: it fills the room a CU
// has beside its tile instead of a launch of its own.
template <typename T, int S>
__global__ __launch_bounds__(wide_impl::THREADS) void gemm_wide_kernel(GemmSlice sl, int row_tiles, int col_tiles) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const BaseGemmArgs& a = sl.g;
  const wide_impl::Role ro = wide_impl::role();
  const int ntile = row_tiles * col_tiles;
  if ((int)blockIdx.x >= ntile) {
    if (blockIdx.y == 0)
      shrink_impl::shrink_reduce_item<T>(sl.side, ((int)blockIdx.x - ntile) * wide_impl::THREADS + (int)threadIdx.x);
    return;
  }
  int t = (int)blockIdx.x;
  if (ntile % 8 == 0) t = (t % 8) * (ntile / 8) + t / 8;
  // Tile order: strips of 8 row tiles, column by column, so the ~32 tiles
  // an XCD runs at once form an 8 x 4 block reading 8 slices of x and 4 of
  // W (each used 4 or 8 times from L2), not a column of every row tile.
  const int strip = 8 * col_tiles;
  const int r_first = (t / strip) * 8, r_rows = min(8, row_tiles - r_first);
  const int rt = r_first + (t % strip) % r_rows, ct = (t % strip) / r_rows;
  const int row0 = rt * 128, col0 = ct * 128;
  const int ks = blockIdx.y;
  const int kbeg = ks * a.kc;
  const int nst = max(0, min(a.d_in - kbeg, a.kc)) / 64;

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
        const int i = row0 + r;
        base = X;  // rows past n read row 0; their results are not stored
        if (i < a.n) {
          base = X + (size_t)i * a.d_in;
          if (a.rot_pos) {
            const int rp = a.rot_pos[i];
            if (rp >= 0) base = XR + (size_t)rp * a.d_in;
          }
        }
      } else {
        base = W + (size_t)(col0 + r - 128) * a.d_in;
      }
      src[j] = base + kbeg + wide_impl::producer_chunk_elems(ro, r);
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

  // Lane holds, for row block 2 grp + mm, 16 consecutive output columns.
#pragma unroll
  for (int mm = 0; mm < 2; ++mm) {
    const int row = row0 + 64 * ro.wr + 16 * (2 * ro.grp + mm) + ro.i16;
    if (row >= a.n) continue;
    const int col = col0 + 64 * ro.wc + 16 * ro.g;
    float v[16];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const f32x4 h4 = acc[b][mm];
#pragma unroll
      for (int q = 0; q < 4; ++q) v[4 * b + q] = h4[q];
    }
    if (a.split == 1 && !a.h_fp32)
      store_run16<T>(static_cast<T*>(a.out) + (size_t)row * a.d_out + col, v);
    else
      store_run16<float>(a.part + ((size_t)ks * a.n + row) * a.d_out + col, v);
  }
}

// ----------------------------------------------------------------- big ----
//
// The same direct-load GEMM with 256 x 256 tiles, for batches large enough
// to give every CU a tile.  Work-group = 8 waves; wave (wr, wc) computes 128
// rows of x by 64 output columns (8 x 4 MFMA tiles, 128 fp32 accumulators
// per lane).  Per 64-element k slice the tile's 256 x rows and 256 W rows
// (64 KB) go straight into one of two LDS buffers (8 loads per wave).  Per
// 32-element k step a wave reads 12 fragments from LDS for 32 MFMAs, and
// the slices' trip from L2 into LDS is 32 B per clock at the MFMA rate
// instead of the 128 x 128 tile's 64.  The two waves of a SIMD work one
// phase apart (below), so one reads fragments while the other multiplies:
// a wave alone reads LDS at about 21 B per clock, its 12 KB per step take
// about as long as its 32 MFMAs.  Tile order, split partials and the
// shrink's reduction in extra work-groups as in the 128 x 128 kernel.
template <typename T>
__global__ __launch_bounds__(512) void gemm_big_kernel(Slices<GemmSlice> ts) {
  typedef typename Frag<T>::V Vt;
  constexpr int S = 2;
  constexpr int STAGE = 512 * 128;  // 256 x rows + 256 W rows, 128 B each
  constexpr int LI = 8;             // loads per wave per slice
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  // Several projections of one input (gate and up) may share the launch:
  // work-group ranges per projection, each its tiles then its side work.
  const int si = slice_of(ts, (int)blockIdx.x);
  const GemmSlice& sl = ts.s[si];
  const int local = (int)blockIdx.x - ts.first[si];
  const BaseGemmArgs& a = sl.g;
  const int row_tiles = (a.n + 255) / 256, col_tiles = a.d_out / 256;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i16 = lane & 15, g = lane >> 4;
  const int wr = wave & 1, wc = wave >> 1;
  const int grp = wave >> 2;
  const int ntile = row_tiles * col_tiles;
  if (local >= ntile) {
    if (blockIdx.y == 0) shrink_impl::shrink_reduce_item<T>(sl.side, (local - ntile) * 512 + tid);
    return;
  }
  int t = local;
  if (ntile % 8 == 0) t = (t % 8) * (ntile / 8) + t / 8;
  const int strip = 8 * col_tiles;
  const int r_first = (t / strip) * 8, r_rows = min(8, row_tiles - r_first);
  const int rt = r_first + (t % strip) % r_rows, ct = (t % strip) / r_rows;
  const int row0 = rt * 256, col0 = ct * 256;
  const int ks = blockIdx.y;
  const int kbeg = ks * a.kc;
  const int nst = max(0, min(a.d_in - kbeg, a.kc)) / 64;
  const T* X = static_cast<const T*>(a.x);
  const T* XR = static_cast<const T*>(a.x_rot);
  const T* W = static_cast<const T*>(a.W);

  // Instruction j < 4 loads x rows 32·wave + 8j .. +8 of the tile, j >= 4
  // W rows 32·wave + 8(j - 4) .. +8; lane = 8 · (row in the instruction) +
  // LDS chunk.
  const int lr = lane >> 3, lc = lane & 7;
  const T* src[LI];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = 32 * wave + 8 * j + lr;
    const int i = row0 + r;
    const T* base = X;  // rows past n read row 0; their results are not stored
    if (i < a.n) {
      base = X + (size_t)i * a.d_in;
      if (a.rot_pos) {
        const int rp = a.rot_pos[i];
        if (rp >= 0) base = XR + (size_t)rp * a.d_in;
      }
    }
    src[j] = base + kbeg + 8 * (lc ^ swz<2>(r));
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = 32 * wave + 8 * j + lr;
    src[4 + j] = W + (size_t)(col0 + r) * a.d_in + kbeg + 8 * (lc ^ swz<4>(r));
  }
  auto issue = [&](int st) {
    unsigned char* buf = smem + (size_t)(st % S) * STAGE;
#pragma unroll
    for (int j = 0; j < LI; ++j)
      __builtin_amdgcn_global_load_lds(
          (const void*)(src[j] + 64 * st),
          (__attribute__((address_space(3))) void*)(buf + (j < 4 ? 0 : 256 * 128) +
                                                    (size_t)(32 * wave + 8 * (j & 3)) * 128),
          16, 0, 0);
  };

  int arow[4], brow[8];
#pragma unroll
  for (int b = 0; b < 4; ++b) arow[b] = 64 * wc + perm_col<4>(i16, b);  // W rows (output columns)
#pragma unroll
  for (int m = 0; m < 8; ++m) brow[m] = 128 * wr + 16 * m + i16;         // x rows
  f32x4 acc[4][8];
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int m = 0; m < 8; ++m) acc[b][m] = f32x4{0.f, 0.f, 0.f, 0.f};
  Vt af[4], bf[8];
  auto R = [&](int st, int kk) {
    const unsigned char* buf = smem + (size_t)(st % S) * STAGE;
    const int q = 4 * kk + g;
#pragma unroll
    for (int b = 0; b < 4; ++b)
      af[b] = *reinterpret_cast<const Vt*>(buf + 256 * 128 + arow[b] * 128 + 16 * (q ^ swz<4>(arow[b])));
#pragma unroll
    for (int m = 0; m < 8; ++m) bf[m] = *reinterpret_cast<const Vt*>(buf + brow[m] * 128 + 16 * (q ^ swz<2>(brow[m])));
    __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  };
  auto M = [&]() {
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int m = 0; m < 8; ++m) acc[b][m] = mma(acc[b][m], af[b], bf[m]);
  };
  auto bar = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };

  // Ping-pong: waves 0..3 and 4..7 (one of each per SIMD) run one phase
  // apart, a phase being one k step's fragment reads or its 32 MFMAs, with a
  // barrier between phases; group 1 enters one barrier later and group 0
  // leaves through one more.  Each wave loads its share of slice it + 1 at
  // the start of its first read phase of slice it (every read of that
  // buffer, slice it - 1, is behind the barrier before it), and has it
  // landed before the barrier that precedes group 0's reads of slice it + 1.
  if (nst > 0) issue(0);
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  bar();
  if (grp == 1) bar();
  for (int it = 0; it < nst; ++it) {
    if (it + 1 < nst) issue(it + 1);
    R(it, 0);
    bar();
    M();
    bar();
    R(it, 1);
    if (grp == 1) __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    bar();
    M();
    if (grp == 0) __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    bar();
  }
  if (grp == 0) bar();

#pragma unroll
  for (int m = 0; m < 8; ++m) {
    const int row = row0 + 128 * wr + 16 * m + i16;
    if (row >= a.n) continue;
    const int col = col0 + 64 * wc + 16 * g;
    float v[16];
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int q = 0; q < 4; ++q) v[4 * b + q] = acc[b][m][q];
    if (a.split == 1 && !a.h_fp32)
      store_run16<T>(static_cast<T*>(a.out) + (size_t)row * a.d_out + col, v);
    else
      store_run16<float>(a.part + ((size_t)ks * a.n + row) * a.d_out + col, v);
  }
}

template <typename T, int G>
hipError_t skinny_dispatch(int nb, const GemmSlice* sl, int count, hipStream_t s) {
  const int mb = sl[0].g.n <= 16 ? 1 : sl[0].g.n <= 32 ? 2 : 4;
  Slices<GemmSlice> t{};
  t.count = count;
  t.first[0] = 0;
  size_t lds = 0;
  for (int i = 0; i < count; ++i) {
    const BaseGemmArgs& a = sl[i].g;
    t.s[i] = sl[i];
    const int n_gemm = (a.d_out / (64 * nb)) * a.split;
    const int n_side = side_workgroups(sl[i], 256 * G);
    t.first[i + 1] = t.first[i] + n_gemm + n_side;
    const size_t stage = (size_t)16 * mb * (a.kc + 16 / sizeof(T)) * sizeof(T);
    const size_t red = G > 1 ? (size_t)4 * nb * mb * 64 * 16 : 0;
    lds = std::max(lds, std::max(stage, red));
  }
  for (int i = count; i < MAX_SLICES; ++i) t.first[i + 1] = t.first[count];
  const dim3 grid((unsigned)t.first[count]);
#define TPA_SK(MBV, NBV)                                                                    \
  if (mb == MBV && nb == NBV) {                                                            \
    hipLaunchKernelGGL((gemm_skinny_kernel<T, MBV, NBV, G>), grid, dim3(256 * G), lds, s, t); \
    return hipGetLastError();                                                              \
  }
  TPA_SK(1, 1) TPA_SK(2, 1) TPA_SK(4, 1)
  TPA_SK(1, 2) TPA_SK(2, 2) TPA_SK(4, 2)
  TPA_SK(1, 4) TPA_SK(2, 4) TPA_SK(4, 4)
#undef TPA_SK
  return hipErrorInvalidValue;
}

template <typename T, int MB, int NB, int G, int S>
hipError_t stream_launch(const Slices<GemmSlice>& t, hipStream_t s, size_t epi_bytes) {
  constexpr size_t lds = (size_t)G * S * stream_stage_bytes<MB, NB>();
  if constexpr (lds > GEMM_STREAM_MAX_LDS) {
    return hipErrorInvalidValue;
  } else {
    if (epi_bytes) {
      if constexpr (S == 3 && MB <= 4 && epi_ring_bytes(MB, NB, G) <= lds) {
        if (lds + epi_bytes > GEMM_STREAM_MAX_LDS) return hipErrorInvalidValue;
        hipLaunchKernelGGL((gemm_stream_kernel<T, MB, NB, G, S, true>), dim3((unsigned)t.first[t.count]),
                           dim3(256 * G), lds + epi_bytes, s, t);
        return hipGetLastError();
      } else {
        return hipErrorInvalidValue;
      }
    }
    hipLaunchKernelGGL((gemm_stream_kernel<T, MB, NB, G, S, false>), dim3((unsigned)t.first[t.count]), dim3(256 * G),
                       lds, s, t);
    return hipGetLastError();
  }
}

// 16-row blocks of x per work-group of the streamed GEMM for n rows.
int stream_mb(int n) { return n <= 16 ? 1 : n <= 32 ? 2 : n <= 64 ? 4 : n <= 128 ? 8 : 16; }

template <typename T, int G, int S>
hipError_t stream_dispatch(int nb, const GemmSlice* sl, int count, hipStream_t s, size_t epi_bytes) {
  const int mb = stream_mb(sl[0].g.n);
  Slices<GemmSlice> t{};
  t.count = count;
  t.first[0] = 0;
  for (int i = 0; i < count; ++i) {
    const BaseGemmArgs& a = sl[i].g;
    t.s[i] = sl[i];
    const int n_gemm = (a.d_out / (64 * nb)) * a.split;
    const int n_side = side_workgroups(sl[i], 256 * G);
    t.first[i + 1] = t.first[i] + n_gemm + n_side;
  }
  for (int i = count; i < MAX_SLICES; ++i) t.first[i + 1] = t.first[count];
#define TPA_ST(MBV, NBV) \
  if (mb == MBV && nb == NBV) return stream_launch<T, MBV, NBV, G, S>(t, s, epi_bytes);
  TPA_ST(1, 1) TPA_ST(2, 1) TPA_ST(4, 1) TPA_ST(8, 1) TPA_ST(16, 1)
  TPA_ST(1, 2) TPA_ST(2, 2) TPA_ST(4, 2) TPA_ST(8, 2) TPA_ST(16, 2)
  TPA_ST(1, 4) TPA_ST(2, 4) TPA_ST(4, 4)
#undef TPA_ST
  return hipErrorInvalidValue;
}

template <typename T>
hipError_t stream_dtype(int nb, int groups, int stages, const GemmSlice* sl, int count, hipStream_t s,
                        size_t epi_bytes) {
  if (groups == 1 && stages == 3) return stream_dispatch<T, 1, 3>(nb, sl, count, s, epi_bytes);
  if (groups == 1 && stages == 4) return stream_dispatch<T, 1, 4>(nb, sl, count, s, epi_bytes);
  if (groups == 1 && stages == 6) return stream_dispatch<T, 1, 6>(nb, sl, count, s, epi_bytes);
  if (groups == 2 && stages == 3) return stream_dispatch<T, 2, 3>(nb, sl, count, s, epi_bytes);
  return hipErrorInvalidValue;
}

}  // namespace

size_t gemm_skinny_lds(int dtype, int n, int nb, int groups, int kc) {
  const int mb = n <= 16 ? 1 : n <= 32 ? 2 : 4;
  const size_t esz = dtype == 0 ? 4 : 2;
  const size_t stage = (size_t)16 * mb * (kc + 16 / esz) * esz;
  const size_t red = groups > 1 ? (size_t)4 * nb * mb * 64 * 16 : 0;
  return stage > red ? stage : red;
}

hipError_t launch_gemm_skinny(int dtype, int nb, int groups, const GemmSlice* slices, int count, hipStream_t s) {
  if (count < 1 || count > MAX_SLICES) return hipErrorInvalidValue;
  for (int i = 0; i < count; ++i) {
    const BaseGemmArgs& a = slices[i].g;
    if (a.n <= 0 || a.n > 64 || a.n != slices[0].g.n || a.kc % 64 || a.d_out % (64 * nb) || slices[i].side_whole)
      return hipErrorInvalidValue;
    if (gemm_skinny_lds(dtype, a.n, nb, dtype == 0 ? 1 : groups, a.kc) > GEMM_SKINNY_MAX_LDS)
      return hipErrorInvalidValue;
  }
  if (dtype == 0) return skinny_dispatch<float, 1>(nb, slices, count, s);
  if (dtype == 1)
    return groups == 1 ? skinny_dispatch<f16, 1>(nb, slices, count, s) : skinny_dispatch<f16, 2>(nb, slices, count, s);
  if (dtype == 2)
    return groups == 1 ? skinny_dispatch<bf16, 1>(nb, slices, count, s)
                       : skinny_dispatch<bf16, 2>(nb, slices, count, s);
  return hipErrorInvalidValue;
}

size_t gemm_stream_lds(int n, int nb, int groups, int stages) {
  const int mb = stream_mb(n);
  return (size_t)groups * stages * (64 * nb + 16 * mb) * 128;
}

size_t gemm_stream_epi_lds(int n, int max_tiles, int steps) {
  return (size_t)epi_lds_layout(16 * stream_mb(n), max_tiles, steps).end;
}

bool gemm_stream_epi_ok(int n, int nb, int groups, int stages) {
  const int mb = stream_mb(n);
  return n <= 64 && stages == 3 && epi_ring_bytes(mb, nb, groups) <= gemm_stream_lds(n, nb, groups, stages);
}

hipError_t launch_gemm_stream(int dtype, int nb, int groups, int stages, const GemmSlice* slices, int count,
                              hipStream_t s, bool epi) {
  if (count < 1 || count > MAX_SLICES || (nb != 1 && nb != 2 && nb != 4)) return hipErrorInvalidValue;
  size_t epi_bytes = 0;
  for (int i = 0; i < count; ++i) {
    const BaseGemmArgs& a = slices[i].g;
    // Whole 64-element slices in every k range, whole column tiles, rows
    // 64-byte aligned for the 16-byte loads.
    if (a.n <= 0 || a.n > 256 || a.n != slices[0].g.n || a.kc <= 0 || a.kc % 64 || a.d_in % 64 ||
        a.d_out % (64 * nb) || (long)a.split * a.kc < a.d_in)
      return hipErrorInvalidValue;
    // Whole-k shrink items in the side work-groups: one k range per wave
    // of a work-group, covering d_in; not beside the fused epilogue.
    const ShrinkArgs& sh = slices[i].side;
    if (slices[i].has_side && slices[i].side_whole &&
        (epi || sh.split < 1 || sh.split > 4 * groups || sh.kc <= 0 || sh.kc % 32 || (long)sh.split * sh.kc < sh.d_in))
      return hipErrorInvalidValue;
    if (epi) {
      // The epilogue's tables: every row, every entry of the tile list (one
      // thread each) and the k steps of the largest factor per entry.
      const ExpandArgs& e = slices[i].e;
      if (!gemm_stream_epi_ok(a.n, nb, groups, stages) || slices[i].has_side || !slices[i].pinfo || !e.out || !e.tiles ||
          !e.slots || !e.apply_scale || e.n != a.n || e.d_out != a.d_out || e.max_tiles < 0 ||
          e.max_tiles > 256 * groups || (a.split > 1 && (!slices[i].cnt || !a.part)))
        return hipErrorInvalidValue;
      const int kcap = std::max(e.kmax, e.r_v);
      if (kcap > 32 * 255) return hipErrorInvalidValue;  // a step names its k step in 8 bits
      epi_bytes = std::max(epi_bytes, gemm_stream_epi_lds(a.n, e.max_tiles, e.max_tiles * ((kcap + 31) / 32)));
    }
  }
  if (gemm_stream_lds(slices[0].g.n, nb, groups, stages) + epi_bytes > GEMM_STREAM_MAX_LDS)
    return hipErrorInvalidValue;
  if (dtype == 1) return stream_dtype<f16>(nb, groups, stages, slices, count, s, epi_bytes);
  if (dtype == 2) return stream_dtype<bf16>(nb, groups, stages, slices, count, s, epi_bytes);
  return hipErrorInvalidValue;
}

hipError_t launch_gemm_wide(int dtype, int stages, const GemmSlice& sl, hipStream_t s) {
  const BaseGemmArgs& a = sl.g;
  if (a.n <= 0 || a.d_out % 128 || a.d_in % 64 || a.kc <= 0 || a.kc % 64 || (long)a.split * a.kc < a.d_in ||
      sl.side_whole)
    return hipErrorInvalidValue;
  if (stages < 2 || stages > 5 || (dtype != 1 && dtype != 2)) return hipErrorInvalidValue;
  const int row_tiles = (a.n + 127) / 128, col_tiles = a.d_out / 128;
  const dim3 grid((unsigned)(row_tiles * col_tiles + side_workgroups(sl, wide_impl::THREADS)), (unsigned)a.split);
  const dim3 block(wide_impl::THREADS);
  const size_t lds = (size_t)stages * wide_impl::STAGE;
#define TPA_WIDE(SV)                                                                                      \
  if (stages == SV) {                                                                                     \
    if (dtype == 1)                                                                                       \
      hipLaunchKernelGGL((gemm_wide_kernel<f16, SV>), grid, block, lds, s, sl, row_tiles, col_tiles);     \
    else                                                                                                  \
      hipLaunchKernelGGL((gemm_wide_kernel<bf16, SV>), grid, block, lds, s, sl, row_tiles, col_tiles);    \
  }
  TPA_WIDE(2) TPA_WIDE(3) TPA_WIDE(4) TPA_WIDE(5)
#undef TPA_WIDE
  return hipGetLastError();
}

hipError_t launch_gemm_big(int dtype, const GemmSlice* slices, int count, hipStream_t s) {
  if (count < 1 || count > MAX_SLICES || (dtype != 1 && dtype != 2)) return hipErrorInvalidValue;
  Slices<GemmSlice> t{};
  t.count = count;
  t.first[0] = 0;
  for (int i = 0; i < count; ++i) {
    const BaseGemmArgs& a = slices[i].g;
    if (a.n <= 0 || a.n != slices[0].g.n || a.d_out % 256 || a.d_in % 64 || a.kc <= 0 || a.kc % 64 ||
        (long)a.split * a.kc < a.d_in || a.split != slices[0].g.split || slices[i].side_whole)
      return hipErrorInvalidValue;
    t.s[i] = slices[i];
    // Each projection's range starts on a multiple of 8 work-groups, so its
    // tile order keeps the XCD mapping (work-group i runs on XCD i % 8).
    const int n_wg = ((a.n + 255) / 256) * (a.d_out / 256) + side_workgroups(slices[i], 512);
    t.first[i + 1] = t.first[i] + (i + 1 < count ? (n_wg + 7) / 8 * 8 : n_wg);
  }
  for (int i = count; i < MAX_SLICES; ++i) t.first[i + 1] = t.first[count];
  const dim3 grid((unsigned)t.first[count], (unsigned)slices[0].g.split);
  const size_t lds = (size_t)2 * 512 * 128;
  if (dtype == 1)
    hipLaunchKernelGGL((gemm_big_kernel<f16>), grid, dim3(512), lds, s, t);
  else
    hipLaunchKernelGGL((gemm_big_kernel<bf16>), grid, dim3(512), lds, s, t);
  return hipGetLastError();
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

}  // namespace tpa
