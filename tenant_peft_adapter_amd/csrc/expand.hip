// The expand: one pass over every output tile that finishes the layer.
//
// Scute paper (arXiv 2611.01089):
//   * §2 "The LoRA schedule": the expand reads h, adds V B and writes the
//     result, one tile of rows (one segment) at a time.
//   * §4.1 route one and §5.2: the output scale s is applied inside the
//     expand as each tile finishes, so a live s costs one extra read of the
//     adapter's vector per tile (the shift b rides along the same way).
//   * §4.1 route two, second GEMM: for VeRA rows, U · B_v over tiles of rows
//     whatever their tenant, each row multiplied by its tenant's e before it
//     is added; B_v is read once per tile, not once per tenant.
//
// Work-group = one wave = one plan tile (up to 16·MB rows in plan order) x
// 64 output columns.  The term is an MFMA product of the factor stored
// [d_out][rank] (a operand: output columns) with the tile's V (or U) rows
// as the shrink left them ([n][kmax], layer type), computed transposed so
// each lane holds 16 consecutive output columns of one row.  The epilogue
// reads h (from `out`, or summed from the base GEMM's split partials in a
// fixed order), applies s and b of the row's slot, adds the term (times e
// for shared-term rows) and writes the row segment once.
#include "internal.h"

namespace tpa {

namespace {

constexpr int THREADS = 256;

// h of one row segment of 16 columns: the split partials added in split
// order, their loads issued 4 splits (16 loads) at a time.  TAIL: the last
// group short of 4 too (2 splits: one round trip, not two; 7: two, not
// four); else the splits past the last full group one at a time, which
// needs fewer registers.
template <bool TAIL>
__device__ __forceinline__ void sum_parts16(const float* hpart, int hsplit, size_t split_stride,
                                            float* v) {
#pragma unroll
  for (int j = 0; j < 16; ++j) v[j] = 0.f;
  int s = 0;
  for (; TAIL ? s < hsplit : s + 4 <= hsplit; s += 4) {
    f32x4 x[4][4];  // (entries past the last split are neither loaded nor added)
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (s + u < hsplit)
#pragma unroll
        for (int q = 0; q < 4; ++q) x[u][q] = gload<f32x4>(hpart + (size_t)(s + u) * split_stride + 4 * q);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (s + u >= hsplit) break;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        v[4 * q] += x[u][q][0];
        v[4 * q + 1] += x[u][q][1];
        v[4 * q + 2] += x[u][q][2];
        v[4 * q + 3] += x[u][q][3];
      }
    }
  }
  for (; s < hsplit; ++s) {
    const float* src = hpart + (size_t)s * split_stride;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      f32x4 x = gload<f32x4>(src + 4 * q);
      v[4 * q] += x[0];
      v[4 * q + 1] += x[1];
      v[4 * q + 2] += x[2];
      v[4 * q + 3] += x[3];
    }
  }
}

// h of one row segment of 8 columns: the split partials added in split
// order, 4 splits (8 loads) at a time, the last group short of 4 included.
__device__ __forceinline__ void sum_parts8(const float* hpart, int hsplit, size_t split_stride, float* v) {
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = 0.f;
  for (int s = 0; s < hsplit; s += 4) {
    f32x4 x[4][2];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (s + u < hsplit)
#pragma unroll
        for (int q = 0; q < 2; ++q) x[u][q] = gload<f32x4>(hpart + (size_t)(s + u) * split_stride + 4 * q);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (s + u >= hsplit) break;
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        v[4 * q] += x[u][q][0];
        v[4 * q + 1] += x[u][q][1];
        v[4 * q + 2] += x[u][q][2];
        v[4 * q + 3] += x[u][q][3];
      }
    }
  }
}

// A shared-term tile at decode sizes (16-bit types, 16-row tiles): work-
// group = one wave = the tile x 32 output columns, so that the term's whole
// rank (up to 8 k steps of 32: VeRA's 256) loads in one round trip, where
// 64 columns take two (their fragments would need twice the registers).
// The same products and sums as the 64-column wave, in the same order; lane
// holds 8 consecutive columns of one row.
template <typename T, bool HPART>
__device__ __forceinline__ void shared_tile32(const ExpandArgs& a, int local, int lane) {
  typedef typename Frag<T>::V Vt;
  constexpr int U = 8;
  const int ncb = a.d_out / 32;
  const int i16 = lane & 15, g = lane >> 4;
  const int ti = local / ncb;
  const int n0 = (local % ncb) * 32;
  const int col = n0 + 8 * g;
  const int4 tl = *reinterpret_cast<const int4*>(a.tiles + 4 * ti);
  const int rw = a.tile_rows_w[(size_t)ti * 16 + i16];
  if (tl.z != CLS_SHARED) return;  // padding past the last shared-term tile
  const int row = rw >= 0 ? (rw & 0xFFFF) : -1;
  const SlotDev* rsd = a.slots + (rw >= 0 ? (rw >> 16) : 0);
  const int K = a.r_v;
  const float* sp = nullptr;
  const float* bq = nullptr;
  const float* ep = nullptr;
  if (row >= 0) {
    if (a.apply_scale) {
      sp = gload<const float*>(&rsd->s);
      bq = gload<const float*>(&rsd->b);
    }
    ep = gload<const float*>(&rsd->e);
  }
  // term = U[p] · B_vᵀ over the 32 columns: a = B_v rows (output columns),
  // b = the tile's U rows.
  const T* bp[2];
#pragma unroll
  for (int b = 0; b < 2; ++b)
    bp[b] = static_cast<const T*>(a.vera_Bt) + (size_t)(n0 + perm_col<2>(i16, b)) * K + 8 * g;
  const bool vv = rw >= 0;
  const T* vp = static_cast<const T*>(a.v) + (size_t)(vv ? tl.x + i16 : 0) * a.kmax + 8 * g;
  f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
  for (int k = 0; k < K; k += 32 * U) {
    Vt af[U][2], bf[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kk = k + 32 * u;
      const bool ok = kk + 8 * g < K;
#pragma unroll
      for (int b = 0; b < 2; ++b) af[u][b] = ok ? load_frag<T>(bp[b] + kk) : zero_frag<T>();
      bf[u] = (ok && vv) ? load_frag<T>(vp + kk) : zero_frag<T>();
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (k + 32 * u >= K) break;
#pragma unroll
      for (int b = 0; b < 2; ++b) acc[b] = mma(acc[b], af[u][b], bf[u]);
    }
  }
  if (row < 0) return;
  T* out = static_cast<T*>(a.out);
  float v[8];
  if (HPART) {
    sum_parts8(a.hpart + (size_t)row * a.d_out + col, a.hsplit, (size_t)a.n * a.d_out, v);
  } else {
    const Vt h8 = *reinterpret_cast<const Vt*>(out + (size_t)row * a.d_out + col);
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = to_f<T>(h8[j]);
  }
  f32x4 s4[2], b4[2], e4[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    s4[q] = sp ? gload<f32x4>(sp + col + 4 * q) : f32x4{1.f, 1.f, 1.f, 1.f};
    b4[q] = bq ? gload<f32x4>(bq + col + 4 * q) : f32x4{0.f, 0.f, 0.f, 0.f};
    e4[q] = ep ? gload<f32x4>(ep + col + 4 * q) : f32x4{1.f, 1.f, 1.f, 1.f};
  }
  // (written as the 64-column wave writes it: h rounded to fp32, then to
  // the layer type.  With the term added unconditionally the compiler fuses
  // the last multiply-add and the conversion into one mixed-precision FMA,
  // a single rounding, and the result differs from the other waves' in the
  // last place now and then.)
  Vt o8;
#pragma unroll
  for (int q = 0; q < 2; ++q)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float h = v[4 * q + j] * s4[q][j] + b4[q][j];
      if (K > 0) h += acc[q][j] * e4[q][j];
      o8[4 * q + j] = to_t<T>(h);
    }
  *reinterpret_cast<Vt*>(out + (size_t)row * a.d_out + col) = o8;
}

// Up to two ranges per projection: its shared-term tiles, then the rest.
typedef Slices<ExpandArgs, 2 * MAX_SLICES> ExpandSlices;

// FEW (16-bit types, 16-row tiles, above 256 rows): two k steps of loads in
// flight instead of four, h and s loaded before the term at any rank, the
// split partials past the last full group of four one at a time: about 128
// registers, four waves per SIMD (2-layer cut of the 1024-tenant Zipf stack
// against four k steps at 158 registers: 1024 rows 1211 -> 1198 µs per
// layer, 4096 rows 2876 -> 2847).  At decode sizes (!FEW) a long term runs
// first, four k steps at a time (two steps per round trip made a rank-256
// VeRA tile's chain longer: decoder layer 203.7 -> 206.2 µs per step), and a
// short one loads one step's fragments; with the occupancy hint that is
// 119 registers, four waves per SIMD as well.

template <typename T, int MB, bool HPART, bool FEW>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(MB == 1 && !FEW ? 3 : 1))) void expand_kernel(
    ExpandSlices t) {
  typedef typename Frag<T>::V Vt;
  // k steps whose loads are issued together (fewer for wide fragments)
  constexpr int U = sizeof(T) == 4 ? (MB == 1 ? 2 : 1) : (MB == 1 && !FEW ? 4 : 2);
  const int si = slice_of(t, (int)blockIdx.x);
  const ExpandArgs& a = t.s[si];
  const int local = (int)blockIdx.x - t.first[si];
  if constexpr (sizeof(T) == 2 && MB == 1 && !FEW) {
    if (a.part == 1) {
      shared_tile32<T, HPART>(a, local, (int)threadIdx.x);
      return;
    }
  }
  const int ncb = a.d_out / 64;
  const int lane = threadIdx.x;
  const int i16 = lane & 15, g = lane >> 4;
  // Tile header and the rows' words load side by side.
  const int ti = local / ncb;
  const int4 tl = *reinterpret_cast<const int4*>(a.tiles + 4 * ti);
  int rw[MB];
#pragma unroll
  for (int m = 0; m < MB; ++m) rw[m] = a.tile_rows_w[(size_t)ti * 16 * MB + 16 * m + i16];
  const int p0 = tl.x, kind = tl.z;
  if (kind < 0) return;  // padding past the plan's last tile
  if (a.part == 2 && kind == CLS_SHARED) return;  // done in the projection's first range
  const int n0 = (local % ncb) * 64;
  const int col = n0 + 16 * g;

  // Row and slot of each of this lane's positions, and the slot record that
  // carries s, b and e (a tile of owned-term rows has one slot).
  int row[MB];
  const SlotDev* rsd[MB];
#pragma unroll
  for (int m = 0; m < MB; ++m) {
    row[m] = rw[m] >= 0 ? (rw[m] & 0xFFFF) : -1;
    rsd[m] = a.slots + (kind == CLS_OWNED ? tl.w : rw[m] >= 0 ? (rw[m] >> 16) : 0);
  }

  // The term's factor (stored [d_out][K]) and rank: kernel arguments for a
  // shared-term tile; an owned tile's come from its slot's record, read
  // beside the rows' pointers.
  int K = 0;
  const T* Bt = nullptr;
  if (kind == CLS_OWNED) {
    K = a.slots[tl.w].rank;
    Bt = static_cast<const T*>(a.slots[tl.w].Bt);
  } else if (kind == CLS_SHARED) {
    K = a.r_v;
    Bt = static_cast<const T*>(a.vera_Bt);
  }
  // The rows' s, b and e pointers.
  const float* sp[MB];
  const float* bq[MB];
  const float* ep[MB];
#pragma unroll
  for (int m = 0; m < MB; ++m) {
    sp[m] = nullptr;
    bq[m] = nullptr;
    ep[m] = nullptr;
    if (row[m] < 0) continue;
    if (a.apply_scale) {
      sp[m] = gload<const float*>(&rsd[m]->s);
      bq[m] = gload<const float*>(&rsd[m]->b);
    }
    if (kind == CLS_SHARED) ep[m] = gload<const float*>(&rsd[m]->e);
  }
  T* out = static_cast<T*>(a.out);
  float v[MB][16];
  f32x4 s4[MB][4], e4[MB][4];
  // h of each row (its split partials summed in order), then the rows' s
  // values (so that a tenant with a live s costs about what one without
  // does); b, rarer, loads in the epilogue.
  auto load_h_s = [&]() {
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      if (row[m] < 0) continue;
      if (HPART)
        sum_parts16<!FEW>(a.hpart + (size_t)row[m] * a.d_out + col, a.hsplit, (size_t)a.n * a.d_out, v[m]);
      else
        load_run16<T>(out + (size_t)row[m] * a.d_out + col, v[m]);
    }
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        s4[m][q] = (row[m] >= 0 && sp[m]) ? gload<f32x4>(sp[m] + col + 4 * q) : f32x4{1.f, 1.f, 1.f, 1.f};
  };
  auto load_e = [&]() {
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        e4[m][q] = (row[m] >= 0 && ep[m]) ? gload<f32x4>(ep[m] + col + 4 * q) : f32x4{1.f, 1.f, 1.f, 1.f};
  };

  // term = V[p] · B'ᵀ over this wave's 64 columns: a = B' rows (output
  // columns), b = V rows of the tile (plan positions).
  f32x4 acc[4][MB];
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int m = 0; m < MB; ++m) acc[b][m] = f32x4{0.f, 0.f, 0.f, 0.f};
  const T* V = static_cast<const T*>(a.v);
  const T* bp[4];
  const T* vp[MB];
  bool vv[MB];
  auto point = [&]() {
#pragma unroll
    for (int b = 0; b < 4; ++b) bp[b] = Bt + (size_t)(n0 + perm_col<4>(i16, b)) * K + 8 * g;
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      const int p = p0 + 16 * m + i16;
      vv[m] = rw[m] >= 0;
      vp[m] = V + (size_t)(vv[m] ? p : 0) * a.kmax + 8 * g;
    }
  };
  // At decode sizes (!FEW) a term of more than one k step (VeRA's shared
  // rank, owned ranks above 32) goes first: its loads need only the tile and
  // the factor, so the first U k steps go out beside the rows' pointers; h,
  // s and e load after it, when the fragments' registers are free again.
  // Its chain of round trips is the launch's longest, and few waves share
  // the chip with it.  Above 256 rows every tile takes h first (stack cut
  // at 4096 rows: 5472-5476 µs per step with h first, 5497-5505 with the
  // term first).
  const bool long_term = !FEW && K > 32;
  if (long_term) {
    point();
    for (int k = 0; k < K; k += 32 * U) {
      Vt af[U][4], bf[U][MB];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int kk = k + 32 * u;
        const bool ok = kk + 8 * g < K;
#pragma unroll
        for (int b = 0; b < 4; ++b) af[u][b] = ok ? load_frag<T>(bp[b] + kk) : zero_frag<T>();
#pragma unroll
        for (int m = 0; m < MB; ++m) bf[u][m] = (ok && vv[m]) ? load_frag<T>(vp[m] + kk) : zero_frag<T>();
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (k + 32 * u >= K) break;
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
          for (int m = 0; m < MB; ++m) acc[b][m] = mma(acc[b][m], af[u][b], bf[u][m]);
      }
    }
    load_h_s();
    load_e();
  } else {
    // h and s first, then the term's loads: at decode sizes no term or one
    // k step, one step's fragments; above 256 rows any rank, U steps at a
    // time.
    load_h_s();
    if (K > 0) {
      point();
      constexpr int U2 = FEW ? U : 1;
      for (int k = 0; k < K; k += 32 * U2) {
        Vt af[U2][4], bf[U2][MB];
#pragma unroll
        for (int u = 0; u < U2; ++u) {
          const int kk = k + 32 * u;
          const bool ok = kk + 8 * g < K;
#pragma unroll
          for (int b = 0; b < 4; ++b) af[u][b] = ok ? load_frag<T>(bp[b] + kk) : zero_frag<T>();
#pragma unroll
          for (int m = 0; m < MB; ++m) bf[u][m] = (ok && vv[m]) ? load_frag<T>(vp[m] + kk) : zero_frag<T>();
        }
#pragma unroll
        for (int u = 0; u < U2; ++u) {
          if (k + 32 * u >= K) break;
#pragma unroll
          for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int m = 0; m < MB; ++m) acc[b][m] = mma(acc[b][m], af[u][b], bf[u][m]);
        }
      }
    }
  }

  // Epilogue: lane holds 16 consecutive columns of one row of the tile.
  // h ⊙ s + b, plus the term (times e for a shared-term row).
#pragma unroll
  for (int m = 0; m < MB; ++m) {
    if (row[m] < 0) continue;
    f32x4 b4[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      b4[q] = bq[m] ? gload<f32x4>(bq[m] + col + 4 * q) : f32x4{0.f, 0.f, 0.f, 0.f};
      if (!long_term) e4[m][q] = ep[m] ? gload<f32x4>(ep[m] + col + 4 * q) : f32x4{1.f, 1.f, 1.f, 1.f};
    }
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float h = v[m][4 * q + j] * s4[m][q][j] + b4[q][j];
        if (K > 0) h += acc[q][m][j] * e4[m][q][j];
        v[m][4 * q + j] = h;
      }
    store_run16<T>(out + (size_t)row[m] * a.d_out + col, v[m]);
  }
}

// Separate scale passes (route comparison).  One thread per 16 columns;
// every vector moves in 16-byte loads and stores.
template <typename T>
__global__ __launch_bounds__(THREADS) void scale_pass_kernel(ScaleArgs a, int mode) {
  const size_t idx = (size_t)blockIdx.x * THREADS + threadIdx.x;
  const int runs = a.d_out / 16;
  if (idx >= (size_t)a.n * runs) return;
  const int row = (int)(idx / runs);
  const int col = 16 * (int)(idx % runs);
  const SlotDev& sd = a.slots[a.row_slot[row]];
  const float* sv = gload<const float*>(&sd.s);
  const float* bv = gload<const float*>(&sd.b);
  T* y = static_cast<T*>(a.y) + (size_t)row * a.d_out + col;
  float v[16], f[16];
  if (mode == 3) {  // index scale, step one: a per-row copy of the scale
    if (sv)
      load_run16<float>(sv + col, f);
    else
#pragma unroll
      for (int j = 0; j < 16; ++j) f[j] = 1.f;
    store_run16<float>(a.srow + (size_t)row * a.d_out + col, f);
    return;
  }
  if (mode == 1 && a.hpart)
    sum_parts16<false>(a.hpart + (size_t)row * a.d_out + col, a.hsplit, (size_t)a.n * a.d_out, v);
  else
    load_run16<T>(y, v);
  if (mode == 4) {  // index scale, step two: multiply by the per-row copy
    load_run16<float>(a.srow + (size_t)row * a.d_out + col, f);
#pragma unroll
    for (int j = 0; j < 16; ++j) v[j] *= f[j];
  } else if (sv) {
    load_run16<float>(sv + col, f);
#pragma unroll
    for (int j = 0; j < 16; ++j) v[j] *= f[j];
  }
  if (bv) {
    load_run16<float>(bv + col, f);
#pragma unroll
    for (int j = 0; j < 16; ++j) v[j] += f[j];
  }
  store_run16<T>(y, v);
}

template <typename T, int MB>
hipError_t expand_launch(const ExpandSlices& t, hipStream_t s) {
  const dim3 grid((unsigned)t.first[t.count]);
  const bool few = sizeof(T) == 2 && MB == 1 && t.s[0].n > 256;
  if (t.s[0].hpart) {
    if (few)
      hipLaunchKernelGGL((expand_kernel<T, MB, true, true>), grid, dim3(64), 0, s, t);
    else
      hipLaunchKernelGGL((expand_kernel<T, MB, true, false>), grid, dim3(64), 0, s, t);
  } else {
    if (few)
      hipLaunchKernelGGL((expand_kernel<T, MB, false, true>), grid, dim3(64), 0, s, t);
    else
      hipLaunchKernelGGL((expand_kernel<T, MB, false, false>), grid, dim3(64), 0, s, t);
  }
  return hipGetLastError();
}

template <typename T>
hipError_t expand_tm(int tile_rows, const ExpandSlices& t, hipStream_t s) {
  if (tile_rows == 16) return expand_launch<T, 1>(t, s);
  if (tile_rows == 64) return expand_launch<T, 4>(t, s);
  return hipErrorInvalidValue;
}

}  // namespace

// Work-groups are dispatched in index order.  At decode sizes a shared-term
// (VeRA) tile's rank-r_v product is the launch's longest chain of dependent
// loads, while most work-groups take owned tiles of a few rows; with the
// shared-term tiles first (their own ranges, from the plan's separate list)
// their chains start in the first wave of dispatch instead of behind every
// owned tile of the launch.  Each work-group's result is unchanged.
hipError_t launch_expand(int dtype, int tile_rows, const ExpandArgs* slices, int count, hipStream_t s) {
  if (count < 1 || count > MAX_SLICES) return hipErrorInvalidValue;
  ExpandSlices t{};
  int m = 0;
  bool sh_first[MAX_SLICES];
  for (int i = 0; i < count; ++i) {
    const ExpandArgs& a = slices[i];
    if ((a.hpart != nullptr) != (slices[0].hpart != nullptr) || a.d_out % 64) return hipErrorInvalidValue;
    sh_first[i] = a.n <= 64 && a.sh_tiles && a.sh_rows_w && a.max_sh_tiles > 0 && a.vera_Bt && a.r_v > 0;
    if (!sh_first[i]) continue;
    t.s[m] = a;
    t.s[m].tiles = a.sh_tiles;
    t.s[m].tile_rows_w = a.sh_rows_w;
    t.s[m].max_tiles = a.max_sh_tiles;
    t.s[m].part = 1;
    ++m;
  }
  for (int i = 0; i < count; ++i) {
    t.s[m] = slices[i];
    t.s[m].part = sh_first[i] ? 2 : 0;
    ++m;
  }
  t.count = m;
  t.first[0] = 0;
  // (a shared-term range of 16-bit types on 16-row tiles runs 32 columns
  // per work-group: shared_tile32)
  const bool narrow = dtype != 0 && tile_rows == 16;
  for (int i = 0; i < m; ++i)
    t.first[i + 1] = t.first[i] + t.s[i].max_tiles * (t.s[i].d_out / (t.s[i].part == 1 && narrow ? 32 : 64));
  for (int i = m; i < 2 * MAX_SLICES; ++i) t.first[i + 1] = t.first[m];
  switch (dtype) {
    case 0: return expand_tm<float>(tile_rows, t, s);
    case 1: return expand_tm<f16>(tile_rows, t, s);
    case 2: return expand_tm<bf16>(tile_rows, t, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_scale_pass(int dtype, int mode, const ScaleArgs& a, hipStream_t s) {
  const size_t work = (size_t)a.n * (a.d_out / 16);
  dim3 grid((unsigned)((work + THREADS - 1) / THREADS));
  switch (dtype) {
    case 0: hipLaunchKernelGGL(scale_pass_kernel<float>, grid, dim3(THREADS), 0, s, a, mode); break;
    case 1: hipLaunchKernelGGL(scale_pass_kernel<f16>, grid, dim3(THREADS), 0, s, a, mode); break;
    case 2: hipLaunchKernelGGL(scale_pass_kernel<bf16>, grid, dim3(THREADS), 0, s, a, mode); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace tpa
