// Internal interface between the C ABI (abi.cpp) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "common.h"

namespace tpa {

// ------------------------------------------------------------- slices ----
// One launch can cover up to MAX_SLICES projections of a fused layer (q, k,
// v; gate, up) that share one row plan: the kernel argument holds one record
// per slice and the work-group ranges [first[i], first[i + 1]) of each.
constexpr int MAX_SLICES = 4;
template <typename A, int N = MAX_SLICES>
struct Slices {
  A s[N];
  int32_t first[N + 1];
  int32_t count;
};
template <typename A, int N>
__device__ __forceinline__ int slice_of(const Slices<A, N>& t, int bid) {
  int i = 0;
#pragma unroll
  for (int j = 1; j < N; ++j)
    if (j < t.count && bid >= t.first[j]) i = j;
  return i;
}

// ---------------------------------------------------------------- plan ----
struct PlanArgs {
  const int32_t* slot_of_row;
  const SlotDev* slots;
  int32_t n;
  int32_t max_slots;
  int32_t tile_rows;
  int32_t* perm;       // [n]
  int32_t* row_slot;   // [n]
  int32_t* rot_pos;    // [n]
  int32_t* seg_ptr;    // [n + 1]
  int32_t* seg_slot;   // [n]
  int32_t* tiles;      // [4 * max_tiles]
  int32_t* oft_tiles;  // [4 * max_tiles]
  int32_t* counts;     // [CNT_WORDS]
  int32_t* flag;       // layer's sticky invalid-slot flag
  int32_t* pinfo;      // [n]: (slot << 16) | row of plan position p
  int32_t max_tiles;   // tile lists are padded to this length with kind / slot -1
  int32_t* sh_tiles;   // [4 * max_sh_tiles]: the shared-term tiles again, on their own
  int32_t max_sh_tiles;  // ceil(n / tile_rows); padded like tiles
  // Row words of each real tile of tiles / sh_tiles / oft_tiles: tile_rows
  // entries per tile, pinfo of position p0 + j, or -1 past p1 (padding
  // entries are left unwritten), so a kernel loads a tile's rows alongside
  // its header instead of after it.
  int32_t* tile_rows_w;      // [tile_rows * max_tiles]
  int32_t* sh_rows_w;        // [tile_rows * max_sh_tiles]
  int32_t* oft_rows_w;       // [tile_rows * max_tiles]
};
constexpr int PLAN_MAX_ROWS = 8192;
hipError_t launch_plan(const PlanArgs& a, hipStream_t stream);

// ---------------------------------------------------------- OFT rotate ----
struct OftArgs {
  const void* x;           // [n][d_in]
  const int32_t* oft_tiles;  // padded with slot -1 to max_tiles
  const int32_t* oft_rows_w; // row words per OFT tile (16·MB each)
  const SlotDev* slots;
  void* x_rot;             // [n][d_in], row p = rotated row perm[p]
  int32_t d_in;
  int32_t block;           // OFT block size of this launch (16, 32 or 64)
  int32_t max_tiles;
  // Blocks per work-group of the split launch (4: one per wave, 16: four
  // per wave); the whole-k launch takes one per wave of its work-groups.
  int32_t bpw;
};

// ---------------------------------------------------------------- GEMMs ---
// Base GEMM h = X_sel Wᵀ for all n rows, where row i of X_sel is x[i] or,
// for an OFT row, x_rot[rot_pos[i]].
struct BaseGemmArgs {
  const void* x;
  const void* x_rot;       // may be null when no row has R
  const int32_t* rot_pos;  // may be null when no row has R
  const void* W;           // [d_out][d_in]
  int32_t n, d_in, d_out;
  int32_t split;           // split-K factor
  int32_t kc;              // k range per split (multiple of 32)
  float* part;             // [split][n][d_out] fp32 partials (split path, or h_fp32)
  void* out;               // [n][d_out] in the layer type (split == 1, tiled)
  int32_t h_fp32;          // split == 1: h to part in fp32 rather than to out
};
// Skinny kernel: n <= 64 rows; 64·nb output columns per work-group (nb = 1,
// 2 or 4; d_out % (64·nb) == 0), kc a multiple of 64 whose staged x fits
// GEMM_SKINNY_MAX_LDS; writes `part`.  groups: k-groups of 4 waves per
// work-group (1 or 2; fp32 uses 1).  Declared with the shrink below.
constexpr size_t GEMM_SKINNY_MAX_LDS = 144 * 1024;
size_t gemm_skinny_lds(int dtype, int n, int nb, int groups, int kc);
// LDS-tiled 128x128 kernel; writes `out` when split == 1, else `part`.
hipError_t launch_gemm_tiled(int dtype, const BaseGemmArgs& a, hipStream_t stream);

// Shrink over the plan's tiles: owned-term tiles V[p] = x[perm[p]] A'ᵀ,
// shared-term tiles U[p] = (x[perm[p]] A_vᵀ) ⊙ d'[slot].  One wave per
// (tile, 16 factor columns, k range of kc); the split partials go to `part`
// ([split][n][kmax] fp32) and a second launch adds them in split order into
// `v` ([n][kmax], layer type) by plan position p.
struct ShrinkArgs {
  const void* x;
  const int32_t* pinfo;    // (slot << 16) | row by plan position
  const int32_t* tiles;    // plan tiles, owned-term tiles first, padded with kind -1
  const int32_t* sh_tiles; // the shared-term tiles, padded with kind -1
  const int32_t* tile_rows_w;  // row words per tile (16·MB each)
  const int32_t* sh_rows_w;    // row words per shared-term tile
  const SlotDev* slots;
  const void* vera_At;     // [r_v][d_in] or null
  int32_t r_v;
  int32_t n, d_in;
  int32_t kmax;            // row stride of part and v
  // Work items: own_tiles x own_nblk x split on the first own_tiles entries of
  // tiles (bound on the owned-term tiles; column blocks of 16·ncb of the
  // largest owned rank), then sh_ntiles x sh_nblk x split on sh_tiles
  // (r_v / (16·ncb)); ncb is the launch's (launch_pre).
  int32_t own_tiles, own_nblk, sh_ntiles, sh_nblk;
  int32_t split, kc;       // k ranges (kc a multiple of 32)
  float* part;
  void* v;
  // Shared-term rows read their x·A_vᵀ partials from here when set (the
  // first projection of a group that shares A_v and the input computed
  // them; row stride kmax_shared), else from part.
  const float* part_shared;
  int32_t kmax_shared;
  // Whole-k shrink (launch_pre with whole): this slice takes its shared-term
  // rows' x·A_vᵀ from the launch's first slice, whose work-groups write
  // this slice's U with this slice's d'.
  int32_t borrows;
};
// One slice of the launch before the base GEMM: the shrink's items and/or
// OFT's rotation of its tiles for the launch's block size.
struct PreSlice {
  ShrinkArgs sh;
  OftArgs of;
  int32_t n_shrink_wg, n_oft_wg, oft_bg;
  // Arrival counters of the fused decode GEMM that follows (one word per
  // column tile), cleared by the launch's first work-group; may be null.
  int32_t* zero;
  int32_t zero_n;
};
// Fills a PreSlice; sh / of may be null (that part gets no work-groups).
// whole: the shrink's layout for launch_pre's whole-k mode.
PreSlice make_pre_slice(const ShrinkArgs* sh, const OftArgs* of, bool whole = false);
// bs: OFT block size of the slices' OFT parts (0 when no slice has one).
// whole (f16 / bf16, 16-row tiles, sh.split <= PRE_WHOLE_WAVES): one
// work-group of PRE_WHOLE_WAVES waves per shrink item (plan tile, 16 factor
// columns), wave w on the w-th k range of kc; the waves' sums meet in LDS
// and are added in wave order (the order the reduce pass adds splits in),
// so V and U are final when the launch ends and no partials are written.
constexpr int PRE_WHOLE_WAVES = 16;
// ncb: 16-column blocks per shrink item (1, or 4 for f16 / bf16 with
// 16-row tiles in split mode); the slices' own_nblk and sh_nblk count
// blocks of 16·ncb columns.
hipError_t launch_pre(int dtype, int tile_rows, int bs, const PreSlice* slices, int count, hipStream_t stream,
                      bool whole = false, int ncb = 1);

// out[row] = h[row] ⊙ s + b + V[p] B'ᵀ (owned tile) or (U[p] B_vᵀ) ⊙ e
// (shared tile), for row = perm[p].  h is read from `out` (in place, layer
// type) or summed from `hpart` (fp32 split-K partials, fixed order).
struct ExpandArgs {
  void* out;
  const float* hpart;      // null: read h from out
  int32_t hsplit;
  const int32_t* tiles;    // padded with kind -1 to max_tiles
  const int32_t* tile_rows_w;  // row words per tile (16·MB each)
  const SlotDev* slots;
  const void* vera_Bt;     // [d_out][r_v]
  int32_t r_v;
  const void* v;           // shrink output [n][kmax], layer type, by plan position
  int32_t kmax;
  int32_t n, d_out;
  int32_t max_tiles;
  int32_t apply_scale;     // 0: leave s and b to a separate pass
  // The plan's shared-term tiles on their own (padded with kind -1 to
  // max_sh_tiles; null or 0 where the layer has no shared term).  At decode
  // sizes launch_expand runs them first, as ranges of their own, and skips
  // them in the full list.
  const int32_t* sh_tiles;
  const int32_t* sh_rows_w;
  int32_t max_sh_tiles;
  int32_t part;            // set by launch_expand: 0 every tile, 2 every tile but shared-term ones
};

// One slice of a decode base-GEMM launch; with has_side, work-groups after
// the slice's GEMM work-groups run the shrink's split reduction.
struct GemmSlice {
  BaseGemmArgs g;
  ShrinkArgs side;
  int32_t has_side;
  // Streamed decode GEMM only: the side work-groups run the shrink itself,
  // one whole-k item each (its k ranges on the work-group's waves, added in
  // LDS in wave order), instead of adding split partials of a launch
  // before; nothing before the GEMM writes V or U.
  int32_t side_whole;
  // Streamed decode GEMM with the expand in its epilogue (launch_gemm_stream
  // with epi): the expand's arguments (out, tiles, slots, vera_Bt, r_v, v,
  // kmax, n, d_out; max_tiles entries of the tile list are read), the
  // plan's pinfo, and one arrival counter per column tile (zero at launch;
  // the last of a tile's split work-groups to arrive finishes it).
  ExpandArgs e;
  const int32_t* pinfo;
  int32_t* cnt;
};
// Work-groups of `threads` threads that a slice's split reduction takes,
// or, with side_whole, one per whole-k shrink item.
inline int side_workgroups(const GemmSlice& sl, int threads) {
  if (!sl.has_side) return 0;
  if (sl.side_whole) return sl.side.own_tiles * sl.side.own_nblk + sl.side.sh_ntiles * sl.side.sh_nblk;
  return (int)(((long)sl.side.n * (sl.side.kmax / 4) + threads - 1) / threads);
}
hipError_t launch_gemm_skinny(int dtype, int nb, int groups, const GemmSlice* slices, int count,
                              hipStream_t stream);
// The same GEMM with W and x streamed into LDS by direct loads (f16 / bf16;
// d_in and kc multiples of 64): `groups` k-groups of 4 waves per work-group
// (1 or 2), `stages` LDS buffers per group (groups 1: 3, 4 or 6; groups 2: 3).
constexpr size_t GEMM_STREAM_MAX_LDS = 160 * 1024;
size_t gemm_stream_lds(int n, int nb, int groups, int stages);
// n > 64, f16 / bf16: 128 x 128 tiles fed by direct global-to-LDS loads
// (d_out % 128 == 0, d_in and kc multiples of 64) through a ring of `stages`
// 32 KB LDS buffers (2..5); writes `out` when split == 1, else `part`.  With
// has_side, extra work-groups run the shrink's split reduction.
hipError_t launch_gemm_wide(int dtype, int stages, const GemmSlice& slice, hipStream_t stream);
// The direct-load GEMM with 256 x 256 tiles (8 waves, two 64 KB LDS
// buffers): d_out % 256 == 0, f16 / bf16; same outputs and side work.
// Several slices (projections of one input, same n and split) may share
// the launch.
hipError_t launch_gemm_big(int dtype, const GemmSlice* slices, int count, hipStream_t stream);
// epi: the expand runs in the epilogue (every slice's e, pinfo and cnt set;
// n <= 64, 3 stages, V and U final before the launch, s applied there: the
// e.apply_scale route); out is then written once and no partials are read
// back by another launch.
hipError_t launch_gemm_stream(int dtype, int nb, int groups, int stages, const GemmSlice* slices, int count,
                              hipStream_t stream, bool epi = false);
// Bytes of LDS the fused epilogue adds after the rings, for n rows, a tile
// list of max_tiles entries and at most `steps` MFMA k steps over it.
size_t gemm_stream_epi_lds(int n, int max_tiles, int steps);
// Whether the fused epilogue exists for this shape (n <= 64, 3 stages, its
// h and e fit in the rings).
bool gemm_stream_epi_ok(int n, int nb, int groups, int stages);
// The shrink's split reduction on its own (when the GEMM cannot carry it).
hipError_t launch_shrink_reduce(int dtype, const ShrinkArgs& a, hipStream_t stream);

// ---------------------------------------------------------------- expand --
// Every slice must have hpart set, or every slice must have it null.
hipError_t launch_expand(int dtype, int tile_rows, const ExpandArgs* slices, int count, hipStream_t stream);

// Prefill base GEMM (n > 64, f16 / bf16, k not split) whose epilogue is the
// expand: rows taken in the plan's tile order (16 row slots per tile of
// tile_rows 16), out written once.  g.x / x_rot / rot_pos / W / n / d_in /
// d_out as for the other GEMMs; e as for the expand (h comes from the GEMM,
// hpart unused, apply_scale must be set).  row_tiles: 128-slot tiles over
// the plan's tile bound; list_tiles: length of the padded tile list.
struct FusedArgs {
  BaseGemmArgs g;
  ExpandArgs e;
  int32_t row_tiles, col_tiles, list_tiles;
};
hipError_t launch_gemm_fused(int dtype, int stages, const FusedArgs& f, hipStream_t stream);

// Separate scale passes, for the route comparison of the appendix "Routes".
//   mode 1 side kernel:  h ← h ⊙ s + b        (before the expand)
//   mode 2 gathered:     out ← out ⊙ s + b    (after the expand)
//   mode 3 index scale, step one:  srow[i] ← s[slot(i)]
//   mode 4 index scale, step two:  out ← out ⊙ srow + b
struct ScaleArgs {
  void* y;                 // [n][d_out] layer type
  const float* hpart;      // side kernel on split partials: sum them into y
  int32_t hsplit;
  const int32_t* row_slot;
  const SlotDev* slots;
  float* srow;             // index scale buffers [n][d_out]
  int32_t n, d_out;
};
hipError_t launch_scale_pass(int dtype, int mode, const ScaleArgs& a, hipStream_t stream);

// ------------------------------------------------------------ load time ---
// DoRA: norm[j] = ‖W[j,:] + c·(A B)[:, j]‖ over d_in; s[j] = m[j] / norm[j];
// Bt[j][k] = B[k][j]·s[j] (k < r), 0 for r <= k < r_pad.  status |= 1 for a
// zero or non-finite norm.
struct DoraArgs {
  const void* W;           // [d_out][d_in]
  const float* At;         // c·A as fp32 [r][d_in]
  const float* B;          // [r][d_out]
  const float* m;          // [d_out]
  int32_t d_in, d_out, r, r_pad;
  float* s;                // [d_out]
  void* Bt;                // [d_out][r_pad], written when fold_e
  int32_t fold_e;
  int32_t* status;
};
hipError_t launch_dora_norm(int dtype, const DoraArgs& a, hipStream_t stream);
// dst[i] = (T)(alpha * src[i]) for i < count.
hipError_t launch_convert(int dtype, const float* src, void* dst, size_t count, float alpha,
                          hipStream_t stream);
// dst[c][r] = (T)(alpha * src[r][c] * colscale[c]) for a [rows][cols] source;
// dst is [cols_pad][ld] with rows < ld; rows >= `rows` and cols >= `cols`
// are zero.  colscale may be null.
hipError_t launch_pack_transpose(int dtype, const float* src, int rows, int cols, float alpha,
                                 const float* colscale, void* dst, int cols_pad, int ld,
                                 hipStream_t stream);

// -------------------------------------------------------------- probes ----
hipError_t launch_copy(void* dst, const void* src, size_t bytes, hipStream_t stream);
// Read-only probe: one 4-byte word per work-group (at most
// PROBE_READ_BLOCKS) goes to sink.
constexpr int PROBE_READ_BLOCKS = 8192;
hipError_t launch_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream);
hipError_t launch_empty(int count, hipStream_t stream);
hipError_t launch_delay(int microseconds, hipStream_t stream);

size_t dtype_size(int dtype);

}  // namespace tpa
