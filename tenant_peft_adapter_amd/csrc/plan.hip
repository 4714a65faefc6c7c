// Row plan: groups the rows of a batch by tenant on the device.
//
// Scute paper (arXiv 2611.01089), §2 "The LoRA schedule": Punica's schedule
// sorts the batch so that each adapter's rows are contiguous (a segment),
// and every tile of rows belongs to one segment so that it reads one
// adapter's factors.  §4.1 route two runs the shared-factor (VeRA) term over
// tiles of rows whatever their adapters; route three rotates OFT rows in a
// pass of their own.  The faangrind "multi-lora-serving" page gives the
// per-row slot index (slot_of_row) this starts from.
//
// Order: rows sorted by (term class, slot, row), with class 0 = term on
// owned factors, 1 = shared-factor term, 2 = no term.  Outputs, in the
// workspace: perm, pinfo ((slot << 16) | row per position, so later kernels
// get both with one load), row_slot, rot_pos (position of a row's rotated
// copy, or -1), segments, tiles and OFT tiles (padded to max_tiles with
// kind / slot -1, so later kernels need no counter), the shared-term tiles
// again in a list of their own (padded to ceil(n / tile_rows)), counters.
//
// One work-group does the whole plan with everything in LDS: the only global
// reads are slot_of_row and the slot records it points to, the rest are
// writes.  A key packs (class, slot, has-R, row) into 32 bits; has-R is a
// function of the slot.  Up to 256 rows, each key is ranked by counting the
// keys below it.  Larger batches take a stable LSD radix sort on the bucket
// class * max_slots + slot (4 bits a pass), which leaves rows of one bucket
// in row order: the order of the keys.  Each thread owns a contiguous run of
// at most 8 elements; a pass counts digits per thread, scans the packed
// counts across the work-group and scatters in order.  Tiles are then
// written position-parallel.  Barriers wait for LDS only: the plan never
// reads its own global writes back.
#include "internal.h"

namespace tpa {

namespace {

constexpr int ROW_BITS = 15;
static_assert(PLAN_MAX_ROWS <= (1 << ROW_BITS), "row index must fit the sort key");

__device__ __forceinline__ int key_cls(uint32_t k) { return (int)(k >> 30); }
__device__ __forceinline__ int key_slot(uint32_t k) { return (int)((k >> 16) & 0x3FFF); }
__device__ __forceinline__ int key_rot(uint32_t k) { return (int)((k >> ROW_BITS) & 1); }
__device__ __forceinline__ int key_row(uint32_t k) { return (int)(k & ((1u << ROW_BITS) - 1)); }

// Exclusive prefix sum over a work-group of T threads; the total goes to
// *total.  `scratch` holds T / 64 ints; callers may run scans back to back.
template <int T>
__device__ __forceinline__ int block_exclusive_scan(int v, int* scratch, int* total) {
  constexpr int W = T / 64;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int incl = (int)wave_incl_scan((uint32_t)v);
  if (W == 1) {
    *total = __builtin_amdgcn_readlane(incl, 63);
    return incl - v;
  }
  if (lane == 63) scratch[wave] = incl;
  lds_barrier();
  int wave_off = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < W; ++w) {
    const int s = scratch[w];
    if (w < wave) wave_off += s;
    tot += s;
  }
  lds_barrier();
  *total = tot;
  return wave_off + incl - v;
}

// Exclusive scan across the work-group of eight packed words per thread
// (sixteen 16-bit counters; no field ever exceeds n <= 8192, so no carry
// crosses a field).  excl gets this thread's exclusive prefix, total the
// work-group's sums.  scratch holds 8 words per wave, 16-byte aligned.
template <int T>
__device__ __forceinline__ void block_scan8(const uint32_t (&v)[8], uint32_t (&excl)[8], uint32_t (&total)[8],
                                            uint32_t* scratch) {
  constexpr int W = T / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t incl[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) incl[q] = wave_incl_scan(v[q]);
  if (lane == 63) {
    uint4* d = reinterpret_cast<uint4*>(scratch + 8 * wave);
    d[0] = make_uint4(incl[0], incl[1], incl[2], incl[3]);
    d[1] = make_uint4(incl[4], incl[5], incl[6], incl[7]);
  }
  lds_barrier();
  uint32_t off[8] = {}, tot[8] = {};
#pragma unroll
  for (int w = 0; w < W; ++w) {
    const uint4* sw = reinterpret_cast<const uint4*>(scratch + 8 * w);
    const uint4 lo = sw[0], hi = sw[1];
    const uint32_t x[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      if (w < wave) off[q] += x[q];
      tot[q] += x[q];
    }
  }
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    excl[q] = off[q] + incl[q] - v[q];
    total[q] = tot[q];
  }
  lds_barrier();
}

template <int T, bool RANK, int TM>
__global__ __launch_bounds__(T) void plan_kernel(PlanArgs a) {
  constexpr int EMAX = 8;  // elements per thread (n <= 8 T)
  extern __shared__ __attribute__((aligned(16))) uint32_t sm[];
  __shared__ int scan_scratch[T / 64 > 0 ? T / 64 : 1];
  __shared__ __attribute__((aligned(16))) uint32_t scan8_scratch[8 * (T / 64)];
  __shared__ int s_cls[4];
  __shared__ int s_bad;
  const int n = a.n;
  const int tid = threadIdx.x;
  uint32_t* kbuf0 = sm;                                         // [n]
  uint32_t* kbuf1 = sm + n;                                     // [n]
  uint16_t* seg_start = reinterpret_cast<uint16_t*>(sm + 2 * n);  // [n + 1]
  uint16_t* seg_of_pos = seg_start + (n + 2);                   // [n]
  uint16_t* own_first = seg_of_pos + n;                         // [n]: first owned tile of a segment
  uint16_t* oft_first = own_first + n;                          // [n]: first OFT tile of a segment

  // 1. Effective slot and key per row (the only global reads).  Each thread
  //    takes a contiguous run of at most EMAX rows; all its slot ids are
  //    loaded before any slot record, so a thread waits for two round trips
  //    whatever its run length.
  if (tid == 0) s_bad = 0;
  lds_barrier();
  const int E = (n + T - 1) / T;
  const int e_lo = min(n, tid * E), e_hi = min(n, e_lo + E);
  int bad = 0;
  {
    int sv[EMAX];
#pragma unroll
    for (int e = 0; e < EMAX; ++e) sv[e] = e_lo + e < e_hi ? a.slot_of_row[e_lo + e] : 0;
    // The record's first 16 bytes, as two 8-byte halves (records are 8-byte
    // aligned): (cls, rank) and (has_R, oft_block).  Every entry loads (slot
    // 0's record where the entry is past the run or its slot out of range)
    // so that all of them go out at once: loaded under a condition, each
    // became a round trip of its own.
    int2 rec[EMAX], rot2[EMAX];
#pragma unroll
    for (int e = 0; e < EMAX; ++e) {
      const bool in = e_lo + e < e_hi && sv[e] >= 0 && sv[e] < a.max_slots;
      const int2* r = reinterpret_cast<const int2*>(a.slots + (in ? sv[e] : 0));
      const int2 r0 = r[0], r1 = r[1];
      rec[e] = make_int2(in ? r0.x : -1, r0.y);
      rot2[e] = make_int2(in ? r1.x : 0, r1.y);
    }
#pragma unroll
    for (int e = 0; e < EMAX; ++e) {
      const int i = e_lo + e;
      if (i >= e_hi) continue;
      int s = sv[e];
      int cls = rec[e].x, rot = rot2[e].x ? 1 : 0;
      if (!(s >= 0 && s < a.max_slots && cls >= 0)) {
        s = 0;
        bad = 1;
      }
      if (s == 0) {
        cls = CLS_NONE;
        rot = 0;
      }
      kbuf0[i] = ((uint32_t)cls << 30) | ((uint32_t)s << 16) | ((uint32_t)rot << ROW_BITS) | (uint32_t)i;
      a.row_slot[i] = s;
    }
  }
  if (__any(bad) && (tid & 63) == 0) atomicOr(&s_bad, 1);
  lds_barrier();
  const int any_bad = s_bad;

  // 2. Sort.  Small batches: each key's rank is the count of smaller keys
  //    (keys are distinct).  Otherwise a stable LSD radix sort on bucket =
  //    class * max_slots + slot.
  const uint32_t nbucket = 3u * (uint32_t)a.max_slots;
  int passes = 0;
  while (!RANK && ((nbucket - 1) >> (4 * passes))) ++passes;
  if (RANK) {
    for (int i = tid; i < n; i += T) {
      const uint32_t k = kbuf0[i];
      int r = 0;
      for (int j = 0; j < n; ++j) r += kbuf0[j] < k ? 1 : 0;
      kbuf1[r] = k;
    }
    lds_barrier();
  }
  uint32_t* src = kbuf0;
  uint32_t* dst = kbuf1;
  for (int pass = 0; pass < passes; ++pass) {
    const int shift = 4 * pass;
    uint32_t kv[EMAX];
    int dg[EMAX];
    uint32_t cnt[16];
#pragma unroll
    for (int d = 0; d < 16; ++d) cnt[d] = 0;
#pragma unroll
    for (int e = 0; e < EMAX; ++e) {
      dg[e] = -1;
      if (e_lo + e < e_hi) {
        kv[e] = src[e_lo + e];
        const uint32_t bucket = (kv[e] >> 30) * (uint32_t)a.max_slots + ((kv[e] >> 16) & 0x3FFFu);
        dg[e] = (int)((bucket >> shift) & 15u);
#pragma unroll
        for (int d = 0; d < 16; ++d) cnt[d] += dg[e] == d ? 1u : 0u;
      }
    }
    uint32_t packed[8], excl[8], total[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) packed[q] = cnt[2 * q] | (cnt[2 * q + 1] << 16);
    block_scan8<T>(packed, excl, total, scan8_scratch);
    uint32_t pos[16];
    uint32_t base = 0;
#pragma unroll
    for (int d = 0; d < 16; ++d) {
      const uint32_t tot = (total[d >> 1] >> (16 * (d & 1))) & 0xFFFFu;
      pos[d] = base + ((excl[d >> 1] >> (16 * (d & 1))) & 0xFFFFu);
      base += tot;
    }
#pragma unroll
    for (int e = 0; e < EMAX; ++e) {
      if (dg[e] < 0) continue;
      uint32_t p = 0;
#pragma unroll
      for (int d = 0; d < 16; ++d)
        if (dg[e] == d) p = pos[d]++;
      dst[p] = kv[e];
    }
    lds_barrier();
    uint32_t* t = src;
    src = dst;
    dst = t;
  }
  if (RANK) {
    src = kbuf1;
    dst = kbuf0;
  }
  const uint32_t* skeys = src;  // sorted keys [n]

  // 3. Positions: perm, rot_pos, segment heads, class boundaries.  Each
  //    thread owns a contiguous chunk of positions, so a scan of per-thread
  //    head counts numbers the segments in order.
  const int chunk = (n + T - 1) / T;
  const int p_lo = min(n, tid * chunk), p_hi = min(n, p_lo + chunk);
  int heads = 0;
  for (int p = p_lo; p < p_hi; ++p)
    if (p == 0 || key_slot(skeys[p - 1]) != key_slot(skeys[p])) ++heads;
  int nseg = 0;
  int seg = block_exclusive_scan<T>(heads, scan_scratch, &nseg);
  // perm, pinfo (by position) and rot_pos (by row, through the LDS copy of
  // the unsorted keys) are written with consecutive lanes on consecutive
  // entries.
  for (int p = tid; p < n; p += T) {
    const uint32_t k = skeys[p];
    const int row = key_row(k);
    a.perm[p] = row;
    a.pinfo[p] = (key_slot(k) << 16) | row;
    dst[row] = key_rot(k) ? (uint32_t)p : 0xFFFFFFFFu;  // the spare key buffer
  }
  for (int p = p_lo; p < p_hi; ++p) {
    const uint32_t k = skeys[p];
    const int s = key_slot(k);
    const int cls = key_cls(k);
    if (p == 0 || key_slot(skeys[p - 1]) != s) {
      seg_start[seg] = (uint16_t)p;
      a.seg_ptr[seg] = p;
      a.seg_slot[seg] = s;
      ++seg;
    }
    seg_of_pos[p] = (uint16_t)(seg - 1);
    const int prev_cls = (p == 0) ? -1 : key_cls(skeys[p - 1]);
    for (int c = prev_cls + 1; c <= cls; ++c) s_cls[c] = p;
    if (p == n - 1)
      for (int c = cls + 1; c <= 3; ++c) s_cls[c] = n;
  }
  if (tid == 0) {
    seg_start[nseg] = (uint16_t)n;
    a.seg_ptr[nseg] = n;
  }
  lds_barrier();
  for (int i = tid; i < n; i += T) a.rot_pos[i] = (int32_t)dst[i];

  // 4. Tiles: owned segments cut into pieces of tile_rows, then the shared-
  //    term and no-term ranges cut from their start; OFT tiles per segment
  //    of a slot with R.  A scan over segments gives each segment its first
  //    owned and OFT tile; then every position writes its own row word, and
  //    the positions that start a tile write its header (and -1 over the
  //    unused words of a short tile).
  const int schunk = (nseg + T - 1) / T;
  const int j_lo = min(nseg, tid * schunk), j_hi = min(nseg, j_lo + schunk);
  int own = 0, oft = 0;
  for (int j = j_lo; j < j_hi; ++j) {
    const int len = (int)seg_start[j + 1] - (int)seg_start[j];
    const uint32_t k = skeys[seg_start[j]];
    const int nt = (len + TM - 1) / TM;
    if (key_cls(k) == CLS_OWNED) own += nt;
    if (key_rot(k)) oft += nt;
  }
  int own_total = 0, oft_total = 0;
  int own_off = block_exclusive_scan<T>(own, scan_scratch, &own_total);
  int oft_off = block_exclusive_scan<T>(oft, scan_scratch, &oft_total);
  for (int j = j_lo; j < j_hi; ++j) {
    const int len = (int)seg_start[j + 1] - (int)seg_start[j];
    const uint32_t k = skeys[seg_start[j]];
    const int nt = (len + TM - 1) / TM;
    own_first[j] = (uint16_t)own_off;
    oft_first[j] = (uint16_t)oft_off;
    if (key_cls(k) == CLS_OWNED) own_off += nt;
    if (key_rot(k)) oft_off += nt;
  }
  lds_barrier();
  const int n_sh = (s_cls[CLS_SHARED + 1] - s_cls[CLS_SHARED] + TM - 1) / TM;
  const int n_none = (s_cls[CLS_NONE + 1] - s_cls[CLS_NONE] + TM - 1) / TM;
  const int nt = own_total + n_sh + n_none;
  for (int p = tid; p < n; p += T) {
    const uint32_t k = skeys[p];
    const int word = (int)(((uint32_t)key_slot(k) << 16) | (uint32_t)key_row(k));
    const int j = seg_of_pos[p];
    const int s0 = seg_start[j], s1 = seg_start[j + 1];
    const int off = p - s0;
    const int cls = key_cls(k);
    // (tile list, its row words, index in the list, start and end of the
    // tile, header) for each list the position belongs to
    auto put = [&](int* list, int* rows, int q, int q0, int q1, int4 hdr) {
      rows[(size_t)q * TM + (p - q0)] = word;
      if (p == q0) {
        *reinterpret_cast<int4*>(list + 4 * q) = hdr;
        for (int u = q1 - q0; u < TM; ++u) rows[(size_t)q * TM + u] = -1;
      }
    };
    if (cls == CLS_OWNED) {
      const int q0 = s0 + off / TM * TM, q1 = min(q0 + TM, s1);
      put(a.tiles, a.tile_rows_w, own_first[j] + off / TM, q0, q1, make_int4(q0, q1, CLS_OWNED, key_slot(k)));
    } else {
      const int c0 = s_cls[cls], c1 = s_cls[cls + 1];
      const int q = (p - c0) / TM;
      const int q0 = c0 + q * TM, q1 = min(q0 + TM, c1);
      const int4 hdr = make_int4(q0, q1, cls, -1);
      put(a.tiles, a.tile_rows_w, own_total + (cls == CLS_NONE ? n_sh : 0) + q, q0, q1, hdr);
      if (cls == CLS_SHARED) put(a.sh_tiles, a.sh_rows_w, q, q0, q1, hdr);
    }
    if (key_rot(k)) {
      const int q0 = s0 + off / TM * TM, q1 = min(q0 + TM, s1);
      put(a.oft_tiles, a.oft_rows_w, oft_first[j] + off / TM, q0, q1, make_int4(q0, q1, key_slot(k), 0));
    }
  }
  for (int q = n_sh + tid; q < a.max_sh_tiles; q += T)
    *reinterpret_cast<int4*>(a.sh_tiles + 4 * q) = make_int4(0, 0, -1, -1);
  // Pad both tile lists to max_tiles so later kernels need no counter.
  for (int q = nt + tid; q < a.max_tiles; q += T) {
    int* t = a.tiles + 4 * q;
    t[0] = 0;
    t[1] = 0;
    t[2] = -1;
    t[3] = -1;
  }
  for (int q = oft_total + tid; q < a.max_tiles; q += T) {
    int* t = a.oft_tiles + 4 * q;
    t[0] = 0;
    t[1] = 0;
    t[2] = -1;
    t[3] = 0;
  }
  if (tid == 0) {
    a.counts[CNT_NSEG] = nseg;
    a.counts[CNT_NTILES] = nt;
    a.counts[CNT_NOFT] = oft_total;
    a.counts[CNT_INVALID] = any_bad ? 1 : 0;
#pragma unroll
    for (int c = 0; c < 4; ++c) a.counts[CNT_CLASS0 + c] = s_cls[c];
    if (any_bad) atomicOr(a.flag, 1);
  }
}

// Tile rows are a template argument so the tile arithmetic is shifts.
template <int T, bool RANK>
hipError_t plan_launch(const PlanArgs& a, hipStream_t stream) {
  const size_t lds = 2 * (size_t)a.n * sizeof(uint32_t) + (4 * (size_t)a.n + 2) * sizeof(uint16_t);
  if (a.tile_rows == 16)
    hipLaunchKernelGGL((plan_kernel<T, RANK, 16>), dim3(1), dim3(T), lds, stream, a);
  else if (a.tile_rows == 64)
    hipLaunchKernelGGL((plan_kernel<T, RANK, 64>), dim3(1), dim3(T), lds, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace

hipError_t launch_plan(const PlanArgs& a, hipStream_t stream) {
  if (a.n <= 0 || a.n > PLAN_MAX_ROWS) return hipErrorInvalidValue;
  if (a.max_slots < 1 || a.max_slots > 16383) return hipErrorInvalidValue;
  if (a.n <= 64) return plan_launch<64, true>(a, stream);
  if (a.n <= 256) return plan_launch<256, true>(a, stream);
  // Thread counts measured per range (graph-replayed plan): 512 threads
  // from 257 to 1024 rows (1024 rows: 11.7 -> 11.1 µs against 256), 1024
  // above (2048 rows: 20.4 -> 16.3 µs against 256).
  if (a.n <= 1024) return plan_launch<512, false>(a, stream);
  return plan_launch<1024, false>(a, stream);
}

}  // namespace tpa
