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
// writes.  A sort key packs (class, slot, has-R, row) into 32 bits; has-R is
// a function of the slot, so it does not change the order.  Up to 1024 rows
// are ranked directly (each thread counts the keys below its own, no
// barriers inside the sort); larger batches use an LDS bitonic network.
#include "internal.h"

namespace tpa {

namespace {

constexpr int ROW_BITS = 15;
static_assert(PLAN_MAX_ROWS <= (1 << ROW_BITS), "row index must fit the sort key");

__device__ __forceinline__ int key_cls(uint32_t k) { return (int)(k >> 30); }
__device__ __forceinline__ int key_slot(uint32_t k) { return (int)((k >> 16) & 0x3FFF); }
__device__ __forceinline__ int key_rot(uint32_t k) { return (int)((k >> ROW_BITS) & 1); }
__device__ __forceinline__ int key_row(uint32_t k) { return (int)(k & ((1u << ROW_BITS) - 1)); }

// Row words (pinfo) of positions [q0, q0 + TM) of a tile ending at q1; -1 past
// it.  TM is a multiple of 4.
__device__ __forceinline__ void put_rows(int32_t* dst, const uint32_t* skeys, int q0, int q1, int TM) {
  for (int j = 0; j < TM; j += 4) {
    int w[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int p = q0 + j + u;
      w[u] = p < q1 ? (int)(((uint32_t)key_slot(skeys[p]) << 16) | (uint32_t)key_row(skeys[p])) : -1;
    }
    *reinterpret_cast<int4*>(dst + j) = make_int4(w[0], w[1], w[2], w[3]);
  }
}

// Exclusive prefix sum over a work-group of T threads; the total goes to
// *total.  `scratch` holds T / 64 ints; callers may run scans back to back.
template <int T>
__device__ __forceinline__ int block_exclusive_scan(int v, int* scratch, int* total) {
  constexpr int W = T / 64;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int t = __shfl_up(incl, off, 64);
    if (lane >= off) incl += t;
  }
  if (W == 1) {
    *total = __shfl(incl, 63, 64);
    return incl - v;
  }
  if (lane == 63) scratch[wave] = incl;
  __syncthreads();
  int wave_off = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < W; ++w) {
    const int s = scratch[w];
    if (w < wave) wave_off += s;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return wave_off + incl - v;
}

template <int T, bool RANK>
__global__ __launch_bounds__(T) void plan_kernel(PlanArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint32_t sm[];
  __shared__ int scan_scratch[T / 64 > 0 ? T / 64 : 1];
  __shared__ int s_cls[4];
  const int n = a.n;
  const int tid = threadIdx.x;
  int np2 = 1;
  while (np2 < n) np2 <<= 1;
  const int nkeys = RANK ? n : np2;
  uint32_t* keys = sm;                               // [nkeys]
  uint32_t* skeys = RANK ? sm + n : sm;              // sorted keys [n]
  uint16_t* seg_start = reinterpret_cast<uint16_t*>(skeys + (RANK ? n : np2));  // [n + 1]

  // 1. Effective slot and sort key per row (the only global reads).
  int bad = 0;
  for (int i = tid; i < nkeys; i += T) {
    uint32_t key = 0xFFFFFFFFu;
    if (i < n) {
      int s = a.slot_of_row[i];
      if (!(s >= 0 && s < a.max_slots && a.slots[s].cls >= 0)) {
        s = 0;
        bad = 1;
      }
      const SlotDev& sd = a.slots[s];
      const int cls = (s == 0) ? CLS_NONE : sd.cls;
      const int rot = (s != 0 && sd.has_R) ? 1 : 0;
      key = ((uint32_t)cls << 30) | ((uint32_t)s << 16) | ((uint32_t)rot << ROW_BITS) | (uint32_t)i;
      a.row_slot[i] = s;
    }
    keys[i] = key;
  }
  const int any_bad = __syncthreads_or(bad);

  // 2. Sort by key, ascending.
  if (RANK) {
    for (int i = tid; i < n; i += T) {
      const uint32_t k = keys[i];
      int r = 0;
      for (int j = 0; j < n; ++j) r += keys[j] < k ? 1 : 0;
      skeys[r] = k;
    }
    __syncthreads();
  } else {
    for (int k = 2; k <= np2; k <<= 1) {
      for (int j = k >> 1; j > 0; j >>= 1) {
        for (int i = tid; i < np2; i += T) {
          const int ixj = i ^ j;
          if (ixj > i) {
            const uint32_t x = keys[i], y = keys[ixj];
            const bool asc = (i & k) == 0;
            if ((x > y) == asc) {
              keys[i] = y;
              keys[ixj] = x;
            }
          }
        }
        __syncthreads();
      }
    }
  }

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
  for (int p = p_lo; p < p_hi; ++p) {
    const uint32_t k = skeys[p];
    const int row = key_row(k);
    const int s = key_slot(k);
    const int cls = key_cls(k);
    a.perm[p] = row;
    a.pinfo[p] = (s << 16) | row;
    a.rot_pos[row] = key_rot(k) ? p : -1;
    if (p == 0 || key_slot(skeys[p - 1]) != s) {
      seg_start[seg] = (uint16_t)p;
      a.seg_ptr[seg] = p;
      a.seg_slot[seg] = s;
      ++seg;
    }
    const int prev_cls = (p == 0) ? -1 : key_cls(skeys[p - 1]);
    for (int c = prev_cls + 1; c <= cls; ++c) s_cls[c] = p;
    if (p == n - 1)
      for (int c = cls + 1; c <= 3; ++c) s_cls[c] = n;
  }
  if (tid == 0) {
    seg_start[nseg] = (uint16_t)n;
    a.seg_ptr[nseg] = n;
  }
  __syncthreads();

  // 4. Tiles: owned segments cut into pieces of tile_rows, then the shared-
  //    term and no-term ranges cut from their start; OFT tiles per segment
  //    of a slot with R.
  const int TM = a.tile_rows;
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
    const int p0 = seg_start[j], p1 = seg_start[j + 1];
    const uint32_t k = skeys[p0];
    const int s = key_slot(k);
    const bool owned = key_cls(k) == CLS_OWNED;
    const bool rot = key_rot(k) != 0;
    for (int q = p0; q < p1; q += TM) {
      const int q1 = min(q + TM, p1);
      if (owned) {
        put_rows(a.tile_rows_w + (size_t)own_off * TM, skeys, q, q1, TM);
        *reinterpret_cast<int4*>(a.tiles + 4 * own_off++) = make_int4(q, q1, CLS_OWNED, s);
      }
      if (rot) {
        put_rows(a.oft_rows_w + (size_t)oft_off * TM, skeys, q, q1, TM);
        *reinterpret_cast<int4*>(a.oft_tiles + 4 * oft_off++) = make_int4(q, q1, s, 0);
      }
    }
  }
  int nt = own_total;
  for (int c = CLS_SHARED; c <= CLS_NONE; ++c) {
    const int p0 = s_cls[c], p1 = s_cls[c + 1];
    const int cnt = (p1 - p0 + TM - 1) / TM;
    for (int q = tid; q < cnt; q += T) {
      const int4 tl = make_int4(p0 + q * TM, min(p0 + (q + 1) * TM, p1), c, -1);
      *reinterpret_cast<int4*>(a.tiles + 4 * (nt + q)) = tl;
      put_rows(a.tile_rows_w + (size_t)(nt + q) * TM, skeys, tl.x, tl.y, TM);
      if (c == CLS_SHARED) {
        *reinterpret_cast<int4*>(a.sh_tiles + 4 * q) = tl;
        put_rows(a.sh_rows_w + (size_t)q * TM, skeys, tl.x, tl.y, TM);
      }
    }
    if (c == CLS_SHARED)
      for (int q = cnt + tid; q < a.max_sh_tiles; q += T)
        *reinterpret_cast<int4*>(a.sh_tiles + 4 * q) = make_int4(0, 0, -1, -1);
    nt += cnt;
  }
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

template <int T, bool RANK>
hipError_t plan_launch(const PlanArgs& a, hipStream_t stream) {
  int np2 = 1;
  while (np2 < a.n) np2 <<= 1;
  const size_t keys = RANK ? 2 * (size_t)a.n : (size_t)np2;
  const size_t lds = keys * sizeof(uint32_t) + ((size_t)a.n + 2) * sizeof(uint16_t);
  hipLaunchKernelGGL((plan_kernel<T, RANK>), dim3(1), dim3(T), lds, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_plan(const PlanArgs& a, hipStream_t stream) {
  if (a.n <= 0 || a.n > PLAN_MAX_ROWS) return hipErrorInvalidValue;
  if (a.n <= 64) return plan_launch<64, true>(a, stream);
  if (a.n <= 256) return plan_launch<256, true>(a, stream);
  if (a.n <= 1024) return plan_launch<1024, true>(a, stream);
  return plan_launch<1024, false>(a, stream);
}

}  // namespace tpa
