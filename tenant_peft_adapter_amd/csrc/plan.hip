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
// workspace: perm, row_slot, rot_pos (position of a row's rotated copy, or
// -1), segments, tiles and OFT tiles, counters.  One work-group of 1024
// threads sorts up to 8192 rows in LDS with a bitonic network.
#include "internal.h"

namespace tpa {

namespace {

constexpr int PLAN_THREADS = 1024;
constexpr int PLAN_WAVES = PLAN_THREADS / 64;

// Exclusive prefix sum over the work-group; returns the prefix of this
// thread and writes the total to *total.  `scratch` holds PLAN_WAVES ints.
__device__ int block_exclusive_scan(int v, int* scratch, int* total) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    int t = __shfl_up(incl, off, 64);
    if (lane >= off) incl += t;
  }
  if (lane == 63) scratch[wave] = incl;
  __syncthreads();
  int wave_off = 0, tot = 0;
  for (int w = 0; w < PLAN_WAVES; ++w) {
    int s = scratch[w];
    if (w < wave) wave_off += s;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return wave_off + incl - v;
}

__device__ __forceinline__ int key_slot(uint32_t k) { return (int)((k >> 16) & 0x3FFF); }
__device__ __forceinline__ int key_cls(uint32_t k) { return (int)(k >> 30); }

}  // namespace

__global__ __launch_bounds__(PLAN_THREADS) void plan_kernel(PlanArgs a) {
  extern __shared__ uint32_t keys[];  // n_pow2 keys
  __shared__ int scan_scratch[PLAN_WAVES];
  __shared__ int s_invalid;
  __shared__ int s_nseg;
  __shared__ int s_nown, s_noft;
  const int n = a.n;
  const int tid = threadIdx.x;
  int np2 = 1;
  while (np2 < n) np2 <<= 1;
  if (tid == 0) s_invalid = 0;
  __syncthreads();

  // 1. Effective slot and sort key per row.
  int bad = 0;
  for (int i = tid; i < np2; i += PLAN_THREADS) {
    uint32_t key = 0xFFFFFFFFu;
    if (i < n) {
      int s = a.slot_of_row[i];
      bool ok = s >= 0 && s < a.max_slots && a.slots[s].cls >= 0;
      if (!ok) {
        s = 0;
        bad = 1;
      }
      int cls = (s == 0) ? CLS_NONE : a.slots[s].cls;
      key = ((uint32_t)cls << 30) | ((uint32_t)s << 16) | (uint32_t)i;
      a.row_slot[i] = s;
    }
    keys[i] = key;
  }
  if (bad) atomicOr(&s_invalid, 1);
  __syncthreads();

  // 2. Bitonic sort, ascending.
  for (int k = 2; k <= np2; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = tid; i < np2; i += PLAN_THREADS) {
        int ixj = i ^ j;
        if (ixj > i) {
          uint32_t x = keys[i], y = keys[ixj];
          bool asc = (i & k) == 0;
          if ((x > y) == asc) {
            keys[i] = y;
            keys[ixj] = x;
          }
        }
      }
      __syncthreads();
    }
  }

  // 3. Positions: perm, rot_pos, segment heads, class boundaries.  Each
  //    thread owns a contiguous chunk of positions so a scan of per-thread
  //    counts numbers the segments in order.
  const int chunk = (n + PLAN_THREADS - 1) / PLAN_THREADS;
  const int p_lo = min(n, tid * chunk), p_hi = min(n, p_lo + chunk);
  int heads = 0;
  for (int p = p_lo; p < p_hi; ++p) {
    uint32_t k = keys[p];
    if (p == 0 || key_slot(keys[p - 1]) != key_slot(k)) ++heads;
  }
  int total = 0;
  int seg = block_exclusive_scan(heads, scan_scratch, &total);
  if (tid == 0) s_nseg = total;
  for (int p = p_lo; p < p_hi; ++p) {
    uint32_t k = keys[p];
    int row = (int)(k & 0xFFFF);
    int s = key_slot(k);
    int cls = key_cls(k);
    a.perm[p] = row;
    a.rot_pos[row] = (s != 0 && a.slots[s].has_R) ? p : -1;
    if (p == 0 || key_slot(keys[p - 1]) != s) {
      a.seg_ptr[seg] = p;
      a.seg_slot[seg] = s;
      ++seg;
    }
    int prev_cls = (p == 0) ? -1 : key_cls(keys[p - 1]);
    for (int c = prev_cls + 1; c <= cls; ++c) a.counts[CNT_CLASS0 + c] = p;
    if (p == n - 1)
      for (int c = cls + 1; c <= 3; ++c) a.counts[CNT_CLASS0 + c] = n;
  }
  if (n == 0 && tid == 0)
    for (int c = 0; c <= 3; ++c) a.counts[CNT_CLASS0 + c] = 0;
  __syncthreads();
  const int nseg = s_nseg;
  if (tid == 0) a.seg_ptr[nseg] = n;
  __syncthreads();

  // 4. Tiles: owned segments cut into pieces of tile_rows, then the shared-
  //    term and no-term ranges cut from their start; OFT tiles per segment
  //    of a slot with R.
  const int TM = a.tile_rows;
  const int schunk = (nseg + PLAN_THREADS - 1) / PLAN_THREADS;
  const int j_lo = min(nseg, tid * schunk), j_hi = min(nseg, j_lo + schunk);
  int own = 0, oft = 0;
  for (int j = j_lo; j < j_hi; ++j) {
    int len = a.seg_ptr[j + 1] - a.seg_ptr[j];
    int s = a.seg_slot[j];
    int nt = (len + TM - 1) / TM;
    if (s != 0 && a.slots[s].cls == CLS_OWNED) own += nt;
    if (s != 0 && a.slots[s].has_R) oft += nt;
  }
  int own_total = 0, oft_total = 0;
  int own_off = block_exclusive_scan(own, scan_scratch, &own_total);
  int oft_off = block_exclusive_scan(oft, scan_scratch, &oft_total);
  for (int j = j_lo; j < j_hi; ++j) {
    int p0 = a.seg_ptr[j], p1 = a.seg_ptr[j + 1];
    int s = a.seg_slot[j];
    bool owned = s != 0 && a.slots[s].cls == CLS_OWNED;
    bool rot = s != 0 && a.slots[s].has_R;
    for (int q = p0; q < p1; q += TM) {
      int q1 = min(q + TM, p1);
      if (owned) {
        int* t = a.tiles + 4 * own_off++;
        t[0] = q;
        t[1] = q1;
        t[2] = CLS_OWNED;
        t[3] = s;
      }
      if (rot) {
        int* t = a.oft_tiles + 4 * oft_off++;
        t[0] = q;
        t[1] = q1;
        t[2] = s;
        t[3] = 0;
      }
    }
  }
  if (tid == 0) {
    s_nown = own_total;
    s_noft = oft_total;
  }
  __syncthreads();
  int nt = s_nown;
  for (int c = CLS_SHARED; c <= CLS_NONE; ++c) {
    int p0 = a.counts[CNT_CLASS0 + c], p1 = a.counts[CNT_CLASS0 + c + 1];
    int cnt = (p1 - p0 + TM - 1) / TM;
    for (int q = tid; q < cnt; q += PLAN_THREADS) {
      int* t = a.tiles + 4 * (nt + q);
      t[0] = p0 + q * TM;
      t[1] = min(p0 + (q + 1) * TM, p1);
      t[2] = c;
      t[3] = -1;
    }
    nt += cnt;
  }
  if (tid == 0) {
    a.counts[CNT_NSEG] = nseg;
    a.counts[CNT_NTILES] = nt;
    a.counts[CNT_NOFT] = s_noft;
    a.counts[CNT_INVALID] = s_invalid;
    if (s_invalid) atomicOr(a.flag, 1);
  }
}

hipError_t launch_plan(const PlanArgs& a, hipStream_t stream) {
  int np2 = 1;
  while (np2 < a.n) np2 <<= 1;
  size_t lds = (size_t)np2 * sizeof(uint32_t);
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(PLAN_THREADS), lds, stream, a);
  return hipGetLastError();
}

}  // namespace tpa
