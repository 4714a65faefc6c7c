// The C ABI of include/tpa.h: layer and slot management, the admission
// converter (normal form and folds), workspace layout and the forward's
// launch sequence.  Kernels live in the .hip files next to this one.
//
// Scute paper (arXiv 2611.01089): §3.1 eq. (1) and Table 1 (the normal form
// and its members), §3.2 and the appendix "Folds" (the fold rule), §5.1
// (admission: DoRA's s at load, VeRA as d, e plus a reference to the shared
// pair, OFT as explicit blocks), §5.2 (per-layer slot buffers set to the
// identity; the forward's steps).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <unordered_map>
#include <vector>

#include "internal.h"
#include "tpa.h"

using tpa::SlotDev;

namespace {

thread_local std::string g_err;

tpa_status fail(tpa_status code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

#define TPA_HIP(expr)                                                                  \
  do {                                                                                 \
    hipError_t e_ = (expr);                                                            \
    if (e_ != hipSuccess) return fail(TPA_ERR_HIP, "%s: %s", #expr, hipGetErrorString(e_)); \
  } while (0)

struct DeviceGuard {
  int prev = -1;
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&prev) != hipSuccess) prev = -1;
    if (prev != dev) (void)hipSetDevice(dev);
  }
  ~DeviceGuard() {
    int cur = -1;
    if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) (void)hipSetDevice(prev);
  }
};

struct HostSlot {
  bool used = false;
  tpa_adapter_info info{};
  void* mem = nullptr;  // block from the layer's slot arena
  size_t bytes = 0;
};

// Device memory of a layer's slots.  Blocks are carved from chunks of 32
// blocks' worth (16 MB to 256 MB) and go back to a free list of their exact
// size on unload, so admitting a tenant mostly allocates nothing, and a
// layer holding a thousand slots holds a few dozen allocations rather than
// a thousand (the equal-sized blocks of one method and shape recycle into
// each other).  A chunk left behind keeps a tail smaller than the block
// that did not fit.
struct SlotArena {
  std::vector<void*> chunks;
  char* cur = nullptr;
  size_t left = 0;
  std::unordered_map<size_t, std::vector<void*>> free_blocks;

  hipError_t take(size_t bytes, void** out) {
    auto it = free_blocks.find(bytes);
    if (it != free_blocks.end() && !it->second.empty()) {
      *out = it->second.back();
      it->second.pop_back();
      return hipSuccess;
    }
    if (bytes > left) {
      const size_t sz = std::max(bytes, std::min(std::max(32 * bytes, size_t(16) << 20), size_t(256) << 20));
      void* c = nullptr;
      if (hipError_t e = hipMalloc(&c, sz)) return e;
      chunks.push_back(c);
      cur = static_cast<char*>(c);
      left = sz;
    }
    *out = cur;
    cur += bytes;
    left -= bytes;
    return hipSuccess;
  }
  void give(void* p, size_t bytes) { free_blocks[bytes].push_back(p); }
  void release() {
    for (void* c : chunks) (void)hipFree(c);
    chunks.clear();
    free_blocks.clear();
    cur = nullptr;
    left = 0;
  }
};

inline int round_up(int v, int m) { return (v + m - 1) / m * m; }
inline size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

bool finite_all(const float* p, size_t n) {
  for (size_t i = 0; i < n; ++i)
    if (!std::isfinite(p[i])) return false;
  return true;
}

// The fold rule (appendix "Folds"): c folds into the first owned neighbour
// among A, d, B, e; d into an owned A or B; e into an owned B; s, b and R
// never fold.  `owned` and `present` use the bits below.
enum { OWN_A = 1, OWN_B = 2, OWN_D = 4, OWN_E = 8, OWN_R = 16 };
enum { PR_S = 1, PR_B = 2, PR_R = 4, PR_C = 8, PR_D = 16, PR_E = 32 };

void fold_rule(int owned, int present, int* fold_mask, int* live_mask) {
  int fm = 0, lm = 0;
  if (present & PR_S) lm |= TPA_LIVE_S;
  if (present & PR_B) lm |= TPA_LIVE_B;
  if (present & PR_R) lm |= TPA_LIVE_R;
  if (present & PR_C) {
    if (owned & OWN_A)
      fm |= TPA_FOLD_C_A;
    else if (owned & OWN_D)
      fm |= TPA_FOLD_C_D;
    // c next to only shared tensors would stay live; no member of Table 1
    // has such a term.
  }
  if (present & PR_D) {
    if (owned & (OWN_A | OWN_B))
      fm |= TPA_FOLD_D_A;
    else
      lm |= TPA_LIVE_D;
  }
  if (present & PR_E) {
    if (owned & OWN_B)
      fm |= TPA_FOLD_E_B;
    else
      lm |= TPA_LIVE_E;
  }
  *fold_mask = fm;
  *live_mask = lm;
}

// Ownership and non-identity slots of each method (Table 1, §2, §5.1).
bool method_shape(int method, int* owned, int* present, int* term) {
  switch (method) {
    case TPA_IDENTITY: *owned = 0; *present = 0; *term = 0; return true;
    case TPA_LORA: *owned = OWN_A | OWN_B; *present = PR_C; *term = 1; return true;
    case TPA_DORA: *owned = OWN_A | OWN_B; *present = PR_S | PR_C | PR_E; *term = 1; return true;
    case TPA_IA3: *owned = 0; *present = PR_S; *term = 0; return true;
    case TPA_VERA: *owned = OWN_D | OWN_E; *present = PR_C | PR_D | PR_E; *term = 2; return true;
    case TPA_OFT: *owned = OWN_R; *present = PR_R; *term = 0; return true;
    case TPA_SSF: *owned = 0; *present = PR_S | PR_B; *term = 0; return true;
    // LoHa and LoKr once expanded into one low-rank term (§3.1): like LoRA.
    case TPA_LOHA: *owned = OWN_A | OWN_B; *present = PR_C; *term = 1; return true;
    case TPA_LOKR: *owned = OWN_A | OWN_B; *present = PR_C; *term = 1; return true;
  }
  return false;
}

// R_jᵀ = (I + Q)^-1 (I - Q) for the Cayley rotation R_j = (I + Q)(I - Q)^-1
// of a skew-symmetric Q (the two factors commute and (I ± Q)ᵀ = I ∓ Q), by
// Gaussian elimination with partial pivoting in float64.  Writes the b x b
// block row-major, which is the transposed storage the rotate kernel reads.
void cayley_transposed(const float* Q, int b, float* out) {
  std::vector<double> M((size_t)b * 2 * b);
  for (int i = 0; i < b; ++i)
    for (int j = 0; j < b; ++j) {
      const double q = Q[(size_t)i * b + j];
      M[(size_t)i * 2 * b + j] = (i == j ? 1.0 : 0.0) + q;
      M[(size_t)i * 2 * b + b + j] = (i == j ? 1.0 : 0.0) - q;
    }
  for (int c = 0; c < b; ++c) {
    int piv = c;
    for (int r = c + 1; r < b; ++r)
      if (std::fabs(M[(size_t)r * 2 * b + c]) > std::fabs(M[(size_t)piv * 2 * b + c])) piv = r;
    if (piv != c)
      for (int j = 0; j < 2 * b; ++j) std::swap(M[(size_t)c * 2 * b + j], M[(size_t)piv * 2 * b + j]);
    const double inv = 1.0 / M[(size_t)c * 2 * b + c];
    for (int j = 0; j < 2 * b; ++j) M[(size_t)c * 2 * b + j] *= inv;
    for (int r = 0; r < b; ++r) {
      if (r == c) continue;
      const double f = M[(size_t)r * 2 * b + c];
      if (f == 0.0) continue;
      for (int j = 0; j < 2 * b; ++j) M[(size_t)r * 2 * b + j] -= f * M[(size_t)c * 2 * b + j];
    }
  }
  for (int i = 0; i < b; ++i)
    for (int j = 0; j < b; ++j) out[(size_t)i * b + j] = (float)M[(size_t)i * 2 * b + b + j];
}

struct Config {
  int tile_rows;
  int gemm_path;  // 0 skinny, 1 tiled, 2 stream, 3 wide
  int gemm_nb, gemm_groups, gemm_stages;
  int gemm_split, gemm_kc;
  int shrink_split, shrink_kc;
  int scale_route;
  int gemm_tile;  // path 3: 128 (128 x 128 tiles) or 256 (256 x 256 tiles)
  int fused;      // path 3, 128 x 128 tiles: the expand runs in the GEMM's epilogue
  int h_fp32;     // h goes to the expand in fp32 even when k is not split
  int fused_dec;  // path 2: the expand runs in the streamed GEMM's epilogue, after a whole-k shrink
  int shrink_in_gemm;  // path 2, no OFT: the shrink runs whole-k in the GEMM's side work-groups
  int shrink_ncb; // 16-column blocks per shrink item (1 or 4)
};

bool decode_path(const Config& c) { return c.gemm_path == 0 || c.gemm_path == 2; }
// The register-fed decode GEMM always writes split partials; the others
// write h into out (in the layer type) when they do not split k.
bool h_partials(const Config& c) { return c.gemm_path == 0 || c.gemm_split > 1 || c.h_fp32; }

// VeRA's shared A_v on the device ([r_v][d_in] in the layer type), held by
// every layer that reads it (one per fused input group: q, k and v share
// one; gate and up another) and freed with its last holder.
struct VeraA {
  void* mem = nullptr;
  int device = 0, dtype = 0, d_in = 0, r_v = 0;
  int refs = 0;
};

struct Layout {
  size_t perm, pinfo, row_slot, rot_pos, seg_ptr, seg_slot, tiles, oft_tiles, counts;
  size_t plan_end;  // the plan arrays come first; a shared plan buffer holds [0, plan_end)
  size_t x_rot, hpart, vpart, v, srow;
  size_t cnt;  // fused decode epilogue: one arrival counter per column tile
  size_t total;
  int max_tiles;
  size_t sh_tiles;
  int max_sh_tiles;
  size_t tile_rows_w, sh_rows_w, oft_rows_w;
};

}  // namespace

struct tpa_layer {
  int device = 0;
  int d_in = 0, d_out = 0, dtype = 0, max_slots = 0, max_rank = 0, kmax = 0;
  const void* W = nullptr;
  SlotDev* slots_dev = nullptr;
  std::vector<SlotDev> slots_host;
  std::vector<HostSlot> hs;
  int32_t* flag_dev = nullptr;
  // VeRA's pair: A_v in a block that layers reading the same input may
  // share (reference-counted, freed with its last holder), B_v in vera_mem.
  VeraA* vera_a = nullptr;
  void* vera_mem = nullptr;
  const void* vera_At = nullptr;
  const void* vera_Bt = nullptr;
  int r_v = 0;
  int n_owned = 0, n_vera = 0, n_dora = 0, n_stack = 0;
  int max_owned_rank = 0;  // largest rank among loaded owned-term slots
  int n_oft_bs[3] = {0, 0, 0};  // loaded OFT slots with block 16, 32, 64
  int opt[13] = {-1, -1, -1, -1, -1, 0, -1, -1, -1, -1, -1, -1, -1};
  // Second stream (default priority) on which the shrink runs beside the
  // base GEMM when overlap is asked for, and the events that fork it from
  // and join it to the caller's stream; created at the first forward that
  // uses them.
  hipStream_t side = nullptr;
  hipEvent_t ev_fork = nullptr, ev_join = nullptr;
  hipEvent_t stage_ev[6] = {};
  bool stage_on = false;
  SlotArena arena;
  float* stage = nullptr;        // fp32 staging of an adapter's raw arrays during its load
  size_t stage_floats = 0;
  int32_t* status_dev = nullptr; // DoRA's norm check
  uint64_t plan_sig = 0;   // hash of every slot's (term class, has R): what a row plan depends on
  uint64_t class_sig = 0;  // the same over term classes only
  int n_rot = 0;           // loaded slots with an OFT rotation
};

// A row plan built by one layer and shared by the layers whose slot classes
// match (same signature), so a batch is grouped once for all of them.
struct tpa_plan {
  uint64_t sig = 0, class_sig = 0;
  int max_slots = 0, n = 0, tile_rows = 0;
  const char* dev = nullptr;
  size_t bytes = 0;
  bool built = false;
};

namespace {

int oft_bs_index(int bs) { return bs == 16 ? 0 : bs == 32 ? 1 : bs == 64 ? 2 : -1; }

// Drops the layer's hold on its VeRA A (freeing it with the last holder).
void release_vera_a(tpa_layer* L) {
  if (!L->vera_a) return;
  if (--L->vera_a->refs == 0) {
    DeviceGuard guard(L->vera_a->device);
    (void)hipFree(L->vera_a->mem);
    delete L->vera_a;
  }
  L->vera_a = nullptr;
  L->vera_At = nullptr;
}


// Scratch memory of tpa_layer_forward_noalloc (for callers that cannot
// allocate): the workspace of one forward, in a file-scope device array of
// which each GPU the library runs on holds its own copy until the process
// ends.  In host code `scratch` names a host-side stand-in, not a device
// address: host code only ever passes the address hipGetSymbolAddress
// returns for the current device (kept per device in g_scratch).
static __device__ __align__(256) unsigned char scratch[TPA_NOALLOC_SCRATCH_BYTES];
std::mutex g_scratch_mu;
std::unordered_map<int, void*> g_scratch;

// Device address of `device`'s scratch array, looked up once per device with
// that device current (the caller holds a DeviceGuard for it).
tpa_status scratch_address(int device, void** out) {
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  auto it = g_scratch.find(device);
  if (it != g_scratch.end()) {
    *out = it->second;
    return TPA_OK;
  }
  void* ptr = nullptr;
  const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (e != hipSuccess || !ptr)
    return fail(TPA_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", device, hipGetErrorString(e));
  g_scratch[device] = ptr;
  *out = ptr;
  return TPA_OK;
}

// k range of the streamed decode GEMM for a grid of `col_tiles` column tiles
// (summed over the projections of one launch) over d_in: the largest power
// of two with at most 16 slices of 64 per k-group and >= 192 work-groups,
// or >= 128 where the launch also carries the whole shrink (its items keep
// the other CUs busy, and half the split partials are written and read
// again: o, 4096 -> 4096 at 64 rows, 23.3 -> 18.8 µs for GEMM + expand).
// (Whole-d_in ranges for gate + up, whose 224 column tiles alone fill the
// grid, write h once in the layer type but made the decode step slower:
// 208 against 200-204 µs.)
int stream_kc(long col_tiles, int d_in, int groups, bool side_shrink) {
  const long min_wgs = side_shrink ? 128 : 192;
  int kc = 64 * groups;
  for (int cand = 4096; cand >= 64 * groups; cand /= 2) {
    if (cand > 1024 * groups) continue;
    if (col_tiles * ((d_in + cand - 1) / cand) >= min_wgs) return cand;
  }
  return kc;
}

// The conditions, other than the GEMM path, for a decode shrink to run in the
// streamed GEMM's own launch: a term to compute, 16-row tiles of a 16-bit
// type, 16-column items, and no option that keeps it in the launch before
// (a pinned shrink split, the second stream, the opt-in fused epilogue).
// OFT's rotation, which the GEMM reads, still runs before it.
bool shrink_in_gemm_ok(const tpa_layer* L, int tile_rows) {
  return L->dtype != TPA_F32 && tile_rows == 16 && (L->n_owned > 0 || L->n_vera > 0) &&
         L->opt[TPA_OPT_SHRINK_SPLIT] <= 0 && L->opt[TPA_OPT_OVERLAP] != 1 && L->opt[TPA_OPT_SHRINK_COLS] != 64 &&
         L->opt[TPA_OPT_FUSE_EXPAND] != 1;
}

// k-groups and k range of one streamed decode-GEMM launch over `count`
// projections (sharing d_in) at column-block width nb: two k-groups (half
// the partials) unless their larger work-groups (one per CU) would take an
// extra round of the grid, counting the work-groups that carry the shrink's
// split reduction.
void stream_pick(const tpa_layer* const* Ls, int count, int n, int nb, int stages, int g_opt, int* groups,
                 int* kc_out) {
  long col_tiles = 0;
  int d_in = 0;
  bool side_shrink = true;
  for (int i = 0; i < count; ++i) {
    col_tiles += Ls[i]->d_out / (64 * nb);
    d_in = std::max(d_in, Ls[i]->d_in);
    side_shrink = side_shrink && shrink_in_gemm_ok(Ls[i], Ls[i]->opt[TPA_OPT_TILE_ROWS] > 0 ? Ls[i]->opt[TPA_OPT_TILE_ROWS] : 16);
  }
  long best_rounds = 0;
  *groups = 0;
  for (int G : {2, 1}) {
    if (g_opt > 0 && G != g_opt) continue;
    if (G > 1 && stages != 3) continue;
    const size_t lds = tpa::gemm_stream_lds(n, nb, G, stages);
    if (lds > tpa::GEMM_STREAM_MAX_LDS) continue;
    const int kc = stream_kc(col_tiles, d_in, G, side_shrink);
    long total = 0;
    for (int i = 0; i < count; ++i) {
      total += (long)(Ls[i]->d_out / (64 * nb)) * ((Ls[i]->d_in + kc - 1) / kc);
      if (Ls[i]->n_owned > 0 || Ls[i]->n_vera > 0) total += ((long)n * (Ls[i]->kmax / 4) + 256 * G - 1) / (256 * G);
    }
    const long slots = 256L * (long)(tpa::GEMM_STREAM_MAX_LDS / lds);
    const long rounds = (total + slots - 1) / slots;
    if (*groups == 0 || rounds < best_rounds) {
      *groups = G;
      *kc_out = kc;
      best_rounds = rounds;
    }
  }
  if (*groups == 0) {  // nothing fits the options: one group, three stages
    *groups = 1;
    *kc_out = stream_kc(col_tiles, d_in, 1, side_shrink);
  }
}

// Shrink: one wave per (tile, 16 factor columns, k range of ~256): short
// waves, as its launch is on the critical path.  From 2048 rows there are
// enough tiles to fill the chip with longer k ranges (~512, at most 8
// splits), which halve the fp32 partials written and summed again (2-layer
// cut of the 1024-tenant Zipf stack at 4096 rows: 2999 -> 2902 µs per
// layer; at 1024 rows the short ranges stay ahead, 1218 vs 1235).
// With the expand in the decode GEMM's epilogue the shrink runs whole-k
// (one work-group per item adds the k ranges itself), so at most
// PRE_WHOLE_WAVES ranges.
void set_shrink_split(const tpa_layer* L, int n, Config* c) {
  int ssplit = L->opt[TPA_OPT_SHRINK_SPLIT];
  if (ssplit <= 0) {
    ssplit = n >= 2048 ? std::max(1, std::min(8, L->d_in / 512)) : std::max(1, std::min(28, L->d_in / 256));
    if (c->fused_dec) ssplit = std::min(ssplit, tpa::PRE_WHOLE_WAVES);
    if (c->shrink_in_gemm) ssplit = 4 * c->gemm_groups;  // one k range per wave of a GEMM work-group
  }
  ssplit = std::min(ssplit, L->d_in / 32);
  c->shrink_kc = round_up((L->d_in + ssplit - 1) / ssplit, 32);
  c->shrink_split = (L->d_in + c->shrink_kc - 1) / c->shrink_kc;
}

int max_tiles_for(const tpa_layer* L, int n, int tile_rows);
int all_tile_bound(const tpa_layer* L, int n, int tr, int max_tiles);

// Rows from which shrink items take 64 factor columns by default.
constexpr int SHRINK_WIDE_ROWS = 512;

// Whether the streamed decode GEMM can carry the expand for n rows at the
// configuration's column blocks and k-groups: one thread per entry of the
// tile list and the epilogue's tables within LDS beside the rings.
bool fused_dec_fits(const tpa_layer* L, int n, const Config& c) {
  const int mt = all_tile_bound(L, n, c.tile_rows, max_tiles_for(L, n, c.tile_rows));
  const int kcap = std::max(L->kmax, L->r_v);
  const size_t lds = tpa::gemm_stream_lds(n, c.gemm_nb, c.gemm_groups, c.gemm_stages) +
                     tpa::gemm_stream_epi_lds(n, mt, mt * ((kcap + 31) / 32));
  return mt <= 256 * c.gemm_groups && lds <= tpa::GEMM_STREAM_MAX_LDS &&
         tpa::gemm_stream_epi_ok(n, c.gemm_nb, c.gemm_groups, c.gemm_stages);
}

Config choose_config(const tpa_layer* L, int n) {
  Config c{};
  // 16-row tiles at every n: measured faster than 64 from 512 to 4096 rows
  // (more work items for the shrink and expand), with identical results.
  c.tile_rows = L->opt[TPA_OPT_TILE_ROWS] > 0 ? L->opt[TPA_OPT_TILE_ROWS] : 16;
  // Decode (n <= 64): the LDS-streamed kernel for f16 / bf16 with d_in a
  // multiple of 64, else the register-fed one; larger batches: tiled.
  const bool stream_ok = L->dtype != TPA_F32 && L->d_in % 64 == 0;
  // n > 64: the direct-load 128 x 128 kernel (3) for f16 / bf16 with
  // d_in % 64 == 0 and d_out % 128 == 0, else the register-staged one (1);
  // options 1 and 3 pin those at any n.
  const int path_opt = L->opt[TPA_OPT_GEMM_PATH];
  if (path_opt == 1 || path_opt == 3)
    c.gemm_path = path_opt;
  else if (path_opt == 2 && n <= 256)
    c.gemm_path = 2;
  else if (n > 64)
    c.gemm_path = 3;
  else
    c.gemm_path = path_opt == 0 || path_opt == 2 ? path_opt : (stream_ok ? 2 : 0);
  if (c.gemm_path == 3 && !(stream_ok && L->d_out % 128 == 0)) c.gemm_path = 1;
  if (c.gemm_path == 2 && !stream_ok) c.gemm_path = 0;
  if (c.gemm_path == 2) {
    // 64·nb columns per work-group; k-groups and k range from stream_pick.
    c.gemm_nb = (L->d_out >= 2048 && L->d_out % 128 == 0) ? 2 : 1;
    if (L->opt[TPA_OPT_GEMM_NB] > 0 && L->d_out % (64 * L->opt[TPA_OPT_GEMM_NB]) == 0) c.gemm_nb = L->opt[TPA_OPT_GEMM_NB];
    const int st = L->opt[TPA_OPT_GEMM_STAGES];
    c.gemm_stages = st == 4 || st == 6 ? st : 3;
    while (c.gemm_stages > 3 && tpa::gemm_stream_lds(n, c.gemm_nb, 1, c.gemm_stages) > tpa::GEMM_STREAM_MAX_LDS)
      c.gemm_stages = c.gemm_stages == 6 ? 4 : 3;
    int kc;
    stream_pick(&L, 1, n, c.gemm_nb, c.gemm_stages, L->opt[TPA_OPT_GEMM_GROUPS], &c.gemm_groups, &kc);
    const int split_opt = L->opt[TPA_OPT_GEMM_SPLIT];
    if (split_opt > 0) kc = round_up((L->d_in + split_opt - 1) / split_opt, 64 * c.gemm_groups);
    c.gemm_kc = std::min(kc, round_up(L->d_in, 64 * c.gemm_groups));
    c.gemm_split = (L->d_in + c.gemm_kc - 1) / c.gemm_kc;
  } else if (c.gemm_path == 0) {
    // 64·nb columns per work-group; the largest k range (1024 ... 64) that
    // still gives ~200 work-groups and whose staged x fits in LDS.
    c.gemm_nb = (L->d_out >= 8192 && L->d_out % 256 == 0) ? 4 : (L->d_out >= 2048 ? 2 : 1);
    if (L->opt[TPA_OPT_GEMM_NB] > 0 && L->d_out % (64 * L->opt[TPA_OPT_GEMM_NB]) == 0) c.gemm_nb = L->opt[TPA_OPT_GEMM_NB];
    c.gemm_groups = L->dtype == TPA_F32 ? 1 : (L->opt[TPA_OPT_GEMM_GROUPS] > 0 ? L->opt[TPA_OPT_GEMM_GROUPS] : 2);
    auto fits = [&](int kc) {
      return tpa::gemm_skinny_lds(L->dtype, n, c.gemm_nb, c.gemm_groups, kc) <= tpa::GEMM_SKINNY_MAX_LDS;
    };
    const int col_tiles = L->d_out / (64 * c.gemm_nb);
    int kc = 0;
    const int split_opt = L->opt[TPA_OPT_GEMM_SPLIT];
    if (split_opt > 0) {
      kc = round_up((L->d_in + split_opt - 1) / split_opt, 64);
      while (kc > 64 && !fits(kc)) kc -= 64;
    } else {
      for (int cand : {1024, 512, 256, 128, 64}) {
        if (!fits(cand)) continue;
        kc = cand;
        if ((long)col_tiles * ((L->d_in + cand - 1) / cand) >= 200) break;
      }
    }
    c.gemm_kc = std::min(kc, round_up(L->d_in, 64));
    c.gemm_split = (L->d_in + c.gemm_kc - 1) / c.gemm_kc;
  } else {
    c.gemm_nb = 4;
    // Path 3: 256 x 256 tiles once they give every CU one (their waves read
    // LDS and L2 at the MFMA rate with room to spare), else 128 x 128.
    c.gemm_tile = 128;
    if (c.gemm_path == 3 && L->d_out % 256 == 0) {
      const int pin = L->opt[TPA_OPT_WIDE_TILE];
      const bool fill = (long)((n + 255) / 256) * (L->d_out / 256) >= 256;
      if (pin == 256 || (pin != 128 && fill)) c.gemm_tile = 256;
    }
    const int tiles = ((n + c.gemm_tile - 1) / c.gemm_tile) * (L->d_out / c.gemm_tile);
    int split = L->opt[TPA_OPT_GEMM_SPLIT];
    if (split <= 0) {
      // The direct-load kernels hold a CU per work-group: split k so that
      // the grid fills at most one round (tiles x split <= 256).  A second,
      // partial round of split work-groups costs more than the CUs it
      // fills (base layer, 256 rows, 14336 outputs, 224 tiles: split 2
      // 75.4 µs against 56.4 with 1; 768 rows, 14336 -> 4096, 192 tiles:
      // 150.1 against 133.7).  The register-staged kernel's small
      // work-groups share CUs: there the grid may overfill.
      const int fill = c.gemm_path == 3 ? std::max(1, 256 / tiles) : (256 + tiles - 1) / tiles;
      split = std::max(1, std::min(L->d_in / 512, fill));
    }
    split = std::min(split, L->d_in / 64);
    c.gemm_kc = round_up((L->d_in + split - 1) / split, 64);
    c.gemm_split = (L->d_in + c.gemm_kc - 1) / c.gemm_kc;
    if (c.gemm_path == 3) {
      // The 128 x 128 kernel runs one work-group of 12 waves per CU, so its
      // ring may take 128 KB: four buffers keep three slices in flight (five
      // measured no better: 1024 x 4096 x 4096 44.6 against 42.5 µs).
      const int st = L->opt[TPA_OPT_GEMM_STAGES];
      c.gemm_stages = st >= 2 && st <= 5 ? st : 4;
    }
  }
  c.scale_route = L->opt[TPA_OPT_SCALE_ROUTE];
  // Expand in the GEMM's epilogue: needs the 128 x 128 prefill kernel with
  // k whole, 16-row plan tiles and s applied in the expand.  The GEMM then
  // runs over plan tiles (16 row slots each, a short tile's unused slots
  // computed for nothing), so by default it is taken only when the plan's
  // tile bound keeps the row slots within 1.5x the rows (prefill q_proj:
  // 1024 rows 75.8-77.1 against 76.7-78.3 µs per layer, 2048 rows 107-109
  // against 111-112).
  c.fused = 0;
  if (c.gemm_path == 3 && c.gemm_tile == 128 && c.gemm_split == 1 && c.tile_rows == 16 && c.scale_route == 0 &&
      L->dtype != TPA_F32 && L->opt[TPA_OPT_FUSE_EXPAND] != 0) {
    const long slots = 16L * ((n + 15) / 16 + std::min(n, L->n_owned) + 2);  // the plan's tile bound
    c.fused = L->opt[TPA_OPT_FUSE_EXPAND] == 1 || 2 * slots <= 3L * n;
  }
  // Decode, by option only: the expand in the streamed GEMM's epilogue
  // (the column tile's last split work-group finishes it) after a whole-k
  // shrink: three launches of a projection group become two, but measured
  // slower (decoder layer, graph-replayed step: 555 µs against 200 with
  // the separate expand).  Each split work-group's release at device scope
  // writes back its XCD's L2 (gate + up GEMM 55 -> 224 µs; 84 µs with the
  // fences left out), the finishing work-group's chain of dependent loads
  // (tables, partials, s / b / e, the term's k steps) is longer than the
  // separate expand, whose thousands of waves overlap theirs, and 16-wave
  // whole-k work-groups leave most CUs idle in the shrink (7-10 -> 13-31
  // µs).  Needs the 3-stage streamed kernel, 16-row tiles, s inside the
  // expand, a shrink of at most PRE_WHOLE_WAVES k ranges and the tables in
  // LDS.
  c.fused_dec = 0;
  if (c.gemm_path == 2 && n <= 64 && c.gemm_stages == 3 && c.tile_rows == 16 && c.scale_route == 0 &&
      L->opt[TPA_OPT_FUSE_EXPAND] == 1 && L->opt[TPA_OPT_SHRINK_SPLIT] <= tpa::PRE_WHOLE_WAVES)
    c.fused_dec = fused_dec_fits(L, n, c);
  // A stacked slot's scale is the product of its members' scales, so h
  // rounded to the layer type before the expand would carry |s|·u·|h| of
  // error: such layers keep h in fp32 between the GEMM and the expand.
  c.h_fp32 = L->n_stack > 0 && !c.fused && !c.fused_dec;
  // Decode on the streamed GEMM: the shrink needs nothing the GEMM makes,
  // so it runs in the GEMM's own grid (side work-groups, one whole-k item
  // each, V and U final when the GEMM ends); the launch before the GEMM
  // goes, or keeps only OFT's rotation.  Not with a pinned shrink split or
  // the second stream.
  c.shrink_in_gemm = c.gemm_path == 2 && !c.fused_dec && shrink_in_gemm_ok(L, c.tile_rows);
  set_shrink_split(L, n, &c);
  // Shrink items of 64 factor columns (one read of the tile's x rows for
  // four column blocks) where there are items enough to fill the chip
  // without them and a factor wider than 16 columns to share the read;
  // decode and rank-16 layers keep 16, whose items issue twice the k steps
  // at once (1024-row q_proj, rank 16: 6.5 against 7.9 µs).  Same bits.
  const int cols = L->opt[TPA_OPT_SHRINK_COLS];
  const bool wide_ok = L->dtype != TPA_F32 && c.tile_rows == 16 && !c.fused_dec;
  const bool wide_pays = L->max_owned_rank > 16 || (L->n_vera > 0 && L->r_v > 16);
  c.shrink_ncb = wide_ok && (cols == 64 || (cols <= 0 && n >= SHRINK_WIDE_ROWS && wide_pays)) ? 4 : 1;
  return c;
}

int max_tiles_for(const tpa_layer* L, int n, int tile_rows) {
  return (n + tile_rows - 1) / tile_rows + std::min(n, L->max_slots) + 2;
}

Layout make_layout(const tpa_layer* L, int n, const Config& c) {
  Layout y{};
  const size_t esz = tpa::dtype_size(L->dtype);
  y.max_tiles = max_tiles_for(L, n, c.tile_rows);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t at = off;
    off = align256(off + bytes);
    return at;
  };
  y.perm = take(4 * (size_t)n);
  y.pinfo = take(4 * (size_t)n);
  y.row_slot = take(4 * (size_t)n);
  y.rot_pos = take(4 * (size_t)n);
  y.seg_ptr = take(4 * (size_t)(n + 1));
  y.seg_slot = take(4 * (size_t)n);
  y.tiles = take(16 * (size_t)y.max_tiles);
  y.oft_tiles = take(16 * (size_t)y.max_tiles);
  y.max_sh_tiles = (n + c.tile_rows - 1) / c.tile_rows;
  y.sh_tiles = take(16 * (size_t)y.max_sh_tiles);
  y.tile_rows_w = take(4 * (size_t)c.tile_rows * y.max_tiles);
  y.sh_rows_w = take(4 * (size_t)c.tile_rows * y.max_sh_tiles);
  y.oft_rows_w = take(4 * (size_t)c.tile_rows * y.max_tiles);
  y.counts = take(4 * tpa::CNT_WORDS);
  y.plan_end = off;
  y.x_rot = take((size_t)n * L->d_in * esz);
  const bool need_hpart = h_partials(c);
  y.hpart = take(need_hpart ? (size_t)c.gemm_split * n * L->d_out * 4 : 0);
  y.vpart = take(c.fused_dec ? 0 : (size_t)c.shrink_split * n * L->kmax * 4);
  y.v = take((size_t)n * L->kmax * esz);
  y.srow = take(c.scale_route == 3 ? (size_t)n * L->d_out * 4 : 0);
  y.cnt = take(c.fused_dec ? 4 * (size_t)(L->d_out / 64) : 0);
  y.total = off;
  return y;
}

tpa::PlanArgs plan_args(tpa_layer* L, const int32_t* sor, int n, char* ws, const Layout& y,
                        const Config& c) {
  tpa::PlanArgs p{};
  p.slot_of_row = sor;
  p.slots = L->slots_dev;
  p.n = n;
  p.max_slots = L->max_slots;
  p.tile_rows = c.tile_rows;
  p.perm = reinterpret_cast<int32_t*>(ws + y.perm);
  p.pinfo = reinterpret_cast<int32_t*>(ws + y.pinfo);
  p.max_tiles = y.max_tiles;
  p.row_slot = reinterpret_cast<int32_t*>(ws + y.row_slot);
  p.rot_pos = reinterpret_cast<int32_t*>(ws + y.rot_pos);
  p.seg_ptr = reinterpret_cast<int32_t*>(ws + y.seg_ptr);
  p.seg_slot = reinterpret_cast<int32_t*>(ws + y.seg_slot);
  p.tiles = reinterpret_cast<int32_t*>(ws + y.tiles);
  p.oft_tiles = reinterpret_cast<int32_t*>(ws + y.oft_tiles);
  p.sh_tiles = reinterpret_cast<int32_t*>(ws + y.sh_tiles);
  p.tile_rows_w = reinterpret_cast<int32_t*>(ws + y.tile_rows_w);
  p.sh_rows_w = reinterpret_cast<int32_t*>(ws + y.sh_rows_w);
  p.oft_rows_w = reinterpret_cast<int32_t*>(ws + y.oft_rows_w);
  p.max_sh_tiles = y.max_sh_tiles;
  p.counts = reinterpret_cast<int32_t*>(ws + y.counts);
  p.flag = L->flag_dev;
  return p;
}

tpa_status stage(tpa_layer* L, int i, hipStream_t s) {
  if (L->stage_on) TPA_HIP(hipEventRecord(L->stage_ev[i], s));
  return TPA_OK;
}

tpa_status check_layer(const tpa_layer* L) {
  if (!L) return fail(TPA_ERR_INVALID, "null layer");
  return TPA_OK;
}

tpa_status upload_slot(tpa_layer* L, int slot, hipStream_t s) {
  TPA_HIP(hipMemcpyAsync(L->slots_dev + slot, &L->slots_host[slot], sizeof(SlotDev), hipMemcpyHostToDevice, s));
  TPA_HIP(hipStreamSynchronize(s));
  return TPA_OK;
}

// FNV-1a over every slot's (term class, has R): the plan depends on nothing
// else of the slot table.
void update_plan_sig(tpa_layer* L) {
  uint64_t h = 1469598103934665603ull, hc = h;
  auto mix = [](uint64_t& x, uint64_t v) {
    for (int i = 0; i < 8; ++i) {
      x ^= (v >> (8 * i)) & 0xFF;
      x *= 1099511628211ull;
    }
  };
  mix(h, (uint64_t)L->max_slots);
  mix(hc, (uint64_t)L->max_slots);
  int rmax = 0, nrot = 0;
  for (const SlotDev& sd : L->slots_host) {
    mix(h, (uint64_t)(uint32_t)sd.cls | ((uint64_t)sd.has_R << 32));
    mix(hc, (uint64_t)(uint32_t)sd.cls);
    if (sd.cls == tpa::CLS_OWNED) rmax = std::max(rmax, (int)sd.rank);
    if (sd.cls >= 0 && sd.has_R) ++nrot;
  }
  L->plan_sig = h;
  L->class_sig = hc;
  L->max_owned_rank = rmax;
  L->n_rot = nrot;
}

// A plan serves a layer whose slots have the builder's term classes and
// rotation flags, or the builder's term classes and no rotation at all: the
// order of rows and the tiles depend only on the classes, and a layer
// without rotated slots reads neither the OFT tiles nor rot_pos.
bool plan_accepts(const tpa_plan* plan, const tpa_layer* L) {
  if (plan->max_slots != L->max_slots) return false;
  return plan->sig == L->plan_sig || (plan->class_sig == L->class_sig && L->n_rot == 0);
}

// Bounds on what a plan of n rows holds for this layer's loaded slots (the
// kernels' grids; the plan pads its lists past the real counts).  Owned-term
// tiles: each owned segment is cut into tiles of tile_rows, so at most
// ceil(n / tile_rows) + (owned segments); the shared-term and no-term ranges
// add at most one partial tile each.  OFT tiles likewise per rotated slot.
int owned_tile_bound(const tpa_layer* L, int n, int tr, int max_tiles) {
  if (L->n_owned == 0) return 0;
  return std::min(max_tiles, (n + tr - 1) / tr + std::min(n, L->n_owned));
}
int all_tile_bound(const tpa_layer* L, int n, int tr, int max_tiles) {
  return std::min(max_tiles, (n + tr - 1) / tr + std::min(n, L->n_owned) + 2);
}
int oft_tile_bound(const tpa_layer* L, int n, int tr, int max_tiles) {
  const int n_rot = L->n_oft_bs[0] + L->n_oft_bs[1] + L->n_oft_bs[2];
  return std::min(max_tiles, (n + tr - 1) / tr + std::min(n, n_rot));
}

// Device float32 staging of an adapter's raw arrays, carved from the
// layer's staging buffer (grown to `floats` first; loads are serialized on
// the caller's stream and synchronized before they return, so one buffer
// serves every load of the layer).
struct Staging {
  tpa_layer* L;
  size_t used = 0;
  tpa_status reserve(size_t floats) {
    if (floats <= L->stage_floats) return TPA_OK;
    if (L->stage) {
      TPA_HIP(hipDeviceSynchronize());
      TPA_HIP(hipFree(L->stage));
      L->stage = nullptr;
      L->stage_floats = 0;
    }
    void* p = nullptr;
    TPA_HIP(hipMalloc(&p, floats * sizeof(float)));
    L->stage = static_cast<float*>(p);
    L->stage_floats = floats;
    return TPA_OK;
  }
  tpa_status alloc(size_t count, float** dev) {
    const size_t padded = (std::max<size_t>(count, 1) + 63) / 64 * 64;
    if (used + padded > L->stage_floats) return fail(TPA_ERR_INVALID, "staging overflow");
    *dev = L->stage + used;
    used += padded;
    return TPA_OK;
  }
  tpa_status put(const float* host, size_t count, float** dev, hipStream_t s) {
    if (tpa_status e = alloc(count, dev)) return e;
    if (count) TPA_HIP(hipMemcpyAsync(*dev, host, count * sizeof(float), hipMemcpyHostToDevice, s));
    return TPA_OK;
  }
};

// Checks one raw adapter against the layer (shapes, ranks, finite values,
// skew-symmetric Q).  Returns TPA_OK or the error with its message set.
tpa_status validate_desc(const tpa_layer* L, const tpa_adapter_desc* d) {
  const int d_in = L->d_in, d_out = L->d_out;
  const int m = d->method;
  if (m == TPA_LORA || m == TPA_DORA) {
    if (d->rank < 1 || d->rank > L->max_rank)
      return fail(TPA_ERR_INVALID, "rank %d outside [1, max_rank=%d]", d->rank, L->max_rank);
    if (!d->A || !d->B) return fail(TPA_ERR_INVALID, "null A or B");
    if (!std::isfinite(d->c) || !finite_all(d->A, (size_t)d_in * d->rank) || !finite_all(d->B, (size_t)d->rank * d_out))
      return fail(TPA_ERR_VALUE, "non-finite LoRA/DoRA factor");
    if (m == TPA_DORA && (!d->m || !finite_all(d->m, d_out))) return fail(TPA_ERR_VALUE, "missing or non-finite DoRA m");
  } else if (m == TPA_IA3) {
    if (!d->l) return fail(TPA_ERR_INVALID, "null l");
    if (!finite_all(d->l, d_out)) return fail(TPA_ERR_VALUE, "non-finite l");
  } else if (m == TPA_SSF) {
    if (!d->s || !d->b) return fail(TPA_ERR_INVALID, "null s or b");
    if (!finite_all(d->s, d_out) || !finite_all(d->b, d_out)) return fail(TPA_ERR_VALUE, "non-finite s or b");
  } else if (m == TPA_VERA) {
    if (L->r_v == 0) return fail(TPA_ERR_INVALID, "VeRA shared pair not set");
    if (d->rank != 0 && d->rank != L->r_v) return fail(TPA_ERR_INVALID, "VeRA rank %d != shared rank %d", d->rank, L->r_v);
    if (!d->d || !d->e) return fail(TPA_ERR_INVALID, "null d or e");
    if (!std::isfinite(d->c) || !finite_all(d->d, L->r_v) || !finite_all(d->e, d_out))
      return fail(TPA_ERR_VALUE, "non-finite VeRA vector");
  } else if (m == TPA_LOHA) {
    const int r2 = d->rank2 ? d->rank2 : d->rank;
    if (d->rank < 1 || r2 < 1 || (long)d->rank * r2 > L->max_rank)
      return fail(TPA_ERR_INVALID, "LoHa ranks %d x %d must be >= 1 with a product <= max_rank=%d", d->rank, r2,
                  L->max_rank);
    if (!d->A || !d->B || !d->A2 || !d->B2) return fail(TPA_ERR_INVALID, "null LoHa factor");
    if (!std::isfinite(d->c) || !finite_all(d->A, (size_t)d_in * d->rank) ||
        !finite_all(d->B, (size_t)d->rank * d_out) || !finite_all(d->A2, (size_t)d_in * r2) ||
        !finite_all(d->B2, (size_t)r2 * d_out))
      return fail(TPA_ERR_VALUE, "non-finite LoHa factor");
  } else if (m == TPA_LOKR) {
    const int p = d->kron_p, q = d->kron_q;
    if (p < 1 || q < 1 || d_in % p || d_out % q)
      return fail(TPA_ERR_INVALID, "LoKr factor shape %d x %d must divide %d x %d", p, q, d_in, d_out);
    if (d->rank < 1 || (long)std::min(p, q) * d->rank > L->max_rank)
      return fail(TPA_ERR_INVALID, "LoKr rank %d x min(%d, %d) outside [1, max_rank=%d]", d->rank, p, q, L->max_rank);
    if (!d->C || !d->A || !d->B) return fail(TPA_ERR_INVALID, "null LoKr factor");
    if (!std::isfinite(d->c) || !finite_all(d->C, (size_t)p * q) ||
        !finite_all(d->A, (size_t)(d_in / p) * d->rank) || !finite_all(d->B, (size_t)d->rank * (d_out / q)))
      return fail(TPA_ERR_VALUE, "non-finite LoKr factor");
  } else if (m == TPA_OFT) {
    const int bs = d->oft_block;
    if (oft_bs_index(bs) < 0 || d_in % bs) return fail(TPA_ERR_INVALID, "OFT block %d must be 16, 32 or 64 and divide d_in", bs);
    if (!d->Q) return fail(TPA_ERR_INVALID, "null Q");
    const size_t cnt = (size_t)d_in * bs;
    if (!finite_all(d->Q, cnt)) return fail(TPA_ERR_VALUE, "non-finite Q");
    for (int j = 0; j < d_in / bs; ++j) {
      const float* q = d->Q + (size_t)j * bs * bs;
      float mx = 0.f;
      for (int i = 0; i < bs * bs; ++i) mx = std::max(mx, std::fabs(q[i]));
      for (int r = 0; r < bs; ++r)
        for (int c = 0; c <= r; ++c)
          if (std::fabs(q[r * bs + c] + q[c * bs + r]) > 1e-6f * (1.f + mx))
            return fail(TPA_ERR_VALUE, "Q block %d is not skew-symmetric at (%d, %d)", j, r, c);
    }
  }
  return TPA_OK;
}

struct StackTerm {
  bool shared = false;          // VeRA term (c·d, e on the layer's pair)
  int r = 0;
  std::vector<double> A;        // owned: c·A as [d_in][r]
  std::vector<double> B;        // owned: B as [r][d_out]
  std::vector<double> dv;       // shared: c·d [r_v]
  std::vector<double> e;        // outer vector [d_out]
  bool e_unit = true;           // e is all ones (nothing to fold into B)
};

// LoHa / LoKr update as one low-rank term without c (§3.1, "Other methods
// fit as well"): A [d_in][R], B [R][d_out] with A B = ΔW / c.
//   LoHa: column (k, l) of A is A1[:,k] ⊙ A2[:,l], row (k, l) of B is
//         B1[k] ⊙ B2[l] (R = r1 · r2).
//   LoKr: C ⊗ (A0 B0) = (C ⊗ A0)(I_q ⊗ B0) when q <= p (R = q · r), else
//         (I_p ⊗ A0)(C ⊗ B0) (R = p · r).
void expand_product(const tpa_layer* L, const tpa_adapter_desc& d, StackTerm* tm) {
  const int d_in = L->d_in, d_out = L->d_out;
  if (d.method == TPA_LOHA) {
    const int r1 = d.rank, r2 = d.rank2 ? d.rank2 : d.rank, R = r1 * r2;
    tm->r = R;
    tm->A.assign((size_t)d_in * R, 0.0);
    tm->B.assign((size_t)R * d_out, 0.0);
    for (int i = 0; i < d_in; ++i)
      for (int k = 0; k < r1; ++k)
        for (int l = 0; l < r2; ++l)
          tm->A[(size_t)i * R + k * r2 + l] = (double)d.A[(size_t)i * r1 + k] * d.A2[(size_t)i * r2 + l];
    for (int k = 0; k < r1; ++k)
      for (int l = 0; l < r2; ++l)
        for (int j = 0; j < d_out; ++j)
          tm->B[(size_t)(k * r2 + l) * d_out + j] = (double)d.B[(size_t)k * d_out + j] * d.B2[(size_t)l * d_out + j];
    return;
  }
  const int p = d.kron_p, q = d.kron_q, r = d.rank, p2 = d_in / p, q2 = d_out / q;
  const bool left_c = q <= p;  // C rides with A (R = q·r), else with B (R = p·r)
  const int R = (left_c ? q : p) * r;
  tm->r = R;
  tm->A.assign((size_t)d_in * R, 0.0);
  tm->B.assign((size_t)R * d_out, 0.0);
  for (int i1 = 0; i1 < p; ++i1)
    for (int i2 = 0; i2 < p2; ++i2)
      for (int k1 = 0; k1 < (left_c ? q : p); ++k1) {
        const double f = left_c ? (double)d.C[(size_t)i1 * q + k1] : (i1 == k1 ? 1.0 : 0.0);
        if (f == 0.0) continue;
        for (int k = 0; k < r; ++k)
          tm->A[(size_t)(i1 * p2 + i2) * R + k1 * r + k] = f * d.A[(size_t)i2 * r + k];
      }
  for (int k1 = 0; k1 < (left_c ? q : p); ++k1)
    for (int k = 0; k < r; ++k)
      for (int j1 = 0; j1 < q; ++j1) {
        const double f = left_c ? (k1 == j1 ? 1.0 : 0.0) : (double)d.C[(size_t)k1 * q + j1];
        if (f == 0.0) continue;
        for (int j2 = 0; j2 < q2; ++j2)
          tm->B[(size_t)(k1 * r + k) * d_out + j1 * q2 + j2] = f * d.B[(size_t)k * q2 + j2];
      }
}

float half_bits_to_float(uint16_t h) {
  const uint32_t sign = (uint32_t)(h >> 15) << 31;
  int exp = (h >> 10) & 0x1F;
  uint32_t man = h & 0x3FF;
  uint32_t bits;
  if (exp == 0x1F) {
    bits = sign | 0x7F800000u | (man << 13);
  } else if (exp == 0) {
    if (man == 0) {
      bits = sign;
    } else {  // subnormal: normalise
      int e = -1;
      do {
        man <<= 1;
        ++e;
      } while (!(man & 0x400));
      bits = sign | ((uint32_t)(127 - 15 - e) << 23) | ((man & 0x3FF) << 13);
    }
  } else {
    bits = sign | ((uint32_t)(exp - 15 + 127) << 23) | (man << 13);
  }
  float f;
  std::memcpy(&f, &bits, 4);
  return f;
}

// Device matrix in the layer type -> host float64.
tpa_status fetch_matrix(const tpa_layer* L, const void* dev, size_t count, std::vector<double>* out) {
  out->resize(count);
  if (L->dtype == TPA_F32) {
    std::vector<float> h(count);
    TPA_HIP(hipMemcpy(h.data(), dev, count * 4, hipMemcpyDeviceToHost));
    for (size_t i = 0; i < count; ++i) (*out)[i] = h[i];
  } else {
    std::vector<uint16_t> h(count);
    TPA_HIP(hipMemcpy(h.data(), dev, count * 2, hipMemcpyDeviceToHost));
    for (size_t i = 0; i < count; ++i) {
      float f;
      if (L->dtype == TPA_BF16) {
        const uint32_t bits = (uint32_t)h[i] << 16;
        std::memcpy(&f, &bits, 4);
      } else {
        f = half_bits_to_float(h[i]);
      }
      (*out)[i] = f;
    }
  }
  return TPA_OK;
}

// DoRA's scale m ⊘ ‖W + cAB‖_c of one member, by the load-time norm kernel.
tpa_status dora_scale_host(tpa_layer* L, const tpa_adapter_desc* d, hipStream_t s, std::vector<double>* out) {
  const int d_in = L->d_in, d_out = L->d_out, r_pad = round_up(d->rank, 16);
  auto pad = [](size_t c) { return (std::max<size_t>(c, 1) + 63) / 64 * 64; };
  Staging st{L};
  if (tpa_status e = st.reserve(pad((size_t)d_in * d->rank) + pad((size_t)d->rank * d_out) +
                                pad((size_t)r_pad * d_in) + 2 * pad(d_out)))
    return e;
  if (!L->status_dev) {
    void* p = nullptr;
    TPA_HIP(hipMalloc(&p, sizeof(int32_t)));
    L->status_dev = static_cast<int32_t*>(p);
  }
  float *a32, *b32, *at32, *m32, *s32;
  if (tpa_status e = st.put(d->A, (size_t)d_in * d->rank, &a32, s)) return e;
  if (tpa_status e = st.put(d->B, (size_t)d->rank * d_out, &b32, s)) return e;
  if (tpa_status e = st.alloc((size_t)r_pad * d_in, &at32)) return e;
  if (tpa_status e = st.put(d->m, d_out, &m32, s)) return e;
  if (tpa_status e = st.alloc(d_out, &s32)) return e;
  TPA_HIP(tpa::launch_pack_transpose(0, a32, d_in, d->rank, d->c, nullptr, at32, r_pad, d_in, s));
  TPA_HIP(hipMemsetAsync(L->status_dev, 0, sizeof(int32_t), s));
  tpa::DoraArgs da{};
  da.W = L->W;
  da.At = at32;
  da.B = b32;
  da.m = m32;
  da.d_in = d_in;
  da.d_out = d_out;
  da.r = d->rank;
  da.r_pad = r_pad;
  da.s = s32;
  da.Bt = nullptr;
  da.fold_e = 0;
  da.status = L->status_dev;
  TPA_HIP(tpa::launch_dora_norm(L->dtype, da, s));
  std::vector<float> sv(d_out);
  int32_t status = 0;
  TPA_HIP(hipMemcpyAsync(sv.data(), s32, (size_t)d_out * 4, hipMemcpyDeviceToHost, s));
  TPA_HIP(hipMemcpyAsync(&status, L->status_dev, sizeof status, hipMemcpyDeviceToHost, s));
  TPA_HIP(hipStreamSynchronize(s));
  if (status) return fail(TPA_ERR_VALUE, "DoRA: zero or non-finite column norm");
  out->assign(sv.begin(), sv.end());
  return TPA_OK;
}


// Installs the layer's VeRA pair: A_v from `va` (taking a hold on it and
// dropping the one on its previous A), B_v [d_out][r_v] uploaded from the
// float32 host array B [r_v][d_out].  Synchronizes s.
tpa_status set_vera_b(tpa_layer* L, VeraA* va, const float* B, hipStream_t s) {
  const size_t esz = tpa::dtype_size(L->dtype);
  const int r_v = va->r_v;
  void* bmem = nullptr;
  TPA_HIP(hipMalloc(&bmem, (size_t)L->d_out * r_v * esz));
  Staging st{L};
  float* b32;
  tpa_status e = st.reserve(((size_t)r_v * L->d_out + 63) / 64 * 64);
  if (!e) e = st.put(B, (size_t)r_v * L->d_out, &b32, s);
  if (e) {
    (void)hipFree(bmem);
    return e;
  }
  // B [r_v][d_out] -> [d_out][r_v].
  hipError_t he = tpa::launch_pack_transpose(L->dtype, b32, r_v, L->d_out, 1.f, nullptr, bmem, L->d_out, r_v, s);
  if (he == hipSuccess) he = hipStreamSynchronize(s);
  if (he != hipSuccess) {
    (void)hipFree(bmem);
    return fail(TPA_ERR_HIP, "%s", hipGetErrorString(he));
  }
  ++va->refs;
  release_vera_a(L);
  if (L->vera_mem) (void)hipFree(L->vera_mem);
  L->vera_a = va;
  L->vera_mem = bmem;
  L->vera_At = va->mem;
  L->vera_Bt = bmem;
  L->r_v = r_v;
  return TPA_OK;
}

}  // namespace

extern "C" {

const char* tpa_last_error(void) { return g_err.c_str(); }

tpa_status tpa_method_info(int32_t method, tpa_adapter_info* out) {
  if (!out) return fail(TPA_ERR_INVALID, "null output");
  int owned, present, term;
  if (!method_shape(method, &owned, &present, &term)) return fail(TPA_ERR_METHOD, "unknown method %d", method);
  std::memset(out, 0, sizeof *out);
  out->method = method;
  out->term_kind = term;
  fold_rule(owned, present, &out->fold_mask, &out->live_mask);
  return TPA_OK;
}

tpa_status tpa_layer_create(int32_t device, int32_t d_in, int32_t d_out, int32_t dtype, const void* W_dev,
                            int32_t max_slots, int32_t max_rank, tpa_layer** out) {
  if (!out) return fail(TPA_ERR_INVALID, "null output");
  *out = nullptr;
  if (d_in <= 0 || d_out <= 0 || d_in % 64 || d_out % 128)
    return fail(TPA_ERR_INVALID, "d_in must be a positive multiple of 64 and d_out of 128 (got %d, %d)", d_in, d_out);
  if (dtype < TPA_F32 || dtype > TPA_BF16) return fail(TPA_ERR_INVALID, "unknown dtype %d", dtype);
  if (!W_dev) return fail(TPA_ERR_INVALID, "null W");
  if (max_slots < 2 || max_slots > 16384) return fail(TPA_ERR_INVALID, "max_slots must be in [2, 16384]");
  if (max_rank < 1 || max_rank > 512) return fail(TPA_ERR_INVALID, "max_rank must be in [1, 512]");
  int ndev = 0;
  TPA_HIP(hipGetDeviceCount(&ndev));
  if (device < 0 || device >= ndev) return fail(TPA_ERR_INVALID, "no device %d", device);
  DeviceGuard guard(device);
  tpa_layer* L = new tpa_layer();
  L->device = device;
  L->d_in = d_in;
  L->d_out = d_out;
  L->dtype = dtype;
  L->W = W_dev;
  L->max_slots = max_slots;
  L->max_rank = max_rank;
  L->kmax = round_up(max_rank, 16);
  L->slots_host.assign(max_slots, SlotDev{});
  for (auto& s : L->slots_host) s.cls = -1;
  L->slots_host[0].cls = tpa::CLS_NONE;  // slot 0: the identity
  L->hs.assign(max_slots, HostSlot{});
  L->hs[0].used = true;
  L->hs[0].info.method = TPA_IDENTITY;
  hipError_t e = hipMalloc(&L->slots_dev, sizeof(SlotDev) * max_slots);
  if (e == hipSuccess) e = hipMemcpy(L->slots_dev, L->slots_host.data(), sizeof(SlotDev) * max_slots, hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipMalloc(&L->flag_dev, sizeof(int32_t));
  if (e == hipSuccess) e = hipMemset(L->flag_dev, 0, sizeof(int32_t));
  if (e != hipSuccess) {
    if (L->slots_dev) (void)hipFree(L->slots_dev);
    if (L->flag_dev) (void)hipFree(L->flag_dev);
    delete L;
    return fail(TPA_ERR_HIP, "layer allocation: %s", hipGetErrorString(e));
  }
  update_plan_sig(L);
  // Set-up of the no-allocation forward: this device's scratch address.
  void* scratch_ptr = nullptr;
  if (tpa_status st = scratch_address(device, &scratch_ptr)) {
    tpa_layer_destroy(L);
    return st;
  }
  *out = L;
  return TPA_OK;
}

tpa_status tpa_layer_destroy(tpa_layer* L) {
  if (!L) return TPA_OK;
  DeviceGuard guard(L->device);
  (void)hipDeviceSynchronize();
  L->arena.release();
  if (L->ev_fork) (void)hipEventDestroy(L->ev_fork);
  if (L->ev_join) (void)hipEventDestroy(L->ev_join);
  if (L->side) (void)hipStreamDestroy(L->side);
  if (L->stage) (void)hipFree(L->stage);
  if (L->status_dev) (void)hipFree(L->status_dev);
  if (L->vera_mem) (void)hipFree(L->vera_mem);
  release_vera_a(L);
  if (L->slots_dev) (void)hipFree(L->slots_dev);
  if (L->flag_dev) (void)hipFree(L->flag_dev);
  delete L;
  return TPA_OK;
}

tpa_status tpa_vera_shared_set(tpa_layer* L, int32_t r_v, const float* A, const float* B, tpa_stream stream) {
  if (tpa_status st = check_layer(L)) return st;
  if (!A || !B) return fail(TPA_ERR_INVALID, "null VeRA factor");
  if (r_v <= 0 || r_v % 16 || r_v > L->max_rank)
    return fail(TPA_ERR_INVALID, "r_v must be a positive multiple of 16 and <= max_rank (got %d)", r_v);
  if (L->n_vera > 0) return fail(TPA_ERR_INVALID, "VeRA slots are loaded; unload them first");
  if (!finite_all(A, (size_t)L->d_in * r_v) || !finite_all(B, (size_t)r_v * L->d_out))
    return fail(TPA_ERR_VALUE, "non-finite VeRA factor");
  DeviceGuard guard(L->device);
  hipStream_t s = static_cast<hipStream_t>(stream);
  TPA_HIP(hipStreamSynchronize(s));
  const size_t esz = tpa::dtype_size(L->dtype);
  VeraA* va = new VeraA();
  va->device = L->device;
  va->dtype = L->dtype;
  va->d_in = L->d_in;
  va->r_v = r_v;
  if (hipError_t e = hipMalloc(&va->mem, (size_t)r_v * L->d_in * esz)) {
    delete va;
    return fail(TPA_ERR_HIP, "%s", hipGetErrorString(e));
  }
  Staging st{L};
  float* a32;
  if (tpa_status e = st.reserve(((size_t)L->d_in * r_v + 63) / 64 * 64)) {
    (void)hipFree(va->mem);
    delete va;
    return e;
  }
  if (tpa_status e = st.put(A, (size_t)L->d_in * r_v, &a32, s)) {
    (void)hipFree(va->mem);
    delete va;
    return e;
  }
  // A [d_in][r_v] -> [r_v][d_in].
  hipError_t e = tpa::launch_pack_transpose(L->dtype, a32, L->d_in, r_v, 1.f, nullptr, va->mem, r_v, L->d_in, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) {
    (void)hipFree(va->mem);
    delete va;
    return fail(TPA_ERR_HIP, "%s", hipGetErrorString(e));
  }
  if (tpa_status st2 = set_vera_b(L, va, B, s)) {
    (void)hipFree(va->mem);
    delete va;
    return st2;
  }
  return TPA_OK;
}

tpa_status tpa_vera_shared_set_from(tpa_layer* L, tpa_layer* from, const float* B, tpa_stream stream) {
  if (tpa_status st = check_layer(L)) return st;
  if (tpa_status st = check_layer(from)) return st;
  if (!B) return fail(TPA_ERR_INVALID, "null VeRA factor");
  if (!from->vera_a) return fail(TPA_ERR_INVALID, "the source layer has no VeRA pair");
  if (from->device != L->device || from->dtype != L->dtype || from->d_in != L->d_in)
    return fail(TPA_ERR_INVALID, "the source layer differs in device, dtype or d_in");
  if (from->r_v > L->max_rank) return fail(TPA_ERR_INVALID, "r_v %d above max_rank %d", from->r_v, L->max_rank);
  if (L->n_vera > 0) return fail(TPA_ERR_INVALID, "VeRA slots are loaded; unload them first");
  if (!finite_all(B, (size_t)from->r_v * L->d_out)) return fail(TPA_ERR_VALUE, "non-finite VeRA factor");
  DeviceGuard guard(L->device);
  hipStream_t s = static_cast<hipStream_t>(stream);
  TPA_HIP(hipStreamSynchronize(s));
  VeraA* va = from->vera_a;
  ++va->refs;  // held across set_vera_b, which releases the layer's old A
  const tpa_status st = set_vera_b(L, va, B, s);
  --va->refs;
  return st;
}

tpa_status tpa_adapter_load(tpa_layer* L, const tpa_adapter_desc* d, int32_t* slot_out, tpa_stream stream) {
  if (tpa_status st = check_layer(L)) return st;
  if (!d || !slot_out) return fail(TPA_ERR_INVALID, "null argument");
  int owned, present, term;
  if (!method_shape(d->method, &owned, &present, &term)) return fail(TPA_ERR_METHOD, "unknown method %d", d->method);
  const int d_in = L->d_in, d_out = L->d_out;
  const int m = d->method;
  if (d->method == TPA_LOHA || d->method == TPA_LOKR) return tpa_adapter_load_stack(L, d, 1, slot_out, stream);
  if (tpa_status e = validate_desc(L, d)) return e;
  int slot = -1;
  for (int i = 1; i < L->max_slots; ++i)
    if (!L->hs[i].used) {
      slot = i;
      break;
    }
  if (slot < 0) return fail(TPA_ERR_NO_SLOT, "all %d slots in use", L->max_slots);

  DeviceGuard guard(L->device);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t esz = tpa::dtype_size(L->dtype);
  const bool post_scale = L->opt[TPA_OPT_SCALE_ROUTE] >= 2;  // s applied after the expand
  SlotDev sd{};
  sd.cls = term == 1 ? tpa::CLS_OWNED : term == 2 ? tpa::CLS_SHARED : tpa::CLS_NONE;
  const int r_pad = (m == TPA_LORA || m == TPA_DORA) ? round_up(d->rank, 16) : 0;
  // One device block per adapter: factors, vectors, blocks.
  size_t off = 0;
  size_t o_At = 0, o_Bt = 0, o_s = 0, o_b = 0, o_d = 0, o_e = 0, o_R = 0;
  auto take = [&](size_t bytes) {
    size_t at = off;
    off = align256(off + bytes);
    return at;
  };
  if (r_pad) {
    o_At = take((size_t)r_pad * d_in * esz);
    o_Bt = take((size_t)d_out * r_pad * esz);
  }
  if (m == TPA_DORA || m == TPA_IA3 || m == TPA_SSF) o_s = take((size_t)d_out * 4);
  if (m == TPA_SSF) o_b = take((size_t)d_out * 4);
  if (m == TPA_VERA) {
    o_d = take((size_t)L->r_v * 4);
    o_e = take((size_t)d_out * 4);
  }
  if (m == TPA_OFT) o_R = take((size_t)d_in * d->oft_block * esz);
  void* mem = nullptr;
  if (off) TPA_HIP(L->arena.take(off, &mem));
  char* base = static_cast<char*>(mem);
  Staging st{L};
  {
    // fp32 staging this load needs (each array padded to 64 floats)
    auto pad = [](size_t c) { return (std::max<size_t>(c, 1) + 63) / 64 * 64; };
    size_t need = 0;
    if (m == TPA_LORA || m == TPA_DORA)
      need = pad((size_t)d_in * d->rank) + pad((size_t)d->rank * d_out) + pad((size_t)r_pad * d_in) +
             (m == TPA_DORA ? pad(d_out) : 0);
    if (m == TPA_OFT) need = pad((size_t)d_in * d->oft_block);
    if (tpa_status e = st.reserve(need)) {
      if (mem) L->arena.give(mem, off);
      return e;
    }
  }
  if (m == TPA_DORA && !L->status_dev) {
    void* p = nullptr;
    if (hipError_t e = hipMalloc(&p, sizeof(int32_t))) {
      if (mem) L->arena.give(mem, off);
      return fail(TPA_ERR_HIP, "%s", hipGetErrorString(e));
    }
    L->status_dev = static_cast<int32_t*>(p);
  }
  int32_t* status_dev = m == TPA_DORA ? L->status_dev : nullptr;
  // Conversion to normal form; TPA_HIP returns from this lambda on error.
  auto convert = [&]() -> tpa_status {
    if (m == TPA_LORA || m == TPA_DORA) {
      float *a32, *b32, *at32;
      if (tpa_status e = st.put(d->A, (size_t)d_in * d->rank, &a32, s)) return e;
      if (tpa_status e = st.put(d->B, (size_t)d->rank * d_out, &b32, s)) return e;
      // A' = c·A stored [r_pad][d_in] (fold c -> A).
      if (tpa_status e = st.alloc((size_t)r_pad * d_in, &at32)) return e;
      TPA_HIP(tpa::launch_pack_transpose(0, a32, d_in, d->rank, d->c, nullptr, at32, r_pad, d_in, s));
      TPA_HIP(tpa::launch_convert(L->dtype, at32, base + o_At, (size_t)r_pad * d_in, 1.f, s));
      sd.A = base + o_At;
      sd.Bt = base + o_Bt;
      sd.rank = r_pad;
      if (m == TPA_LORA || post_scale)  // B stored [d_out][r_pad]
        TPA_HIP(tpa::launch_pack_transpose(L->dtype, b32, d->rank, d_out, 1.f, nullptr, base + o_Bt, d_out, r_pad, s));
      if (m == TPA_DORA) {
        float* m32;
        if (tpa_status e = st.put(d->m, d_out, &m32, s)) return e;
        TPA_HIP(hipMemsetAsync(status_dev, 0, sizeof(int32_t), s));
        // s = m ⊘ ‖W + cAB‖_c on the device from W; e = s folds into B
        // unless s is applied after the expand.
        tpa::DoraArgs da{};
        da.W = L->W;
        da.At = at32;
        da.B = b32;
        da.m = m32;
        da.d_in = d_in;
        da.d_out = d_out;
        da.r = d->rank;
        da.r_pad = r_pad;
        da.s = reinterpret_cast<float*>(base + o_s);
        da.Bt = base + o_Bt;
        da.fold_e = post_scale ? 0 : 1;
        da.status = status_dev;
        TPA_HIP(tpa::launch_dora_norm(L->dtype, da, s));
        sd.s = da.s;
      }
    } else if (m == TPA_IA3 || m == TPA_SSF) {
      const float* sv = m == TPA_IA3 ? d->l : d->s;
      TPA_HIP(hipMemcpyAsync(base + o_s, sv, (size_t)d_out * 4, hipMemcpyHostToDevice, s));
      sd.s = reinterpret_cast<float*>(base + o_s);
      if (m == TPA_SSF) {
        TPA_HIP(hipMemcpyAsync(base + o_b, d->b, (size_t)d_out * 4, hipMemcpyHostToDevice, s));
        sd.b = reinterpret_cast<float*>(base + o_b);
      }
      TPA_HIP(hipStreamSynchronize(s));
    } else if (m == TPA_VERA) {
      // d' = c·d (fold c -> d); e stays live.
      std::vector<float> dd(L->r_v);
      for (int k = 0; k < L->r_v; ++k) dd[k] = d->c * d->d[k];
      TPA_HIP(hipMemcpyAsync(base + o_d, dd.data(), (size_t)L->r_v * 4, hipMemcpyHostToDevice, s));
      TPA_HIP(hipMemcpyAsync(base + o_e, d->e, (size_t)d_out * 4, hipMemcpyHostToDevice, s));
      TPA_HIP(hipStreamSynchronize(s));
      sd.d = reinterpret_cast<float*>(base + o_d);
      sd.e = reinterpret_cast<float*>(base + o_e);
      sd.rank = L->r_v;
    } else if (m == TPA_OFT) {
      const int bs = d->oft_block;
      const size_t cnt = (size_t)d_in * bs;
      std::vector<float> rt(cnt);
      for (int j = 0; j < d_in / bs; ++j)
        cayley_transposed(d->Q + (size_t)j * bs * bs, bs, rt.data() + (size_t)j * bs * bs);
      float* r32;
      if (tpa_status e = st.put(rt.data(), cnt, &r32, s)) return e;
      TPA_HIP(tpa::launch_convert(L->dtype, r32, base + o_R, cnt, 1.f, s));
      sd.Rt = base + o_R;
      sd.has_R = 1;
      sd.oft_block = bs;
    }
    TPA_HIP(hipStreamSynchronize(s));
    if (status_dev) {
      int32_t status = 0;
      TPA_HIP(hipMemcpy(&status, status_dev, sizeof status, hipMemcpyDeviceToHost));
      if (status) return fail(TPA_ERR_VALUE, "DoRA: zero or non-finite column norm");
    }
    return TPA_OK;
  };
  tpa_status err = convert();
  if (err) {
    (void)hipStreamSynchronize(s);
    if (mem) L->arena.give(mem, off);
    return err;
  }
  L->slots_host[slot] = sd;
  if ((err = upload_slot(L, slot, s))) {
    L->slots_host[slot] = SlotDev{};
    L->slots_host[slot].cls = -1;
    if (mem) L->arena.give(mem, off);
    return err;
  }
  HostSlot& h = L->hs[slot];
  h.used = true;
  h.mem = mem;
  h.bytes = off;
  h.info = tpa_adapter_info{};
  h.info.method = m;
  h.info.term_kind = term;
  int pres = present;
  if (m == TPA_DORA && post_scale) pres &= ~PR_E;  // e rides with s in the post-expand pass
  fold_rule(owned, pres, &h.info.fold_mask, &h.info.live_mask);
  h.info.rank = (m == TPA_LORA || m == TPA_DORA) ? d->rank : (m == TPA_VERA ? L->r_v : 0);
  h.info.oft_block = m == TPA_OFT ? d->oft_block : 0;
  if (term == 1) ++L->n_owned;
  if (term == 2) ++L->n_vera;
  if (m == TPA_DORA) ++L->n_dora;
  if (m == TPA_OFT) ++L->n_oft_bs[oft_bs_index(d->oft_block)];
  update_plan_sig(L);
  *slot_out = slot;
  return TPA_OK;
}

// A stack (§3.2 "Stacking", appendix "Stacking"): members applied in order
// at one hook, each to the previous member's output.  The composition is
// again one member of eq. (1): scale Π s_j, shift folded through the later
// scales (b1⊙s2 + b2), and every member's term, each multiplied by the
// scales of the members after it through its outer vector e.  The members'
// own folds are made on the host in float64 (DoRA's scale comes from the
// device norm kernel, as for a single DoRA load); then the terms are stored
// as one slot:
//   * one shared (VeRA) term and nothing else: a shared-term slot (d' = c·d,
//     e' = e ⊙ later scales);
//   * otherwise every term becomes part of one owned term whose rank is the
//     sum of the members' ranks (a shared term enters through its exact
//     owned form A_v diag(c·d), B_v diag(e'), from the layer's stored pair),
//     so the stack runs as one segment of the same kernels.
// Only the first member may hold an input transform R (OFT).
tpa_status tpa_adapter_load_stack(tpa_layer* L, const tpa_adapter_desc* members, int32_t count, int32_t* slot_out,
                                  tpa_stream stream) {
  if (tpa_status st = check_layer(L)) return st;
  if (!members || !slot_out) return fail(TPA_ERR_INVALID, "null argument");
  if (count < 1 || count > TPA_MAX_STACK) return fail(TPA_ERR_INVALID, "a stack holds 1..%d members (got %d)",
                                                      TPA_MAX_STACK, count);
  const bool product1 = count == 1 && (members[0].method == TPA_LOHA || members[0].method == TPA_LOKR);
  if (count == 1 && !product1) return tpa_adapter_load(L, members, slot_out, stream);
  if (L->opt[TPA_OPT_SCALE_ROUTE] >= 2)
    return fail(TPA_ERR_INVALID, "stacks fold later scales into the terms; use a scale route inside the expand");
  for (int j = 0; j < count; ++j) {
    int owned, present, term;
    if (!method_shape(members[j].method, &owned, &present, &term))
      return fail(TPA_ERR_METHOD, "member %d: unknown method %d", j, members[j].method);
    if (j > 0 && members[j].method == TPA_OFT)
      return fail(TPA_ERR_INVALID, "member %d: only the first member of a stack may rotate the input", j);
    if (tpa_status e = validate_desc(L, &members[j])) return e;
  }
  int slot = -1;
  for (int i = 1; i < L->max_slots; ++i)
    if (!L->hs[i].used) {
      slot = i;
      break;
    }
  if (slot < 0) return fail(TPA_ERR_NO_SLOT, "all %d slots in use", L->max_slots);

  DeviceGuard guard(L->device);
  hipStream_t s = static_cast<hipStream_t>(stream);
  TPA_HIP(hipStreamSynchronize(s));
  const int d_in = L->d_in, d_out = L->d_out;
  // Compose on the host: y <- y ⊙ s_j + b_j + (terms of member j).
  std::vector<double> S, Bsh;
  std::vector<StackTerm> terms;
  int fold_mask = 0;
  for (int j = 0; j < count; ++j) {
    const tpa_adapter_desc& d = members[j];
    std::vector<double> sj, bj;
    if (d.method == TPA_DORA) {
      if (tpa_status e = dora_scale_host(L, &d, s, &sj)) return e;
    } else if (d.method == TPA_IA3) {
      sj.assign(d.l, d.l + d_out);
    } else if (d.method == TPA_SSF) {
      sj.assign(d.s, d.s + d_out);
      bj.assign(d.b, d.b + d_out);
    }
    if (!sj.empty()) {
      if (S.empty()) S.assign(d_out, 1.0);
      for (int c = 0; c < d_out; ++c) S[c] *= sj[c];
      if (!Bsh.empty())
        for (int c = 0; c < d_out; ++c) Bsh[c] *= sj[c];
      for (StackTerm& tm : terms) {
        for (int c = 0; c < d_out; ++c) tm.e[c] *= sj[c];
        tm.e_unit = false;
      }
    }
    if (!bj.empty()) {
      if (Bsh.empty()) Bsh.assign(d_out, 0.0);
      for (int c = 0; c < d_out; ++c) Bsh[c] += bj[c];
    }
    if (d.method == TPA_LORA || d.method == TPA_DORA) {
      StackTerm tm;
      tm.r = d.rank;
      tm.A.resize((size_t)d_in * d.rank);
      for (size_t i = 0; i < tm.A.size(); ++i) tm.A[i] = (double)d.c * d.A[i];
      tm.B.assign(d.B, d.B + (size_t)d.rank * d_out);
      tm.e = d.method == TPA_DORA ? sj : std::vector<double>(d_out, 1.0);
      tm.e_unit = d.method != TPA_DORA;
      terms.push_back(std::move(tm));
      fold_mask |= TPA_FOLD_C_A;
    } else if (d.method == TPA_LOHA || d.method == TPA_LOKR) {
      StackTerm tm;
      expand_product(L, d, &tm);
      for (double& v : tm.A) v *= (double)d.c;
      tm.e.assign(d_out, 1.0);
      terms.push_back(std::move(tm));
      fold_mask |= TPA_FOLD_C_A;
    } else if (d.method == TPA_VERA) {
      StackTerm tm;
      tm.shared = true;
      tm.e_unit = false;
      tm.r = L->r_v;
      tm.dv.resize(L->r_v);
      for (int k = 0; k < L->r_v; ++k) tm.dv[k] = (double)d.c * d.d[k];
      tm.e.assign(d.e, d.e + d_out);
      terms.push_back(std::move(tm));
    }
  }
  const bool has_R = members[0].method == TPA_OFT;
  const bool one_shared = terms.size() == 1 && terms[0].shared;
  int r_tot = 0;
  for (const StackTerm& tm : terms) r_tot += tm.r;
  const int r_pad = one_shared ? 0 : round_up(r_tot, 16);
  if (!one_shared && r_tot > L->max_rank)
    return fail(TPA_ERR_INVALID, "stacked rank %d exceeds max_rank=%d", r_tot, L->max_rank);
  const int cls = terms.empty() ? tpa::CLS_NONE : one_shared ? tpa::CLS_SHARED : tpa::CLS_OWNED;

  // Owned form of every term: A_all [d_in][r_tot] and B_all [r_tot][d_out]
  // with e folded into B (a shared term through A_v diag(c·d), B_v).
  std::vector<float> A_all, B_all;
  if (cls == tpa::CLS_OWNED) {
    std::vector<double> Av, Bv;  // the layer's pair as stored: [r_v][d_in], [d_out][r_v]
    for (const StackTerm& tm : terms)
      if (tm.shared && Av.empty()) {
        if (tpa_status e = fetch_matrix(L, L->vera_At, (size_t)L->r_v * d_in, &Av)) return e;
        if (tpa_status e = fetch_matrix(L, L->vera_Bt, (size_t)d_out * L->r_v, &Bv)) return e;
      }
    A_all.assign((size_t)d_in * r_tot, 0.f);
    B_all.assign((size_t)r_tot * d_out, 0.f);
    int k0 = 0;
    for (const StackTerm& tm : terms) {
      for (int i = 0; i < d_in; ++i)
        for (int k = 0; k < tm.r; ++k)
          A_all[(size_t)i * r_tot + k0 + k] =
              (float)(tm.shared ? Av[(size_t)k * d_in + i] * tm.dv[k] : tm.A[(size_t)i * tm.r + k]);
      for (int k = 0; k < tm.r; ++k)
        for (int c = 0; c < d_out; ++c)
          B_all[(size_t)(k0 + k) * d_out + c] =
              (float)((tm.shared ? Bv[(size_t)c * L->r_v + k] : tm.B[(size_t)k * d_out + c]) * tm.e[c]);
      if (tm.shared) fold_mask |= TPA_FOLD_D_A;
      if (!tm.e_unit) fold_mask |= TPA_FOLD_E_B;
      k0 += tm.r;
    }
  } else if (cls == tpa::CLS_SHARED) {
    fold_mask |= TPA_FOLD_C_D;
  }

  const size_t esz = tpa::dtype_size(L->dtype);
  size_t off = 0;
  size_t o_At = 0, o_Bt = 0, o_s = 0, o_b = 0, o_d = 0, o_e = 0, o_R = 0;
  auto take = [&](size_t bytes) {
    size_t at = off;
    off = align256(off + bytes);
    return at;
  };
  if (cls == tpa::CLS_OWNED) {
    o_At = take((size_t)r_pad * d_in * esz);
    o_Bt = take((size_t)d_out * r_pad * esz);
  }
  if (!S.empty()) o_s = take((size_t)d_out * 4);
  if (!Bsh.empty()) o_b = take((size_t)d_out * 4);
  if (cls == tpa::CLS_SHARED) {
    o_d = take((size_t)L->r_v * 4);
    o_e = take((size_t)d_out * 4);
  }
  const int bs = has_R ? members[0].oft_block : 0;
  if (has_R) o_R = take((size_t)d_in * bs * esz);
  void* mem = nullptr;
  if (off) TPA_HIP(L->arena.take(off, &mem));
  char* base = static_cast<char*>(mem);
  SlotDev sd{};
  sd.cls = cls;
  auto upload = [&]() -> tpa_status {
    auto pad = [](size_t c) { return (std::max<size_t>(c, 1) + 63) / 64 * 64; };
    Staging st{L};
    size_t need = has_R ? pad((size_t)d_in * bs) : 0;
    if (cls == tpa::CLS_OWNED) need += pad(A_all.size()) + pad(B_all.size());
    if (tpa_status e = st.reserve(need)) return e;
    auto to_f32 = [](const std::vector<double>& v) { return std::vector<float>(v.begin(), v.end()); };
    std::vector<float> s32 = to_f32(S), b32 = to_f32(Bsh), dd, ee;
    if (cls == tpa::CLS_OWNED) {
      float *a32, *bb32;
      if (tpa_status e = st.put(A_all.data(), A_all.size(), &a32, s)) return e;
      if (tpa_status e = st.put(B_all.data(), B_all.size(), &bb32, s)) return e;
      // A_all [d_in][r_tot] -> [r_pad][d_in];  B_all [r_tot][d_out] -> [d_out][r_pad].
      TPA_HIP(tpa::launch_pack_transpose(L->dtype, a32, d_in, r_tot, 1.f, nullptr, base + o_At, r_pad, d_in, s));
      TPA_HIP(tpa::launch_pack_transpose(L->dtype, bb32, r_tot, d_out, 1.f, nullptr, base + o_Bt, d_out, r_pad, s));
      sd.A = base + o_At;
      sd.Bt = base + o_Bt;
      sd.rank = r_pad;
    } else if (cls == tpa::CLS_SHARED) {
      dd = to_f32(terms[0].dv);
      ee = to_f32(terms[0].e);
      TPA_HIP(hipMemcpyAsync(base + o_d, dd.data(), dd.size() * 4, hipMemcpyHostToDevice, s));
      TPA_HIP(hipMemcpyAsync(base + o_e, ee.data(), ee.size() * 4, hipMemcpyHostToDevice, s));
      sd.d = reinterpret_cast<float*>(base + o_d);
      sd.e = reinterpret_cast<float*>(base + o_e);
      sd.rank = L->r_v;
    }
    if (!S.empty()) {
      TPA_HIP(hipMemcpyAsync(base + o_s, s32.data(), s32.size() * 4, hipMemcpyHostToDevice, s));
      sd.s = reinterpret_cast<float*>(base + o_s);
    }
    if (!Bsh.empty()) {
      TPA_HIP(hipMemcpyAsync(base + o_b, b32.data(), b32.size() * 4, hipMemcpyHostToDevice, s));
      sd.b = reinterpret_cast<float*>(base + o_b);
    }
    if (has_R) {
      const size_t cnt = (size_t)d_in * bs;
      std::vector<float> rt(cnt);
      for (int j = 0; j < d_in / bs; ++j)
        cayley_transposed(members[0].Q + (size_t)j * bs * bs, bs, rt.data() + (size_t)j * bs * bs);
      float* r32;
      if (tpa_status e = st.put(rt.data(), cnt, &r32, s)) return e;
      TPA_HIP(tpa::launch_convert(L->dtype, r32, base + o_R, cnt, 1.f, s));
      sd.Rt = base + o_R;
      sd.has_R = 1;
      sd.oft_block = bs;
    }
    TPA_HIP(hipStreamSynchronize(s));  // host vectors above must outlive the copies
    return TPA_OK;
  };
  tpa_status err = upload();
  if (!err) {
    L->slots_host[slot] = sd;
    err = upload_slot(L, slot, s);
    if (err) {
      L->slots_host[slot] = SlotDev{};
      L->slots_host[slot].cls = -1;
    }
  }
  if (err) {
    (void)hipStreamSynchronize(s);
    if (mem) L->arena.give(mem, off);
    return err;
  }
  HostSlot& h = L->hs[slot];
  h.used = true;
  h.mem = mem;
  h.bytes = off;
  h.info = tpa_adapter_info{};
  h.info.method = count == 1 ? members[0].method : TPA_STACK;
  h.info.term_kind = cls == tpa::CLS_OWNED ? 1 : cls == tpa::CLS_SHARED ? 2 : 0;
  h.info.rank = cls == tpa::CLS_OWNED ? r_tot : cls == tpa::CLS_SHARED ? L->r_v : 0;
  h.info.oft_block = bs;
  h.info.fold_mask = fold_mask;
  h.info.live_mask = (S.empty() ? 0 : TPA_LIVE_S) | (Bsh.empty() ? 0 : TPA_LIVE_B) | (has_R ? TPA_LIVE_R : 0) |
                     (cls == tpa::CLS_SHARED ? TPA_LIVE_D | TPA_LIVE_E : 0);
  if (cls == tpa::CLS_OWNED) ++L->n_owned;
  if (cls == tpa::CLS_SHARED) ++L->n_vera;
  if (count > 1) ++L->n_stack;
  if (has_R) ++L->n_oft_bs[oft_bs_index(bs)];
  update_plan_sig(L);
  *slot_out = slot;
  return TPA_OK;
}

tpa_status tpa_adapter_unload(tpa_layer* L, int32_t slot, tpa_stream stream) {
  if (tpa_status st = check_layer(L)) return st;
  if (slot <= 0 || slot >= L->max_slots || !L->hs[slot].used) return fail(TPA_ERR_UNKNOWN_SLOT, "slot %d is not loaded", slot);
  DeviceGuard guard(L->device);
  hipStream_t s = static_cast<hipStream_t>(stream);
  TPA_HIP(hipStreamSynchronize(s));
  const tpa_adapter_info info = L->hs[slot].info;
  L->slots_host[slot] = SlotDev{};
  L->slots_host[slot].cls = -1;
  if (tpa_status e = upload_slot(L, slot, s)) return e;
  if (L->hs[slot].mem) L->arena.give(L->hs[slot].mem, L->hs[slot].bytes);
  L->hs[slot] = HostSlot{};
  if (info.term_kind == 1) --L->n_owned;
  if (info.term_kind == 2) --L->n_vera;
  if (info.method == TPA_DORA) --L->n_dora;
  if (info.method == TPA_STACK) --L->n_stack;
  if (info.live_mask & TPA_LIVE_R) --L->n_oft_bs[oft_bs_index(info.oft_block)];
  update_plan_sig(L);
  return TPA_OK;
}

tpa_status tpa_adapter_info_get(const tpa_layer* L, int32_t slot, tpa_adapter_info* out) {
  if (tpa_status st = check_layer(L)) return st;
  if (!out) return fail(TPA_ERR_INVALID, "null output");
  if (slot < 0 || slot >= L->max_slots || !L->hs[slot].used) return fail(TPA_ERR_UNKNOWN_SLOT, "slot %d is not loaded", slot);
  *out = L->hs[slot].info;
  return TPA_OK;
}

tpa_status tpa_workspace_size(const tpa_layer* L, int32_t n_max, size_t* bytes) {
  if (tpa_status st = check_layer(L)) return st;
  if (!bytes || n_max < 0 || n_max > tpa::PLAN_MAX_ROWS)
    return fail(TPA_ERR_INVALID, "n_max must be in [0, %d]", tpa::PLAN_MAX_ROWS);
  if (n_max == 0) {
    *bytes = 0;
    return TPA_OK;
  }
  // Split and tile choices depend on n, so take the largest layout of any
  // batch size up to n_max.
  size_t best = 0;
  for (int n = 1; n <= n_max; ++n) best = std::max(best, make_layout(L, n, choose_config(L, n)).total);
  *bytes = best;
  return TPA_OK;
}

tpa_status tpa_plan_max_tiles(const tpa_layer* L, int32_t n, int32_t* max_tiles, int32_t* tile_rows) {
  if (tpa_status st = check_layer(L)) return st;
  if (n < 0 || n > tpa::PLAN_MAX_ROWS) return fail(TPA_ERR_INVALID, "bad n");
  const Config c = choose_config(L, std::max(n, 1));
  if (max_tiles) *max_tiles = max_tiles_for(L, n, c.tile_rows);
  if (tile_rows) *tile_rows = c.tile_rows;
  return TPA_OK;
}

}  // extern "C"

namespace {

// One projection of a forward: its layer, input, output, workspace and the
// kernel configuration and workspace layout it runs with.
struct SliceCtx {
  tpa_layer* L;
  const void* x;
  void* out;
  char* w;
  Layout y;
  Config c;
};

// Configurations of projections forwarded together with one plan: on the
// decode path their base GEMMs share one launch, so they take one column-block
// width (that of the widest projection, when it divides every d_out), one
// k-group count and one k range, chosen as for one projection but over the
// combined grid (a split pinned on the first projection is kept).
// The fused decode epilogue is a property of the group's launches (the
// shrink's mode and the GEMM's): all projections take it or none does.
void uniform_fused_dec(tpa_layer* const* Ls, int count, Config* cs, bool allowed) {
  bool all = allowed;
  for (int i = 0; i < count; ++i) all = all && cs[i].fused_dec;
  for (int i = 0; i < count; ++i) {
    cs[i].fused_dec = all ? 1 : 0;
    cs[i].h_fp32 = Ls[i]->n_stack > 0 && !cs[i].fused && !cs[i].fused_dec;
  }
}

void group_configs(tpa_layer* const* Ls, int count, int n, Config* cs) {
  for (int i = 0; i < count; ++i) cs[i] = choose_config(Ls[i], n);
  if (count < 2) return;
  for (int i = 0; i < count; ++i)
    if (cs[i].gemm_path != cs[0].gemm_path || !decode_path(cs[i])) {
      uniform_fused_dec(Ls, count, cs, false);
      return;
    }
  const bool stream = cs[0].gemm_path == 2;
  int ref = 0;
  for (int i = 1; i < count; ++i)
    if (Ls[i]->d_out > Ls[ref]->d_out) ref = i;
  int nb = cs[ref].gemm_nb;
  for (int i = 0; i < count; ++i)
    if (Ls[i]->d_out % (64 * nb)) nb = 1;
  int G = cs[0].gemm_groups, S = cs[0].gemm_stages;
  int kc = 64;
  if (stream) {
    while (S > 3 && tpa::gemm_stream_lds(n, nb, 1, S) > tpa::GEMM_STREAM_MAX_LDS) S = S == 6 ? 4 : 3;
    stream_pick(Ls, count, n, nb, S, Ls[0]->opt[TPA_OPT_GEMM_GROUPS], &G, &kc);
  }
  if (Ls[0]->opt[TPA_OPT_GEMM_SPLIT] > 0) {
    kc = round_up((Ls[0]->d_in + Ls[0]->opt[TPA_OPT_GEMM_SPLIT] - 1) / Ls[0]->opt[TPA_OPT_GEMM_SPLIT],
                  64 * (stream ? G : 1));
    if (!stream)
      while (kc > 64 && tpa::gemm_skinny_lds(Ls[0]->dtype, n, nb, G, kc) > tpa::GEMM_SKINNY_MAX_LDS) kc -= 64;
  } else if (!stream) {
    for (int cand : {1024, 512, 256, 128, 64}) {
      if (tpa::gemm_skinny_lds(Ls[0]->dtype, n, nb, G, cand) > tpa::GEMM_SKINNY_MAX_LDS) continue;
      kc = cand;
      long wgs = 0;
      for (int i = 0; i < count; ++i) wgs += (long)(Ls[i]->d_out / (64 * nb)) * ((Ls[i]->d_in + cand - 1) / cand);
      if (wgs >= 200) break;
    }
  }
  bool fits = stream && S == 3;
  for (int i = 0; i < count; ++i) {
    cs[i].gemm_nb = nb;
    cs[i].gemm_groups = G;
    cs[i].gemm_stages = S;
    cs[i].gemm_kc = std::min(kc, round_up(Ls[i]->d_in, 64 * (stream ? G : 1)));
    cs[i].gemm_split = (Ls[i]->d_in + cs[i].gemm_kc - 1) / cs[i].gemm_kc;
    if (cs[i].shrink_in_gemm) set_shrink_split(Ls[i], n, &cs[i]);  // one k range per wave of the launch's groups
    fits = fits && fused_dec_fits(Ls[i], n, cs[i]);
  }
  // (a shrink capped for the fused epilogue stays valid without it)
  uniform_fused_dec(Ls, count, cs, fits);
}

// Everything after the plan, for `count` projections that share it: the
// shrink with OFT's rotation, the base GEMM (with the shrink's split
// reduction), the expand (and any separate scale pass).  Each kernel is one
// launch over all projections whose configurations allow it.  Stage events
// are those of the first projection's layer.
tpa_status forward_group_after_plan(SliceCtx* sl, int count, const tpa::PlanArgs& p, int n, hipStream_t s,
                                    bool allow_side = true) {
  tpa_layer* L0 = sl[0].L;
  const int dtype = L0->dtype;
  const int tile_rows = sl[0].c.tile_rows;
  const int ncb = sl[0].c.shrink_ncb;  // one shrink launch: the first projection's item width for all
  tpa::ShrinkArgs sh[tpa::MAX_SLICES];
  tpa::OftArgs of[tpa::MAX_SLICES];
  bool term[tpa::MAX_SLICES], oft[tpa::MAX_SLICES];
  bool any_term_all = false;
  for (int i = 0; i < count; ++i) {
    tpa_layer* L = sl[i].L;
    const Layout& y = sl[i].y;
    const Config& c = sl[i].c;
    term[i] = L->n_owned > 0 || L->n_vera > 0;
    oft[i] = L->n_oft_bs[0] + L->n_oft_bs[1] + L->n_oft_bs[2] > 0;
    any_term_all = any_term_all || term[i];
    sh[i] = tpa::ShrinkArgs{};
    if (term[i]) {
      sh[i].x = sl[i].x;
      sh[i].pinfo = p.pinfo;
      sh[i].tiles = p.tiles;
      sh[i].slots = L->slots_dev;
      sh[i].vera_At = L->vera_At;
      sh[i].r_v = L->r_v;
      sh[i].n = n;
      sh[i].d_in = L->d_in;
      sh[i].kmax = L->kmax;
      sh[i].sh_tiles = p.sh_tiles;
      sh[i].tile_rows_w = p.tile_rows_w;
      sh[i].sh_rows_w = p.sh_rows_w;
      sh[i].own_tiles = owned_tile_bound(L, n, tile_rows, y.max_tiles);
      sh[i].own_nblk = std::max(1, (L->max_owned_rank + 16 * ncb - 1) / (16 * ncb));
      sh[i].sh_ntiles = L->n_vera > 0 ? y.max_sh_tiles : 0;
      sh[i].sh_nblk = std::max(1, (L->r_v + 16 * ncb - 1) / (16 * ncb));
      sh[i].split = c.shrink_split;
      sh[i].kc = c.shrink_kc;
      sh[i].part = reinterpret_cast<float*>(sl[i].w + y.vpart);
      sh[i].v = sl[i].w + y.v;
    }
    sh[i].part_shared = nullptr;
    sh[i].kmax_shared = 0;
    sh[i].borrows = 0;
    of[i] = tpa::OftArgs{};
    of[i].x = sl[i].x;
    of[i].oft_tiles = p.oft_tiles;
    of[i].oft_rows_w = p.oft_rows_w;
    of[i].slots = L->slots_dev;
    of[i].x_rot = sl[i].w + y.x_rot;
    of[i].d_in = L->d_in;
    of[i].max_tiles = oft_tile_bound(L, n, tile_rows, y.max_tiles);
    // One block per wave at decode sizes, where the launch is a chain of
    // round trips (q/k/v of the decoder layer at 64 rows: 180.3 -> 178.5 µs
    // per step); four per wave above, where more, smaller work-groups lost
    // more than they overlapped (2-layer stack cut at 4096 rows +0.9%).
    of[i].bpw = n <= 64 ? 4 : 16;
  }

  // VeRA's A_v read once per fused input (Table 2's route-two count; the
  // appendix "Byte counts"): a projection of the group whose layer holds the
  // first projection's A_v and reads the same input computes no x·A_vᵀ of
  // its own; its reduction takes the first projection's partials and
  // applies its own d'.  Same bits as computing them again.
  // The expand in the decode GEMM's epilogue (all projections of the group
  // or none, by their configurations): the shrink then runs whole-k, and a
  // launch before the GEMM clears its arrival counters (the shrink's or
  // OFT's; with k whole in the GEMM no counter is read).
  bool any_oft = false, all_unsplit = true;
  for (int i = 0; i < count; ++i) {
    any_oft = any_oft || oft[i];
    all_unsplit = all_unsplit && sl[i].c.gemm_split == 1;
  }
  const bool fdec = sl[0].c.fused_dec && (any_term_all || any_oft || all_unsplit);
  // Decode projections on the streamed GEMM: the shrink runs in the GEMM's
  // side work-groups (every projection of the group or none); OFT's
  // rotation keeps its launch before the GEMM.
  bool sgemm = !fdec && any_term_all;
  for (int i = 0; i < count; ++i)
    sgemm = sgemm && sl[i].c.shrink_in_gemm && sl[i].c.shrink_ncb == 1 && sl[i].c.gemm_path == 2;
  for (int i = 1; i < count; ++i) {
    const tpa_layer* L = sl[i].L;
    if (term[i] && term[0] && L->n_vera > 0 && L0->n_vera > 0 && L->vera_At && L->vera_At == L0->vera_At &&
        sl[i].x == sl[0].x && L->r_v == L0->r_v && sh[i].split == sh[0].split && sh[i].kc == sh[0].kc) {
      sh[i].sh_ntiles = 0;
      if (fdec || sgemm) {
        sh[i].borrows = 1;
      } else {
        sh[i].part_shared = sh[0].part;
        sh[i].kmax_shared = sh[0].kmax;
      }
    }
  }
  int32_t* cnt[tpa::MAX_SLICES];
  for (int i = 0; i < count; ++i)
    cnt[i] = fdec && sl[i].c.gemm_split > 1 ? reinterpret_cast<int32_t*>(sl[i].w + sl[i].y.cnt) : nullptr;
  bool cnt_cleared = false;
  auto clear_counters = [&](tpa::PreSlice* ps) {
    if (cnt_cleared) return;
    for (int i = 0; i < count; ++i) {
      ps[i].zero = cnt[i];
      ps[i].zero_n = cnt[i] ? sl[i].L->d_out / (64 * sl[i].c.gemm_nb) : 0;
    }
    cnt_cleared = true;
  };

  // 2. The shrink and OFT's rotation: one launch per OFT block size present
  //    (the shrink rides in the first), or one for the shrink alone.  With
  //    overlap on, the shrink and its split reduction run on the layer's
  //    second stream beside OFT's rotation and the base GEMM (neither reads
  //    V or U), and the expand waits for them.  Only when asked for
  //    (TPA_OPT_OVERLAP = 1): in a graph-replayed decode step the fork and
  //    join cost more than the launch they hide (222 vs 202 µs per decoder
  //    layer), and larger batches gain 1-4% (2-layer cut of the
  //    1024-tenant Zipf stack: 192 rows 442.5 -> 436-437 µs per layer,
  //    1024 rows 1203-1219 -> 1156-1159, 4096 rows 2890 -> 2876-2879).
  //    Never where the expand rides in the GEMM's epilogue: that GEMM reads
  //    V and U, so nothing could overlap.  The second stream and its events
  //    are made on first use, outside graph capture (a captured forward
  //    before then runs on one stream; both orders give the same bits).
  bool any_fused_cfg = fdec;
  for (int i = 0; i < count; ++i) any_fused_cfg = any_fused_cfg || sl[i].c.fused;
  const int ov_opt = L0->opt[TPA_OPT_OVERLAP];
  bool overlap = allow_side && any_term_all && !any_fused_cfg && ov_opt == 1;
  if (overlap && !(L0->side && L0->ev_fork && L0->ev_join)) {
    hipStreamCaptureStatus cap = hipStreamCaptureStatusActive;
    if (hipStreamIsCapturing(s, &cap) != hipSuccess) {
      (void)hipGetLastError();
      cap = hipStreamCaptureStatusActive;
    }
    overlap = cap == hipStreamCaptureStatusNone;
  }
  if (overlap) {
    if (!L0->side) TPA_HIP(hipStreamCreateWithFlags(&L0->side, hipStreamNonBlocking));
    if (!L0->ev_fork) TPA_HIP(hipEventCreateWithFlags(&L0->ev_fork, hipEventDisableTiming));
    if (!L0->ev_join) TPA_HIP(hipEventCreateWithFlags(&L0->ev_join, hipEventDisableTiming));
    TPA_HIP(hipEventRecord(L0->ev_fork, s));
    TPA_HIP(hipStreamWaitEvent(L0->side, L0->ev_fork, 0));
    tpa::PreSlice ps[tpa::MAX_SLICES];
    for (int i = 0; i < count; ++i) ps[i] = tpa::make_pre_slice(term[i] ? &sh[i] : nullptr, nullptr);
    TPA_HIP(tpa::launch_pre(dtype, tile_rows, 0, ps, count, L0->side, false, ncb));
    for (int i = 0; i < count; ++i)
      if (term[i]) TPA_HIP(tpa::launch_shrink_reduce(dtype, sh[i], L0->side));
    TPA_HIP(hipEventRecord(L0->ev_join, L0->side));
  }
  static const int kBs[3] = {16, 32, 64};
  tpa::PreSlice ps[tpa::MAX_SLICES];
  bool sh_done = overlap;
  for (int b = 0; b < 3; ++b) {
    bool any = false;
    for (int i = 0; i < count; ++i) any = any || sl[i].L->n_oft_bs[b] > 0;
    if (!any) continue;
    for (int i = 0; i < count; ++i) {
      of[i].block = kBs[b];
      ps[i] = tpa::make_pre_slice(!sh_done && !sgemm && term[i] ? &sh[i] : nullptr,
                                  sl[i].L->n_oft_bs[b] ? &of[i] : nullptr, fdec);
    }
    if (fdec) clear_counters(ps);
    TPA_HIP(tpa::launch_pre(dtype, tile_rows, kBs[b], ps, count, s, fdec, ncb));
    sh_done = true;
  }
  if (!sh_done && any_term_all && !sgemm) {
    for (int i = 0; i < count; ++i) ps[i] = tpa::make_pre_slice(term[i] ? &sh[i] : nullptr, nullptr, fdec);
    if (fdec) clear_counters(ps);
    TPA_HIP(tpa::launch_pre(dtype, tile_rows, 0, ps, count, s, fdec, ncb));
  }
  if (tpa_status st = stage(L0, 2, s)) return st;

  auto expand_args = [&](int i) {
    tpa_layer* L = sl[i].L;
    const Config& c = sl[i].c;
    tpa::ExpandArgs ea{};
    ea.out = sl[i].out;
    ea.hpart = nullptr;
    ea.hsplit = c.gemm_split;
    ea.tiles = p.tiles;
    ea.tile_rows_w = p.tile_rows_w;
    ea.slots = L->slots_dev;
    ea.vera_Bt = L->vera_Bt;
    ea.r_v = L->r_v;
    ea.v = sl[i].w + sl[i].y.v;
    ea.kmax = L->kmax;
    ea.n = n;
    ea.d_out = L->d_out;
    ea.max_tiles = all_tile_bound(L, n, tile_rows, sl[i].y.max_tiles);
    ea.apply_scale = c.scale_route == 0;
    ea.sh_tiles = L->n_vera > 0 ? p.sh_tiles : nullptr;
    ea.sh_rows_w = L->n_vera > 0 ? p.sh_rows_w : nullptr;
    ea.max_sh_tiles = L->n_vera > 0 ? p.max_sh_tiles : 0;
    return ea;
  };

  // 3. Base GEMM.  Decode path: one launch over the projections (they share
  //    the column-block width and k-groups), the shrink's split reduction
  //    riding in the same grid; otherwise the LDS-tiled kernel per projection.
  tpa::GemmSlice gs[tpa::MAX_SLICES];
  bool one_launch = true;
  for (int i = 0; i < count; ++i) {
    const Config& c = sl[i].c;
    tpa_layer* L = sl[i].L;
    tpa::BaseGemmArgs& g = gs[i].g;
    g = tpa::BaseGemmArgs{};
    g.x = sl[i].x;
    g.x_rot = oft[i] ? sl[i].w + sl[i].y.x_rot : nullptr;
    g.rot_pos = oft[i] ? p.rot_pos : nullptr;
    g.W = L->W;
    g.n = n;
    g.d_in = L->d_in;
    g.d_out = L->d_out;
    g.split = c.gemm_split;
    g.h_fp32 = c.h_fp32;
    g.kc = c.gemm_kc;
    g.part = reinterpret_cast<float*>(sl[i].w + sl[i].y.hpart);
    g.out = sl[i].out;
    gs[i].side = sh[i];
    gs[i].has_side = term[i] && !overlap && !fdec ? 1 : 0;
    gs[i].side_whole = sgemm ? 1 : 0;
    gs[i].e = tpa::ExpandArgs{};
    gs[i].pinfo = nullptr;
    gs[i].cnt = nullptr;
    if (fdec) {
      gs[i].e = expand_args(i);
      gs[i].pinfo = p.pinfo;
      gs[i].cnt = cnt[i];
    }
    if (c.gemm_path != sl[0].c.gemm_path || !decode_path(c) || c.gemm_nb != sl[0].c.gemm_nb ||
        c.gemm_groups != sl[0].c.gemm_groups || (c.gemm_path == 2 && c.gemm_stages != sl[0].c.gemm_stages))
      one_launch = false;
  }
  // Prefill projections on 256 x 256 tiles (gate and up) share one launch:
  // their tiles fill whole rounds of the grid together where each alone
  // leaves the last round half empty.
  bool big_group = count > 1;
  for (int i = 0; i < count; ++i)
    big_group = big_group && sl[i].c.gemm_path == 3 && sl[i].c.gemm_tile == 256 && !sl[i].c.fused &&
                sl[i].c.gemm_split == sl[0].c.gemm_split;
  if (big_group) {
    TPA_HIP(tpa::launch_gemm_big(dtype, gs, count, s));  // carries the shrinks' reductions
  } else if (one_launch) {
    if (sl[0].c.gemm_path == 2)
      TPA_HIP(tpa::launch_gemm_stream(dtype, sl[0].c.gemm_nb, sl[0].c.gemm_groups, sl[0].c.gemm_stages, gs, count, s,
                                      fdec));
    else
      TPA_HIP(tpa::launch_gemm_skinny(dtype, sl[0].c.gemm_nb, sl[0].c.gemm_groups, gs, count, s));
  } else {
    for (int i = 0; i < count; ++i) {
      const Config& c = sl[i].c;
      if (c.gemm_path == 2) {
        TPA_HIP(tpa::launch_gemm_stream(dtype, c.gemm_nb, c.gemm_groups, c.gemm_stages, &gs[i], 1, s, fdec));
      } else if (c.gemm_path == 0) {
        TPA_HIP(tpa::launch_gemm_skinny(dtype, c.gemm_nb, c.gemm_groups, &gs[i], 1, s));
      } else {
        if (c.fused) {
          // launched with the expand's arguments below
        } else if (c.gemm_path == 3 && c.gemm_tile == 256) {
          TPA_HIP(tpa::launch_gemm_big(dtype, &gs[i], 1, s));  // carries the shrink's reduction
        } else if (c.gemm_path == 3) {
          TPA_HIP(tpa::launch_gemm_wide(dtype, c.gemm_stages, gs[i], s));  // carries the shrink's reduction
        } else {
          TPA_HIP(tpa::launch_gemm_tiled(dtype, gs[i].g, s));
          if (term[i] && !overlap) TPA_HIP(tpa::launch_shrink_reduce(dtype, sh[i], s));
        }
      }
    }
  }
  // Join the side stream here, so the stage event after the GEMM also
  // covers the shrink that ran beside it (only the expand reads V and U).
  if (overlap) TPA_HIP(hipStreamWaitEvent(s, L0->ev_join, 0));
  if (tpa_status st = stage(L0, 3, s)) return st;

  // 4. Expand (with the comparison routes' separate scale passes), unless
  //    the GEMM's epilogue ran it.
  if (fdec) {
    if (tpa_status st = stage(L0, 4, s)) return st;
    return stage(L0, 5, s);
  }
  tpa::ExpandArgs e[tpa::MAX_SLICES];
  tpa::ScaleArgs sc[tpa::MAX_SLICES];
  for (int i = 0; i < count; ++i) {
    tpa_layer* L = sl[i].L;
    const Config& c = sl[i].c;
    const bool hsplit = h_partials(c);
    sc[i] = tpa::ScaleArgs{};
    sc[i].y = sl[i].out;
    sc[i].hpart = hsplit ? reinterpret_cast<const float*>(sl[i].w + sl[i].y.hpart) : nullptr;
    sc[i].hsplit = c.gemm_split;
    sc[i].row_slot = p.row_slot;
    sc[i].slots = L->slots_dev;
    sc[i].srow = reinterpret_cast<float*>(sl[i].w + sl[i].y.srow);
    sc[i].n = n;
    sc[i].d_out = L->d_out;
    bool h_in_out = !hsplit;
    if (c.scale_route == 1) {  // side kernel: h ⊙ s + b written before the expand
      TPA_HIP(tpa::launch_scale_pass(dtype, 1, sc[i], s));
      h_in_out = true;
    }
    e[i] = expand_args(i);
    e[i].hpart = h_in_out ? nullptr : reinterpret_cast<const float*>(sl[i].w + sl[i].y.hpart);
    if (c.fused) {
      // The shrink's reduction as a launch of its own (V / U must be final
      // before the GEMM's epilogue reads them), then the GEMM with the
      // expand in its epilogue over the plan's tiles.
      if (term[i]) TPA_HIP(tpa::launch_shrink_reduce(dtype, sh[i], s));
      tpa::FusedArgs f{};
      f.g = gs[i].g;
      f.e = e[i];
      f.list_tiles = p.max_tiles;
      f.row_tiles = (std::min(e[i].max_tiles, p.max_tiles) + 7) / 8;
      f.col_tiles = L->d_out / 128;
      TPA_HIP(tpa::launch_gemm_fused(dtype, c.gemm_stages, f, s));
    }
  }
  if (tpa_status st = stage(L0, 4, s)) return st;
  bool same_h = true, any_fused = false;
  for (int i = 0; i < count; ++i) {
    same_h = same_h && ((e[i].hpart != nullptr) == (e[0].hpart != nullptr));
    any_fused = any_fused || sl[i].c.fused;
  }
  if (same_h && !any_fused) {
    TPA_HIP(tpa::launch_expand(dtype, tile_rows, e, count, s));
  } else {
    for (int i = 0; i < count; ++i)
      if (!sl[i].c.fused) TPA_HIP(tpa::launch_expand(dtype, tile_rows, &e[i], 1, s));
  }
  for (int i = 0; i < count; ++i) {
    sc[i].hpart = nullptr;
    if (sl[i].c.scale_route == 2) TPA_HIP(tpa::launch_scale_pass(dtype, 2, sc[i], s));
    if (sl[i].c.scale_route == 3) {
      TPA_HIP(tpa::launch_scale_pass(dtype, 3, sc[i], s));
      TPA_HIP(tpa::launch_scale_pass(dtype, 4, sc[i], s));
    }
  }
  return stage(L0, 5, s);
}

tpa_status forward_after_plan(tpa_layer* L, const tpa::PlanArgs& p, const void* x, int n, void* out, char* w,
                              const Layout& y, const Config& c, hipStream_t s, bool allow_side = true) {
  SliceCtx one{L, x, out, w, y, c};
  return forward_group_after_plan(&one, 1, p, n, s, allow_side);
}

}  // namespace

extern "C" {

tpa_status tpa_layer_forward(tpa_layer* L, const void* x, const int32_t* sor, int32_t n, void* out, void* ws,
                             size_t ws_bytes, tpa_stream stream) {
  if (tpa_status st = check_layer(L)) return st;
  if (n < 0 || n > tpa::PLAN_MAX_ROWS) return fail(TPA_ERR_INVALID, "n=%d outside [0, %d]", n, tpa::PLAN_MAX_ROWS);
  if (n == 0) return TPA_OK;
  if (!x || !sor || !out || !ws) return fail(TPA_ERR_INVALID, "null pointer");
  if (reinterpret_cast<uintptr_t>(ws) & 255) return fail(TPA_ERR_INVALID, "workspace must be 256-byte aligned");
  if (x == out) return fail(TPA_ERR_INVALID, "out may not alias x");
  const Config c = choose_config(L, n);
  const Layout y = make_layout(L, n, c);
  if (ws_bytes < y.total) return fail(TPA_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, y.total);
  DeviceGuard guard(L->device);
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* w = static_cast<char*>(ws);
  const tpa::PlanArgs p = plan_args(L, sor, n, w, y, c);
  if (tpa_status st = stage(L, 0, s)) return st;
  TPA_HIP(tpa::launch_plan(p, s));
  if (tpa_status st = stage(L, 1, s)) return st;
  return forward_after_plan(L, p, x, n, out, w, y, c, s);
}

tpa_status tpa_layer_forward_noalloc(tpa_layer* L, const void* x, const int32_t* sor, int32_t n, void* out,
                                     tpa_stream stream) {
  if (tpa_status st = check_layer(L)) return st;
  if (n < 0 || n > tpa::PLAN_MAX_ROWS) return fail(TPA_ERR_INVALID, "n=%d outside [0, %d]", n, tpa::PLAN_MAX_ROWS);
  if (n == 0) return TPA_OK;
  if (!x || !sor || !out) return fail(TPA_ERR_INVALID, "null pointer");
  if (x == out) return fail(TPA_ERR_INVALID, "out may not alias x");
  const Config c = choose_config(L, n);
  const Layout y = make_layout(L, n, c);
  if (y.total > (size_t)TPA_NOALLOC_SCRATCH_BYTES)
    return fail(TPA_ERR_WORKSPACE, "a forward of %d rows on this layer needs %zu bytes of workspace, more than the "
                "%zu bytes of scratch the no-allocation forward holds", n, y.total, (size_t)TPA_NOALLOC_SCRATCH_BYTES);
  DeviceGuard guard(L->device);
  void* ws = nullptr;
  if (tpa_status st = scratch_address(L->device, &ws)) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* w = static_cast<char*>(ws);
  // Nothing in the workspace needs clearing: the plan kernel writes every
  // entry later kernels read, and the GEMM and shrink write their partials
  // before they are summed.  The shrink stays on `stream` (no second stream
  // or event is created), which gives the same bits as the overlapped order.
  const tpa::PlanArgs p = plan_args(L, sor, n, w, y, c);
  if (tpa_status st = stage(L, 0, s)) return st;
  TPA_HIP(tpa::launch_plan(p, s));
  if (tpa_status st = stage(L, 1, s)) return st;
  return forward_after_plan(L, p, x, n, out, w, y, c, s, false);
}

tpa_status tpa_layer_plan_signature(const tpa_layer* L, uint64_t* sig) {
  if (tpa_status st = check_layer(L)) return st;
  if (!sig) return fail(TPA_ERR_INVALID, "null output");
  *sig = L->plan_sig;
  return TPA_OK;
}

tpa_status tpa_plan_accepts(const tpa_plan* plan, const tpa_layer* L, int32_t* ok) {
  if (tpa_status st = check_layer(L)) return st;
  if (!plan || !ok) return fail(TPA_ERR_INVALID, "null argument");
  *ok = plan->built && plan_accepts(plan, L) ? 1 : 0;
  return TPA_OK;
}

tpa_status tpa_plan_create(tpa_plan** out) {
  if (!out) return fail(TPA_ERR_INVALID, "null output");
  *out = new tpa_plan();
  return TPA_OK;
}

tpa_status tpa_plan_destroy(tpa_plan* plan) {
  delete plan;
  return TPA_OK;
}

tpa_status tpa_plan_size(const tpa_layer* L, int32_t n_max, size_t* bytes) {
  if (tpa_status st = check_layer(L)) return st;
  if (!bytes || n_max < 0 || n_max > tpa::PLAN_MAX_ROWS)
    return fail(TPA_ERR_INVALID, "n_max must be in [0, %d]", tpa::PLAN_MAX_ROWS);
  size_t best = 0;
  for (int n = 1; n <= n_max; ++n) best = std::max(best, make_layout(L, n, choose_config(L, n)).plan_end);
  *bytes = best;
  return TPA_OK;
}

tpa_status tpa_plan_build(tpa_plan* plan, tpa_layer* L, const int32_t* sor, int32_t n, void* plan_dev,
                          size_t plan_bytes, tpa_stream stream) {
  if (tpa_status st = check_layer(L)) return st;
  if (!plan) return fail(TPA_ERR_INVALID, "null plan");
  if (n < 0 || n > tpa::PLAN_MAX_ROWS) return fail(TPA_ERR_INVALID, "n=%d outside [0, %d]", n, tpa::PLAN_MAX_ROWS);
  if (n > 0 && (!sor || !plan_dev)) return fail(TPA_ERR_INVALID, "null pointer");
  if (reinterpret_cast<uintptr_t>(plan_dev) & 255) return fail(TPA_ERR_INVALID, "plan buffer must be 256-byte aligned");
  const Config c = choose_config(L, std::max(n, 1));
  const Layout y = make_layout(L, n, c);
  if (plan_bytes < y.plan_end) return fail(TPA_ERR_WORKSPACE, "plan buffer %zu < %zu bytes", plan_bytes, y.plan_end);
  plan->built = false;
  if (n > 0) {
    DeviceGuard guard(L->device);
    const tpa::PlanArgs p = plan_args(L, sor, n, static_cast<char*>(plan_dev), y, c);
    TPA_HIP(tpa::launch_plan(p, static_cast<hipStream_t>(stream)));
  }
  plan->sig = L->plan_sig;
  plan->class_sig = L->class_sig;
  plan->max_slots = L->max_slots;
  plan->n = n;
  plan->tile_rows = c.tile_rows;
  plan->dev = static_cast<const char*>(plan_dev);
  plan->bytes = plan_bytes;
  plan->built = true;
  return TPA_OK;
}

tpa_status tpa_layer_forward_planned(tpa_layer* L, const tpa_plan* plan, const void* x, void* out, void* ws,
                                     size_t ws_bytes, tpa_stream stream) {
  if (tpa_status st = check_layer(L)) return st;
  if (!plan || !plan->built) return fail(TPA_ERR_INVALID, "plan is not built");
  const int n = plan->n;
  if (n == 0) return TPA_OK;
  if (!x || !out || !ws) return fail(TPA_ERR_INVALID, "null pointer");
  if (reinterpret_cast<uintptr_t>(ws) & 255) return fail(TPA_ERR_INVALID, "workspace must be 256-byte aligned");
  if (x == out) return fail(TPA_ERR_INVALID, "out may not alias x");
  const Config c = choose_config(L, n);
  if (!plan_accepts(plan, L) || plan->tile_rows != c.tile_rows)
    return fail(TPA_ERR_INVALID, "plan was built for a layer with other slot classes or tiling");
  const Layout y = make_layout(L, n, c);
  if (ws_bytes < y.total) return fail(TPA_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, y.total);
  if (plan->bytes < y.plan_end) return fail(TPA_ERR_WORKSPACE, "plan buffer too small");
  DeviceGuard guard(L->device);
  hipStream_t s = static_cast<hipStream_t>(stream);
  // The plan arrays come from the shared buffer (same offsets as a
  // workspace's head); the rest of the workspace is this forward's.
  const tpa::PlanArgs p = plan_args(L, nullptr, n, const_cast<char*>(plan->dev), y, c);
  if (tpa_status st = stage(L, 0, s)) return st;
  if (tpa_status st = stage(L, 1, s)) return st;
  return forward_after_plan(L, p, x, n, out, static_cast<char*>(ws), y, c, s);
}

tpa_status tpa_group_workspace_size(tpa_layer* const* layers, int32_t count, int32_t n_max, size_t* bytes) {
  if (!layers || !bytes || count < 1 || count > tpa::MAX_SLICES) return fail(TPA_ERR_INVALID, "bad group");
  if (n_max < 0 || n_max > tpa::PLAN_MAX_ROWS) return fail(TPA_ERR_INVALID, "n_max must be in [0, %d]", tpa::PLAN_MAX_ROWS);
  for (int i = 0; i < count; ++i) {
    if (tpa_status st = check_layer(layers[i])) return st;
    bytes[i] = 0;
  }
  Config cs[tpa::MAX_SLICES];
  for (int n = 1; n <= n_max; ++n) {
    group_configs(layers, count, n, cs);
    for (int i = 0; i < count; ++i) bytes[i] = std::max(bytes[i], make_layout(layers[i], n, cs[i]).total);
  }
  return TPA_OK;
}

tpa_status tpa_group_forward_planned(tpa_layer* const* layers, int32_t count, const tpa_plan* plan,
                                     const void* const* x, void* const* out, void* const* ws, const size_t* ws_bytes,
                                     tpa_stream stream) {
  if (!layers || !x || !out || !ws || !ws_bytes || count < 1 || count > tpa::MAX_SLICES)
    return fail(TPA_ERR_INVALID, "bad group");
  if (!plan || !plan->built) return fail(TPA_ERR_INVALID, "plan is not built");
  for (int i = 0; i < count; ++i) {
    tpa_layer* L = layers[i];
    if (tpa_status st = check_layer(L)) return st;
    if (L->dtype != layers[0]->dtype || L->device != layers[0]->device)
      return fail(TPA_ERR_INVALID, "group layers differ in dtype or device");
    if (!plan_accepts(plan, L)) return fail(TPA_ERR_INVALID, "plan was built for a layer with other slot classes");
  }
  const int n = plan->n;
  if (n == 0) return TPA_OK;
  Config cs[tpa::MAX_SLICES];
  group_configs(layers, count, n, cs);
  SliceCtx sl[tpa::MAX_SLICES];
  for (int i = 0; i < count; ++i) {
    if (!x[i] || !out[i] || !ws[i]) return fail(TPA_ERR_INVALID, "null pointer");
    if (reinterpret_cast<uintptr_t>(ws[i]) & 255) return fail(TPA_ERR_INVALID, "workspace must be 256-byte aligned");
    if (x[i] == out[i]) return fail(TPA_ERR_INVALID, "out may not alias x");
    if (cs[i].tile_rows != plan->tile_rows) return fail(TPA_ERR_INVALID, "plan was built with other tiling");
    sl[i] = SliceCtx{layers[i], x[i], out[i], static_cast<char*>(ws[i]), make_layout(layers[i], n, cs[i]), cs[i]};
    if (ws_bytes[i] < sl[i].y.total) return fail(TPA_ERR_WORKSPACE, "workspace %d: %zu < %zu bytes", i, ws_bytes[i], sl[i].y.total);
    if (plan->bytes < sl[i].y.plan_end) return fail(TPA_ERR_WORKSPACE, "plan buffer too small");
  }
  DeviceGuard guard(layers[0]->device);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const tpa::PlanArgs p = plan_args(layers[0], nullptr, n, const_cast<char*>(plan->dev), sl[0].y, cs[0]);
  if (tpa_status st = stage(layers[0], 0, s)) return st;
  if (tpa_status st = stage(layers[0], 1, s)) return st;
  return forward_group_after_plan(sl, count, p, n, s);
}

tpa_status tpa_error_flag(tpa_layer* L, int32_t* flag_host, int32_t clear, tpa_stream stream) {
  if (tpa_status st = check_layer(L)) return st;
  if (!flag_host) return fail(TPA_ERR_INVALID, "null output");
  DeviceGuard guard(L->device);
  hipStream_t s = static_cast<hipStream_t>(stream);
  TPA_HIP(hipStreamSynchronize(s));
  TPA_HIP(hipMemcpy(flag_host, L->flag_dev, sizeof(int32_t), hipMemcpyDeviceToHost));
  if (clear) {
    const int32_t zero = 0;
    TPA_HIP(hipMemcpy(L->flag_dev, &zero, sizeof zero, hipMemcpyHostToDevice));
  }
  return TPA_OK;
}

tpa_status tpa_plan_debug(tpa_layer* L, const int32_t* sor, int32_t n, void* ws, size_t ws_bytes, tpa_plan_host* o,
                          tpa_stream stream) {
  if (tpa_status st = check_layer(L)) return st;
  if (!o || n < 0 || n > tpa::PLAN_MAX_ROWS || (n > 0 && (!sor || !ws))) return fail(TPA_ERR_INVALID, "bad argument");
  const Config c = choose_config(L, std::max(n, 1));
  const Layout y = make_layout(L, n, c);
  if (ws_bytes < y.total) return fail(TPA_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, y.total);
  DeviceGuard guard(L->device);
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* w = static_cast<char*>(ws);
  if (n == 0) {
    if (o->counts) std::memset(o->counts, 0, 4 * sizeof(int32_t));
    if (o->class_ptr) std::memset(o->class_ptr, 0, 4 * sizeof(int32_t));
    if (o->seg_ptr) o->seg_ptr[0] = 0;
    return TPA_OK;
  }
  const tpa::PlanArgs p = plan_args(L, sor, n, w, y, c);
  TPA_HIP(tpa::launch_plan(p, s));
  TPA_HIP(hipStreamSynchronize(s));
  int32_t cnt[tpa::CNT_WORDS];
  TPA_HIP(hipMemcpy(cnt, p.counts, sizeof cnt, hipMemcpyDeviceToHost));
  const int nseg = cnt[tpa::CNT_NSEG], nt = cnt[tpa::CNT_NTILES], no = cnt[tpa::CNT_NOFT];
  if (o->perm) TPA_HIP(hipMemcpy(o->perm, p.perm, 4 * (size_t)n, hipMemcpyDeviceToHost));
  if (o->row_slot) TPA_HIP(hipMemcpy(o->row_slot, p.row_slot, 4 * (size_t)n, hipMemcpyDeviceToHost));
  if (o->seg_ptr) TPA_HIP(hipMemcpy(o->seg_ptr, p.seg_ptr, 4 * (size_t)(nseg + 1), hipMemcpyDeviceToHost));
  if (o->seg_slot) TPA_HIP(hipMemcpy(o->seg_slot, p.seg_slot, 4 * (size_t)nseg, hipMemcpyDeviceToHost));
  if (o->tiles) TPA_HIP(hipMemcpy(o->tiles, p.tiles, 16 * (size_t)nt, hipMemcpyDeviceToHost));
  if (o->oft_tiles) TPA_HIP(hipMemcpy(o->oft_tiles, p.oft_tiles, 16 * (size_t)no, hipMemcpyDeviceToHost));
  if (o->class_ptr) std::memcpy(o->class_ptr, cnt + tpa::CNT_CLASS0, 4 * sizeof(int32_t));
  if (o->counts) {
    o->counts[0] = nseg;
    o->counts[1] = nt;
    o->counts[2] = no;
    o->counts[3] = cnt[tpa::CNT_INVALID];
  }
  return TPA_OK;
}

tpa_status tpa_layer_set_option(tpa_layer* L, int32_t key, int32_t value) {
  if (tpa_status st = check_layer(L)) return st;
  if (key < TPA_OPT_GEMM_SPLIT || key > TPA_OPT_SHRINK_COLS) return fail(TPA_ERR_INVALID, "unknown option %d", key);
  if (key == TPA_OPT_SHRINK_COLS && value > 0 && value != 16 && value != 64)
    return fail(TPA_ERR_INVALID, "shrink columns must be 16 or 64");
  if (key == TPA_OPT_FUSE_EXPAND && value > 1) return fail(TPA_ERR_INVALID, "fused expand must be 0 or 1");
  if (key == TPA_OPT_WIDE_TILE && value > 0 && value != 128 && value != 256)
    return fail(TPA_ERR_INVALID, "wide tile must be 128 or 256");
  if (key == TPA_OPT_OVERLAP && value > 1) return fail(TPA_ERR_INVALID, "overlap must be 0 or 1");
  if (key == TPA_OPT_GEMM_STAGES && value > 0 && (value < 2 || value > 6))
    return fail(TPA_ERR_INVALID, "gemm stages must be 2..6");
  if (key == TPA_OPT_GEMM_NB && value > 0 && value != 1 && value != 2 && value != 4)
    return fail(TPA_ERR_INVALID, "gemm nb must be 1, 2 or 4");
  if (key == TPA_OPT_GEMM_GROUPS && value > 2) return fail(TPA_ERR_INVALID, "gemm groups must be 1 or 2");
  if (key == TPA_OPT_TILE_ROWS && value > 0 && value != 16 && value != 64)
    return fail(TPA_ERR_INVALID, "tile rows must be 16 or 64");
  if (key == TPA_OPT_GEMM_PATH && value > 3) return fail(TPA_ERR_INVALID, "gemm path must be 0, 1, 2 or 3");
  if (key == TPA_OPT_SCALE_ROUTE) {
    if (value < 0) value = 0;
    if (value > 3) return fail(TPA_ERR_INVALID, "scale route must be 0..3");
    const bool was_post = L->opt[TPA_OPT_SCALE_ROUTE] >= 2, post = value >= 2;
    if (was_post != post && (L->n_dora > 0 || L->n_stack > 0))
      return fail(TPA_ERR_INVALID, "DoRA or stacked slots are folded for the current route; unload them first");
  }
  L->opt[key] = value;
  return TPA_OK;
}

tpa_status tpa_layer_config(const tpa_layer* L, int32_t n, tpa_config* out) {
  if (tpa_status st = check_layer(L)) return st;
  if (!out || n < 0 || n > tpa::PLAN_MAX_ROWS) return fail(TPA_ERR_INVALID, "bad argument");
  const Config c = choose_config(L, std::max(n, 1));
  out->tile_rows = c.tile_rows;
  out->gemm_path = c.gemm_path;
  out->gemm_nb = c.gemm_nb;
  out->gemm_split = c.gemm_split;
  out->gemm_kc = c.gemm_kc;
  out->shrink_split = c.shrink_split;
  out->shrink_kc = c.shrink_kc;
  out->scale_route = c.scale_route;
  out->gemm_groups = c.gemm_groups;
  out->gemm_stages = c.gemm_path == 2 || c.gemm_path == 3 ? c.gemm_stages : 0;
  out->gemm_tile = c.gemm_path == 3 ? c.gemm_tile : 0;
  // The decode epilogue also needs a launch before the GEMM to clear its
  // counters: a term, an OFT rotation, or k not split.
  const bool pre = L->n_owned > 0 || L->n_vera > 0 || L->n_oft_bs[0] + L->n_oft_bs[1] + L->n_oft_bs[2] > 0;
  out->fused_expand = c.fused || (c.fused_dec && (pre || c.gemm_split == 1));
  out->shrink_cols = 16 * c.shrink_ncb;
  out->shrink_in_gemm = c.shrink_in_gemm;
  return TPA_OK;
}

tpa_status tpa_layer_set_stage_events(tpa_layer* L, void* const* events, int32_t count) {
  if (tpa_status st = check_layer(L)) return st;
  if (!events) {
    L->stage_on = false;
    return TPA_OK;
  }
  if (count != 6) return fail(TPA_ERR_INVALID, "stage events: count must be 6");
  for (int i = 0; i < 6; ++i) {
    if (!events[i]) return fail(TPA_ERR_INVALID, "stage events: null event %d", i);
    L->stage_ev[i] = static_cast<hipEvent_t>(events[i]);
  }
  L->stage_on = true;
  return TPA_OK;
}

tpa_status tpa_timing_event_create(void** event) {
  if (!event) return fail(TPA_ERR_INVALID, "null output");
  hipEvent_t e = nullptr;
  TPA_HIP(hipEventCreateWithFlags(&e, hipEventDisableSystemFence));
  *event = e;
  return TPA_OK;
}

tpa_status tpa_timing_event_destroy(void* event) {
  if (event) TPA_HIP(hipEventDestroy(static_cast<hipEvent_t>(event)));
  return TPA_OK;
}

tpa_status tpa_timing_event_elapsed(void* start, void* end, float* ms) {
  if (!start || !end || !ms) return fail(TPA_ERR_INVALID, "null argument");
  TPA_HIP(hipEventSynchronize(static_cast<hipEvent_t>(end)));
  TPA_HIP(hipEventElapsedTime(ms, static_cast<hipEvent_t>(start), static_cast<hipEvent_t>(end)));
  return TPA_OK;
}

tpa_status tpa_probe_copy(void* dst, const void* src, size_t bytes, tpa_stream stream) {
  if (!dst || !src || (bytes & 15) || (reinterpret_cast<uintptr_t>(dst) & 15) || (reinterpret_cast<uintptr_t>(src) & 15))
    return fail(TPA_ERR_INVALID, "copy needs 16-byte aligned pointers and a multiple of 16 bytes");
  TPA_HIP(tpa::launch_copy(dst, src, bytes, static_cast<hipStream_t>(stream)));
  return TPA_OK;
}

tpa_status tpa_probe_read(const void* src, size_t bytes, void* sink, tpa_stream stream) {
  if (!src || !sink || (bytes & 15) || (reinterpret_cast<uintptr_t>(src) & 15) || (reinterpret_cast<uintptr_t>(sink) & 3))
    return fail(TPA_ERR_INVALID, "read probe needs a 16-byte aligned source, a multiple of 16 bytes and a sink");
  TPA_HIP(tpa::launch_read(src, bytes, static_cast<uint32_t*>(sink), static_cast<hipStream_t>(stream)));
  return TPA_OK;
}

tpa_status tpa_probe_empty(int32_t count, tpa_stream stream) {
  if (count < 0) return fail(TPA_ERR_INVALID, "negative count");
  TPA_HIP(tpa::launch_empty(count, static_cast<hipStream_t>(stream)));
  return TPA_OK;
}

tpa_status tpa_probe_delay(int32_t microseconds, tpa_stream stream) {
  if (microseconds < 0 || microseconds > 1000000) return fail(TPA_ERR_INVALID, "delay must be 0 .. 1e6 us");
  TPA_HIP(tpa::launch_delay(microseconds, static_cast<hipStream_t>(stream)));
  return TPA_OK;
}

}  // extern "C"
