/*
 * tpa.h -- C ABI of the batched multi-adapter layer in normal form, for
 * AMD Instinct MI355X (gfx950).
 *
 * One `tpa_layer` is one adapted projection: a shared base weight W and a
 * table of slots, each holding one tenant's adapter in normal form
 * (Scute paper, arXiv 2611.01089, §3.1 eq. (1)):
 *
 *   F_a(x) = ((x R) W) ⊙ s + b + Σ_k c_k (((x A_k) ⊙ d_k) B_k ⊙ e_k)
 *
 * `tpa_layer_forward` evaluates F_{a(i)} for every row i of one batch whose
 * rows belong to many tenants (slot_of_row[i] = the row's slot), following
 * §2 "The LoRA schedule" and the three routes of §4.1: the output scale s
 * (and shift b) is applied inside the expand, VeRA's shared-factor term
 * runs over row tiles whatever their tenant, and OFT's rotation R runs in a
 * pass of its own before the shared GEMM.
 *
 * Conventions
 *   - Layer element type (`dtype`): TPA_F32, TPA_F16 or TPA_BF16.  x, W and
 *     out use it; accumulation is always fp32.
 *   - W is row-major [d_out][d_in] (an nn.Linear weight; the paper's math W
 *     is its transpose).  x is row-major [n][d_in]; out is [n][d_out].
 *   - Raw adapter parameters are float32 host arrays in the paper's math
 *     layout: A [d_in][r], B [r][d_out], Q [d_in / b][b][b].
 *   - All device work is enqueued on the caller's stream; nothing here
 *     synchronizes except where a function says so.  A `tpa_layer` is not
 *     thread-safe: serialize calls on one layer.
 *   - Errors: every function returns a tpa_status; on failure a message for
 *     the calling thread is available from tpa_last_error().
 */
#ifndef TPA_H
#define TPA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t tpa_status;
#define TPA_OK 0
#define TPA_ERR_INVALID (-1)      /* bad argument or shape */
#define TPA_ERR_METHOD (-2)       /* unknown method */
#define TPA_ERR_NO_SLOT (-3)      /* every slot is in use */
#define TPA_ERR_UNKNOWN_SLOT (-4) /* slot not loaded (or slot 0) */
#define TPA_ERR_VALUE (-5)        /* non-skew Q, non-finite or zero-norm input */
#define TPA_ERR_WORKSPACE (-6)    /* workspace too small */
#define TPA_ERR_HIP (-7)          /* HIP runtime error */

typedef struct tpa_layer tpa_layer;
typedef void* tpa_stream; /* a hipStream_t; NULL = the null stream */

enum tpa_dtype { TPA_F32 = 0, TPA_F16 = 1, TPA_BF16 = 2 };

/* Methods of Table 1 (§3.1).  TPA_IDENTITY loads a slot that leaves its rows
 * unchanged, so a tenant that does not adapt this projection can keep the
 * same slot id in every layer. */
enum tpa_method {
  TPA_IDENTITY = 0,
  TPA_LORA = 1,
  TPA_DORA = 2,
  TPA_IA3 = 3,
  TPA_VERA = 4,
  TPA_OFT = 5,
  TPA_SSF = 6,
  TPA_STACK = 7, /* reported by tpa_adapter_info_get for a stacked slot; not loadable by itself */
  TPA_LOHA = 8,
  TPA_LOKR = 9
};

/* Most members in one stack (tpa_adapter_load_stack). */
#define TPA_MAX_STACK 8

/* Raw parameters of one adapter (host memory, float32, copied before
 * tpa_adapter_load returns).  Fields a method does not use are ignored.
 *   LoRA : A [d_in][rank], B [rank][d_out], c
 *   DoRA : A, B, c as LoRA, m [d_out] magnitude (§5.1: s = m ⊘ ‖W + cAB‖_c)
 *   (IA)3: l [d_out]
 *   VeRA : d [r_v], e [d_out], c; the shared pair is set per layer with
 *          tpa_vera_shared_set; rank must be 0 or r_v
 *   OFT  : Q [d_in / oft_block][oft_block][oft_block], skew-symmetric
 *   SSF  : s [d_out], b [d_out]
 *   LoHa : ΔW = c · (A B) ⊙ (A2 B2) (§3.1 "Other methods fit as well": a
 *          product of small factors, expanded at load).  A [d_in][rank],
 *          B [rank][d_out], A2 [d_in][rank2], B2 [rank2][d_out]
 *          (rank2 = 0: rank2 = rank); stored as one owned term of rank
 *          rank · rank2, which must not exceed max_rank.
 *   LoKr : ΔW = c · (C ⊗ (A B)), C [kron_p][kron_q], A [d_in / kron_p][rank],
 *          B [rank][d_out / kron_q]; kron_p divides d_in and kron_q d_out.
 *          Stored as one owned term of rank min(kron_p, kron_q) · rank
 *          (C ⊗ AB = (C ⊗ A)(I ⊗ B) or (I ⊗ A)(C ⊗ B)), at most max_rank.  */
typedef struct {
  int32_t method;
  int32_t rank;
  int32_t oft_block;
  float c;
  const float* A;
  const float* B;
  const float* m;
  const float* l;
  const float* d;
  const float* e;
  const float* Q;
  const float* s;
  const float* b;
  int32_t rank2;   /* LoHa */
  int32_t kron_p;  /* LoKr */
  int32_t kron_q;  /* LoKr */
  int32_t reserved;
  const float* A2; /* LoHa */
  const float* B2; /* LoHa */
  const float* C;  /* LoKr */
} tpa_adapter_desc;

/* Merged-slot metadata (Table 1 and the fold rule of §3.2).
 *   live_mask: which slots stay live   S=1, B(shift)=2, R=4, D=8, E=16
 *   fold_mask: which folds were made   C->A=1, E->B=2, C->D=4, D->A=8
 *   term_kind: 0 no term, 1 term on owned factors, 2 term on shared factors */
#define TPA_LIVE_S 1
#define TPA_LIVE_B 2
#define TPA_LIVE_R 4
#define TPA_LIVE_D 8
#define TPA_LIVE_E 16
#define TPA_FOLD_C_A 1
#define TPA_FOLD_E_B 2
#define TPA_FOLD_C_D 4
#define TPA_FOLD_D_A 8
typedef struct {
  int32_t method;
  int32_t live_mask;
  int32_t fold_mask;
  int32_t term_kind;
  int32_t rank;
  int32_t oft_block;
} tpa_adapter_info;

/* Metadata a method gets by the fold rule (appendix "Folds": c folds into
 * the first owned neighbour among A, d, B, e; d into an owned A or B; e into
 * an owned B; s, b, R never fold).  Host only; needs no GPU. */
tpa_status tpa_method_info(int32_t method, tpa_adapter_info* out);

/* Create one adapted projection on `device`.
 *   W_dev: device pointer to W [d_out][d_in] in `dtype`; borrowed, must
 *          outlive the layer and not change while adapters are loaded
 *          (DoRA's scale is computed from it at load).
 *   max_slots: slots 0..max_slots-1; slot 0 is the permanent identity.
 *   max_rank : largest rank of any term (owned rank or VeRA r_v); sizes the
 *              workspace.
 * Requires d_in a multiple of 64, d_out a multiple of 128, 2 <= max_slots <= 16384,
 * 1 <= max_rank <= 512. */
/* Per-layer slot storage: Scute paper §5.2 (each adapted layer keeps one
 * buffer per slot for s, d, e and R beside the LoRA factors). */
tpa_status tpa_layer_create(int32_t device, int32_t d_in, int32_t d_out, int32_t dtype,
                            const void* W_dev, int32_t max_slots, int32_t max_rank,
                            tpa_layer** out);
/* Frees the layer's slot storage (§5.2); W stays the caller's.  A null
 * layer is a no-op. */
tpa_status tpa_layer_destroy(tpa_layer* layer);

/* Set VeRA's frozen pair shared by every VeRA slot of this layer
 * (§2 "The methods", §3.2): A [d_in][r_v], B [r_v][d_out], float32 host.
 * Stored once; r_v a multiple of 16, <= max_rank.  Must precede any VeRA
 * load and cannot change while VeRA slots are loaded. */
tpa_status tpa_vera_shared_set(tpa_layer* layer, int32_t r_v, const float* A, const float* B,
                               tpa_stream stream);

/* VeRA's A read once per fused input (Table 2's route-two count; appendix
 * "Byte counts": the shared A once per input a fused layer reads, B once
 * per slice): `layer` takes `from`'s stored A_v (the same device copy, held
 * until both layers drop it; r_v from `from`) and its own B [r_v][d_out]
 * (float32 host).  `from` must have a VeRA pair and the same device, dtype
 * and d_in.  A group forward (tpa_group_forward_planned) whose projections
 * hold one A_v and read one input pointer computes x·A_vᵀ once for all of
 * them; each applies its own d' and B_v.  Same rules as
 * tpa_vera_shared_set otherwise (no VeRA slot loaded; synchronizes). */
tpa_status tpa_vera_shared_set_from(tpa_layer* layer, tpa_layer* from, const float* B, tpa_stream stream);

/* Admit one adapter (§5.1): validate, convert to normal form and fold what
 * the fold rule allows, upload to the device, and return its slot (the
 * lowest free slot >= 1).  Runs on `stream` and synchronizes it before
 * returning; host arrays may be reused when the call returns.  Folds: LoRA and DoRA c -> A; DoRA
 * s = m ⊘ ‖W + cAB‖_c computed on the device from W, then e = s -> B;
 * VeRA c -> d; OFT blocks R_j = (I + Q_j)(I - Q_j)^-1 computed in float64 on
 * the host.  Errors: -1 shapes/rank, -2 method, -3 no free slot, -5 Q not
 * skew-symmetric, a non-finite value, or a zero column norm. */
tpa_status tpa_adapter_load(tpa_layer* layer, const tpa_adapter_desc* desc, int32_t* slot_out,
                            tpa_stream stream);

/* Admit a stack of adapters at this hook as one slot (§3.2 paragraph
 * "Stacking", appendix "Stacking"): members[0] is applied first, and each
 * later member takes the previous member's output in place of its base
 * output xW (its terms still read x).  The result is one member of eq. (1):
 * scale s_1⊙…⊙s_K, shift folded through the later scales (b1⊙s2 + b2 for
 * two members), and every member's term multiplied by the scales of the
 * members after it through its outer vector e.  Order matters.
 *   members: `count` raw descriptors (1 <= count <= TPA_MAX_STACK), each
 *            valid for tpa_adapter_load; host memory, copied before return.
 *            Only members[0] may be TPA_OFT (a later member's base path is
 *            the previous output, so it cannot rotate the input).
 * Storage: a stack whose only term is one VeRA term stays a shared-term
 * slot (d' = c·d, e' = e ⊙ later scales); otherwise all terms become one
 * owned term whose rank is the sum of the members' ranks (a VeRA term
 * enters in its exact owned form A_v diag(c·d), B_v diag(e'), from the
 * layer's stored pair), which must not exceed max_rank.  DoRA members get
 * their scale from the device norm kernel as in tpa_adapter_load; the
 * composition runs on the host in float64.  count == 1 is tpa_adapter_load.
 * tpa_adapter_info_get reports method TPA_STACK.  Synchronizes `stream`.
 * Errors: as tpa_adapter_load; -1 also for a count out of range, OFT after
 * the first member, a stacked rank above max_rank, or a layer whose scale
 * route applies s after the expand (TPA_OPT_SCALE_ROUTE >= 2). */
tpa_status tpa_adapter_load_stack(tpa_layer* layer, const tpa_adapter_desc* members, int32_t count,
                                  int32_t* slot_out, tpa_stream stream);

/* Free a slot (admission of §5.1 undone).  Synchronizes `stream` before
 * releasing device memory, so forwards enqueued on it earlier still see the
 * adapter (faangrind "multi-lora-serving" page, failure mode "Adapter
 * evicted while in use").  -4 if the slot is not loaded. */
tpa_status tpa_adapter_unload(tpa_layer* layer, int32_t slot, tpa_stream stream);

/* The slot's metadata (Table 1; the fold rule of §3.2): method, the slots
 * that stay live, the folds made, term kind, rank and OFT block.  Host only.
 * -4 if the slot is not loaded (slot 0 reports the identity). */
tpa_status tpa_adapter_info_get(const tpa_layer* layer, int32_t slot, tpa_adapter_info* out);

/* Bytes of device workspace a forward of any n <= n_max rows needs under
 * the layer's current options; n_max <= 8192.  The workspace holds the row
 * plan (§2 "The LoRA schedule"), the rotated rows of OFT tenants (§4.1
 * route three), the shrink's V and U between the two halves of the term
 * (§2), the base GEMM's split partials and, when the decode GEMM carries
 * the expand, its arrival counters (one word per column tile, cleared on
 * every forward by the launch before the GEMM).  Host only. */
tpa_status tpa_workspace_size(const tpa_layer* layer, int32_t n_max, size_t* bytes);

/* out[i] = F_{slot_of_row[i]}(x[i]) for i < n (eq. (1)).
 *   x_dev [n][d_in], out_dev [n][d_out] in the layer dtype (out may not
 *   alias x); slot_of_row_dev int32 [n] on the device; ws_dev of at least
 *   tpa_workspace_size(n) bytes, 256-byte aligned, not shared by forwards
 *   that may run concurrently.
 * n <= 8192.  A row whose slot is out of range or not loaded is computed as
 * the identity
 * and raises the layer's sticky error flag (tpa_error_flag).  n = 0 is a
 * no-op.  No host synchronization; capturable in a HIP graph. */
tpa_status tpa_layer_forward(tpa_layer* layer, const void* x_dev, const int32_t* slot_of_row_dev,
                             int32_t n, void* out_dev, void* ws_dev, size_t ws_bytes,
                             tpa_stream stream);

/* Bytes of scratch each GPU holds for tpa_layer_forward_noalloc. */
#define TPA_NOALLOC_SCRATCH_BYTES (64u << 20)
/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * forward as tpa_layer_forward, same kernels and same bits, with its
 * workspace in a scratch array the library holds, one copy per GPU, of
 * TPA_NOALLOC_SCRATCH_BYTES, kept until the process ends.  The call
 * allocates nothing (no hipMalloc or hipFree, no stream or event is
 * created: the shrink runs on `stream`, never on a second stream).
 *   x_dev, slot_of_row_dev, out_dev: as for tpa_layer_forward.
 * Errors: as tpa_layer_forward; -6 when a forward of n rows on this layer
 * needs more workspace than the scratch holds (tpa_workspace_size(layer, n)
 * gives the bytes; nothing is launched then).  Every call on one GPU uses
 * that GPU's one scratch array: calls whose work may overlap on a GPU
 * (other streams, other threads, other layers) race and must be
 * serialized by the caller; calls queued on one stream are ordered. */
tpa_status tpa_layer_forward_noalloc(tpa_layer* layer, const void* x_dev, const int32_t* slot_of_row_dev,
                                     int32_t n, void* out_dev, tpa_stream stream);

/* Shared row plans.  The plan of a batch (rows grouped by term class and
 * slot, tiles, OFT tiles; §2 "The LoRA schedule") depends only on
 * slot_of_row and on each slot's term class and whether it holds an OFT
 * rotation, so projections whose slot tables agree on those (for example
 * q, k and v of one decoder layer) can group the batch once:
 *   tpa_plan_size(layer, n_max, &bytes): device bytes of a plan buffer;
 *   tpa_plan_build(plan, layer, slot_of_row_dev, n, plan_dev, bytes, s):
 *     enqueue the plan kernel on s into plan_dev (caller-owned, 256-byte
 *     aligned, must stay allocated and unmodified while forwards use it) and
 *     record layer's slot-class signature; raises layer's sticky flag for
 *     invalid slots;
 *   tpa_layer_forward_planned(layer, plan, x, out, ws, ws_bytes, s): as
 *     tpa_layer_forward for the plan's rows, without the plan kernel; -1 if
 *     the plan does not accept the layer (below) or its tiling differs (any
 *     load or unload can change that).  ws as for tpa_layer_forward;
 *   tpa_plan_accepts(plan, layer, &ok): host only; ok = 1 when the plan is
 *     built and layer's slots have the building layer's term classes and
 *     either the same OFT flags or no OFT rotation at all (such a layer reads
 *     neither the OFT tiles nor the rotated-row map), and the same slot
 *     count.  In a decoder layer whose OFT tenants adapt q, k and v only, a
 *     plan built by q serves all seven projections.
 * The tpa_plan handle is host memory (create/destroy); it holds no device
 * memory. */
typedef struct tpa_plan tpa_plan;
/* Layers whose signatures are equal can share a plan of the same rows
 * (§2 "The LoRA schedule"; appendix "CUDA graphs": the row mapping is built
 * once per step for every layer). */
tpa_status tpa_layer_plan_signature(const tpa_layer* layer, uint64_t* sig);
/* §2 "The LoRA schedule": whether a plan's grouping serves this layer. */
tpa_status tpa_plan_accepts(const tpa_plan* plan, const tpa_layer* layer, int32_t* ok);
/* Host handle of a shared row plan (§2 "The LoRA schedule"). */
tpa_status tpa_plan_create(tpa_plan** out);
tpa_status tpa_plan_destroy(tpa_plan* plan); /* §2 "The LoRA schedule" */
/* Device bytes of a plan of n_max rows (§2 "The LoRA schedule"). */
tpa_status tpa_plan_size(const tpa_layer* layer, int32_t n_max, size_t* bytes);
/* Groups the rows once per step (§2 "The LoRA schedule"; appendix "CUDA
 * graphs"). */
tpa_status tpa_plan_build(tpa_plan* plan, tpa_layer* layer, const int32_t* slot_of_row_dev, int32_t n,
                          void* plan_dev, size_t plan_bytes, tpa_stream stream);
/* eq. (1) for the plan's rows, steps after the plan (§2, §4.1). */
tpa_status tpa_layer_forward_planned(tpa_layer* layer, const tpa_plan* plan, const void* x_dev,
                                     void* out_dev, void* ws_dev, size_t ws_bytes, tpa_stream stream);

/* Projections of one fused layer (q, k and v; gate and up) forwarded in one
 * launch per kernel (Scute paper §5.2: one launch covers all slices of a layer), with
 * a plan that accepts each of them.  count <= 4; layers[i] with
 * x[i] [n][d_in_i], out[i] [n][d_out_i], ws[i] of ws_bytes[i] bytes (at least
 * tpa_group_workspace_size's bytes[i] for this group; 256-byte aligned).  The
 * plan must accept every layer; one dtype and one device.  On the
 * decode path (n <= 64) the group shares one base-GEMM configuration (column
 * blocks per work-group and k range), so results may differ from separate
 * forwards by the rounding of a different split-K order.  Stage events are
 * those of layers[0]. */
/* Workspace bytes of each projection of a group (§5.2, one launch per
 * kernel for every slice); bytes[count]. */
tpa_status tpa_group_workspace_size(tpa_layer* const* layers, int32_t count, int32_t n_max, size_t* bytes);
/* eq. (1) for every projection of the group, one launch per kernel (§5.2). */
tpa_status tpa_group_forward_planned(tpa_layer* const* layers, int32_t count, const tpa_plan* plan,
                                     const void* const* x_dev, void* const* out_dev, void* const* ws_dev,
                                     const size_t* ws_bytes, tpa_stream stream);

/* Read (and optionally clear) the layer's sticky invalid-slot flag: set by
 * any forward or plan whose slot_of_row names a slot that is out of range
 * or not loaded (such rows are computed as the identity, never with another
 * tenant's weights: faangrind "multi-lora-serving" page, failure mode
 * "Wrong adapter applied").  Synchronizes `stream`. */
tpa_status tpa_error_flag(tpa_layer* layer, int32_t* flag_host, int32_t clear, tpa_stream stream);

/* The row plan a forward of these rows uses, copied to host arrays
 * (synchronizes `stream`).  Rows are ordered by (term class of the slot,
 * slot, row), class 0 = term on owned factors, 1 = shared-factor term,
 * 2 = no term.  Arrays (each may be NULL):
 *   perm[n], row_slot[n], seg_ptr[n+1], seg_slot[n], class_ptr[4],
 *   tiles[4 * max_tiles] as (p0, p1, kind, slot), oft_tiles[4 * max_tiles]
 *   as (p0, p1, slot, 0), counts[4] = (n_seg, n_tiles, n_oft_tiles, invalid),
 * with max_tiles from tpa_plan_max_tiles. */
typedef struct {
  int32_t* perm;
  int32_t* row_slot;
  int32_t* seg_ptr;
  int32_t* seg_slot;
  int32_t* class_ptr;
  int32_t* tiles;
  int32_t* oft_tiles;
  int32_t* counts;
} tpa_plan_host;
/* Padded tile-list length and rows per tile of a plan of n rows (§2 "The
 * LoRA schedule": one adapter per tile).  Host only. */
tpa_status tpa_plan_max_tiles(const tpa_layer* layer, int32_t n, int32_t* max_tiles,
                              int32_t* tile_rows);
/* Runs the plan kernel (§2 "The LoRA schedule") and copies the plan out. */
tpa_status tpa_plan_debug(tpa_layer* layer, const int32_t* slot_of_row_dev, int32_t n,
                          void* ws_dev, size_t ws_bytes, tpa_plan_host* out, tpa_stream stream);

/* Kernel configuration pins, for tests and tuning.  value < 0 restores the
 * automatic choice.
 *   TPA_OPT_GEMM_SPLIT   : split-K factor of the base GEMM
 *   TPA_OPT_SHRINK_SPLIT : split-K factor of the shrink
 *   TPA_OPT_TILE_ROWS    : rows per tile of the plan (16, the default, or
 *                          64)
 *   TPA_OPT_GEMM_PATH    : n <= 64: 0 register-fed decode kernel; n <= 256:
 *                          2 decode kernel fed by direct global-to-LDS
 *                          loads (f16 / bf16 with d_in % 64 == 0, else 0;
 *                          the default where it applies up to 64 rows, by
 *                          option up to 256); any n: 1 LDS-tiled kernel
 *                          with register-staged loads, 3 128 x 128 tiles fed
 *                          by direct global-to-LDS loads (f16 / bf16, d_in
 *                          % 64 == 0, d_out % 128 == 0, else 1; the default
 *                          for n > 64)
 *   TPA_OPT_SCALE_ROUTE  : where s (and b) are applied (§4.3, appendix
 *                          "Routes"): 0 inside the expand (route one),
 *                          1 side kernel writing h⊙s before the expand,
 *                          2 gathered scale pass after the expand,
 *                          3 index scale: write s per row, then multiply
 *   TPA_OPT_GEMM_NB      : decode GEMM, 64-column blocks per work-group (1,
 *                          2 or 4)
 *   TPA_OPT_GEMM_GROUPS  : decode GEMM, k-groups of 4 waves per work-group
 *                          (1 or 2; fp32 layers always use 1; the streamed
 *                          kernel takes 2 only with 3 stages)
 *   TPA_OPT_GEMM_STAGES  : LDS buffers of the direct-load GEMMs (2..6):
 *                          streamed decode kernel, per k-group 3, 4 or 6
 *                          (other values take 3; fewer where they do not
 *                          fit); 128 x 128 kernel, 32 KB each, 2..5 (6
 *                          takes the automatic choice, 4)
 *   TPA_OPT_OVERLAP      : 1 runs the shrink and its split
 *                          reduction on a second stream of the layer
 *                          (default priority) beside OFT's rotation and
 *                          the base GEMM, forked from and joined to the
 *                          caller's stream with events, so the forward
 *                          still behaves as one ordered call on `stream`
 *                          (and is captured whole into a HIP graph); 0 or
 *                          < 0 (the default) runs every step on `stream`.
 *                          Never where the expand runs in the GEMM's
 *                          epilogue (that GEMM reads the shrink's output).
 *                          The second stream and its two events are
 *                          created on the first forward that overlaps
 *                          outside graph capture; a captured forward
 *                          before then runs on `stream` alone.  Both ways
 *                          give the same bits.  Stage event 3 (after the
 *                          GEMM) is recorded after the join, so it covers
 *                          the overlapped shrink.  The group forward uses
 *                          the first layer's setting.
 *   TPA_OPT_WIDE_TILE    : direct-load kernel for n > 64: 256 (256 x 256
 *                          tiles, 8 waves; needs d_out % 256 == 0) or 128;
 *                          by default 256 when that gives at least 256
 *                          tiles, else 128.
 *   TPA_OPT_FUSE_EXPAND  : the expand in the base GEMM's epilogue (§2 "The
 *                          LoRA schedule"; §5.2).  128 x 128 direct-load
 *                          kernel with k whole: 1 runs it there (the GEMM
 *                          takes the rows in the plan's tile order, 16 row
 *                          slots per tile, keeps h in fp32 and writes out
 *                          once; the shrink's reduction becomes a launch
 *                          before it); by default when the plan's tile
 *                          bound keeps the row slots within 1.5x the rows.
 *                          Streamed decode kernel (n <= 64, 3 stages,
 *                          16-row tiles, route 0, shrink split <= 16): 1
 *                          runs it in the work-group that completes a
 *                          column tile (the last of its split work-groups
 *                          to arrive, counted on counters in the workspace
 *                          that the launch before the GEMM clears), which
 *                          adds the splits, applies s and b and adds the
 *                          term; the shrink then adds its k ranges inside
 *                          one work-group, so two launches per forward
 *                          instead of three, but slower on MI355X (each
 *                          split's device-scope release writes back an L2).
 *                          It needs a launch before the GEMM (a term or an
 *                          OFT rotation on the layer) unless k is whole,
 *                          and rounds the last sum to the layer type once,
 *                          so it may differ from the separate expand by one
 *                          unit in the last place.  Default (< 0) at
 *                          decode and 0 everywhere: the separate expand.
 *   TPA_OPT_SHRINK_COLS  : factor columns per shrink work item, 16 or 64
 *                          (f16 / bf16, 16-row tiles, split-k shrink): 64
 *                          reads a tile's x rows once for four column
 *                          blocks instead of once per block; the same
 *                          bits.  By default 64 from 512 rows when an
 *                          owned rank or VeRA's r_v exceeds 16, else 16.
 *                          The group forward uses the first layer's. */
#define TPA_OPT_GEMM_SPLIT 1
#define TPA_OPT_SHRINK_SPLIT 2
#define TPA_OPT_TILE_ROWS 3
#define TPA_OPT_GEMM_PATH 4
#define TPA_OPT_SCALE_ROUTE 5
#define TPA_OPT_GEMM_NB 6
#define TPA_OPT_GEMM_GROUPS 7
#define TPA_OPT_GEMM_STAGES 8
#define TPA_OPT_OVERLAP 9
#define TPA_OPT_WIDE_TILE 10
#define TPA_OPT_FUSE_EXPAND 11
#define TPA_OPT_SHRINK_COLS 12
/* Scale routes of §4.3 and the appendix "Routes"; the other keys pin the
 * kernel configuration the appendix "Tuned kernels" would tune. */
tpa_status tpa_layer_set_option(tpa_layer* layer, int32_t key, int32_t value);

/* The kernel configuration a forward of n rows would use (host only, no
 * device work): plan tile rows, base GEMM path (0 register-fed decode
 * kernel, 1 LDS-tiled kernel, 2 streamed decode kernel, 3 direct-load
 * tiled kernel), its 64-column
 * blocks per work-group (nb), split-K factor and k range, the shrink's split
 * and k range, the scale route, the decode GEMM's k-groups per work-group
 * and (direct-load kernels, else 0) its LDS buffers (per k-group for the
 * streamed kernel), path 3's tile edge (128 or 256; else 0), and whether
 * the expand runs in the GEMM's epilogue (prefill or decode kernel), the
 * factor columns per shrink item, and whether the shrink runs in the decode
 * GEMM's own launch (one whole-k item per side work-group; a group forward
 * does so only when every layer of the group can).  For tests and
 * measurement. */
typedef struct {
  int32_t tile_rows, gemm_path, gemm_nb, gemm_split, gemm_kc, shrink_split, shrink_kc, scale_route,
      gemm_groups, gemm_stages, gemm_tile, fused_expand, shrink_cols, shrink_in_gemm;
} tpa_config;
/* Appendix "Tuned kernels": the configuration in force for n rows. */
tpa_status tpa_layer_config(const tpa_layer* layer, int32_t n, tpa_config* out);

/* Stage timing: when `events` is non-null, each forward records events[0]
 * before its first kernel and events[1..5] after the plan, the launch of the
 * shrink with OFT's rotation (none where the decode GEMM carries the whole
 * shrink), the base GEMM (which also carries the shrink's split reduction,
 * or the whole shrink, on the decode path), any scale pass that runs before the
 * expand, and the expand (with any scale pass after it), all on its stream.
 * `events` are hipEvent_t handles owned by the caller; count must be 6 (or 0
 * with null to stop).  For profiling only. */
/* Appendix "Kernel timing": per-kernel times of one forward. */
tpa_status tpa_layer_set_stage_events(tpa_layer* layer, void* const* events, int32_t count);

/* Events for tpa_layer_set_stage_events.  A default HIP event performs a
 * system-scope fence (cache write-back and invalidate) when it is recorded,
 * which costs microseconds and lands inside the interval being timed; these
 * are created without it, so an event pair around one kernel measures that
 * kernel.  elapsed waits for `end` and returns milliseconds. */
tpa_status tpa_timing_event_create(void** event);          /* appendix "Kernel timing" */
tpa_status tpa_timing_event_destroy(void* event);          /* appendix "Kernel timing" */
tpa_status tpa_timing_event_elapsed(void* start, void* end, float* ms); /* appendix "Kernel timing" */

/* Calibration probes (appendix "Constants"): a plain device copy of `bytes`
 * (a multiple of 16, 16-byte aligned pointers) by a streaming kernel, and
 * `count` chained one-block empty kernels for the launch cost.
 * tpa_probe_delay enqueues one wave that idles for `microseconds` (0 .. 1e6)
 * of the device's constant-rate clock and touches no memory: work queued
 * behind it on the stream starts back to back once it ends, so host launch
 * gaps drop out of event timings. */
tpa_status tpa_probe_copy(void* dst_dev, const void* src_dev, size_t bytes, tpa_stream stream); /* β, appendix "Constants" */
/* Read ceiling beside β (appendix "Constants" measures copies; a kernel
 * that mostly reads, like the decode GEMM streaming W, is also set against
 * a plain read): streams `bytes` (a multiple of 16, 16-byte aligned) from
 * src_dev and writes one 4-byte word per work-group to sink_dev, which
 * must hold 8192 words. */
tpa_status tpa_probe_read(const void* src_dev, size_t bytes, void* sink_dev, tpa_stream stream);
tpa_status tpa_probe_empty(int32_t count, tpa_stream stream);    /* λ, appendix "Constants" */
tpa_status tpa_probe_delay(int32_t microseconds, tpa_stream stream); /* appendix "Kernel timing" */

/* Message of the last error on this thread ("" if none): why an adapter
 * was refused at admission (shape, rank or value checks: faangrind
 * "multi-lora-serving" page, failure mode "Corrupt or untrusted adapter
 * file") or why a call failed. */
const char* tpa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* TPA_H */
