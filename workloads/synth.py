"""Seeded synthetic inputs with the shapes and value distributions of the
Scute paper's workloads (arXiv 2611.01089: §6.1 "Setup" for the
Llama-3.1-8B projection shapes, the appendix "Training" for ranks, block
size and which projections each method adapts, "Amplified adapters" for
vectors pulled away from the identity).

Every array is float32 holding a value already rounded to the layer's
storage type (f32, f16 or bf16), so the oracle (which upcasts to float64)
and the HIP path see exactly the same numbers.

Layouts: the base weight ``W`` is stored like an nn.Linear weight,
[d_out, d_in] (the oracle uses its transpose, the paper's math layout);
adapter parameters are in the paper's math layout, A [d_in, r],
B [r, d_out], Q [d_in / b, b, b].

Distributions (one reading of the workload descriptions, used everywhere):
  W ~ N(0, 1/d_in); x ~ N(0, 1); LoRA and DoRA A ~ N(0, 1/d_in),
  B ~ N(0, 1/r), c = 2 (alpha 32 over rank 16); DoRA magnitude
  m = sqrt(1 + c²) · (1 + 0.1 z); (IA)3 l = 1 + 0.3 z; VeRA shared
  A ~ N(0, 1/d_in), B ~ N(0, 1/r_v), d, e = 1 + 0.3 z, c = 1; OFT skew Q
  with upper entries 0.1 z, blocks of 32.

The DoRA magnitude's sqrt(1 + c²) is the expected column norm of the
adapted weight under these draws (a column of W has expected squared norm
1, one of cAB has c², and the cross term has mean 0), a constant of the
recipe, not a norm formed from the drawn values: the scale that both sides
compute from m on their own is then about 1 + 0.1 z.  This module does none
of the methods' arithmetic.
"""
import numpy as np

# Llama-3.1-8B projection shapes (d_in, d_out), §6.1.
LLAMA8B_PROJECTIONS = (
    ("q", 4096, 4096),
    ("k", 4096, 1024),
    ("v", 4096, 1024),
    ("o", 4096, 4096),
    ("gate", 4096, 14336),
    ("up", 4096, 14336),
    ("down", 14336, 4096),
)


def round_to(a, dtype):
    """Round float data to the storage type (once, to nearest even) and
    return it as float32."""
    a = np.asarray(a)
    if a.dtype not in (np.float32, np.float64):
        a = a.astype(np.float64)
    if dtype == "f32":
        return a.astype(np.float32)
    if dtype == "f16":
        return a.astype(np.float16).astype(np.float32)
    if dtype == "bf16":
        u = a.astype(np.float32).view(np.uint32).astype(np.uint64)
        bias = ((u >> 16) & 1) + 0x7FFF
        r = ((u + bias) >> 16) << 16
        return r.astype(np.uint32).view(np.float32)
    raise ValueError(dtype)


def _normal(rng, shape, std):
    """float32 draws of N(0, std^2)."""
    a = rng.standard_normal(shape, dtype=np.float32)
    a *= np.float32(std)
    return a


def _lora(rng, d_in, d_out, r, dtype, c=2.0):
    A = round_to(_normal(rng, (d_in, r), 1.0 / np.sqrt(d_in)), dtype)
    B = round_to(_normal(rng, (r, d_out), 1.0 / np.sqrt(r)), dtype)
    return {"method": "lora", "A": A, "B": B, "c": float(c)}


def _dora(rng, W, r, dtype, c=2.0):
    """DoRA tenant: LoRA factors of rank r and a magnitude
    m = sqrt(1 + c²) · (1 + 0.1 z) (W gives the shapes only)."""
    d_out, d_in = W.shape
    rec = _lora(rng, d_in, d_out, r, dtype, c)
    g = 1.0 + 0.1 * rng.standard_normal(d_out)
    rec["method"] = "dora"
    rec["m"] = (np.sqrt(1.0 + c * c) * g).astype(np.float32)
    return rec


def _ia3(rng, d_out):
    return {"method": "ia3", "l": (1.0 + 0.3 * rng.standard_normal(d_out)).astype(np.float32)}


def _vera(rng, r_v, d_out, c=1.0):
    return {"method": "vera",
            "d": (1.0 + 0.3 * rng.standard_normal(r_v)).astype(np.float32),
            "e": (1.0 + 0.3 * rng.standard_normal(d_out)).astype(np.float32),
            "c": float(c)}


def _oft(rng, d_in, block=32, std=0.1):
    nb = d_in // block
    Q = np.zeros((nb, block, block))
    iu = np.triu_indices(block, 1)
    for j in range(nb):
        v = std * rng.standard_normal(len(iu[0]))
        Q[j][iu] = v
        Q[j][(iu[1], iu[0])] = -v
    return {"method": "oft", "Q": Q.astype(np.float32), "block": block}


def _ssf(rng, d_out):
    return {"method": "ssf", "s": (1.0 + 0.3 * rng.standard_normal(d_out)).astype(np.float32),
            "b": (0.3 * rng.standard_normal(d_out)).astype(np.float32)}


def _loha(rng, d_in, d_out, r1, r2, dtype, c=1.0):
    """LoHa factors with A ~ N(0, 1/sqrt(d_in)), B ~ N(0, 1/r): each of the
    two products has entries of variance d_in^-1/2, so their elementwise
    product has the size of a LoRA update's entries."""
    return {"method": "loha",
            "A": round_to(_normal(rng, (d_in, r1), d_in ** -0.25), dtype),
            "B": round_to(_normal(rng, (r1, d_out), 1.0 / np.sqrt(r1)), dtype),
            "A2": round_to(_normal(rng, (d_in, r2), d_in ** -0.25), dtype),
            "B2": round_to(_normal(rng, (r2, d_out), 1.0 / np.sqrt(r2)), dtype),
            "c": float(c)}


def _lokr(rng, d_in, d_out, p, q, r, dtype, c=1.0):
    """LoKr factors: C [p, q] ~ N(0, 1), A [d_in/p, r] ~ N(0, 1/d_in),
    B [r, d_out/q] ~ N(0, 1/r) (update entries of a LoRA update's size)."""
    return {"method": "lokr",
            "C": round_to(rng.standard_normal((p, q)), dtype),
            "A": round_to(_normal(rng, (d_in // p, r), 1.0 / np.sqrt(d_in)), dtype),
            "B": round_to(_normal(rng, (r, d_out // q), 1.0 / np.sqrt(r)), dtype),
            "c": float(c)}


def _vera_shared(rng, d_in, d_out, r_v, dtype):
    return {"A": round_to(_normal(rng, (d_in, r_v), 1.0 / np.sqrt(d_in)), dtype),
            "B": round_to(_normal(rng, (r_v, d_out), 1.0 / np.sqrt(r_v)), dtype)}


def make_projection(rng, name, d_in, d_out, dtype, n):
    """Base weight and input rows of one projection."""
    W = round_to(_normal(rng, (d_out, d_in), 1.0 / np.sqrt(d_in)), dtype)
    x = round_to(rng.standard_normal((n, d_in)), dtype)
    return {"name": name, "d_in": d_in, "d_out": d_out, "dtype": dtype,
            "W": W, "x": x, "shared": None, "adapters": {}}


def tiny_mixed(seed=0, n=64, d=256, dtype="f32", with_identity=False, d_out=None):
    """Tiny single layer: W [d x d] (d_out x d when d_out is given), n rows
    assigned uniformly at random to five tenants, one per method (LoRA r8,
    DoRA r8, (IA)3, VeRA with a shared rank-32 pair, OFT with blocks of 32).
    Slots 1..5 in that order; with_identity also draws rows onto slot 0 (base
    only)."""
    rng = np.random.default_rng(seed)
    do = d if d_out is None else d_out
    p = make_projection(rng, "tiny", d, do, dtype, n)
    p["shared"] = _vera_shared(rng, d, do, 32, dtype)
    p["adapters"] = {
        1: _lora(rng, d, do, 8, dtype),
        2: _dora(rng, p["W"], 8, dtype),
        3: _ia3(rng, do),
        4: _vera(rng, 32, do),
        5: _oft(rng, d, 32),
    }
    lo = 0 if with_identity else 1
    slot_of_row = rng.integers(lo, 6, size=n).astype(np.int32)
    return {"name": "tiny_mixed", "dtype": dtype, "n": n,
            "slot_of_row": slot_of_row, "projections": [p]}


def decode_ranks(seed=7000, n=64, d_in=512, d_out=384, dtype="f16", r_v=96):
    """Decode-size layer whose terms span one, several and a partial group of
    32-wide k steps: LoRA r16, LoRA r48, DoRA r64, LoRA r160, VeRA with a
    shared rank-r_v pair, (IA)3, and identity rows.  Slots 1..6 in that
    order; rows uniform over slots 0..6."""
    rng = np.random.default_rng(seed)
    p = make_projection(rng, "decode_ranks", d_in, d_out, dtype, n)
    p["shared"] = _vera_shared(rng, d_in, d_out, r_v, dtype)
    p["adapters"] = {
        1: _lora(rng, d_in, d_out, 16, dtype),
        2: _lora(rng, d_in, d_out, 48, dtype),
        3: _dora(rng, p["W"], 64, dtype),
        4: _lora(rng, d_in, d_out, 160, dtype),
        5: _vera(rng, r_v, d_out),
        6: _ia3(rng, d_out),
    }
    slot_of_row = rng.integers(0, 7, size=n).astype(np.int32)
    return {"name": "decode_ranks", "dtype": dtype, "n": n,
            "slot_of_row": slot_of_row, "projections": [p]}


def oft_blocks(seed=6000, n=64, d_in=256, d_out=256, dtype="f32", blocks=(16, 32, 64)):
    """One layer with OFT tenants of every block size the rotation accepts
    (appendix "Training" names 32; 16 and 64 are the other sizes a d_in that
    is a multiple of 64 divides into), two per size, beside a LoRA r8 tenant
    and identity rows.  Slots 1, 2: blocks[0]; 3, 4: blocks[1]; 5, 6:
    blocks[2]; 7 LoRA; rows uniform over slots 0..7."""
    rng = np.random.default_rng(seed)
    p = make_projection(rng, "oft_blocks", d_in, d_out, dtype, n)
    p["shared"] = None
    p["adapters"] = {}
    slot = 1
    for b in blocks:
        for _ in range(2):
            p["adapters"][slot] = _oft(rng, d_in, b)
            slot += 1
    p["adapters"][slot] = _lora(rng, d_in, d_out, 8, dtype)
    slot_of_row = rng.integers(0, slot + 1, size=n).astype(np.int32)
    return {"name": "oft_blocks", "dtype": dtype, "n": n,
            "slot_of_row": slot_of_row, "projections": [p]}


def tiny_stacks(seed=5000, n=64, d=256, dtype="f32", r=8, r_v=32):
    """Tiny single layer with stacked adapters (several members applied in
    order at one hook) beside single ones.
    SSF (absent from the other workloads) draws s = 1 + 0.3 z, b = 0.3 z.
      1 LoRA then (IA)3        2 (IA)3 then LoRA        3 SSF, DoRA, (IA)3
      4 OFT then LoRA          5 VeRA then (IA)3        6 LoRA then VeRA
      7 OFT, VeRA, SSF         8 (IA)3 then SSF         9 LoRA alone
     10 VeRA alone            11 DoRA then LoRA
    and the members expanded at load: 12 LoHa (ranks 4 x 4), 13 LoKr with
    C 4 x 4 and rank 4, 14 LoKr with C 2 x 8 and rank 4, 15 LoKr then (IA)3,
    16 SSF alone; rows uniform over slots 0..16."""
    rng = np.random.default_rng(seed)
    p = make_projection(rng, "tiny", d, d, dtype, n)
    p["shared"] = _vera_shared(rng, d, d, r_v, dtype)
    W = p["W"]
    st = lambda *m: {"method": "stack", "members": list(m)}
    p["adapters"] = {
        1: st(_lora(rng, d, d, r, dtype), _ia3(rng, d)),
        2: st(_ia3(rng, d), _lora(rng, d, d, r, dtype)),
        3: st(_ssf(rng, d), _dora(rng, W, r, dtype), _ia3(rng, d)),
        4: st(_oft(rng, d, 32), _lora(rng, d, d, r, dtype)),
        5: st(_vera(rng, r_v, d), _ia3(rng, d)),
        6: st(_lora(rng, d, d, r, dtype), _vera(rng, r_v, d)),
        7: st(_oft(rng, d, 32), _vera(rng, r_v, d), _ssf(rng, d)),
        8: st(_ia3(rng, d), _ssf(rng, d)),
        9: _lora(rng, d, d, r, dtype),
        10: _vera(rng, r_v, d),
        11: st(_dora(rng, W, r, dtype), _lora(rng, d, d, r, dtype)),
        12: _loha(rng, d, d, 4, 4, dtype),
        13: _lokr(rng, d, d, 4, 4, 4, dtype),
        14: _lokr(rng, d, d, 2, 8, 4, dtype),
        15: st(_lokr(rng, d, d, 8, 4, 2, dtype), _ia3(rng, d)),
        16: _ssf(rng, d),
    }
    slot_of_row = rng.integers(0, 17, size=n).astype(np.int32)
    return {"name": "tiny_stacks", "dtype": dtype, "n": n,
            "slot_of_row": slot_of_row, "projections": [p]}


def prefill_lora_dora(seed=1000, n=1024, d=4096, r=16, dtype="f16", tenants=16, d_out=None, methods="mixed"):
    """q_proj 4096 -> 4096 (d_out x d when d_out is given), n prefill rows in
    `tenants` contiguous segments of n / tenants rows; even segments LoRA,
    odd segments DoRA, rank r (methods "lora" or "dora": every segment)."""
    rng = np.random.default_rng(seed)
    do = d if d_out is None else d_out
    p = make_projection(rng, "q", d, do, dtype, n)
    for t in range(tenants):
        dora = methods == "dora" or (methods == "mixed" and t % 2 == 1)
        p["adapters"][t + 1] = (_dora(rng, p["W"], r, dtype) if dora
                                else _lora(rng, d, do, r, dtype))
    seg = max(1, n // tenants)
    slot_of_row = np.minimum(np.arange(n) // seg + 1, tenants).astype(np.int32)
    return {"name": "prefill_lora_dora", "dtype": dtype, "n": n,
            "slot_of_row": slot_of_row, "projections": [p]}


# Projections that read one input in the model (the fused layers q/k/v and
# gate/up): they share the input rows and VeRA's A (appendix "Byte counts":
# the shared A is read once per fused input, B once per slice).
FUSED_INPUT_OF = {"q": "q", "k": "q", "v": "q", "o": "o", "gate": "gate", "up": "gate", "down": "down"}


def decoder_layer_mixed(seed=2000, n=64, dtype="f16", per_method=4, r=16, r_v=256,
                        oft_block=32, shapes=LLAMA8B_PROJECTIONS, pure_lora=False):
    """One decoder layer's seven projections with 5 * per_method tenants:
    LoRA r16 and DoRA r16 on all seven, (IA)3 on k, v and up, VeRA (shared
    rank-256 pair) on all seven, OFT (blocks of 32) on q, k and v.  Tenant t
    has slot t + 1 in every projection; where its method does not adapt a
    projection the slot holds the identity.  Row j belongs to tenant
    j mod (5 * per_method), then the rows are shuffled so segments are not
    contiguous.  Inputs are N(0, 1) rows, one draw per fused input (q, k and
    v read the same rows, gate and up the same rows, o and down their own),
    and VeRA's A is drawn once per fused input (B per projection); a
    projection that takes them from an earlier one records its name in
    p["input_of"] and p["shared"]["a_from"].

    pure_lora: the same rows and slots, every tenant a rank-r LoRA (the
    equal-size pure-LoRA batch)."""
    rng = np.random.default_rng(seed)
    T = 5 * per_method
    order = ["lora", "dora", "ia3", "vera", "oft"]
    methods = [order[t // per_method] for t in range(T)]
    projs = []
    by_name = {}
    for name, d_in, d_out in shapes:
        p = make_projection(rng, name, d_in, d_out, dtype, n)
        src = by_name.get(FUSED_INPUT_OF.get(name, name))
        if src is not None and src["d_in"] == d_in:
            p["x"] = src["x"]
            p["input_of"] = src["name"]
        if not pure_lora:
            p["shared"] = _vera_shared(rng, d_in, d_out, r_v, dtype)
            if src is not None and src["d_in"] == d_in:
                p["shared"]["A"] = src["shared"]["A"]
                p["shared"]["a_from"] = src["name"]
        for t, m in enumerate(methods):
            slot = t + 1
            if pure_lora or m == "lora":
                p["adapters"][slot] = _lora(rng, d_in, d_out, r, dtype)
            elif m == "dora":
                p["adapters"][slot] = _dora(rng, p["W"], r, dtype)
            elif m == "ia3":
                p["adapters"][slot] = (_ia3(rng, d_out) if name in ("k", "v", "up")
                                       else {"method": "identity"})
            elif m == "vera":
                p["adapters"][slot] = _vera(rng, r_v, d_out)
            elif m == "oft":
                p["adapters"][slot] = (_oft(rng, d_in, oft_block) if name in ("q", "k", "v")
                                       else {"method": "identity"})
        projs.append(p)
        by_name.setdefault(name, p)
    slot_of_row = (np.arange(n) % T + 1).astype(np.int32)
    slot_of_row = slot_of_row[rng.permutation(n)]
    return {"name": "decoder_layer_mixed" + ("_pure_lora" if pure_lora else ""),
            "dtype": dtype, "n": n, "slot_of_row": slot_of_row, "projections": projs}


def vera_sweep(seed=3000, n=256, d_in=4096, d_out=4096, tenants=16, r_v=256, dtype="f16",
               as_lora=False):
    """VeRA tenant sweep: n rows drawn uniformly over `tenants` VeRA tenants
    sharing one rank-r_v pair.  as_lora: the same tenants stored as their
    exact rank-r_v LoRA conversion, A_a = A diag(c d_a), B_a = B diag(e_a)
    (§4.2; the factors are rounded to the storage type after scaling)."""
    rng = np.random.default_rng(seed)
    p = make_projection(rng, "vera_%dx%d" % (d_in, d_out), d_in, d_out, dtype, n)
    shared = _vera_shared(rng, d_in, d_out, r_v, dtype)
    p["shared"] = shared
    for t in range(tenants):
        rec = _vera(rng, r_v, d_out)
        if as_lora:
            A = round_to(shared["A"].astype(np.float64) * (rec["c"] * rec["d"].astype(np.float64))[None, :], dtype)
            B = round_to(shared["B"].astype(np.float64) * rec["e"].astype(np.float64)[None, :], dtype)
            rec = {"method": "lora", "A": A, "B": B, "c": 1.0}
        p["adapters"][t + 1] = rec
    if as_lora:
        p["shared"] = None
    slot_of_row = rng.integers(1, tenants + 1, size=n).astype(np.int32)
    return {"name": "vera_sweep", "dtype": dtype, "n": n, "slot_of_row": slot_of_row,
            "projections": [p]}
