"""The byte model: bytes and launches each route and each kernel moves, and
the time they predict.

Scute paper (arXiv 2611.01089):
  * §4.1 Proposition 2 and the appendix "Byte counts" / "Propositions
    A2-A4": a slot carried by a pass that already reads and writes its
    tensor adds at most k·d_out elements; a slot in a pass of its own adds
    2N·d_out elements and a launch (4N·d_out if it first writes a per-row
    copy); an input transform in its own pass moves 2N·d_in + k·d_in·b_R
    elements; shared factors are read once per step, r(d_in + d_out), plus
    k(r + d_out) vector elements, against k·r(d_in + d_out) for k
    conversions to LoRA.
  * §4.2 Table 2: bytes each route reads per decode step, 16 tenants,
    Llama-3.1-8B in fp16, every adapted projection of 32 layers, and that
    time at the copy bandwidth β.
  * §4.3: predicted time t0 + ΔQ/β + ΔL·λ.

Pure Python; no GPU needed.
"""
from dataclasses import dataclass, field

# Llama-3.1-8B projections (d_in, d_out), §6.1; fused groups share an input.
LLAMA8B = {"q": (4096, 4096), "k": (4096, 1024), "v": (4096, 1024), "o": (4096, 4096),
           "gate": (4096, 14336), "up": (4096, 14336), "down": (14336, 4096)}
LLAMA8B_LAYERS = 32
FUSED_GROUPS = (("q", "k", "v"), ("o",), ("gate", "up"), ("down",))
A6000_BETA = 680e9          # bytes/s, §2 "GPU cost terms"
A6000_LAMBDA = 0.96e-6      # s per launch inside a graph


def predict_time(t0, dq_bytes, dl_launches, beta, lam):
    """§4.3: t0 + ΔQ/β + ΔL·λ."""
    return t0 + dq_bytes / beta + dl_launches * lam


# ----------------------------------------------- Table 2 (model-level) -----

def lora_bytes(rank, tenants, q=2, projections=LLAMA8B, layers=LLAMA8B_LAYERS):
    """k conversions (or LoRA tenants) of rank r read their own factors:
    k·r·(d_in + d_out) per projection (§4.2)."""
    per_layer = sum(rank * (di + do) for di, do in projections.values())
    return tenants * per_layer * q * layers


def vera_route2_bytes(rank, tenants, q=2, projections=LLAMA8B, layers=LLAMA8B_LAYERS,
                      groups=FUSED_GROUPS):
    """Route two: the shared A is read once per fused input group and B once
    per slice, r·d_in + r·d_out, plus k·(r + d_out) vector elements per
    projection (appendix "Byte counts")."""
    per_layer = 0
    for grp in groups:
        per_layer += rank * projections[grp[0]][0]
        for p in grp:
            d_out = projections[p][1]
            per_layer += rank * d_out + tenants * (rank + d_out)
    return per_layer * q * layers


def oft_route3_block_bytes(tenants, block=32, q=2, projections=LLAMA8B, layers=LLAMA8B_LAYERS):
    """Route three's blocks: k·d_in·b_R elements per projection (the 2N·d_in
    row traffic is counted apart, see oft_rows_bytes)."""
    return tenants * sum(di * block for di, _ in projections.values()) * q * layers


def oft_rows_bytes(n_rows, q=2, projections=LLAMA8B, layers=LLAMA8B_LAYERS):
    return 2 * n_rows * sum(di for di, _ in projections.values()) * q * layers


def ia3_route1_bytes(tenants, q=2, layers=LLAMA8B_LAYERS, d_outs=(1024, 1024, 14336)):
    """Route one: at most k·d_out extra elements per adapted projection;
    (IA)3 scales k, v and (as s of up) the FFN activation."""
    return tenants * sum(d_outs) * q * layers


def table2(tenants=16, beta=A6000_BETA):
    """The rows of Table 2 in bytes and seconds at β."""
    ia3_conv = {"k": LLAMA8B["k"], "v": LLAMA8B["v"], "down": LLAMA8B["down"]}
    rows = {
        "lora_r16_expand": lora_bytes(16, tenants),
        "vera_route2": vera_route2_bytes(256, tenants),
        "vera_as_lora_r256": lora_bytes(256, tenants),
        "vera_as_lora_r64": lora_bytes(64, tenants),
        "oft_route3": oft_route3_block_bytes(tenants),
        "oft_as_lora_r64": lora_bytes(64, tenants),
        "ia3_route1": ia3_route1_bytes(tenants),
        "ia3_as_lora_r64": lora_bytes(64, tenants, projections=ia3_conv),
    }
    return {k: (v, v / beta) for k, v in rows.items()}


def per_tenant_decode(beta=A6000_BETA):
    """Table A9's predicted column: decode time one more tenant adds."""
    return {
        "vera_scute": (vera_route2_bytes(256, 1) - vera_route2_bytes(256, 0)) / beta,
        "oft_scute": oft_route3_block_bytes(1) / beta,
        "ia3_scute": ia3_route1_bytes(1) / beta,
        "rank64": lora_bytes(64, 1) / beta,
        "rank256": lora_bytes(256, 1) / beta,
    }


# ----------------------------------------- this library's kernels ----------

@dataclass
class BatchShape:
    """What one forward of one projection touches.  Counts are of rows and
    of distinct tenants present in the batch."""
    n: int
    d_in: int
    d_out: int
    q: int = 2                       # bytes per element of x, W, out, factors
    f_v: int = 4                     # bytes per element of s, b, d, e (fp32)
    owned_ranks: list = field(default_factory=list)   # rank of each distinct owned-term tenant
    owned_ranks_stored: list = field(default_factory=list)  # the same, padded to 16 as stored
    n_owned: int = 0                 # rows with an owned term
    v_elems: int = 0                 # Σ over owned rows of the row's rank
    f_uv: int = 0                    # bytes per element of V and U between shrink and expand (0: q)
    r_v: int = 0
    n_vera: int = 0
    k_vera: int = 0
    k_s: int = 0                     # distinct tenants with a live s
    k_b: int = 0
    n_oft: int = 0
    k_oft: int = 0
    oft_block: int = 32
    vera_a_read: bool = True         # False: another projection of the fused input reads A_v


def shape_of(n, d_in, d_out, slot_of_row, adapters, q=2, r_v=0, vera_a_read=True):
    """BatchShape from per-row slots and raw adapter records.  vera_a_read
    False: the projection shares its input and VeRA's A with an earlier one
    of its fused layer, which reads A_v and computes x·A_vᵀ for both
    (appendix "Byte counts")."""
    present = {}
    for s in slot_of_row:
        present[int(s)] = present.get(int(s), 0) + 1
    bs = BatchShape(n=n, d_in=d_in, d_out=d_out, q=q, r_v=r_v, vera_a_read=vera_a_read)
    for s, rows in present.items():
        ad = adapters.get(s, {"method": "identity"})
        m = ad["method"]
        if m in ("lora", "dora"):
            r = ad["A"].shape[1]
            bs.owned_ranks.append(r)
            bs.owned_ranks_stored.append(r + (-r) % 16)
            bs.n_owned += rows
            bs.v_elems += rows * r
        if m == "dora" or m == "ia3" or m == "ssf":
            bs.k_s += 1
        if m == "ssf":
            bs.k_b += 1
        if m == "vera":
            bs.n_vera += rows
            bs.k_vera += 1
        if m == "oft":
            bs.n_oft += rows
            bs.k_oft += 1
            bs.oft_block = ad["Q"].shape[1]
    return bs


def kernel_bytes(b):
    """Algorithmic bytes (what each kernel must read and write) and flops.

    Factors count at their true rank (the stored copy is padded to 16 rows;
    stored_factor_bytes gives that), and V and U once written by the shrink
    and once read by the expand, in the layer type (as stored)."""
    sum_r = sum(b.owned_ranks)
    fuv = b.f_uv or b.q
    out = {}
    out["oft"] = {"bytes": b.q * (2 * b.n_oft * b.d_in + b.k_oft * b.d_in * b.oft_block),
                  "flops": 2 * b.oft_block * b.n_oft * b.d_in, "launches": 1 if b.k_oft else 0}
    out["gemm"] = {"bytes": b.q * (b.n * b.d_in + b.d_in * b.d_out + b.n * b.d_out),
                   "flops": 2 * b.n * b.d_in * b.d_out, "launches": 1}
    sh = b.q * (b.n_owned * b.d_in + sum_r * b.d_in) + fuv * b.v_elems
    if b.k_vera:
        if b.vera_a_read:
            sh += b.q * (b.n_vera * b.d_in + b.r_v * b.d_in)
        else:                        # reads the fused input's x·A_v instead of x and A_v
            sh += fuv * b.n_vera * b.r_v
        sh += fuv * b.n_vera * b.r_v + b.f_v * b.k_vera * b.r_v
    out["shrink"] = {"bytes": sh, "flops": 2 * b.d_in * (b.v_elems + b.n_vera * b.r_v),
                     "launches": 1 if (b.owned_ranks or b.k_vera) else 0}
    ex = b.q * (2 * b.n * b.d_out + sum_r * b.d_out) + fuv * (b.v_elems + b.n_vera * b.r_v)
    ex += b.f_v * (b.k_s + b.k_b + b.k_vera) * b.d_out
    if b.k_vera:
        ex += b.q * b.r_v * b.d_out
    out["expand"] = {"bytes": ex, "flops": 2 * b.d_out * (b.v_elems + b.n_vera * b.r_v),
                     "launches": 1}
    out["plan"] = {"bytes": 4 * b.n * 7, "flops": 0, "launches": 1}
    return out


def stored_factor_bytes(b):
    """Bytes of the owned factors as stored (rank padded to 16), read once by
    the shrink (A') and once by the expand (B')."""
    return b.q * sum(b.owned_ranks_stored) * (b.d_in + b.d_out)


def adapter_path_bytes(b):
    """Bytes of the adapter kernels (everything but the base GEMM)."""
    kb = kernel_bytes(b)
    return sum(v["bytes"] for k, v in kb.items() if k != "gemm")


def scale_route_extra(n, d_out, route, q=2):
    """Extra bytes and launches of applying s outside the expand (appendix
    "Routes"): side kernel or gathered scale 2N·d_out and one launch; index
    scale 4N·d_out and two launches (here the per-row copy is fp32)."""
    if route in (1, 2):
        return 2 * n * d_out * q, 1
    if route == 3:
        return 2 * n * d_out * q + 2 * n * d_out * 4, 2
    return 0, 0
