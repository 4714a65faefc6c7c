"""Seeded synthetic inputs for the full adapter stack: 32 decoder layers of
Llama-3.1-8B projection shapes, 1024 resident tenants in an equal method
mix, rows drawn from a Zipf(1.1) popularity over tenants (Scute paper,
arXiv 2611.01089: §6.1 "Setup" for the shapes, the appendix "Training" for
ranks, block size and which projections each method adapts).

Readings (where the workload description leaves a step open):
  * tenant t (0-based) has popularity rank t + 1, p(rank i) ∝ i^-1.1, and
    method t mod 5 in the order LoRA, DoRA, (IA)3, VeRA, OFT; it sits in
    slot t + 1 of every projection, as the identity where its method does
    not adapt that projection (placement as in the single decoder layer:
    LoRA, DoRA, VeRA on all seven, (IA)3 on k, v, up, OFT on q, k, v);
  * LoRA and DoRA at rank 64, VeRA's shared pair at rank 256, OFT blocks of
    32, with the value distributions of the other workloads;
  * raw parameters are drawn once per (projection, method); tenant t's own
    record is that prototype with a factor f_t in [0.75, 1.25) of its own
    (a golden-ratio sequence, so no two tenants share one) applied to its
    adapter's deviation from the identity and rounded to the layer type
    again: LoRA and DoRA A·f_t (DoRA also m·f_t), (IA)3 1 + (l − 1)·f_t,
    VeRA 1 + (d − 1)·f_t and 1 + (e − 1)·f_t, OFT Q·f_t.  So every tenant
    has distinct values (a row routed to another tenant of the same method
    gives another output) while drawing 1024 full records stays cheap; the
    base weights and inputs are drawn per layer and projection on the
    device;
  * DoRA's magnitude is m = 1 + 0.1 z per column: with these weights the
    column norms of W + cAB are close to 1, so the scale stays near 1 ± 0.1
    without forming the norms on the host for all 32 layers.

Every host array is float32 holding a value rounded to the layer type, as in
``synth``.
"""
import numpy as np

from . import synth

METHODS = ("lora", "dora", "ia3", "vera", "oft")
IA3_ON = ("k", "v", "up")
OFT_ON = ("q", "k", "v")


def method_of(t):
    return METHODS[t % len(METHODS)]


def zipf_rows(n, tenants=1024, s=1.1, seed=4100):
    """slot_of_row for n rows: tenant t drawn with probability ∝ (t + 1)^-s."""
    rng = np.random.default_rng(seed + n)
    p = np.arange(1, tenants + 1, dtype=np.float64) ** -s
    p /= p.sum()
    return (rng.choice(tenants, size=n, p=p) + 1).astype(np.int32)


def prototypes(seed=4000, r=64, r_v=256, dtype="f16", shapes=synth.LLAMA8B_PROJECTIONS):
    """Per projection: its shapes, VeRA's shared pair and one raw-parameter
    record per method (the identity where the method does not adapt it)."""
    rng = np.random.default_rng(seed)
    out = {}
    for name, d_in, d_out in shapes:
        dora = synth._lora(rng, d_in, d_out, r, dtype)
        dora["method"] = "dora"
        dora["m"] = (1.0 + 0.1 * rng.standard_normal(d_out)).astype(np.float32)
        recs = {
            "lora": synth._lora(rng, d_in, d_out, r, dtype),
            "dora": dora,
            "ia3": synth._ia3(rng, d_out) if name in IA3_ON else {"method": "identity"},
            "vera": synth._vera(rng, r_v, d_out),
            "oft": synth._oft(rng, d_in, 32) if name in OFT_ON else {"method": "identity"},
        }
        out[name] = {"name": name, "d_in": d_in, "d_out": d_out, "r_v": r_v,
                     "shared": synth._vera_shared(rng, d_in, d_out, r_v, dtype), "records": recs}
    return out


def tenant_factor(t):
    """f_t in [0.75, 1.25): 0.75 + 0.5 · frac(t · φ), distinct for every t."""
    return 0.75 + 0.5 * ((t * 0.6180339887498949) % 1.0)


def tenant_record(proto, t, dtype="f16"):
    """Raw-parameter record of tenant t (0-based) for one projection: the
    method's prototype with the tenant's factor applied (module docstring)."""
    rec = proto["records"][method_of(t)]
    f = np.float64(tenant_factor(t))
    m = rec["method"]
    if m in ("lora", "dora"):
        out = dict(rec)
        out["A"] = synth.round_to(rec["A"].astype(np.float64) * f, dtype)
        if m == "dora":
            out["m"] = (rec["m"].astype(np.float64) * f).astype(np.float32)
        return out
    if m == "ia3":
        return {"method": "ia3", "l": (1.0 + (rec["l"].astype(np.float64) - 1.0) * f).astype(np.float32)}
    if m == "vera":
        return {"method": "vera", "c": rec["c"],
                "d": (1.0 + (rec["d"].astype(np.float64) - 1.0) * f).astype(np.float32),
                "e": (1.0 + (rec["e"].astype(np.float64) - 1.0) * f).astype(np.float32)}
    if m == "oft":
        return {"method": "oft", "block": rec["block"], "Q": (rec["Q"].astype(np.float64) * f).astype(np.float32)}
    return rec


class TenantRecords:
    """slot -> raw-parameter record (slot t + 1 holds tenant t), made on
    access: only the tenants a check touches are materialized."""

    def __init__(self, proto, tenants=1024):
        self.proto, self.tenants = proto, tenants
        self._memo = {}

    def __len__(self):
        return self.tenants

    def __contains__(self, slot):
        return 1 <= int(slot) <= self.tenants

    def __iter__(self):
        return iter(range(1, self.tenants + 1))

    def __getitem__(self, slot):
        slot = int(slot)
        if slot not in self:
            raise KeyError(slot)
        if slot not in self._memo:
            self._memo[slot] = tenant_record(self.proto, slot - 1)
        return self._memo[slot]

    def get(self, slot, default=None):
        return self[slot] if slot in self else default

    def items(self):
        return ((s, self[s]) for s in self)


def adapters_of(proto, tenants=1024):
    """slot -> raw-parameter record for one projection of the stack (made on
    access)."""
    return TenantRecords(proto, tenants)


def device_weight(torch, layer, name, d_out, d_in, seed=4200):
    """W [d_out, d_in] ~ N(0, 1/d_in) in fp16, drawn on the device from a
    seed of its own per (layer, projection)."""
    idx = [p[0] for p in synth.LLAMA8B_PROJECTIONS].index(name)
    g = torch.Generator(device="cuda")
    g.manual_seed(seed + 16 * layer + idx)
    W = torch.empty((d_out, d_in), dtype=torch.float16, device="cuda")
    for r0 in range(0, d_out, 2048):   # bounded fp32 temporaries
        r1 = min(d_out, r0 + 2048)
        W[r0:r1] = (torch.randn((r1 - r0, d_in), generator=g, device="cuda") / np.sqrt(d_in)).half()
    return W


def device_input(torch, n, d_in, name, seed=4300):
    """x [n, d_in] ~ N(0, 1) in fp16, per projection."""
    idx = [p[0] for p in synth.LLAMA8B_PROJECTIONS].index(name)
    g = torch.Generator(device="cuda")
    g.manual_seed(seed + idx)
    return torch.randn((n, d_in), generator=g, device="cuda").half()
