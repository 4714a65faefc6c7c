"""Helpers shared by the GPU tests: build layers through the C ABI from the
seeded workloads, run them, and compute the oracle's reference."""
import sys

import numpy as np
import torch

import oracle

TORCH = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def make_layer(proj, max_slots=64, max_rank=256, options=None, skip=()):
    from tenant_peft_adapter_amd.layer import AdaptedLayer
    W = torch.tensor(proj["W"]).to(TORCH[proj["dtype"]]).cuda()
    L = AdaptedLayer(W, max_slots=max_slots, max_rank=max_rank)
    for k, v in (options or {}).items():
        L.set_option(k, v)
    if proj["shared"] is not None:
        L.set_vera_shared(proj["shared"]["A"], proj["shared"]["B"])
    for slot in sorted(proj["adapters"]):
        rec = proj["adapters"][slot]
        if slot in skip:
            rec = {"method": "identity"}
        got = L.load(rec)
        assert got == slot, (got, slot)
    return L


def run(L, x_np, sor_np, dtype):
    x = torch.tensor(x_np).to(TORCH[dtype]).cuda()
    sor = torch.tensor(np.asarray(sor_np, dtype=np.int32)).cuda()
    out = L.forward(x, sor)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64)


def reference(proj, sor, rows=None):
    """Oracle output y, base output h and plain xW for the given rows."""
    x = proj["x"].astype(np.float64)
    W = proj["W"].astype(np.float64).T
    sor = np.asarray(sor)
    if rows is not None:
        x, sor = x[rows], sor[rows]
    y, h = oracle.layer_forward(x, W, sor, proj["adapters"], proj["shared"])
    return y, h, x @ W


def check(y_gpu, y, h, xw, mean_tol=0.01, max_tol=2e-3, label=""):
    m = oracle.parity_metrics(y_gpu, y, h, xw)
    say(label, {k: (round(v, 8) if isinstance(v, float) else v) for k, v in m.items()})
    assert m["mean_rel"] <= mean_tol, (label, m)
    assert m["max_abs"] <= max_tol * m["max_h"], (label, m)
    return m


def slot_classes(proj, max_slots):
    """Term class per slot for the oracle's plan (-1 = not loaded)."""
    cls = [-1] * max_slots
    has_R = [0] * max_slots
    cls[0] = 2
    for slot, ad in proj["adapters"].items():
        m = ad["method"]
        cls[slot] = 0 if m in ("lora", "dora") else 1 if m == "vera" else 2
        has_R[slot] = 1 if m == "oft" else 0
    return cls, has_R
