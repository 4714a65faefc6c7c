"""GPU parity of stacked adapters (§3.2 paragraph "Stacking", appendix
"Stacking"): several members applied in order at one hook, loaded through
tpa_adapter_load_stack as one slot, against the oracle's sequential
application of each member's own definition; and of LoHa and LoKr, expanded
at load into one low-rank term (§3.1, "Other methods fit as well"), against
their own definitions.  Same tolerances as the other
parity tests: fp32 layers 1e-4 (mean relative) and 2e-5 · max|h| (max);
f16 layers 1% and 2e-3 · max|h|."""
import numpy as np
import pytest
import torch

from gpu_util import check, make_layer, reference, run, say
from tenant_peft_adapter_amd import binding as B
from workloads import synth

pytestmark = pytest.mark.gpu

# bf16 keeps 8 mantissa bits: its bounds scale with the type's unit
# roundoff, as in the single-member tests.
TOL = {"f32": dict(mean_tol=1e-4, max_tol=2e-5), "f16": dict(mean_tol=0.01, max_tol=2e-3),
       "bf16": dict(mean_tol=0.05, max_tol=1.6e-2)}


@pytest.mark.parametrize("dtype,n", [("f32", 64), ("f16", 64), ("f16", 17), ("f16", 300), ("bf16", 64),
                                     ("bf16", 300)])
def test_stacks_match_oracle(dtype, n):
    wl = synth.tiny_stacks(seed=5000 + n, n=n, dtype=dtype)
    p = wl["projections"][0]
    say("tiny_stacks %s n=%d" % (dtype, n))
    L = make_layer(p, max_slots=24, max_rank=64)
    y_gpu = run(L, p["x"], wl["slot_of_row"], dtype)
    y, h, xw = reference(p, wl["slot_of_row"])
    check(y_gpu, y, h, xw, label="stacks %s n=%d" % (dtype, n), **TOL[dtype])
    # every slot on its own rows too (a stack's error must not hide in the mean)
    for slot in range(1, 17):
        rows = np.nonzero(wl["slot_of_row"] == slot)[0]
        if len(rows):
            check(y_gpu[rows], y[rows], h[rows], xw[rows], label="slot %d" % slot, **TOL[dtype])
    L.close()


def test_stack_metadata():
    wl = synth.tiny_stacks(n=8, dtype="f16")
    p = wl["projections"][0]
    L = make_layer(p, max_slots=24, max_rank=64)
    want = {  # slot: (term_kind, rank, live bits)
        1: (1, 8, B.LIVE_S), 2: (1, 8, B.LIVE_S), 3: (1, 8, B.LIVE_S | B.LIVE_B), 4: (1, 8, B.LIVE_R),
        5: (2, 32, B.LIVE_S | B.LIVE_D | B.LIVE_E), 6: (1, 40, 0),
        7: (2, 32, B.LIVE_S | B.LIVE_B | B.LIVE_R | B.LIVE_D | B.LIVE_E), 8: (0, 0, B.LIVE_S | B.LIVE_B),
        11: (1, 16, B.LIVE_S),
    }
    for slot, (kind, rank, live) in want.items():
        info = L.info(slot)
        say(slot, info)
        assert info["method"] == B.METHODS["stack"], (slot, info)
        assert (info["term_kind"], info["rank"], info["live_mask"]) == (kind, rank, live), (slot, info)
    assert L.info(9)["method"] == B.METHODS["lora"]
    # LoHa and LoKr: one owned term of the expanded rank, c folded into A
    for slot, meth, rank in ((12, "loha", 16), (13, "lokr", 16), (14, "lokr", 8)):
        info = L.info(slot)
        assert (info["method"], info["term_kind"], info["rank"]) == (B.METHODS[meth], 1, rank), (slot, info)
        assert (info["fold_mask"], info["live_mask"]) == (B.FOLD_C_A, 0), (slot, info)
    info = L.info(15)
    assert (info["method"], info["rank"], info["live_mask"]) == (B.METHODS["stack"], 8, B.LIVE_S), info
    assert L.info(16)["method"] == B.METHODS["ssf"]
    assert L.info(6)["fold_mask"] & B.FOLD_D_A  # the VeRA term entered in owned form
    L.close()


def test_stack_rejections_and_reload():
    wl = synth.tiny_stacks(n=64, dtype="f16")
    p = wl["projections"][0]
    L = make_layer(p, max_slots=24, max_rank=64)
    ads = p["adapters"]
    oft = ads[4]["members"][0]
    lora = ads[9]
    with pytest.raises(B.TpaError) as ei:  # OFT after the first member
        L.load({"method": "stack", "members": [lora, oft]})
    assert ei.value.code == -1
    small = make_layer({**p, "adapters": {}}, max_slots=16, max_rank=32)
    rng = np.random.default_rng(3)
    big = (ads[6],  # stacked rank 8 + 32, LoHa 8 x 8, LoKr 16 x 4: all above max_rank 32
           synth._loha(rng, 256, 256, 8, 8, "f16"), synth._lokr(rng, 256, 256, 16, 16, 4, "f16"))
    for rec in big:
        with pytest.raises(B.TpaError) as ei:
            small.load(rec)
        assert ei.value.code == -1
    small.close()
    # unload the rotated stacks and load them again: same outputs
    before = run(L, p["x"], wl["slot_of_row"], "f16")
    for slot in (4, 7):
        L.unload(slot)
    assert L.load(ads[4]) == 4
    assert L.load(ads[7]) == 7
    after = run(L, p["x"], wl["slot_of_row"], "f16")
    np.testing.assert_array_equal(before, after)
    # a one-member stack is the plain load
    s1 = L.load({"method": "stack", "members": [lora]})
    assert L.info(s1)["method"] == B.METHODS["lora"]
    L.close()


def test_stack_argument_errors():
    """Counts outside 1..TPA_MAX_STACK and null pointers are rejected
    before anything is uploaded; the layer keeps working."""
    import ctypes
    wl = synth.tiny_stacks(n=16, dtype="f16")
    p = wl["projections"][0]
    L = make_layer({**p, "adapters": {}}, max_slots=8, max_rank=64)
    lib = B.library()
    slot = ctypes.c_int32()
    descs = (B.tpa_adapter_desc * 9)()
    for count in (0, 9, -1):
        assert lib.tpa_adapter_load_stack(L.handle, descs, count, ctypes.byref(slot), None) == -1
    assert lib.tpa_adapter_load_stack(L.handle, None, 2, ctypes.byref(slot), None) == -1
    assert lib.tpa_adapter_load_stack(L.handle, descs, 2, None, None) == -1
    descs[0].method, descs[1].method = 42, 1
    assert lib.tpa_adapter_load_stack(L.handle, descs, 2, ctypes.byref(slot), None) == -2
    assert L.load(p["adapters"][1]) == 1
    L.close()


@pytest.mark.parametrize("n", [16, 300])
def test_stacks_and_products_in_a_group(n):
    """Stacked, LoHa and LoKr slots through a fused group forward (one
    launch per kernel over three projections sharing the plan) match the
    separate forwards' outputs within the parity bound and the oracle."""
    from tenant_peft_adapter_amd.layer import LayerGroup, RowPlan
    wls = [synth.tiny_stacks(seed=700 + 10 * i + n, n=n, dtype="f16") for i in range(3)]
    for w in wls[1:]:
        w["slot_of_row"] = wls[0]["slot_of_row"]
    ps = [w["projections"][0] for w in wls]
    Ls = [make_layer(p, max_slots=24, max_rank=64) for p in ps]
    sor = torch.tensor(wls[0]["slot_of_row"]).cuda()
    xs = [torch.tensor(p["x"]).half().cuda() for p in ps]
    plan = RowPlan(Ls[0], n).build(Ls[0], sor)
    outs = LayerGroup(Ls, n).forward(plan, xs)
    torch.cuda.synchronize()
    for o, p in zip(outs, ps):
        y, h, xw = reference(p, wls[0]["slot_of_row"])
        check(o.float().cpu().numpy().astype(np.float64), y, h, xw, label="group n=%d" % n, **TOL["f16"])
    plan.close()
    for L in Ls:
        L.close()
