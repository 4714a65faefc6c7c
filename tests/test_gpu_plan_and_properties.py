"""GPU tests of the row plan, the merged-slot metadata, and properties the
layer must have beyond parity: identity rows equal the base-only output bit
for bit, a row's output does not depend on the rest of the batch, one
tenant's weights never reach another tenant's rows, invalid slots raise the
sticky flag and compute as the identity, runs are deterministic, a captured
HIP graph replays correctly, and the error paths return their codes."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from gpu_util import TORCH, check, make_layer, reference, run, say, slot_classes
from workloads import synth

pytestmark = pytest.mark.gpu

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "table1_members.json")))["methods"]


def _tiny(seed=3, n=64, dtype="f16"):
    wl = synth.tiny_mixed(seed=seed, n=n, dtype=dtype, with_identity=True)
    return wl, wl["projections"][0]


# ------------------------------------------------------------------ plan ---

@pytest.mark.parametrize("n,tile_rows", [(1, 16), (64, 16), (300, 16), (1000, 16), (1000, 64), (4096, 16),
                                         (4096, 64), (8192, 16), (8192, 64)])
def test_plan_bit_exact_against_oracle(n, tile_rows):
    wl, p = _tiny()
    L = make_layer(p, max_slots=8, max_rank=32, options={3: tile_rows})
    rng = np.random.default_rng(n)
    sor = rng.integers(-1, 9, size=n).astype(np.int32)     # includes invalid ids
    say("plan n=%d tile_rows=%d" % (n, tile_rows))
    got = L.plan(torch.tensor(sor).cuda())
    cls, has_R = slot_classes(p, 8)
    want = oracle.plan(sor.tolist(), cls, tile_rows, has_R)
    for k in ("perm", "row_slot", "seg_ptr", "seg_slot", "class_ptr", "tiles", "oft_tiles", "invalid"):
        assert got[k] == (list(want[k]) if isinstance(want[k], list) else want[k]), k


def test_plan_empty_and_single_class():
    wl, p = _tiny()
    L = make_layer(p, max_slots=8, max_rank=32)
    got = L.plan(torch.zeros(0, dtype=torch.int32).cuda())
    assert got["perm"] == [] and got["tiles"] == [] and got["invalid"] == 0
    sor = np.full(40, 4, np.int32)                            # all VeRA
    got = L.plan(torch.tensor(sor).cuda())
    cls, has_R = slot_classes(p, 8)
    want = oracle.plan(sor.tolist(), cls, 16, has_R)
    assert got["tiles"] == want["tiles"] and got["class_ptr"] == want["class_ptr"]


def test_metadata_matches_table1():
    wl, p = _tiny()
    L = make_layer(p, max_slots=8, max_rank=32)
    names = {1: "lora", 2: "dora", 3: "ia3", 4: "vera", 5: "oft"}
    from tenant_peft_adapter_amd import binding as B
    for slot, meth in names.items():
        info = L.info(slot)
        assert info == {**B.tpa_method_info(meth), "rank": info["rank"], "oft_block": info["oft_block"]}
        assert info["rank"] == {"lora": 8, "dora": 8, "vera": 32}.get(meth, 0)
        assert info["oft_block"] == (32 if meth == "oft" else 0)
    assert L.info(0)["method"] == 0


# ------------------------------------------------------------ properties ---

def test_identity_rows_equal_base_only_output_bitwise():
    wl, p = _tiny(seed=4)
    sor = wl["slot_of_row"]
    L = make_layer(p, max_slots=8, max_rank=32)
    y_mixed = run(L, p["x"], sor, "f16")
    base = make_layer({**p, "adapters": {}, "shared": None}, max_slots=8, max_rank=32)
    y_base = run(base, p["x"], np.zeros_like(sor), "f16")
    ident = sor == 0
    assert ident.sum() > 0
    assert np.array_equal(y_mixed[ident], y_base[ident])


@pytest.mark.parametrize("n,path", [(20, 0), (20, 2), (64, 0), (64, 2), (200, 1), (200, 3)])
def test_batch_invariance_row_alone_vs_in_batch(n, path):
    """With the kernel configuration pinned, a row computed alone equals the
    same row inside a batch of other tenants, bit for bit."""
    wl, p = _tiny(seed=5, n=n)
    opts = {1: 2, 2: 2, 3: 16, 4: path}
    L = make_layer(p, max_slots=8, max_rank=32, options=opts)
    sor = wl["slot_of_row"]
    y_all = run(L, p["x"], sor, "f16")
    for i in [0, n // 2, n - 1]:
        y_one = run(L, p["x"][i:i + 1], sor[i:i + 1], "f16")
        assert np.array_equal(y_one[0], y_all[i]), i


def test_isolation_canary_tenant():
    """A canary adapter with a huge update changes only its own rows."""
    wl, p = _tiny(seed=6)
    sor = wl["slot_of_row"].copy()
    d_in, d_out = p["d_in"], p["d_out"]
    canary = {"method": "lora", "A": np.ones((d_in, 8), np.float32) * 0.5,
              "B": np.ones((8, d_out), np.float32) * 0.5, "c": 8.0}
    with_canary = {**p, "adapters": {**p["adapters"], 6: canary}}
    without = {**p, "adapters": {**p["adapters"], 6: {"method": "identity"}}}
    sor[::7] = 6
    La = make_layer(with_canary, max_slots=8, max_rank=32)
    Lb = make_layer(without, max_slots=8, max_rank=32)
    ya = run(La, p["x"], sor, "f16")
    yb = run(Lb, p["x"], sor, "f16")
    other = sor != 6
    assert np.array_equal(ya[other], yb[other])
    assert np.all(np.abs(ya[~other] - yb[~other]).max(axis=1) > 1.0)


def test_invalid_slots_compute_identity_and_flag():
    wl, p = _tiny(seed=7)
    sor = wl["slot_of_row"].copy()
    L = make_layer(p, max_slots=8, max_rank=32)
    assert L.error_flag(clear=True) == 0
    y_ok = run(L, p["x"], sor, "f16")
    assert L.error_flag() == 0
    bad = sor.copy()
    bad[3], bad[10], bad[20] = 99, -4, 7          # out of range, negative, not loaded
    y_bad = run(L, p["x"], bad, "f16")
    assert L.error_flag(clear=True) == 1
    assert L.error_flag() == 0
    base = make_layer({**p, "adapters": {}, "shared": None}, max_slots=8, max_rank=32)
    y_base = run(base, p["x"], np.zeros_like(sor), "f16")
    for i in (3, 10, 20):
        assert np.array_equal(y_bad[i], y_base[i])
    keep = np.ones(len(sor), bool)
    keep[[3, 10, 20]] = False
    assert np.array_equal(y_bad[keep], y_ok[keep])


def test_deterministic_runs():
    wl = synth.decoder_layer_mixed(shapes=(("q", 4096, 4096),))
    p = wl["projections"][0]
    L = make_layer(p, max_slots=32, max_rank=256)
    a = run(L, p["x"], wl["slot_of_row"], "f16")
    b = run(L, p["x"], wl["slot_of_row"], "f16")
    assert np.array_equal(a, b)


def test_graph_capture_replays_match_eager():
    wl = synth.decoder_layer_mixed(shapes=(("k", 4096, 1024),))
    p = wl["projections"][0]
    L = make_layer(p, max_slots=32, max_rank=256)
    x = torch.tensor(p["x"]).half().cuda()
    sor = torch.tensor(wl["slot_of_row"]).cuda()
    out = torch.empty((x.shape[0], p["d_out"]), dtype=torch.float16, device="cuda")
    ws = L.workspace(x.shape[0])
    L.forward(x, sor, out=out, ws=ws)
    torch.cuda.synchronize()
    eager = out.clone()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            L.forward(x, sor, out=out, ws=ws)
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(4):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), rep
        # eager work between replays
        L.forward(x, sor)
        torch.cuda.synchronize()


@pytest.mark.parametrize("route", [1, 2, 3])
def test_scale_routes_outside_the_expand(route):
    """The comparison routes (side kernel, gathered scale, index scale) give
    the same layer as the fused route, within the parity tolerance."""
    wl = synth.prefill_lora_dora(n=256, tenants=4)
    p = wl["projections"][0]
    say("route", route)
    L = make_layer(p, max_slots=8, max_rank=16, options={5: route})
    y_gpu = run(L, p["x"], wl["slot_of_row"], "f16")
    rows = np.arange(0, 256, 5)
    y, h, xw = reference(p, wl["slot_of_row"], rows)
    check(y_gpu[rows], y, h, xw, label="route %d" % route)


def test_unload_and_reload():
    wl, p = _tiny(seed=8)
    L = make_layer(p, max_slots=8, max_rank=32)
    sor = wl["slot_of_row"]
    y0 = run(L, p["x"], sor, "f16")
    L.unload(1)
    assert L.load(p["adapters"][1]) == 1              # lowest free slot again
    y1 = run(L, p["x"], sor, "f16")
    assert np.array_equal(y0, y1)
    L.error_flag(clear=True)


def test_slot_churn_recycles_blocks():
    """Unloaded slots return their device block to the layer's arena and
    later loads reuse it: repeated unload / load / extra-copy cycles leave
    the outputs bitwise unchanged."""
    wl, p = _tiny(seed=12)
    L = make_layer(p, max_slots=12, max_rank=32)
    sor = wl["slot_of_row"]
    y0 = run(L, p["x"], sor, "f16")
    for _ in range(3):
        L.unload(2)
        L.unload(1)
        assert L.load(p["adapters"][1]) == 1
        assert L.load(p["adapters"][2]) == 2
        extra = [L.load(p["adapters"][k]) for k in (2, 1, 5)]
        assert extra == [6, 7, 8]
        for slot in extra:
            L.unload(slot)
    y1 = run(L, p["x"], sor, "f16")
    assert np.array_equal(y0, y1)
    assert L.error_flag(clear=True) == 0


def test_error_codes():
    from tenant_peft_adapter_amd import binding as B
    wl, p = _tiny(seed=9)
    L = make_layer(p, max_slots=7, max_rank=32)       # slots 1..5 used, 6 free
    d_in, d_out = p["d_in"], p["d_out"]

    def code(fn):
        with pytest.raises(B.TpaError) as e:
            fn()
        return e.value.code

    Q = np.zeros((d_in // 32, 32, 32), np.float32)
    Q[0, 0, 1] = 0.3                                   # not skew
    assert code(lambda: L.load({"method": "oft", "Q": Q})) == -5
    big = {"method": "lora", "A": np.zeros((d_in, 64), np.float32), "B": np.zeros((64, d_out), np.float32), "c": 1.0}
    assert code(lambda: L.load(big)) == -1              # rank > max_rank
    nan = {"method": "ia3", "l": np.full(d_out, np.nan, np.float32)}
    assert code(lambda: L.load(nan)) == -5
    assert code(lambda: B.tpa_adapter_load(L.handle, 42)) == -2
    zero_dora = {"method": "dora", "A": np.zeros((d_in, 8), np.float32), "B": np.zeros((8, d_out), np.float32),
                 "c": 1.0, "m": np.ones(d_out, np.float32)}
    W0 = torch.zeros((d_out, d_in), dtype=torch.float16, device="cuda")
    from tenant_peft_adapter_amd.layer import AdaptedLayer
    Lz = AdaptedLayer(W0, max_slots=4, max_rank=16)
    assert code(lambda: Lz.load(zero_dora)) == -5       # zero column norm
    assert L.load({"method": "identity"}) == 6
    assert code(lambda: L.load({"method": "identity"})) == -3
    assert code(lambda: L.unload(6 + 1)) == -4
    assert code(lambda: L.unload(0)) == -4
    Lv = make_layer({**p, "adapters": {}, "shared": None}, max_slots=4, max_rank=32)
    assert code(lambda: Lv.load(p["adapters"][4])) == -1   # VeRA without the shared pair
    x = torch.zeros((64, d_in), dtype=torch.float16, device="cuda")
    sor = torch.zeros(64, dtype=torch.int32, device="cuda")
    out = torch.empty((64, d_out), dtype=torch.float16, device="cuda")
    ws = L.workspace(64)
    assert code(lambda: B.tpa_layer_forward(L.handle, x.data_ptr(), sor.data_ptr(), 64, out.data_ptr(),
                                            ws.data_ptr(), 16, 0)) == -6
    assert code(lambda: B.tpa_layer_forward(L.handle, x.data_ptr(), sor.data_ptr(), 9000, out.data_ptr(),
                                            ws.data_ptr(), ws.numel(), 0)) == -1
    L.forward(x[:0], sor[:0])                            # n = 0 is a no-op


def test_probes_copy_and_launch():
    from tenant_peft_adapter_amd import binding as B
    src = torch.randint(0, 255, (1 << 20,), dtype=torch.uint8, device="cuda")
    dst = torch.zeros_like(src)
    B.tpa_probe_copy(dst.data_ptr(), src.data_ptr(), src.numel(), torch.cuda.current_stream().cuda_stream)
    B.tpa_probe_empty(8, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)
    # The delay probe idles for about the time asked.
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    B.tpa_probe_delay(2000, torch.cuda.current_stream().cuda_stream)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    assert 1.9 <= ms <= 50.0, ms


def test_shared_plan_forward_matches_plain_forward():
    """A row plan built by one projection and reused by another with the same
    slot classes gives the same output, bit for bit, as each projection's own
    forward; so does a projection with the same classes and no OFT rotation
    (OFT tenants are the identity on o); a projection with other slot
    classes, or one whose slot table changed after the build, is refused."""
    from tenant_peft_adapter_amd import binding as B
    from tenant_peft_adapter_amd.layer import RowPlan
    wl = synth.decoder_layer_mixed(shapes=(("q", 4096, 4096), ("k", 4096, 1024), ("o", 4096, 4096)))
    pq, pk, po = wl["projections"]
    Ls = [make_layer(p, max_slots=32, max_rank=256) for p in (pq, pk, po)]
    Lq, Lk, Lo = Ls
    assert Lq.plan_signature() == Lk.plan_signature()      # OFT on both, (IA)3 is a no-term class
    assert Lq.plan_signature() != Lo.plan_signature()      # OFT tenants are the identity on o
    sor = torch.tensor(wl["slot_of_row"]).cuda()
    n = sor.numel()
    plan = RowPlan(Lq, n).build(Lq, sor)
    assert plan.accepts(Lq) and plan.accepts(Lk) and plan.accepts(Lo)
    for L, p in ((Lq, pq), (Lk, pk), (Lo, po)):
        x = torch.tensor(p["x"]).half().cuda()
        want = L.forward(x, sor).clone()
        got = L.forward_planned(plan, x)
        torch.cuda.synchronize()
        assert torch.equal(got, want), p["name"]
    # o's plan has no rotation flags: q (which rotates) may not use it.
    plan_o = RowPlan(Lo, n).build(Lo, sor)
    assert plan_o.accepts(Lo) and not plan_o.accepts(Lq)
    with pytest.raises(B.TpaError) as e:
        Lq.forward_planned(plan_o, torch.tensor(pq["x"]).half().cuda())
    assert e.value.code == -1
    plan_o.close()
    # A layer whose owned slot 1 is loaded as the identity has other classes.
    owned = [s for s, ad in po["adapters"].items() if ad["method"] in ("lora", "dora")][0]
    Lx = make_layer(po, max_slots=32, max_rank=256, skip=(owned,))
    assert not plan.accepts(Lx)
    with pytest.raises(B.TpaError) as e:
        Lx.forward_planned(plan, torch.tensor(po["x"]).half().cuda())
    assert e.value.code == -1
    Lk.unload(1)
    assert not plan.accepts(Lk)
    with pytest.raises(B.TpaError) as e:
        Lk.forward_planned(plan, torch.tensor(pk["x"]).half().cuda())
    assert e.value.code == -1
    plan.close()


@pytest.mark.parametrize("n,path,fuse", [(64, 2, 0), (64, 2, 1), (64, 0, 0), (17, 2, 0), (17, 2, 1), (100, 3, 0),
                                         (300, 3, 0), (300, 3, 1), (300, 1, 0)])
def test_overlap_matches_one_stream(n, path, fuse):
    """The shrink on the layer's second stream gives the same bits as every
    step on the caller's stream (option 0): same kernels, same order of the
    split sums; forced on (1), automatic (-1, one stream), and with the
    expand in the GEMM's epilogue (fuse 1), where overlap does not apply."""
    wl = synth.tiny_mixed(seed=70 + n, n=n, dtype="f16", with_identity=True)
    p = wl["projections"][0]
    say("overlap n=%d path=%d fuse=%d" % (n, path, fuse))
    outs = []
    for ov in (1, -1, 0):
        opts = {4: path, 9: ov}
        if fuse >= 0:
            opts[11] = fuse
        L = make_layer(p, max_slots=8, max_rank=32, options=opts)
        assert L.config(n)["fused_expand"] == fuse
        outs.append(run(L, p["x"], wl["slot_of_row"], "f16"))
        L.close()
    np.testing.assert_array_equal(outs[0], outs[2])
    np.testing.assert_array_equal(outs[1], outs[2])
    y, h, xw = reference(p, wl["slot_of_row"])
    check(outs[0], y, h, xw, label="overlap n=%d" % n)


def test_first_forward_inside_graph_capture_with_overlap():
    """A fresh layer with overlap on whose first forward is captured runs
    that forward on the capturing stream alone (no stream is made during
    capture); eager forwards afterwards overlap; replays and eager calls
    give the same bits."""
    n = 200
    wl = synth.tiny_mixed(seed=777, n=n, dtype="f16", with_identity=True)
    p = wl["projections"][0]
    L = make_layer(p, max_slots=8, max_rank=32, options={11: 0, 9: 1})
    x = torch.tensor(p["x"]).half().cuda()
    sor = torch.tensor(wl["slot_of_row"]).cuda()
    out = torch.empty((n, L.d_out), dtype=torch.float16, device="cuda")
    L.workspace(n)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            L.forward(x, sor, out=out)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    eager = L.forward(x, sor).clone()   # overlapped: the side stream is made now
    torch.cuda.synchronize()
    for rep in range(3):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), rep
        L.forward(x, sor)
    torch.cuda.synchronize()
    y, h, xw = reference(p, wl["slot_of_row"])
    check(eager.float().cpu().numpy().astype(np.float64), y, h, xw, label="captured first forward")


def test_graph_capture_group_with_overlap():
    """A captured plan + group forward (q, k, v with OFT rows: rotation on
    the caller's stream, shrink on the second stream) replays to the eager
    result, with eager work between replays."""
    from tenant_peft_adapter_amd.layer import LayerGroup, RowPlan
    shapes = (("q", 512, 512), ("k", 512, 256), ("v", 512, 256))
    wl = synth.decoder_layer_mixed(shapes=shapes, r_v=64)
    Ls = [make_layer(p, max_slots=32, max_rank=64, options={9: 1}) for p in wl["projections"]]
    xs = [torch.tensor(p["x"]).half().cuda() for p in wl["projections"]]
    sor = torch.tensor(wl["slot_of_row"]).cuda()
    plan = RowPlan(Ls[0], wl["n"])
    grp = LayerGroup(Ls, wl["n"])
    outs = [torch.empty((wl["n"], L.d_out), dtype=torch.float16, device="cuda") for L in Ls]
    grp.forward(plan.build(Ls[0], sor), xs, outs)
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            grp.forward(plan.build(Ls[0], sor), xs, outs)
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(3):
        for o in outs:
            o.zero_()
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, eager):
            assert torch.equal(o, e), rep
        grp.forward(plan.build(Ls[0], sor), xs)
        torch.cuda.synchronize()

