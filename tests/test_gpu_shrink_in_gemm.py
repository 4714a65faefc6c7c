"""GPU tests of the decode path whose shrink runs in the streamed GEMM's own
launch (Scute paper, §2 "The LoRA schedule": the shrink V = x A of each
tile; §4.1: the base product and the terms of one layer in one pass).

The shrink needs nothing the base GEMM makes, so the work-groups past the
GEMM's tiles each take one (tile, 16 factor columns) item of the shrink
over the whole of k: one k range per wave, added in wave order.  The launch
before the GEMM is gone (or, on a projection with OFT tenants, keeps only
their rotation), and V comes out with the bits the split shrink and its
reduction give on the same k ranges (a pinned shrink split of 4 ranges per
k-group keeps the separate launch).  Checked here:

  * every projection of the decoder-layer workload (q, k and v with OFT
    tenants), f16 and bf16, at 64, 17 (a ragged last tile), 16 (one full
    tile) and 1 row: the
    same bits as the pinned split and the oracle's bar;
  * the gate / up group, whose up projection borrows VeRA's x A_v from gate
    (one item writes both projections' scaled columns), the q / k / v group
    (OFT rotation before the GEMM, VeRA's x A_v borrowed by k and v), and
    an o / down group with two inputs;
  * repeated calls give the same bits (every item overwrites its V)."""
import numpy as np
import pytest
import torch

from gpu_util import check, make_layer, reference, run, say
from workloads import synth

pytestmark = pytest.mark.gpu

SHRINK_SPLIT, GROUPS, GEMM_SPLIT, TILE_ROWS = 2, 7, 1, 3

_WL = {}


def _workload(dtype):
    if dtype not in _WL:
        _WL[dtype] = synth.decoder_layer_mixed(dtype=dtype)
    return _WL[dtype]


def _proj(wl, name):
    return next(p for p in wl["projections"] if p["name"] == name)


def _tol(dtype):
    return dict(mean_tol=0.01, max_tol=2e-3) if dtype == "f16" else dict(mean_tol=0.05, max_tol=1.6e-2)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("name", ["q", "k", "v", "o", "gate", "up", "down"])
@pytest.mark.parametrize("n", [64, 17, 16, 1])
def test_shrink_in_gemm_matches_split_shrink(dtype, name, n):
    wl = _workload(dtype)
    p = _proj(wl, name)
    rows = np.arange(n)
    sor = np.asarray(wl["slot_of_row"])[:n]
    x = p["x"][:n]
    say("shrink in GEMM %s %s n=%d" % (dtype, name, n))
    L = make_layer(p, max_slots=32, max_rank=256)
    cfg = L.config(n)
    assert cfg["gemm_path"] == 2 and cfg["shrink_in_gemm"] == 1, cfg
    groups = cfg["gemm_groups"]
    assert cfg["shrink_split"] <= 4 * groups and cfg["shrink_split"] * cfg["shrink_kc"] >= p["d_in"], cfg
    got = run(L, x, sor, dtype)
    again = run(L, x, sor, dtype)
    L.close()
    assert np.array_equal(got, again)
    # (the GEMM's k-groups and split pinned too: a launch that carries the
    # shrink may take longer k ranges)
    Lp = make_layer(p, max_slots=32, max_rank=256,
                    options={SHRINK_SPLIT: 4 * groups, GROUPS: groups, GEMM_SPLIT: cfg["gemm_split"]})
    cp = Lp.config(n)
    assert cp["shrink_in_gemm"] == 0 and cp["shrink_kc"] == cfg["shrink_kc"], (cp, cfg)
    assert (cp["gemm_kc"], cp["gemm_groups"]) == (cfg["gemm_kc"], groups), (cp, cfg)
    want = run(Lp, x, sor, dtype)
    Lp.close()
    assert np.array_equal(got, want), float(np.abs(got - want).max())
    y, h, xw = reference(p, wl["slot_of_row"], rows=rows)
    check(got, y, h, xw, label="shrink in GEMM %s %s n=%d" % (dtype, name, n), **_tol(dtype))


def _group_outputs(projs, n, sor, opts, borrow):
    from tenant_peft_adapter_amd.layer import AdaptedLayer, LayerGroup, RowPlan
    Ls = []
    for i, p in enumerate(projs):
        if i > 0 and borrow:
            L = AdaptedLayer(torch.tensor(p["W"]).half().cuda(), max_slots=32, max_rank=256)
            for k, v in opts.items():
                L.set_option(k, v)
            L.set_vera_shared_from(Ls[0], p["shared"]["B"])
            for slot in sorted(p["adapters"]):
                assert L.load(p["adapters"][slot]) == slot
            Ls.append(L)
        else:
            Ls.append(make_layer(p, max_slots=32, max_rank=256, options=opts))
    sor_t = torch.tensor(np.asarray(sor, dtype=np.int32)).cuda()
    plan = RowPlan(Ls[0], n).build(Ls[0], sor_t)
    xs = [torch.tensor(projs[0]["x"] if borrow else p["x"]).half().cuda() for p in projs]
    outs = [o.float().cpu().numpy().astype(np.float64) for o in LayerGroup(Ls, n).forward(plan, xs)]
    torch.cuda.synchronize()
    cfgs = [L.config(n) for L in Ls]
    plan.close()
    for L in Ls:
        L.close()
    return cfgs, outs


@pytest.mark.parametrize("names,borrow", [(("gate", "up"), True), (("q", "k", "v"), True), (("o", "down"), False)])
def test_shrink_in_gemm_group(names, borrow):
    wl = _workload("f16")
    projs = [_proj(wl, nm) for nm in names]
    n = wl["n"]
    say("shrink in GEMM group %s borrow=%d" % ("+".join(names), borrow))
    # The group's launch takes one k-group count for all its projections
    # (and with it the shrink's k ranges); pinned here so that both runs
    # take the same ranges.
    cd, got = _group_outputs(projs, n, wl["slot_of_row"], {GROUPS: 2}, borrow)
    assert all(c["shrink_in_gemm"] == 1 and c["gemm_groups"] == 2 for c in cd), cd
    cp, want = _group_outputs(projs, n, wl["slot_of_row"], {GROUPS: 2, SHRINK_SPLIT: 8}, borrow)
    assert all(c["shrink_in_gemm"] == 0 for c in cp), cp
    for nm, g, w, p in zip(names, got, want, projs):
        assert np.array_equal(g, w), (nm, float(np.abs(g - w).max()))
        y, h, xw = reference({**p, "x": projs[0]["x"]} if borrow else p, wl["slot_of_row"])
        check(g, y, h, xw, label="shrink in GEMM group " + nm)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("n", [64, 33, 17, 16, 1])
@pytest.mark.parametrize("r_v", [96, 256])
def test_decode_terms_of_several_k_steps(dtype, n, r_v):
    """Owned ranks of one (16), two (48, 64) and five (160: a full group of
    four steps and one more) 32-wide k steps and VeRA ranks 96 and 256 at
    decode sizes: the expand runs a term of more than one step first (its
    shared-term tiles in a range of their own, ahead of the rest) and a
    one-step term after h; the shrink rides in the GEMM's launch.  Against
    the oracle, and bitwise against a second call."""
    wl = synth.decode_ranks(seed=7000 + n + r_v, n=n, dtype=dtype, r_v=r_v)
    p = wl["projections"][0]
    say("decode ranks %s n=%d r_v=%d" % (dtype, n, r_v))
    L = make_layer(p, max_slots=8, max_rank=256)
    cfg = L.config(n)
    assert cfg["gemm_path"] == 2 and cfg["shrink_in_gemm"] == 1, cfg
    got = run(L, p["x"], wl["slot_of_row"], dtype)
    again = run(L, p["x"], wl["slot_of_row"], dtype)
    L.close()
    assert np.array_equal(got, again)
    y, h, xw = reference(p, wl["slot_of_row"])
    check(got, y, h, xw, label="decode ranks %s n=%d r_v=%d" % (dtype, n, r_v), **_tol(dtype))


@pytest.mark.parametrize("name,n", [("gate", 64), ("gate", 17), ("down", 64)])
def test_vera_narrow_waves_match_wide_tiles(name, n):
    """The decode expand's VeRA tiles on 32-column waves (16-row tiles)
    against the same layer on 64-row tiles (64-column waves, another code
    path) with the GEMM's split and k-groups and the shrink's k ranges
    pinned alike: every output element is the same sum in the same order,
    so the outputs agree bit for bit."""
    wl = _workload("f16")
    p = _proj(wl, name)
    sor = np.asarray(wl["slot_of_row"])[:n]
    x = p["x"][:n]
    L = make_layer(p, max_slots=32, max_rank=256)
    cfg = L.config(n)
    assert cfg["tile_rows"] == 16 and cfg["shrink_in_gemm"] == 1, cfg
    got = run(L, x, sor, "f16")
    L.close()
    opts = {TILE_ROWS: 64, GEMM_SPLIT: cfg["gemm_split"], GROUPS: cfg["gemm_groups"],
            SHRINK_SPLIT: cfg["shrink_split"]}
    Lw = make_layer(p, max_slots=32, max_rank=256, options=opts)
    cw = Lw.config(n)
    assert (cw["tile_rows"], cw["gemm_kc"], cw["shrink_kc"]) == (64, cfg["gemm_kc"], cfg["shrink_kc"]), (cw, cfg)
    want = run(Lw, x, sor, "f16")
    Lw.close()
    say("narrow vs wide %s n=%d: max |diff| %g" % (name, n, float(np.abs(got - want).max())))
    assert np.array_equal(got, want)
