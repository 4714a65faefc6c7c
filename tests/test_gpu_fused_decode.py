"""GPU tests of the decode path whose expand runs in the streamed GEMM's
epilogue (option 1 of the fused-expand key; Scute paper, §2 "The LoRA
schedule": the expand finishes each tile of h; §4.1 route one and §5.2: s
applied as the tile finishes; route two: the shared factor's term times e),
after a whole-k shrink:

  * the decoder-layer workload, every projection, against the oracle and
    against the same layer with the expand as a launch of its own and the
    same shrink k ranges.  The epilogue adds the splits and the term's
    products in the expand's order (V, h ⊙ s + b and the term come out with
    the same bits), but it rounds term ⊙ e + (h ⊙ s + b) to the layer type
    once (gfx950's mixed-precision FMA), where the separate expand rounds
    it to fp32 first: the two differ by one unit in the last place of the
    layer type, in the rare elements where that second rounding flips;
  * each row-block count, column-block width, split count (1: no arrival
    counters) and k-group count of the streamed kernel on a tiny layer;
  * groups (q/k/v with OFT rows; gate/up with VeRA's A read once) against
    the oracle and the separate expand;
  * repeated calls and graph replays (the launch before the GEMM clears the
    counters every time), and rows of unknown slots;
  * the fall-backs: a layer with no term and no rotation (nothing runs
    before the GEMM to clear counters) and the routes that apply s outside
    the expand."""
import numpy as np
import pytest
import torch

from gpu_util import check, make_layer, reference, run, say
from workloads import synth

pytestmark = pytest.mark.gpu

FUSE, SHRINK_SPLIT, GEMM_SPLIT, PATH, NB, GROUPS, ROUTE = 11, 2, 1, 4, 6, 7, 5


def _one_ulp(a, b, dtype):
    """a and b (values of the layer type, as float64) differ by at most one
    unit in the last place of that type, in at most 1 element in 1000 (or 4
    elements of a small output)."""
    mant = {"f16": 10, "bf16": 7}[dtype]
    m = np.maximum(np.abs(a), np.abs(b))
    ulp = np.exp2(np.floor(np.log2(np.maximum(m, 1e-30))) - mant)
    diff = np.abs(a - b)
    assert np.all(diff <= ulp), float((diff / ulp).max())
    apart = int(np.count_nonzero(diff))
    say("elements one ulp apart: %d of %d" % (apart, diff.size))
    assert apart <= max(4, diff.size // 1000), apart


def _pair(p, n, sor, dtype="f16", opts=None, max_slots=32, max_rank=256):
    """Outputs of the layer with the fused epilogue (option 1) and with the
    separate expand (the default at decode), both on 16 shrink k ranges."""
    outs = []
    for fuse in (1, -1):
        o = {SHRINK_SPLIT: 16, FUSE: fuse}
        o.update(opts or {})
        L = make_layer(p, max_slots=max_slots, max_rank=max_rank, options=o)
        cfg = L.config(n)
        outs.append((cfg, run(L, p["x"], sor, dtype)))
        L.close()
    return outs


_DEC = {}


def _decoder():
    if "wl" not in _DEC:
        _DEC["wl"] = synth.decoder_layer_mixed()
    return _DEC["wl"]


@pytest.mark.parametrize("name", ["q", "k", "v", "o", "gate", "up", "down"])
def test_decoder_layer_fused_matches_separate_expand(name):
    wl = _decoder()
    p = [q for q in wl["projections"] if q["name"] == name][0]
    say("fused decode", name, p["d_in"], p["d_out"])
    (cf, yf), (cs, ys) = _pair(p, wl["n"], wl["slot_of_row"])
    assert cf["gemm_path"] == 2 and cf["fused_expand"] == 1, cf
    assert cs["fused_expand"] == 0 and cf["gemm_split"] == cs["gemm_split"] > 1, (cf, cs)
    y, h, xw = reference(p, wl["slot_of_row"])
    check(yf, y, h, xw, label="fused " + name)
    _one_ulp(yf, ys, "f16")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("n", [1, 16, 17, 40, 64])
@pytest.mark.parametrize("nb,split,groups", [(1, 1, 1), (2, 4, 1), (4, 2, 1), (1, 2, 2), (2, 1, 2), (2, 3, 2)])
def test_fused_stream_configurations(dtype, n, nb, split, groups):
    """Every row-block count (n up to 16, 32, 64, ragged), column-block
    width, split count and k-group count; with k whole the separate expand
    reads h rounded to the layer type, so only the oracle decides there."""
    d = 384 if split == 3 else 256
    wl = synth.tiny_mixed(seed=900 + n + 7 * nb + split, n=n, d=d, dtype=dtype, with_identity=True, d_out=256)
    p = wl["projections"][0]
    say("fused tiny", dtype, "n=%d nb=%d split=%d groups=%d" % (n, nb, split, groups))
    opts = {PATH: 2, NB: nb, GEMM_SPLIT: split, GROUPS: groups}
    (cf, yf), (cs, ys) = _pair(p, n, wl["slot_of_row"], dtype, opts, max_slots=8, max_rank=32)
    assert (cf["gemm_nb"], cf["gemm_split"], cf["gemm_groups"]) == (nb, split, groups), cf
    # 4 column blocks of 64 rows leave no room for the epilogue's h and e
    assert cf["fused_expand"] == (0 if nb == 4 and groups == 1 and n > 32 else 1), cf
    y, h, xw = reference(p, wl["slot_of_row"])
    tol = dict(mean_tol=0.01, max_tol=2e-3) if dtype == "f16" else dict(mean_tol=0.05, max_tol=1.6e-2)
    check(yf, y, h, xw, label="fused tiny", **tol)
    check(ys, y, h, xw, label="separate tiny", **tol)
    if split > 1:
        _one_ulp(yf, ys, dtype)


def _group(projs, n, sor, fuse, borrow):
    from tenant_peft_adapter_amd.layer import AdaptedLayer, LayerGroup, RowPlan
    opts = {SHRINK_SPLIT: 16, FUSE: fuse}
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
    sor_t = torch.tensor(sor).cuda()
    plan = RowPlan(Ls[0], n).build(Ls[0], sor_t)
    x0 = torch.tensor(projs[0]["x"]).half().cuda()
    xs = [x0] * len(projs) if borrow else [torch.tensor(p["x"]).half().cuda() for p in projs]
    outs = [o.float().cpu().numpy().astype(np.float64) for o in LayerGroup(Ls, n).forward(plan, xs)]
    torch.cuda.synchronize()
    cfg = Ls[0].config(n)
    plan.close()
    for L in Ls:
        L.close()
    return cfg, outs


@pytest.mark.parametrize("names,borrow", [(("q", "k", "v"), False), (("q", "k", "v"), True),
                                          (("gate", "up"), True)])
def test_fused_group_forward(names, borrow):
    """One launch before the GEMM for the group (OFT's rotation and the
    shrink; with borrow, VeRA's x·A_vᵀ computed once and scaled by each
    projection's d'), one GEMM launch carrying every projection's expand."""
    shapes = tuple(s for s in synth.LLAMA8B_PROJECTIONS if s[0] in names)
    wl = synth.decoder_layer_mixed(n=64, shapes=shapes)
    projs = wl["projections"]
    say("fused group %s borrow=%d" % ("+".join(names), borrow))
    cf, got = _group(projs, wl["n"], wl["slot_of_row"], 1, borrow)
    cs, want = _group(projs, wl["n"], wl["slot_of_row"], -1, borrow)
    assert cf["fused_expand"] == 1 and cs["fused_expand"] == 0
    for nm, g, w, p in zip(names, got, want, projs):
        _one_ulp(g, w, "f16")
        # (a borrowing group reads the first projection's input, which is
        # every projection's input in this workload)
        y, h, xw = reference({**p, "x": projs[0]["x"]} if borrow else p, wl["slot_of_row"])
        check(g, y, h, xw, label="fused group " + nm)


def test_fused_repeated_calls_and_graph_replays():
    """The arrival counters start from zero on every call: eager calls,
    graph replays with eager calls between them, and a call with fewer rows
    give the same bits."""
    wl = _decoder()
    p = [q for q in wl["projections"] if q["name"] == "down"][0]
    n = wl["n"]
    L = make_layer(p, max_slots=32, max_rank=256, options={FUSE: 1})
    assert L.config(n)["fused_expand"] == 1 and L.config(n)["gemm_split"] > 1
    x = torch.tensor(p["x"]).half().cuda()
    sor = torch.tensor(wl["slot_of_row"]).cuda()
    first = L.forward(x, sor).clone()
    for _ in range(3):
        assert torch.equal(L.forward(x, sor), first)
    out = torch.empty_like(first)
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
    for rep in range(4):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, first), rep
        L.forward(x[:17], sor[:17])
    small = L.forward(x[:17], sor[:17])
    torch.cuda.synchronize()
    y, h, xw = reference(p, wl["slot_of_row"])
    check(first.float().cpu().numpy().astype(np.float64), y, h, xw, label="fused down")
    ys, hs, xws = reference(p, wl["slot_of_row"], np.arange(17))
    check(small.float().cpu().numpy().astype(np.float64), ys, hs, xws, label="fused down 17 rows")
    L.close()


def test_fused_unknown_slots():
    """Rows naming an unloaded or out-of-range slot: the identity, the
    sticky flag raised."""
    wl = synth.tiny_mixed(seed=931, n=64, dtype="f16", with_identity=True)
    p = wl["projections"][0]
    sor = wl["slot_of_row"].copy()
    sor[::9] = 99
    L = make_layer(p, max_slots=24, max_rank=64, options={PATH: 2, FUSE: 1})
    assert L.config(64)["fused_expand"] == 1
    y_gpu = run(L, p["x"], sor, "f16")
    assert L.error_flag(clear=True) == 1
    y, h, xw = reference(p, np.where(sor == 99, 0, sor))
    check(y_gpu, y, h, xw, label="fused unknown slots")
    L.close()


def test_fused_fallbacks():
    """No term and no rotation on the layer: with k split nothing runs before
    the GEMM to clear counters, so the separate expand is kept; with k whole
    the epilogue needs none.  Routes that apply s outside the expand keep
    the separate expand too."""
    wl = synth.tiny_mixed(seed=932, n=64, dtype="f16", with_identity=True)
    p = wl["projections"][0]
    # every slot but the (IA)3 ones loaded as the identity
    ia3 = {k: v for k, v in p["adapters"].items() if v["method"] == "ia3"}
    assert ia3
    pi = {**p, "adapters": {k: (v if k in ia3 else {"method": "identity"}) for k, v in p["adapters"].items()},
          "shared": None}
    sor = np.array([s if s in ia3 else 0 for s in wl["slot_of_row"]], dtype=np.int32)
    y, h, xw = reference(pi, sor)
    for split, fused in ((2, 0), (1, 1)):
        L = make_layer(pi, max_slots=24, max_rank=64, options={PATH: 2, GEMM_SPLIT: split, FUSE: 1})
        assert L.config(64)["fused_expand"] == fused, (split, L.config(64))
        check(run(L, pi["x"], sor, "f16"), y, h, xw, label="ia3 only split=%d" % split)
        L.close()
    y, h, xw = reference(p, wl["slot_of_row"])
    for route in (1, 2, 3):
        L = make_layer(p, max_slots=24, max_rank=64, options={PATH: 2, ROUTE: route, FUSE: 1})
        assert L.config(64)["fused_expand"] == 0
        check(run(L, p["x"], wl["slot_of_row"], "f16"), y, h, xw, label="route %d" % route)
        L.close()
