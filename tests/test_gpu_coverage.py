"""GPU tests that widen the parity cases to the sizes the workloads reach:

  * the row plan, bit for bit against the oracle's canonical plan, on slot
    tables of 1025 slots (1024 tenants and the identity: the full stack) and
    16383 (the largest the plan's key holds), with Zipf and uniform rows, at
    batch sizes that take the rank sort (n <= 256) and the radix sort with
    three and four digit passes (Scute paper, §2 "The LoRA schedule":
    rows grouped into one segment per adapter);
  * OFT's rotation with blocks of 16, 32 and 64 (§4.1 route three), on a
    tiny layer and on a 4096-wide one, on the decode and the prefill
    kernels, against the oracle's direct definition y = (x R) W;
  * VeRA's A stored and read once per fused input (q/k/v, gate/up), against
    the same group with a copy per projection and the oracle."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import check, make_layer, reference, run, say
from workloads import synth

pytestmark = pytest.mark.gpu

# ------------------------------------------------------------------ plan ---

# Method of slot k (k >= 1) by k mod 6; every term class and the rotation
# flag occur across the whole slot range.
_CYCLE = ("identity", "lora", "vera", "ia3", "oft", "dora")
_HOLES = (7, 1000, 1024)   # unloaded again after the fill: rows naming them are invalid


def _slot_record(rng_recs, k):
    return rng_recs[_CYCLE[k % len(_CYCLE)]]


@pytest.fixture(scope="module", params=[1025, 16383])
def big_table(request):
    """A 64 -> 128 f16 layer whose slots 1 .. max_slots-1 are all loaded
    (method by slot, see _CYCLE), then a few unloaded again."""
    from tenant_peft_adapter_amd.layer import AdaptedLayer
    max_slots = request.param
    d_in, d_out = 64, 128
    rng = np.random.default_rng(7000 + max_slots)
    W = synth.round_to(synth._normal(rng, (d_out, d_in), 1.0 / np.sqrt(d_in)), "f16")
    shared = synth._vera_shared(rng, d_in, d_out, 16, "f16")
    recs = {"identity": {"method": "identity"}, "lora": synth._lora(rng, d_in, d_out, 1, "f16"),
            "vera": synth._vera(rng, 16, d_out), "ia3": synth._ia3(rng, d_out), "oft": synth._oft(rng, d_in, 32),
            "dora": synth._dora(rng, W, 1, "f16")}
    L = AdaptedLayer(torch.tensor(W).half().cuda(), max_slots=max_slots, max_rank=16)
    L.set_vera_shared(shared["A"], shared["B"])
    say("big slot table: loading %d slots" % (max_slots - 1))
    for k in range(1, max_slots):
        assert L.load(_slot_record(recs, k)) == k
    holes = [h for h in _HOLES if h < max_slots]
    for h in holes:
        L.unload(h)
    cls = [-1] * max_slots
    has_R = [0] * max_slots
    cls[0] = 2
    for k in range(1, max_slots):
        m = _CYCLE[k % len(_CYCLE)]
        cls[k] = 0 if m in ("lora", "dora") else 1 if m == "vera" else 2
        has_R[k] = 1 if m == "oft" else 0
    for h in holes:
        cls[h] = -1
        has_R[h] = 0
    say("big slot table: %d slots loaded, holes %s" % (max_slots - 1 - len(holes), holes))
    yield L, max_slots, cls, has_R, holes
    L.close()


def _rows(kind, n, max_slots, holes, seed):
    rng = np.random.default_rng(seed)
    if kind == "zipf":
        p = np.arange(1, max_slots, dtype=np.float64) ** -1.1
        p /= p.sum()
        sor = rng.choice(np.arange(1, max_slots), size=n, p=p)
    else:
        sor = rng.integers(0, max_slots, size=n)
    sor = sor.astype(np.int32)
    # A few invalid ids: unloaded slots, out of range on both sides.
    if n >= 8:
        bad = [holes[0] if holes else -1, -1, max_slots, max_slots + 5]
        idx = rng.choice(n, size=len(bad), replace=False)
        sor[idx] = bad
    return sor


@pytest.mark.parametrize("kind", ["zipf", "uniform"])
@pytest.mark.parametrize("n", [1, 256, 257, 4096, 8192])
def test_plan_bit_exact_large_slot_tables(big_table, kind, n):
    L, max_slots, cls, has_R, holes = big_table
    sor = _rows(kind, n, max_slots, holes, seed=n * 31 + max_slots)
    say("plan max_slots=%d n=%d rows=%s distinct=%d" % (max_slots, n, kind, len(set(sor.tolist()))))
    got = L.plan(torch.tensor(sor).cuda())
    want = oracle.plan(sor.tolist(), cls, 16, has_R)
    for k in ("perm", "row_slot", "seg_ptr", "seg_slot", "class_ptr", "tiles", "oft_tiles", "invalid"):
        assert got[k] == (list(want[k]) if isinstance(want[k], list) else want[k]), k
    if n >= 8:
        assert got["invalid"] == 1


def test_plan_large_table_64_row_tiles(big_table):
    L, max_slots, cls, has_R, holes = big_table
    L.set_option(3, 64)
    try:
        sor = _rows("zipf", 4096, max_slots, holes, seed=99)
        got = L.plan(torch.tensor(sor).cuda())
        want = oracle.plan(sor.tolist(), cls, 64, has_R)
        for k in ("perm", "seg_ptr", "seg_slot", "class_ptr", "tiles", "oft_tiles", "invalid"):
            assert got[k] == (list(want[k]) if isinstance(want[k], list) else want[k]), k
    finally:
        L.set_option(3, -1)


# ------------------------------------------------------------ OFT blocks ---

@pytest.mark.parametrize("dtype,n", [("f32", 64), ("f16", 64), ("f16", 300), ("bf16", 64)])
def test_oft_block_sizes_tiny(dtype, n):
    wl = synth.oft_blocks(n=n, dtype=dtype)
    p = wl["projections"][0]
    L = make_layer(p, max_slots=16, max_rank=16)
    for slot, b in ((1, 16), (3, 32), (5, 64)):
        assert L.info(slot)["oft_block"] == b
    y_gpu = run(L, p["x"], wl["slot_of_row"], dtype)
    y, h, xw = reference(p, wl["slot_of_row"])
    tol = {"f32": (1e-4, 2e-5), "f16": (0.01, 2e-3), "bf16": (0.05, 1.6e-2)}[dtype]
    check(y_gpu, y, h, xw, mean_tol=tol[0], max_tol=tol[1], label="oft blocks %s n=%d" % (dtype, n))
    L.close()


@pytest.mark.parametrize("n", [64, 300])
def test_oft_block_sizes_4096_wide(n):
    """4096 -> 4096 f16 (a q projection's shape): the decode kernels at 64
    rows, the prefill kernels at 300 rows."""
    wl = synth.oft_blocks(seed=6100 + n, n=n, d_in=4096, d_out=4096, dtype="f16")
    p = wl["projections"][0]
    L = make_layer(p, max_slots=16, max_rank=16)
    say("oft 4096 n=%d config %s" % (n, L.config(n)))
    y_gpu = run(L, p["x"], wl["slot_of_row"], "f16")
    y, h, xw = reference(p, wl["slot_of_row"])
    check(y_gpu, y, h, xw, label="oft blocks 4096 n=%d" % n)
    L.close()


# ------------------------------------------------ VeRA's A once per group ---

def _borrowing_layers(projs, max_slots=32, max_rank=256):
    """Layers of one fused input: the first stores VeRA's pair, the others
    take its A (tpa_vera_shared_set_from) with their own B."""
    from tenant_peft_adapter_amd.layer import AdaptedLayer
    Ls = []
    for i, p in enumerate(projs):
        if i == 0:
            Ls.append(make_layer(p, max_slots=max_slots, max_rank=max_rank))
            continue
        assert p["shared"]["A"] is projs[0]["shared"]["A"]
        L = AdaptedLayer(torch.tensor(p["W"]).half().cuda(), max_slots=max_slots, max_rank=max_rank)
        L.set_vera_shared_from(Ls[0], p["shared"]["B"])
        for slot in sorted(p["adapters"]):
            assert L.load(p["adapters"][slot]) == slot
        Ls.append(L)
    return Ls


@pytest.mark.parametrize("names,n", [(("q", "k", "v"), 64), (("q", "k", "v"), 300), (("gate", "up"), 64)])
def test_vera_a_read_once_per_fused_group(names, n):
    """Appendix "Byte counts": VeRA's A is read once per fused input.  The
    group forward over projections that hold one A_v and read one input
    computes x·A_vᵀ once; its outputs equal, bit for bit, those of the same
    group with a copy of A per projection and an input tensor per
    projection, and match the oracle.  Closing the layer that stored A
    leaves the others working (the A block is held by all of them)."""
    from tenant_peft_adapter_amd.layer import LayerGroup, RowPlan
    shapes = tuple(s for s in synth.LLAMA8B_PROJECTIONS if s[0] in names)
    wl = synth.decoder_layer_mixed(n=n, shapes=shapes)
    projs = wl["projections"]
    sor = torch.tensor(wl["slot_of_row"]).cuda()
    say("shared A group %s n=%d" % ("+".join(names), n))
    Ls = _borrowing_layers(projs)
    x = torch.tensor(projs[0]["x"]).half().cuda()
    plan = RowPlan(Ls[0], n).build(Ls[0], sor)
    got = [o.clone() for o in LayerGroup(Ls, n).forward(plan, [x] * len(Ls))]
    Lo = [make_layer(p, max_slots=32, max_rank=256) for p in projs]
    xs = [torch.tensor(p["x"]).half().cuda() for p in projs]
    plan2 = RowPlan(Lo[0], n).build(Lo[0], sor)
    want = LayerGroup(Lo, n).forward(plan2, xs)
    torch.cuda.synchronize()
    for nm, g, w, p in zip(names, got, want, projs):
        assert torch.equal(g, w), nm
        rows = np.arange(0, n, max(1, n // 64))
        y, h, xw = reference(p, wl["slot_of_row"], rows)
        check(g.float().cpu().numpy().astype(np.float64)[rows], y, h, xw, label="shared A %s n=%d" % (nm, n))
    Ls[0].close()
    y1 = Ls[1].forward(x, sor)
    w1 = Lo[1].forward(xs[1], sor)
    torch.cuda.synchronize()
    assert torch.equal(y1, w1)
    plan.close()
    plan2.close()
    for L in Ls[1:] + Lo:
        L.close()


# ------------------------------------------------- shrink item widths ---

@pytest.mark.parametrize("n", [65, 300, 1024])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_shrink_items_of_64_columns_same_bits(n, dtype):
    """§2 "The LoRA schedule", shrink: work items of 64 factor columns (the
    tile's x rows read once for four column blocks) give the same V and U,
    hence the same outputs, as items of 16: each block's products are the
    same MFMA steps in the same k order.  Ranks 16, 48 and 64 and VeRA's
    shared r_v = 64 leave some of an item's blocks past the rank (masked),
    and the layer matches the oracle."""
    rng = np.random.default_rng(7100 + n)
    d_in, d_out = 256, 256
    W = synth.round_to(synth._normal(rng, (d_out, d_in), 1.0 / np.sqrt(d_in)), dtype)
    shared = synth._vera_shared(rng, d_in, d_out, 64, dtype)
    adapters = {1: synth._lora(rng, d_in, d_out, 16, dtype), 2: synth._lora(rng, d_in, d_out, 48, dtype),
                3: synth._lora(rng, d_in, d_out, 64, dtype), 4: synth._vera(rng, 64, d_out),
                5: synth._dora(rng, W, 16, dtype), 6: synth._ia3(rng, d_out)}
    x = synth.round_to(synth._normal(rng, (n, d_in), 1.0), dtype)
    sor = rng.integers(0, 7, size=n).astype(np.int32)
    p = {"W": W, "x": x, "adapters": adapters, "shared": shared, "dtype": dtype, "d_in": d_in, "d_out": d_out}
    outs = []
    for cols in (16, 64):
        L = make_layer(p, max_slots=8, max_rank=64, options={12: cols})
        assert L.config(n)["shrink_cols"] == cols
        outs.append(run(L, x, sor, dtype))
        L.close()
    say("shrink items of 16 / 64 columns n=%d %s: max diff %g" % (n, dtype, np.abs(outs[0] - outs[1]).max()))
    np.testing.assert_array_equal(outs[0], outs[1])
    y, h, xw = reference(p, sor)
    tol = {"f16": (0.01, 2e-3), "bf16": (0.05, 1.6e-2)}[dtype]
    check(outs[1], y, h, xw, mean_tol=tol[0], max_tol=tol[1], label="shrink 64 columns n=%d" % n)


# ------------------------------------------------ short k in the prefill GEMMs ---

@pytest.mark.gpu
@pytest.mark.parametrize("n,d_in,d_out,tile,split,stages,dtype", [
    (65, 64, 128, 128, 0, 4, "f16"),     # one slice: the ring holds fewer slices than it could
    (130, 128, 256, 128, 2, 4, "f16"),   # one slice per split, the shrink's reduction in the grid
    (300, 192, 256, 128, 0, 5, "bf16"),  # three slices, a ring of five
    (257, 192, 384, 128, 3, 2, "f16"),   # split 3 of one slice each, two buffers, ragged rows
    (257, 64, 256, 256, 0, 0, "f16"),    # 256 x 256 tiles over one slice
    (300, 128, 512, 256, 2, 0, "bf16"),  # 256 x 256 tiles, one slice per split
])
def test_direct_load_gemms_short_k(n, d_in, d_out, tile, split, stages, dtype):
    """§2 "The LoRA schedule", base GEMM h = (xR)W: the direct-load prefill
    kernels where the k range is shorter than their LDS ring (one to three
    64-element slices per work-group, split or not), with ragged row tiles,
    against the oracle.  The producer waves of the 128 x 128 kernel then
    issue fewer slices before the loop than the ring holds, and the 256 x
    256 kernel's two phases per slice run over a single slice."""
    wl = synth.tiny_mixed(seed=7300 + n + d_in, n=n, d=d_in, dtype=dtype, with_identity=True, d_out=d_out)
    p = wl["projections"][0]
    opts = {4: 3, 10: tile, 11: 0}
    if split:
        opts[1] = split
    if stages:
        opts[8] = stages
    L = make_layer(p, max_slots=8, max_rank=32, options=opts)
    cfg = L.config(n)
    assert (cfg["gemm_path"], cfg["gemm_tile"]) == (3, tile), cfg
    if split:
        assert cfg["gemm_split"] == split, cfg
    if stages:
        assert cfg["gemm_stages"] == stages, cfg
    say("short k n=%d d_in=%d d_out=%d tile=%d split=%d stages=%d %s" % (n, d_in, d_out, tile, cfg["gemm_split"],
                                                                        cfg["gemm_stages"], dtype))
    y_gpu = run(L, p["x"], wl["slot_of_row"], dtype)
    L.close()
    y, h, xw = reference(p, wl["slot_of_row"])
    tol = dict(mean_tol=0.01, max_tol=2e-3) if dtype == "f16" else dict(mean_tol=0.05, max_tol=1.6e-2)
    check(y_gpu, y, h, xw, label="short k %d/%d/%d" % (n, d_in, d_out), **tol)
