"""GPU parity: the HIP path through the C ABI against the CPU float64 oracle,
element by element, on the seeded workloads.

Tolerance (written here, from the target the layer is held to): for fp16 and
bf16 layers with fp32 accumulation, the mean over rows of
‖y_gpu,i − y_ref,i‖ / ‖y_ref,i − x_i W‖ is at most 1%, and the largest
elementwise error is at most 2e-3 · max|h| with h = (x R_a) W the oracle's
base output.  fp32 layers are held to 1e-4 and 2e-5.
"""
import numpy as np
import pytest
import torch

import oracle

from gpu_util import check, make_layer, reference, run, say
from workloads import synth

pytestmark = pytest.mark.gpu

F32_TOL = dict(mean_tol=1e-4, max_tol=2e-5)


@pytest.mark.parametrize("with_identity", [False, True])
def test_tiny_mixed_fp32(with_identity):
    wl = synth.tiny_mixed(seed=0, with_identity=with_identity)
    p = wl["projections"][0]
    say("tiny_mixed fp32 identity=%s n=%d" % (with_identity, wl["n"]))
    L = make_layer(p, max_slots=8, max_rank=32)
    y_gpu = run(L, p["x"], wl["slot_of_row"], "f32")
    y, h, xw = reference(p, wl["slot_of_row"])
    check(y_gpu, y, h, xw, label="tiny f32", **F32_TOL)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_tiny_mixed_half(dtype):
    wl = synth.tiny_mixed(seed=1, dtype=dtype, with_identity=True)
    p = wl["projections"][0]
    say("tiny_mixed", dtype)
    L = make_layer(p, max_slots=8, max_rank=32)
    y_gpu = run(L, p["x"], wl["slot_of_row"], dtype)
    y, h, xw = reference(p, wl["slot_of_row"])
    # bf16 keeps 8 bits of mantissa: the output rounding alone is 2^-9
    # relative, so the max bound is scaled by the type's unit roundoff.
    max_tol = 2e-3 if dtype == "f16" else 1.6e-2
    check(y_gpu, y, h, xw, max_tol=max_tol, mean_tol=0.01 if dtype == "f16" else 0.05, label="tiny " + dtype)


@pytest.mark.parametrize("n", [1, 5, 16, 17, 63, 64, 65, 100, 129, 300])
def test_ragged_batch_sizes(n):
    """Sizes that span several tiles with a ragged tail, on both GEMM paths
    (n <= 64 takes the skinny kernel, larger n the tiled one)."""
    wl = synth.tiny_mixed(seed=10 + n, n=n, dtype="f16", with_identity=True)
    p = wl["projections"][0]
    say("ragged n=%d" % n)
    L = make_layer(p, max_slots=8, max_rank=32)
    y_gpu = run(L, p["x"], wl["slot_of_row"], "f16")
    y, h, xw = reference(p, wl["slot_of_row"])
    check(y_gpu, y, h, xw, label="ragged n=%d" % n)


@pytest.mark.parametrize("n,path,stages,d", [
    (100, 1, 0, 256), (300, 1, 0, 256),
    (40, 3, 2, 256), (129, 3, 2, 256), (129, 3, 3, 640), (200, 3, 4, 640), (129, 3, 5, 640), (300, 3, 5, 256)])
def test_pinned_prefill_kernels(n, path, stages, d):
    """The register-staged tiled kernel (1) pinned at prefill sizes, and the
    direct-load 128 x 128 kernel (3) pinned at a decode size and ragged
    prefill sizes with each LDS ring depth (2..5 buffers; d_in = 256 gives
    fewer k slices than a 5-deep ring holds, 640 more)."""
    wl = synth.tiny_mixed(seed=50 + n + d, n=n, d=d, dtype="f16", with_identity=True)
    p = wl["projections"][0]
    say("pinned path=%d stages=%d n=%d d=%d" % (path, stages, n, d))
    opts = {4: path}
    if stages:
        opts[8] = stages
    L = make_layer(p, max_slots=8, max_rank=32, options=opts)
    cfg = L.config(n)
    assert cfg["gemm_path"] == path
    if stages:
        assert cfg["gemm_stages"] == stages
    y_gpu = run(L, p["x"], wl["slot_of_row"], "f16")
    y, h, xw = reference(p, wl["slot_of_row"])
    check(y_gpu, y, h, xw, label="pinned path=%d stages=%d n=%d d=%d" % (path, stages, n, d))


@pytest.mark.parametrize("n", [100, 300])
def test_tile_rows_64_pinned(n):
    """64-row plan tiles (four 16-row blocks per shrink and expand item)
    against the oracle, ragged."""
    wl = synth.tiny_mixed(seed=70 + n, n=n, dtype="f16", with_identity=True)
    p = wl["projections"][0]
    say("tile_rows=64 n=%d" % n)
    L = make_layer(p, max_slots=8, max_rank=32, options={3: 64})
    assert L.config(n)["tile_rows"] == 64
    y_gpu = run(L, p["x"], wl["slot_of_row"], "f16")
    y, h, xw = reference(p, wl["slot_of_row"])
    check(y_gpu, y, h, xw, label="tile_rows=64 n=%d" % n)


def test_prefill_lora_dora_q_proj():
    """q_proj 4096 -> 4096, 1024 rows in 16 segments of 64, 8 LoRA + 8 DoRA
    rank 16: every row checked."""
    wl = synth.prefill_lora_dora()
    p = wl["projections"][0]
    say("prefill_lora_dora n=1024 4096x4096")
    L = make_layer(p, max_slots=32, max_rank=16)
    y_gpu = run(L, p["x"], wl["slot_of_row"], "f16")
    y, h, xw = reference(p, wl["slot_of_row"])
    check(y_gpu, y, h, xw, label="prefill q")


_DECODER = {}


def _decoder_layer():
    """The decoder-layer workload and its oracle outputs, computed once."""
    if not _DECODER:
        wl = synth.decoder_layer_mixed()
        _DECODER["wl"] = wl
        _DECODER["ref"] = {p["name"]: reference(p, wl["slot_of_row"]) for p in wl["projections"]}
    return _DECODER["wl"], _DECODER["ref"]


@pytest.mark.parametrize("path", [0, 2])
def test_decoder_layer_mixed_all_projections(path):
    """One Llama-3.1-8B decoder layer (7 projections), 64 decode rows over 20
    tenants of 5 methods, rows shuffled: every row of every projection, with
    the register-fed (0) and the LDS-streamed (2) decode GEMM."""
    wl, ref = _decoder_layer()
    for p in wl["projections"]:
        say("decoder_layer_mixed path=%d" % path, p["name"], p["d_in"], p["d_out"])
        L = make_layer(p, max_slots=32, max_rank=256, options={4: path})
        y_gpu = run(L, p["x"], wl["slot_of_row"], "f16")
        y, h, xw = ref[p["name"]]
        check(y_gpu, y, h, xw, label="decoder " + p["name"])
        L.close()


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("n", [1, 16, 17, 40, 64])
@pytest.mark.parametrize("d,nb,split,groups", [(256, 1, 1, 1), (256, 2, 4, 1), (256, 4, 2, 1),
                                               (256, 1, 2, 2), (256, 2, 1, 2), (448, 1, 1, 2)])
def test_stream_gemm_tiny(dtype, n, d, nb, split, groups):
    """The LDS-streamed decode GEMM over each row-block count (n up to 16,
    32, 64, ragged), each column-block width, several k ranges (one
    64-element slice up to the whole row) and one or two k-groups per
    work-group (d_in = 448: seven slices shared 4 + 3)."""
    wl = synth.tiny_mixed(seed=400 + n, n=n, d=d, dtype=dtype, with_identity=True, d_out=256)
    p = wl["projections"][0]
    say("stream tiny", dtype, "n=%d d_in=%d nb=%d split=%d groups=%d" % (n, d, nb, split, groups))
    L = make_layer(p, max_slots=8, max_rank=32, options={4: 2, 6: nb, 1: split, 7: groups})
    cfg = L.config(n)
    assert (cfg["gemm_path"], cfg["gemm_nb"], cfg["gemm_split"], cfg["gemm_groups"]) == (2, nb, split, groups), cfg
    y_gpu = run(L, p["x"], wl["slot_of_row"], dtype)
    y, h, xw = reference(p, wl["slot_of_row"])
    max_tol = 2e-3 if dtype == "f16" else 1.6e-2
    check(y_gpu, y, h, xw, max_tol=max_tol, mean_tol=0.01 if dtype == "f16" else 0.05,
          label="stream " + dtype)


@pytest.mark.parametrize("path,n", [(0, 64), (2, 64), (-1, 300)])
def test_group_forward_qkv_against_oracle(path, n):
    """q, k and v of the decoder-layer workload forwarded as one group (one
    launch per kernel, a shared plan): every row of every projection against
    the oracle.  At 300 rows the default configuration: 128 x 128 tiles, OFT's
    rotation on the caller's stream and the shrink on the second stream."""
    from tenant_peft_adapter_amd.layer import LayerGroup, RowPlan
    wl = synth.decoder_layer_mixed(n=n, shapes=(("q", 4096, 4096), ("k", 4096, 1024), ("v", 4096, 1024)))
    projs = wl["projections"]
    Ls = [make_layer(p, max_slots=32, max_rank=256, options={4: path}) for p in projs]
    say("group q+k+v n=%d path=%d" % (wl["n"], path))
    sor = torch.tensor(wl["slot_of_row"]).cuda()
    plan = RowPlan(Ls[0], wl["n"]).build(Ls[0], sor)
    grp = LayerGroup(Ls, wl["n"])
    xs = [torch.tensor(p["x"]).half().cuda() for p in projs]
    outs = grp.forward(plan, xs)
    torch.cuda.synchronize()
    for p, o in zip(projs, outs):
        y, h, xw = reference(p, wl["slot_of_row"])
        check(o.float().cpu().numpy().astype(np.float64), y, h, xw, label="group " + p["name"])
    plan.close()


def test_group_forward_gate_up_matches_separate_forwards():
    """gate and up as one group give the separate forwards' outputs up to the
    rounding of the shared split-K configuration."""
    from tenant_peft_adapter_amd import binding as B
    from tenant_peft_adapter_amd.layer import LayerGroup, RowPlan
    wl = synth.decoder_layer_mixed(shapes=(("gate", 4096, 14336), ("up", 4096, 14336), ("o", 4096, 4096)))
    pg, pu, po = wl["projections"]
    Lg, Lu, Lo = [make_layer(p, max_slots=32, max_rank=256) for p in (pg, pu, po)]
    sor = torch.tensor(wl["slot_of_row"]).cuda()
    xs = [torch.tensor(p["x"]).half().cuda() for p in (pg, pu)]
    sep = [Lg.forward(xs[0], sor).float(), Lu.forward(xs[1], sor).float()]
    plan = RowPlan(Lg, wl["n"]).build(Lg, sor)
    outs = LayerGroup([Lg, Lu], wl["n"]).forward(plan, xs)
    torch.cuda.synchronize()
    for a, b, nm in zip(outs, sep, ("gate", "up")):
        err = (a.float() - b).abs().max().item()
        scale = b.abs().max().item()
        say("group vs separate", nm, err, scale)
        assert err <= 2e-3 * scale, nm
    # o has the same slot classes as gate and up in this workload (OFT and
    # (IA)3 tenants are no-term classes there), so it may join the group; a
    # layer with other slot classes may not.
    Lq = make_layer(synth.decoder_layer_mixed(shapes=(("q", 4096, 4096),))["projections"][0],
                    max_slots=32, max_rank=256)
    with pytest.raises(B.TpaError) as e:
        LayerGroup([Lg, Lq], wl["n"]).forward(plan, [xs[0], torch.zeros(wl["n"], 4096, dtype=torch.half,
                                                                         device="cuda")])
    assert e.value.code == -1
    plan.close()


@pytest.mark.parametrize("n,d,d_out,split", [(300, 256, 256, 0), (513, 640, 512, 0), (200, 256, 768, 2),
                                             (1024, 512, 256, 3)])
def test_big_tile_kernel(n, d, d_out, split):
    """The 256 x 256-tile direct-load kernel pinned at small shapes with
    ragged row tiles, several column tiles, split-K partials and the
    shrink's reduction in its grid; against the oracle and bitwise against
    itself across runs."""
    wl = synth.tiny_mixed(seed=130 + n + d, n=n, d=d, dtype="f16", with_identity=True, d_out=d_out)
    p = wl["projections"][0]
    say("big tile n=%d d=%d d_out=%d split=%d" % (n, d, d_out, split))
    opts = {4: 3, 10: 256}
    if split:
        opts[1] = split
    L = make_layer(p, max_slots=8, max_rank=32, options=opts)
    cfg = L.config(n)
    assert (cfg["gemm_path"], cfg["gemm_tile"]) == (3, 256), cfg
    if split:
        assert cfg["gemm_split"] == split, cfg
    y_gpu = run(L, p["x"], wl["slot_of_row"], "f16")
    y_again = run(L, p["x"], wl["slot_of_row"], "f16")
    np.testing.assert_array_equal(y_gpu, y_again)
    y, h, xw = reference(p, wl["slot_of_row"])
    check(y_gpu, y, h, xw, label="big n=%d" % n)


def test_big_tile_chosen_at_prefill_sizes():
    """At 4096 rows of a 4096 x 4096 projection the 256 x 256 tiles give one
    per CU and are chosen; at 1024 rows the 128 x 128 tiles are."""
    from tenant_peft_adapter_amd.layer import AdaptedLayer
    W = torch.zeros((4096, 4096), dtype=torch.float16, device="cuda")
    L = AdaptedLayer(W, max_slots=4, max_rank=16)
    assert L.config(4096)["gemm_tile"] == 256
    assert L.config(1024)["gemm_tile"] == 128
    assert L.config(64)["gemm_tile"] == 0
    L.close()


@pytest.mark.parametrize("d_out,tenants", [(4096, 1), (4096, 16), (4096, 1024), (14336, 16), (14336, 1024)])
def test_vera_sweep_full_size(d_out, tenants):
    """The VeRA tenant sweep at its own sizes (4096 -> 4096 / 14336, 256
    rows, shared rank-256 pair): sampled rows against the oracle, and the
    shared-factor path against the same tenants stored as their exact
    rank-256 LoRA conversion through the owned-factor path (§4.2 equates
    the two; the conversion rounds its scaled factors to f16 once more)."""
    wl = synth.vera_sweep(d_out=d_out, tenants=tenants)
    p = wl["projections"][0]
    say("vera sweep d_out=%d tenants=%d" % (d_out, tenants))
    L = make_layer(p, max_slots=tenants + 1, max_rank=256)
    y_gpu = run(L, p["x"], wl["slot_of_row"], "f16")
    L.close()
    rows = np.arange(0, wl["n"], 7)
    y, h, xw = reference(p, wl["slot_of_row"], rows)
    check(y_gpu[rows], y, h, xw, label="vera sweep")
    if tenants > 16:
        return  # the conversion arm of 1024 tenants is 9.6 GB of factors; the smaller sweeps cover it
    wl2 = synth.vera_sweep(d_out=d_out, tenants=tenants, as_lora=True)
    p2 = wl2["projections"][0]
    assert np.array_equal(wl2["slot_of_row"], wl["slot_of_row"])
    L2 = make_layer(p2, max_slots=tenants + 1, max_rank=256)
    y_lora = run(L2, p2["x"], wl2["slot_of_row"], "f16")
    L2.close()
    check(y_lora[rows], y, h, xw, label="rank-256 LoRA arm")
    eff = np.linalg.norm(y - xw, axis=1)
    gap = np.linalg.norm(y_gpu[rows] - y_lora[rows], axis=1)
    assert np.mean(gap / eff) <= 0.01


def test_largest_batch():
    """The largest batch the plan takes (8192 rows) through every kernel."""
    wl = synth.tiny_mixed(seed=8192, n=8192, dtype="f16", with_identity=True)
    p = wl["projections"][0]
    say("n=8192")
    L = make_layer(p, max_slots=8, max_rank=32)
    y_gpu = run(L, p["x"], wl["slot_of_row"], "f16")
    y, h, xw = reference(p, wl["slot_of_row"])
    check(y_gpu, y, h, xw, label="n=8192")


@pytest.mark.parametrize("n,splits", [(2047, 8), (2048, 4)])
def test_shrink_split_either_side_of_2048_rows(n, splits):
    """d_in = 2048: below 2048 rows the shrink takes k ranges of 256 (8
    splits), from 2048 rows ranges of 512 (4 splits); both against the
    oracle, every row."""
    wl = synth.tiny_mixed(seed=2040 + n, n=n, d=2048, dtype="f16", with_identity=True, d_out=512)
    p = wl["projections"][0]
    say("shrink split boundary n=%d" % n)
    L = make_layer(p, max_slots=8, max_rank=32)
    assert L.config(n)["shrink_split"] == splits
    y_gpu = run(L, p["x"], wl["slot_of_row"], "f16")
    y, h, xw = reference(p, wl["slot_of_row"])
    check(y_gpu, y, h, xw, label="shrink split n=%d" % n)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_large_batch_defaults_every_type(dtype):
    """2100 rows, d_in 1024 -> 512, default configuration in each layer
    type: the shrink's long k ranges (2 splits from 2048 rows), the shrink
    on the second stream (automatic above 128 rows), the tiled GEMM of the
    type (register-staged for fp32, direct loads for 16-bit types)."""
    n = 2100
    wl = synth.tiny_mixed(seed=2100, n=n, d=1024, dtype=dtype, with_identity=True, d_out=512)
    p = wl["projections"][0]
    say("large batch defaults", dtype)
    L = make_layer(p, max_slots=8, max_rank=32)
    cfg = L.config(n)
    assert cfg["shrink_split"] == 2 and cfg["gemm_path"] == (1 if dtype == "f32" else 3)
    y_gpu = run(L, p["x"], wl["slot_of_row"], dtype)
    y, h, xw = reference(p, wl["slot_of_row"])
    tol = F32_TOL if dtype == "f32" else dict(max_tol=2e-3, mean_tol=0.01) if dtype == "f16" else \
        dict(max_tol=1.6e-2, mean_tol=0.05)
    check(y_gpu, y, h, xw, label="large batch " + dtype, **tol)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_deep_ring_default_for_long_split_k(dtype):
    """128 rows of a 14336 -> 4096 projection: 32 tiles x split 8, k ranges
    of 1792, through the 128 x 128 kernel with its default ring of four LDS
    buffers."""
    n = 128
    wl = synth.tiny_mixed(seed=1280, n=n, d=14336, dtype=dtype, with_identity=True, d_out=4096)
    p = wl["projections"][0]
    say("deep ring", dtype)
    L = make_layer(p, max_slots=8, max_rank=32)
    cfg = L.config(n)
    assert (cfg["gemm_path"], cfg["gemm_split"], cfg["gemm_stages"]) == (3, 8, 4), cfg
    y_gpu = run(L, p["x"], wl["slot_of_row"], dtype)
    y, h, xw = reference(p, wl["slot_of_row"])
    tol = dict(max_tol=2e-3, mean_tol=0.01) if dtype == "f16" else dict(max_tol=1.6e-2, mean_tol=0.05)
    check(y_gpu, y, h, xw, label="deep ring " + dtype, **tol)


def test_empty_batch_through_the_abi():
    """n = 0 is a valid call that launches nothing and leaves out alone;
    n above the plan's limit is rejected before any launch."""
    from tenant_peft_adapter_amd import binding as B
    wl = synth.tiny_mixed(seed=3, n=4, dtype="f16")
    p = wl["projections"][0]
    L = make_layer(p, max_slots=8, max_rank=32)
    out = torch.full((4, p["d_out"]), 7.0, dtype=torch.float16, device="cuda")
    x = torch.tensor(p["x"]).half().cuda()
    sor = torch.tensor(wl["slot_of_row"]).cuda()
    ws = L.workspace(4)
    st = torch.cuda.current_stream().cuda_stream
    B.tpa_layer_forward(L.handle, x.data_ptr(), sor.data_ptr(), 0, out.data_ptr(), ws.data_ptr(), ws.numel(), st)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
    with pytest.raises(B.TpaError) as ei:
        B.tpa_layer_forward(L.handle, x.data_ptr(), sor.data_ptr(), 8193, out.data_ptr(), ws.data_ptr(),
                            ws.numel(), st)
    assert ei.value.code == -1
    L.close()


@pytest.mark.parametrize("wl_name,n,d,dtype", [("tiny_mixed", 65, 256, "f16"), ("tiny_mixed", 300, 640, "f16"),
                                               ("tiny_mixed", 1024, 256, "f16"), ("tiny_mixed", 300, 256, "bf16"),
                                               ("tiny_stacks", 300, 256, "f16")])
def test_fused_expand_epilogue(wl_name, n, d, dtype):
    """The expand in the prefill GEMM's epilogue (rows in plan-tile order)
    against the oracle, and against the same layer with the expand as a
    launch of its own (which reads h back rounded to the layer type, so the
    two differ by that rounding times s)."""
    if wl_name == "tiny_mixed":
        wl = synth.tiny_mixed(seed=170 + n + d, n=n, d=d, dtype=dtype, with_identity=True)
    else:
        wl = synth.tiny_stacks(seed=170 + n, n=n, dtype=dtype)
    p = wl["projections"][0]
    sor = wl["slot_of_row"].copy()
    sor[::37] = 99  # rows of an unknown slot: computed as the identity, flag raised
    say("fused expand %s n=%d d=%d %s" % (wl_name, n, d, dtype))
    outs = []
    for fuse in (1, 0):
        L = make_layer(p, max_slots=24, max_rank=64, options={4: 3, 10: 128, 1: 1, 11: fuse})
        cfg = L.config(n)
        assert (cfg["gemm_path"], cfg["gemm_tile"], cfg["gemm_split"], cfg["fused_expand"]) == (3, 128, 1, fuse), cfg
        outs.append(run(L, p["x"], sor, dtype))
        assert L.error_flag(clear=True) == 1
        L.close()
    ref_sor = np.where(sor == 99, 0, sor)
    y, h, xw = reference(p, ref_sor)
    tol = dict(mean_tol=0.01, max_tol=2e-3) if dtype == "f16" else dict(mean_tol=0.05, max_tol=1.6e-2)
    check(outs[0], y, h, xw, label="fused", **tol)
    # The separate expand reads h back rounded to the layer type (adding up
    # to |s| · u · |h|), except on layers with stacked slots, whose scales
    # multiply: those keep h in fp32 (this seed's stacks exceeded the max
    # bound with a rounded h).
    check(outs[1], y, h, xw, label="separate", **tol)
    diff = np.abs(outs[0] - outs[1]).max()
    say("fused vs separate expand: max diff", diff)
    assert diff <= tol["max_tol"] * np.abs(h).max()


def test_fused_expand_default_at_prefill():
    """At the prefill workload (16 segments of 64 rows, 1024 rows) the fused
    epilogue is the default and matches the oracle; with many loaded owned
    slots the tile bound is loose and the separate expand is kept."""
    wl = synth.prefill_lora_dora(n=1024, tenants=16)
    p = wl["projections"][0]
    L = make_layer(p, max_slots=32, max_rank=16)
    cfg = L.config(1024)
    assert cfg["fused_expand"] == 1, cfg
    assert L.config(128)["fused_expand"] == 0  # k is split at 128 rows
    y_gpu = run(L, p["x"], wl["slot_of_row"], "f16")
    rows = np.arange(0, 1024, 9)
    y, h, xw = reference(p, wl["slot_of_row"], rows)
    check(y_gpu[rows], y, h, xw, label="fused prefill")
    L.close()


@pytest.mark.parametrize("n", [300, 600])
def test_group_big_tiles_one_launch(n):
    """Two projections on 256 x 256 tiles as a group run in one launch (the
    projections' work-group ranges side by side) and give the separate
    forwards' bits, each matching the oracle."""
    from tenant_peft_adapter_amd.layer import LayerGroup, RowPlan
    wa = synth.tiny_mixed(seed=400 + n, n=n, d=256, dtype="f16", with_identity=True, d_out=512)
    wb = synth.tiny_mixed(seed=401 + n, n=n, d=256, dtype="f16", with_identity=True, d_out=768)
    wb["slot_of_row"] = wa["slot_of_row"]
    pa, pb = wa["projections"][0], wb["projections"][0]
    say("big-tile group n=%d" % n)
    La = make_layer(pa, max_slots=8, max_rank=32, options={4: 3, 10: 256})
    Lb = make_layer(pb, max_slots=8, max_rank=32, options={4: 3, 10: 256})
    assert La.config(n)["gemm_tile"] == 256 and La.config(n)["fused_expand"] == 0
    sor = torch.tensor(wa["slot_of_row"]).cuda()
    xs = [torch.tensor(p["x"]).half().cuda() for p in (pa, pb)]
    sep = [La.forward(xs[0], sor).float().cpu().numpy(), Lb.forward(xs[1], sor).float().cpu().numpy()]
    plan = RowPlan(La, n).build(La, sor)
    outs = LayerGroup([La, Lb], n).forward(plan, xs)
    torch.cuda.synchronize()
    for o, s_, p in zip(outs, sep, (pa, pb)):
        np.testing.assert_array_equal(o.float().cpu().numpy(), s_)
        y, h, xw = reference(p, wa["slot_of_row"])
        check(s_.astype(np.float64), y, h, xw, label="big group")
    plan.close()


@pytest.mark.parametrize("n", [65, 100, 128, 200, 256])
@pytest.mark.parametrize("d", [256, 640])
def test_stream_gemm_up_to_256_rows(n, d):
    """The streamed GEMM (W read once, all rows of x in each work-group) at
    65 to 256 rows: 8 or 16 row blocks per work-group, ragged tails."""
    wl = synth.tiny_mixed(seed=500 + n + d, n=n, d=d, dtype="f16", with_identity=True)
    p = wl["projections"][0]
    say("stream n=%d d=%d" % (n, d))
    L = make_layer(p, max_slots=8, max_rank=32, options={4: 2})
    assert L.config(n)["gemm_path"] == 2
    y_gpu = run(L, p["x"], wl["slot_of_row"], "f16")
    y, h, xw = reference(p, wl["slot_of_row"])
    check(y_gpu, y, h, xw, label="stream n=%d" % n)
    L.close()
