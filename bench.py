"""Benchmark of the batched multi-adapter layer on one MI355X.

Workload (default): one Llama-3.1-8B decoder layer's seven adapted
projections (q, k, v, o, gate, up, down) in fp16, 64 decode rows over 20
tenants -- 4 each of LoRA r16, DoRA r16, (IA)3 on k/v/up, VeRA with a shared
rank-256 pair, OFT with blocks of 32 on q/k/v -- rows shuffled so segments
are not contiguous.  Inputs are seeded synthetic data of those shapes.

A step is one forward of all seven projections, captured in one HIP graph:
the row plan of the batch (built once and used by every projection it
accepts: here all seven), then for each projection the shrink with OFT's
rotation, the base GEMM (carrying the shrink's split reduction) and the
expand.  `value` is adapted-
layer rows/s: rows through one adapted projection per second, i.e.
7 · n / t_step, with t_step the mean over exactly `--steps` graph replays
whose buffer sets rotate (`--sets` copies of the layer's weights, inputs
and adapters), so every step reads its weights from HBM as consecutive
decoder layers do.  `timing` adds the appendix "Kernel timing" protocol
(graph chains of at least 2 ms, rebuilt five times, median), cold and warm.

The same run also times other workloads of the layer (`side_targets`):
the prefill q_proj (1024 rows in 16 segments of LoRA / DoRA r16) warm and
cold, with its base GEMM against the fp16 MFMA peak; DoRA's expand against
an equal-shape LoRA expand (§4.3 "DoRA in vLLM"); VeRA's layer time at 1
and 1024 tenants (256 rows, 4096 -> 14336, shared rank 256); and
(`routes_vs_byte_model`) the routes of the appendix "Routes" against the
byte model, Table A7's medians.

Prints one JSON line.  `python bench.py --gpus N` with N > 1 exits: this
build measures one GPU.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "adapted-layer rows/s, mixed 5-method batch; adapter-path HBM GB/s vs byte model"
HBM_PEAK = 8.0e12          # B/s, MI355X HBM3E
MFMA_F16_PEAK = 2.5e15     # flop/s, dense fp16


def log(msg):
    """Progress line on stderr (the JSON result is the only stdout line)."""
    print("[bench] " + msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-pure-lora", action="store_true", help="skip the pure-LoRA comparison batch")
    ap.add_argument("--no-side-targets", action="store_true",
                    help="skip the prefill q_proj layer and the VeRA tenant sweep")
    ap.add_argument("--stage-reps", type=int, default=30)
    ap.add_argument("--sets", type=int, default=4,
                    help="buffer sets the timed chain rotates over (cold weights; 4 sets hold 1.8 GB of W)")
    ap.add_argument("--routes", action="store_true",
                    help="also measure the routes-against-the-byte-model table (eager, event-timed forwards)")
    ap.add_argument("--only-routes", action="store_true", help="calibrate and measure the routes table only")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="minimum oracle time in the CPU sample")
    ap.add_argument("--workload", default="decoder_layer_mixed",
                    choices=("decoder_layer_mixed", "stack", "prefill_q_proj"),
                    help="stack: the 32-layer, 1024-tenant Zipf stack against the byte model; prefill_q_proj: "
                         "only the 1024-row q_proj layer (8 LoRA + 8 DoRA r16), for profiling")
    ap.add_argument("--layers", type=int, default=32, help="stack: decoder layers")
    ap.add_argument("--tenants", type=int, default=1024, help="stack: resident tenants")
    ap.add_argument("--stack-n", default="16,256,4096", help="stack: batch sizes")
    ap.add_argument("--stack-eager", choices=("mixed", "base"), default=None,
                    help="stack: two eager steps per batch size on Zipf (mixed) or identity (base) rows and the "
                         "byte model's bytes per kernel class, no timing (for hardware counters)")
    return ap.parse_args()


def build_step(wl, torch):
    from tenant_peft_adapter_amd.layer import AdaptedLayer
    n = wl["n"]
    sor = torch.tensor(wl["slot_of_row"]).cuda()
    layers, xs, outs, wss = [], [], [], []
    by_name, x_dev = {}, {}
    for p in wl["projections"]:
        W = torch.tensor(p["W"]).half().cuda()
        L = AdaptedLayer(W, max_slots=32, max_rank=256)
        if p["shared"] is not None:
            if p["shared"].get("a_from") in by_name:   # VeRA's A stored once per fused input
                L.set_vera_shared_from(by_name[p["shared"]["a_from"]], p["shared"]["B"])
            else:
                L.set_vera_shared(p["shared"]["A"], p["shared"]["B"])
        for slot in sorted(p["adapters"]):
            assert L.load(p["adapters"][slot]) == slot
        layers.append(L)
        by_name[p["name"]] = L
        # Projections of one fused input read the same device rows.
        if id(p["x"]) not in x_dev:
            x_dev[id(p["x"])] = torch.tensor(p["x"]).half().cuda()
        xs.append(x_dev[id(p["x"])])
        outs.append(torch.empty((n, p["d_out"]), dtype=torch.float16, device="cuda"))
        wss.append(L.workspace(n))

    # One row plan per step serves every projection it accepts (same slot
    # classes, and the builder's OFT flags or no rotation at all: here q's
    # plan serves all seven, OFT adapting q, k and v only).  The projections
    # of one fused layer -- q, k, v and gate, up, which read the same input in
    # the model -- run as one group (one launch per kernel); o and down
    # depend on earlier results in the model and run alone.
    from tenant_peft_adapter_amd.layer import LayerGroup, RowPlan
    names = [p["name"] for p in wl["projections"]]
    fused = [("q", "k", "v"), ("gate", "up")]
    owner = []   # (RowPlan, builder index, [layer indices])
    for i, L in enumerate(layers):
        for rp, b, idx in owner:
            if rp.accepts(L):
                idx.append(i)
                break
        else:
            rp = RowPlan(L, n).build(L, sor)
            owner.append((rp, i, [i]))
    plans = []
    for rp, b, idx in owner:
        launch_groups, seen = [], set()
        for i in idx:
            if i in seen:
                continue
            members = [i]
            for f in fused:
                if names[i] in f:
                    members = [j for j in idx if names[j] in f]
            seen.update(members)
            launch_groups.append((members, LayerGroup([layers[j] for j in members], n) if len(members) > 1
                                  else None))
        plans.append((rp, b, launch_groups))

    def step():
        for plan, b, launch_groups in plans:
            plan.build(layers[b], sor)
            for members, grp in launch_groups:
                if grp is None:
                    layers[members[0]].forward_planned(plan, xs[members[0]], out=outs[members[0]],
                                                       ws=wss[members[0]])
                else:
                    grp.forward(plan, [xs[j] for j in members], [outs[j] for j in members])
    step.plans = plans
    units = [members for _, _, lg in plans for members, _ in lg]
    return layers, step, units


def capture(step, torch, warm=True):
    if warm:
        step()
        torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    return g


def capture_chain(call, count, torch):
    """One graph holding `count` calls call(0) .. call(count - 1) (each call
    runs once eagerly first, which also warms caches and code)."""
    for i in range(min(count, 8)):
        call(i)
    torch.cuda.synchronize()
    return capture(lambda: [call(i) for i in range(count)], torch, warm=False)


def time_chain(call, torch, min_s=2e-3, rebuilds=5):
    """Appendix "Kernel timing": enough copies of a call chained into one
    graph that the timed interval reaches `min_s`, divided by the copies;
    the graph rebuilt `rebuilds` times and the median of the per-call times
    taken.  call(i) is the i-th copy (callers rotate buffer sets with i for
    cold measurements).  Returns (median seconds per call, samples, copies)."""
    import statistics
    g = capture_chain(call, 1, torch)
    t1 = time_graph(g, 10, 2, torch)
    del g
    copies = max(1, int(min_s / max(t1, 1e-7)) + 1)
    samples = []
    for _ in range(rebuilds):
        g = capture_chain(call, copies, torch)
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        samples.append(e0.elapsed_time(e1) * 1e-3 / copies)
        del g
    return statistics.median(samples), samples, copies


def time_graph(g, steps, warmup, torch):
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        g.replay()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps


def stage_times(layers, step, reps, torch):
    """Per projection and stage durations (µs) from HIP events the library
    records on the forward's stream around each kernel.  The events are the
    library's timing events (no system-scope fence on record, so a pair
    around one kernel measures that kernel).  Events recorded while a graph
    is captured do not time anything, so the step runs eagerly, queued behind
    a 5 ms idle wave that touches no memory: the host has enqueued every
    launch before the GPU reaches the first event, so each event pair
    brackets only GPU work, and the caches hold what the previous step left
    in them, as in the replayed graph.
    Stage 3 (between the base GEMM and the expand) holds no kernel on this
    path: its interval is the cost of an event pair itself."""
    from tenant_peft_adapter_amd import binding as B
    evs = []
    for L in layers:
        e = [B.tpa_timing_event_create() for _ in range(6)]
        B.tpa_layer_set_stage_events(L.handle, e)
        evs.append(e)
    st = torch.cuda.current_stream().cuda_stream
    acc = [[0.0] * 5 for _ in layers]
    step()
    torch.cuda.synchronize()
    for _ in range(reps):
        B.tpa_probe_delay(5000, st)
        step()
        torch.cuda.synchronize()
        for i, e in enumerate(evs):
            for k in range(5):
                acc[i][k] += B.tpa_timing_event_elapsed(e[k], e[k + 1]) * 1e3
    for L, e in zip(layers, evs):
        B.tpa_layer_set_stage_events(L.handle, None)
        for x in e:
            B.tpa_timing_event_destroy(x)
    return [[v / reps for v in row] for row in acc]


def _copy_rate(torch, nbytes, reps):
    """Bytes read plus written per second by the library's copy probe over a
    buffer pair of `nbytes`, timed over `reps` back-to-back copies."""
    from tenant_peft_adapter_amd import binding as B
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    st = torch.cuda.current_stream().cuda_stream
    for _ in range(3):
        B.tpa_probe_copy(dst.data_ptr(), src.data_ptr(), nbytes, st)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        B.tpa_probe_copy(dst.data_ptr(), src.data_ptr(), nbytes, st)
    e1.record()
    torch.cuda.synchronize()
    rate = 2 * nbytes * reps / (e0.elapsed_time(e1) * 1e-3)
    del src, dst
    return rate


def _read_rate(torch, nbytes, reps):
    """Bytes read per second by the library's read probe over `nbytes`."""
    from tenant_peft_adapter_amd import binding as B
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.empty(B.PROBE_READ_SINK_WORDS, dtype=torch.int32, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    for _ in range(3):
        B.tpa_probe_read(src.data_ptr(), nbytes, sink.data_ptr(), st)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        B.tpa_probe_read(src.data_ptr(), nbytes, sink.data_ptr(), st)
    e1.record()
    torch.cuda.synchronize()
    rate = nbytes * reps / (e0.elapsed_time(e1) * 1e-3)
    del src, sink
    return rate


def _copy_rate_graph(torch, nbytes, copies=400):
    """Copy rate of `copies` chained copies of one small buffer pair inside a
    graph (read + written bytes per second)."""
    from tenant_peft_adapter_amd import binding as B
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for _ in range(copies):
                B.tpa_probe_copy(dst.data_ptr(), src.data_ptr(), nbytes, s.cuda_stream)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    rate = 2 * nbytes * copies / (e0.elapsed_time(e1) * 1e-3)
    del g, src, dst
    return rate


L2_BYTES = 8 * (4 << 20)     # MI355X: 4 MB of L2 in each of the 8 XCDs
MALL_BYTES = 256 << 20       # Infinity Cache


def calibrate(torch, full=False):
    """β_HBM: a 2 GiB device copy (1 GiB read + 1 GiB written, larger than the
    256 MB MALL); β_MALL: the fastest of copies of 16, 32 and 64 MB (1/16 to
    1/4 of the MALL, read and written back from it); λ: 200 chained one-block
    kernels in one graph (appendix "Constants", sizes rescaled to this
    chip's caches).  Returns (β_HBM, λ, β_MALL), or with full=True a dict
    that also holds β_L2 (the fastest of copies of 1/16, 1/8 and 1/4 of the
    chip's L2, each XCD's share in its own L2, chained in a graph) and the
    read ceiling (a 1 GiB read-only stream)."""
    from tenant_peft_adapter_amd import binding as B
    beta = _copy_rate(torch, 1 << 30, 10)
    beta_mall = max(_copy_rate(torch, mb << 20, 200) for mb in (16, 32, 64))
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            B.tpa_probe_empty(200, s.cuda_stream)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(20):
        g.replay()
    torch.cuda.synchronize()
    lam = (time.perf_counter() - t0) / 20 / 200
    if not full:
        return beta, lam, beta_mall
    beta_l2 = max(_copy_rate_graph(torch, L2_BYTES // f) for f in (16, 8, 4))
    read = _read_rate(torch, 1 << 30, 10)
    return {"beta_hbm": beta, "lambda": lam, "beta_mall": beta_mall, "beta_l2": beta_l2, "read_hbm": read}


PROFILE = os.path.join(ROOT, "profiles", "gemm_stream_decoder_layer_mixed.md")


def profiled_traffic(kernel, config):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 PMC
    summary, or None when the summary covers another kernel or launch
    configuration, or the kernel's sources changed since the counters were
    taken (sha256 over the files it lists)."""
    import hashlib
    import re
    try:
        text = open(PROFILE).read()
    except OSError:
        return None
    k = re.search(r"^kernel: (\S+)", text, re.M)
    c = re.search(r"^config: (.+)$", text, re.M)
    sha = re.search(r"^source_sha256: (\w+)", text, re.M)
    files = re.search(r"^\(sha256 over ([^;]+);", text, re.M)
    val = re.search(r"^traffic_bytes_per_launch: (\d+)", text, re.M)
    if not (k and c and sha and files and val) or k.group(1) != kernel or c.group(1).strip() != config:
        return None
    h = hashlib.sha256()
    for f in files.group(1).split(", "):
        with open(os.path.join(ROOT, f.strip()), "rb") as fh:
            h.update(fh.read())
    return int(val.group(1)) if h.hexdigest()[:16] == sha.group(1) else None


def cpu_baseline(wl, min_seconds=10.0, chunk=4):
    """The oracle, untuned, on a bounded sample of the same batch: chunks of
    `chunk` rows (in batch order) through all seven projections until at
    least `min_seconds` have passed."""
    import contextlib

    import numpy as np
    import oracle
    # The cores this process may run on; BLAS gets one thread per core.
    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_limits
        limit = threadpool_limits(limits=cores, user_api="blas")
    except Exception:  # pragma: no cover
        limit = contextlib.nullcontext()
    rows = 0
    with limit:
        t0 = time.perf_counter()
        while rows < wl["n"]:
            sel = np.arange(rows, min(rows + chunk, wl["n"]))
            for p in wl["projections"]:
                x = p["x"][sel].astype(np.float64)
                oracle.layer_forward(x, p["W"].astype(np.float64).T, wl["slot_of_row"][sel], p["adapters"],
                                     p["shared"])
            rows += len(sel)
            if time.perf_counter() - t0 >= min_seconds:
                break
        dt = time.perf_counter() - t0
    return {"value": rows * len(wl["projections"]) / dt, "unit": "rows/s", "cores": cores, "kind": "oracle",
            "sample": "first %d of the %d rows, in calls of %d rows, through all %d projections (%.1f s)"
                      % (rows, wl["n"], chunk, len(wl["projections"]), dt)}


def stack_main(args):
    """The full adapter stack: `layers` decoder layers of the seven
    Llama-3.1-8B projections with `tenants` resident tenants (methods in
    turn, LoRA/DoRA at rank 64), batches of Zipf(1.1)-drawn rows.  A step is
    one forward of every projection of every layer on the batch (one row
    plan, q/k/v and gate/up as groups), captured in one graph.  Measured
    step time is set beside the byte model (Scute paper §4.3: t0 + ΔQ/β +
    ΔL·λ), with t0 the same step on identity rows (the base GEMMs and the
    launches), ΔQ the adapter kernels' algorithmic bytes and ΔL = 0: the
    identity batch launches the same kernels."""
    import numpy as np
    import torch
    from tenant_peft_adapter_amd import binding as B
    from tenant_peft_adapter_amd import bytemodel as bm
    from tenant_peft_adapter_amd.layer import AdaptedLayer, LayerGroup, RowPlan
    from workloads import stack, synth

    torch.cuda.set_device(0)
    shapes = synth.LLAMA8B_PROJECTIONS
    names = [s[0] for s in shapes]
    ns = [int(v) for v in args.stack_n.split(",")]
    nmax, T, NL = max(ns), args.tenants, args.layers
    protos = stack.prototypes()
    xs = {name: stack.device_input(torch, nmax, d_in, name) for name, d_in, _ in shapes}
    outs = {name: torch.empty((nmax, d_out), dtype=torch.float16, device="cuda") for name, _, d_out in shapes}
    log("stack: loading %d tenants into %d layers x 7 projections" % (T, NL))
    t_load = time.perf_counter()
    layers = []
    for li in range(NL):
        row = []
        for name, d_in, d_out in shapes:
            W = stack.device_weight(torch, li, name, d_out, d_in)
            L = AdaptedLayer(W, max_slots=T + 1, max_rank=256)
            pr = protos[name]
            L.set_vera_shared(pr["shared"]["A"], pr["shared"]["B"])
            for t in range(T):
                L.load(stack.tenant_record(pr, t))
            row.append(L)
        layers.append(row)
        log("stack: layer %d loaded, %.0f s, %.1f GB in use" % (li, time.perf_counter() - t_load,
                                                                  torch.cuda.mem_get_info()[1] / 1e9 -
                                                                  torch.cuda.mem_get_info()[0] / 1e9))
    t_load = time.perf_counter() - t_load

    # Workspaces shared by every layer (one projection runs at a time).
    qkv, gu = [0, 1, 2], [4, 5]
    ws_qkv = [torch.empty(max(sz, 256), dtype=torch.uint8, device="cuda")
              for sz in B.tpa_group_workspace_size([layers[0][i].handle for i in qkv], nmax)]
    ws_gu = [torch.empty(max(sz, 256), dtype=torch.uint8, device="cuda")
             for sz in B.tpa_group_workspace_size([layers[0][i].handle for i in gu], nmax)]
    ws_o = torch.empty(B.tpa_workspace_size(layers[0][3].handle, nmax), dtype=torch.uint8, device="cuda")
    ws_down = torch.empty(B.tpa_workspace_size(layers[0][6].handle, nmax), dtype=torch.uint8, device="cuda")
    g_qkv = [LayerGroup([row[i] for i in qkv], nmax, ws=ws_qkv) for row in layers]
    g_gu = [LayerGroup([row[i] for i in gu], nmax, ws=ws_gu) for row in layers]
    plan = RowPlan(layers[0][0], nmax)

    def make_step(sor):
        n = sor.numel()
        x = {k: v[:n] for k, v in xs.items()}
        o = {k: v[:n] for k, v in outs.items()}

        def step():
            plan.build(layers[0][0], sor)
            for li in range(NL):
                g_qkv[li].forward(plan, [x["q"], x["k"], x["v"]], [o["q"], o["k"], o["v"]])
                layers[li][3].forward_planned(plan, x["o"], out=o["o"], ws=ws_o)
                g_gu[li].forward(plan, [x["gate"], x["up"]], [o["gate"], o["up"]])
                layers[li][6].forward_planned(plan, x["down"], out=o["down"], ws=ws_down)
        return step

    if args.stack_eager:
        # Two eager steps per batch size (the first warms caches and code);
        # the byte model's algorithmic bytes per kernel class for one step.
        # One 1 GiB device copy first: the reference that scales the
        # hardware byte counters.
        nb = 1 << 30
        src = torch.empty(nb, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        B.tpa_probe_copy(dst.data_ptr(), src.data_ptr(), nb, torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        del src, dst
        out = []
        for n in ns:
            sor_np = stack.zipf_rows(n, T) if args.stack_eager == "mixed" else np.zeros(n, np.int32)
            step = make_step(torch.tensor(sor_np).cuda())
            for _ in range(2):
                step()
            torch.cuda.synchronize()
            per = {}
            for name, d_in, d_out in shapes:
                kb = bm.kernel_bytes(bm.shape_of(n, d_in, d_out, sor_np, stack.adapters_of(protos[name], T),
                                                 r_v=protos[name]["r_v"]))
                for k, v in kb.items():
                    per[k] = per.get(k, 0) + NL * v["bytes"]
            out.append({"n": n, "rows": args.stack_eager, "bytes_per_step": per})
        print(json.dumps({"workload": "stack eager steps", "layers": NL, "tenants": T, "results": out}))
        return

    beta, lam, beta_mall = calibrate(torch)
    results = []
    for n in ns:
        sor_np = stack.zipf_rows(n, T)
        sor = torch.tensor(sor_np).cuda()
        base = torch.zeros(n, dtype=torch.int32, device="cuda")
        plan.build(layers[0][0], sor)
        torch.cuda.synchronize()
        assert all(plan.accepts(L) for row in layers for L in row)
        steps = max(3, min(50, int(2e6 / (n * NL))))
        t = {}
        for tag, rows in (("mixed", sor), ("base", base)):
            g = capture(make_step(rows), torch)
            t[tag] = time_graph(g, steps, 2, torch)
            del g
        q_ad = q_gemm = fl = 0
        for name, d_in, d_out in shapes:
            kb = bm.kernel_bytes(bm.shape_of(n, d_in, d_out, sor_np, stack.adapters_of(protos[name], T),
                                             r_v=protos[name]["r_v"]))
            q_gemm += NL * kb["gemm"]["bytes"]
            fl += NL * kb["gemm"]["flops"]
            q_ad += NL * sum(v["bytes"] for k, v in kb.items() if k != "gemm")
        pred = t["base"] + q_ad / beta
        res = {"n": n, "distinct_tenants": int(len(set(sor_np.tolist()))), "steps": steps,
               "step_us": round(t["mixed"] * 1e6, 1), "base_step_us": round(t["base"] * 1e6, 1),
               "adapter_bytes": int(q_ad), "gemm_bytes": int(q_gemm), "gemm_flops": int(fl),
               "predicted_step_us": round(pred * 1e6, 1), "measured_over_predicted": round(t["mixed"] / pred, 3),
               "adapter_GBps": round(q_ad / max(t["mixed"] - t["base"], 1e-9) / 1e9, 1),
               "base_step_mfma_frac": round(fl / t["base"] / MFMA_F16_PEAK, 3),
               "base_step_hbm_frac": round(q_gemm / t["base"] / HBM_PEAK, 3)}
        log("stack n=%d: %s" % (n, res))
        results.append(res)
    print(json.dumps({
        "metric": "full adapter stack: measured step time against the byte model",
        "workload": "stack: %d Llama-3.1-8B decoder layers x 7 projections, fp16, %d resident tenants "
                    "(LoRA r64, DoRA r64, (IA)3 k/v/up, VeRA r256, OFT b32 in turn), Zipf(1.1) rows" % (NL, T),
        "data": "synthetic (seeded; raw parameters shared per projection and method, one device copy per tenant)",
        "load_s": round(t_load, 1), "calibration": {"beta_hbm_GBps": beta / 1e9, "beta_mall_GBps": beta_mall / 1e9,
                        "lambda_us": lam * 1e6},
        "dL_launches": 0, "results": results}))


def load_layer(p, torch, max_rank=256, options=None, copies=1):
    """A layer (or `copies` layers, each with its own W and adapters) of a
    single-projection workload."""
    from tenant_peft_adapter_amd.layer import AdaptedLayer
    out = []
    for _ in range(copies):
        L = AdaptedLayer(torch.tensor(p["W"]).half().cuda(), max_slots=max(2, len(p["adapters"]) + 1), max_rank=max_rank)
        for k, v in (options or {}).items():
            L.set_option(k, v)
        if p["shared"] is not None:
            L.set_vera_shared(p["shared"]["A"], p["shared"]["B"])
        for slot in sorted(p["adapters"]):
            assert L.load(p["adapters"][slot]) == slot
        out.append(L)
    return out if copies > 1 else out[0]


def layer_call(Ls, xs, sor, torch):
    """call(i): the forward of buffer set i mod len(Ls)."""
    n = sor.numel()
    outs = [torch.empty((n, L.d_out), dtype=torch.float16, device="cuda") for L in Ls]
    wss = [L.workspace(n) for L in Ls]

    def call(i):
        k = i % len(Ls)
        Ls[k].forward(xs[k], sor, out=outs[k], ws=wss[k])
    return call


def single_layer_time(wl, torch, copies=1, max_rank=256, options=None):
    """Chained-graph time of one forward of a single-projection workload;
    with copies > 1 the chain rotates over that many layers (own W, adapters,
    input and output: a cold measurement)."""
    p = wl["projections"][0]
    Ls = load_layer(p, torch, max_rank=max_rank, options=options, copies=copies)
    Ls = Ls if copies > 1 else [Ls]
    xs = [torch.tensor(p["x"]).half().cuda() for _ in Ls]
    sor = torch.tensor(wl["slot_of_row"]).cuda()
    t, samples, chained = time_chain(layer_call(Ls, xs, sor, torch), torch)
    cfg = Ls[0].config(wl["n"])
    for L in Ls:
        L.close()
    return t, cfg


def prefill_targets(torch, cold_sets=12, stage_reps=20):
    """The prefill q_proj workload (1024 rows in 16 segments, 8 LoRA + 8
    DoRA r16): layer time warm and cold (the chain rotating over
    `cold_sets` layers, > 512 MB in all), the kernel stages of the default
    path, and the base GEMM alone (a layer without adapters, expand apart)
    against the fp16 MFMA peak."""
    import numpy as np
    from tenant_peft_adapter_amd import binding as B
    from workloads import synth
    n = 1024
    wl = synth.prefill_lora_dora(n=n, tenants=16)
    p = wl["projections"][0]
    t_warm, cfg = single_layer_time(wl, torch)
    t_cold, _ = single_layer_time(wl, torch, copies=cold_sets)
    L = load_layer(p, torch)
    x = torch.tensor(p["x"]).half().cuda()
    sor = torch.tensor(wl["slot_of_row"]).cuda()
    call = layer_call([L], [x], sor, torch)
    st = stage_times([L], lambda: call(0), stage_reps, torch)[0]
    L.close()
    # Base GEMM alone: no adapters, identity rows, the expand in its own launch.
    Lb = load_layer({**p, "adapters": {}, "shared": None}, torch, options={B.TPA_OPT_FUSE_EXPAND: 0})
    callb = layer_call([Lb], [x], torch.zeros(n, dtype=torch.int32, device="cuda"), torch)
    stb = stage_times([Lb], lambda: callb(0), stage_reps, torch)[0]
    cfgb = Lb.config(n)
    Lb.close()
    flops = 2.0 * n * 4096 * 4096
    t_gemm = stb[2] * 1e-6
    kern = "gemm_%s_kernel<f16%s>" % ("big" if cfgb["gemm_tile"] == 256 else "wide",
                                      "" if cfgb["gemm_tile"] == 256 else ",%d" % cfgb["gemm_stages"])
    return {
        "us_per_layer": t_warm * 1e6, "us_per_layer_cold": t_cold * 1e6, "cold_sets": cold_sets,
        "rows_per_s": n / t_warm, "layer_flops_over_mfma_peak": flops / t_warm / MFMA_F16_PEAK,
        "fused_expand": bool(cfg["fused_expand"]), "gemm_tile": cfg["gemm_tile"],
        "stages_us": dict(zip(("plan", "shrink", "gemm", "reduce+fused gemm", "expand"), [round(v, 2) for v in st])),
        "roofline_base_gemm": {"kernel": kern + " (1024 x 4096 x 4096, no adapters)", "bound": "mfma",
                               "achieved": flops / t_gemm / 1e12, "peak": MFMA_F16_PEAK / 1e12,
                               "unit": "TFLOP/s", "frac": flops / t_gemm / MFMA_F16_PEAK,
                               "us_per_launch": t_gemm * 1e6,
                               "config": "tile=%d stages=%d split=%d" % (cfgb["gemm_tile"], cfgb["gemm_stages"],
                                                                         cfgb["gemm_split"])},
    }


def dora_expand_ratio(torch, ns=(1024, 4096), stage_reps=20):
    """§4.3 "DoRA in vLLM": the expand of a DoRA batch (s inside the expand,
    route one) against the expand of an equal-shape LoRA batch (16 segments
    of rank 16, q_proj 4096 -> 4096), and the same DoRA batch with s
    applied after the expand by the index-scale route (a per-row copy of s,
    then a multiply).  Expand stages from the library's timing events; the
    expand runs in its own launch here."""
    from tenant_peft_adapter_amd import binding as B
    from workloads import synth
    out = {}
    for n in ns:
        t = {}
        for methods, route in (("lora", 0), ("dora", 0), ("dora", 3)):
            wl = synth.prefill_lora_dora(n=n, tenants=16, methods=methods)
            p = wl["projections"][0]
            opts = {B.TPA_OPT_FUSE_EXPAND: 0}
            if route:
                opts[B.TPA_OPT_SCALE_ROUTE] = route
            L = load_layer(p, torch, options=opts)
            call = layer_call([L], [torch.tensor(p["x"]).half().cuda()], torch.tensor(wl["slot_of_row"]).cuda(),
                              torch)
            t[(methods, route)] = stage_times([L], lambda: call(0), stage_reps, torch)[0][4]
            L.close()
        out["n%d" % n] = {"lora_expand_us": t[("lora", 0)], "dora_expand_us": t[("dora", 0)],
                          "dora_over_lora": t[("dora", 0)] / t[("lora", 0)],
                          "index_scale_expand_and_passes_us": t[("dora", 3)],
                          "index_scale_over_lora": t[("dora", 3)] / t[("lora", 0)]}
    return out


def route_table(torch, cal, ns=(256, 512, 1024, 2048, 4096), d_outs=(1024, 4096, 14336), oft_k=(1, 4, 16), reps=10):
    """Appendix "Routes" and Table A7, on this chip: measured layer time of
    each route that applies DoRA's s outside the expand (side kernel,
    gathered scale, index scale) and of OFT's input transform, against the
    byte model t0 + ΔQ/β + ΔL·λ (§4.3), t0 the same batch without the extra
    pass.  Times are the library's timing events around each forward, run
    eagerly behind an idle wave (as `stage_times`), first event to last,
    mean of `reps`.  β is β_L2 when the extra bytes fit the L2, β_MALL when
    they fit the MALL, else β_HBM (§4.3: the cache's rate when the extra
    read and write fit in it).  Cells: 16 DoRA r16 segments, d_in 4096, n
    rows x d_out; OFT: k tenants (b = 32) over n rows, d_in 4096 and 14336,
    against the same weight without adapters (one launch fewer).  Returns
    the cells and, per route, the median absolute error of the increment and
    of the total over bandwidth-regime cells (ΔQ/β > λ) and of the total
    over the launch-bound rest."""
    import statistics

    import numpy as np
    from tenant_peft_adapter_amd import binding as B
    from tenant_peft_adapter_amd import bytemodel as bm
    from workloads import synth
    lam = cal["lambda"]

    def beta_for(dq):
        if dq <= L2_BYTES:
            return cal["beta_l2"], "l2"
        if dq <= MALL_BYTES:
            return cal["beta_mall"], "mall"
        return cal["beta_hbm"], "hbm"

    def layer_time(L, x, sor):
        call = layer_call([L], [x], sor, torch)
        return sum(stage_times([L], lambda: call(0), reps, torch)[0]) * 1e-6

    cells = []

    def add(route, n, d, t0, t, dq, dl):
        beta, where = beta_for(dq)
        extra = dq / beta + dl * lam
        inc = t - t0
        cells.append({"route": route, "n": n, "d": d, "t0_us": round(t0 * 1e6, 2), "t_us": round(t * 1e6, 2),
                      "pred_us": round((t0 + extra) * 1e6, 2), "beta": where, "dq_bytes": int(dq),
                      "bandwidth_regime": dq / beta > lam,
                      "inc_err": abs(inc - extra) / max(abs(inc), 1e-9), "total_err": abs(t - t0 - extra) / t})

    names = {1: "side kernel", 2: "gathered scale", 3: "index scale"}
    nmax = max(ns)
    for d_out in d_outs:
        wl = synth.prefill_lora_dora(seed=7000 + d_out, n=nmax, tenants=16, d_out=d_out, methods="dora")
        p = wl["projections"][0]
        La = load_layer(p, torch, options={B.TPA_OPT_FUSE_EXPAND: 0})
        Lb = load_layer(p, torch, options={B.TPA_OPT_FUSE_EXPAND: 0, B.TPA_OPT_SCALE_ROUTE: 2})
        x_all = torch.tensor(p["x"]).half().cuda()
        for n in ns:
            sor = torch.tensor(np.minimum(np.arange(n) // max(1, n // 16) + 1, 16).astype(np.int32)).cuda()
            x = x_all[:n].contiguous()
            t = {}
            for route in (0, 1, 2, 3):
                L = La if route < 2 else Lb
                L.set_option(B.TPA_OPT_SCALE_ROUTE, route)
                log("routes: cell d_out=%d n=%d route=%d" % (d_out, n, route))
                t[route] = layer_time(L, x, sor)
            for route in (1, 2, 3):
                dq, dl = bm.scale_route_extra(n, d_out, route)
                add(names[route], n, d_out, t[0], t[route], dq, dl)
        La.close()
        Lb.close()
    for d_in in (4096, 14336):
        rng = np.random.default_rng(7100 + d_in)
        p = synth.make_projection(rng, "oft", d_in, 4096, "f16", 1)
        p["adapters"] = {t + 1: synth._oft(rng, d_in, 32) for t in range(max(oft_k))}
        L = load_layer(p, torch, options={B.TPA_OPT_FUSE_EXPAND: 0})
        L0 = load_layer({**p, "adapters": {}}, torch, options={B.TPA_OPT_FUSE_EXPAND: 0})
        x_all = torch.randn((nmax, d_in), device="cuda").half()
        for n in ns:
            x = x_all[:n].contiguous()
            log("routes: OFT base d_in=%d n=%d" % (d_in, n))
            t0 = layer_time(L0, x, torch.zeros(n, dtype=torch.int32, device="cuda"))
            for k in oft_k:
                log("routes: OFT cell d_in=%d n=%d k=%d" % (d_in, n, k))
                sor = torch.tensor((np.arange(n) * k // n + 1).astype(np.int32)).cuda()
                t = layer_time(L, x, sor)
                add("OFT transform", n, d_in, t0, t, 2 * (2 * n * d_in + k * d_in * 32), 1)
        L.close()
        L0.close()
    summary = {}
    for route in list(names.values()) + ["OFT transform"]:
        bw = [c for c in cells if c["route"] == route and c["bandwidth_regime"]]
        lb = [c for c in cells if c["route"] == route and not c["bandwidth_regime"]]
        summary[route] = {
            "cells": len(bw) + len(lb), "bandwidth_cells": len(bw),
            "increment_median_err": statistics.median([c["inc_err"] for c in bw]) if bw else None,
            "total_median_err": statistics.median([c["total_err"] for c in bw]) if bw else None,
            "launch_median_err": statistics.median([c["total_err"] for c in lb]) if lb else None}
    return {"summary": summary, "cells": cells}


def side_targets(torch, args):
    """The other targets on their own workloads, in the same run: the
    prefill q_proj layer (1024 rows, 16 segments of LoRA / DoRA r16) with
    its base GEMM's share of the fp16 MFMA peak, DoRA's expand against
    LoRA's, and VeRA's step time from 1 to 1024 tenants (256 rows, 4096 ->
    14336, shared rank 256)."""
    from workloads import synth
    pre = prefill_targets(torch, stage_reps=args.stage_reps)
    log("prefill q_proj: %.1f us warm, %.1f us cold" % (pre["us_per_layer"], pre["us_per_layer_cold"]))
    dora = dora_expand_ratio(torch, stage_reps=args.stage_reps)
    vera = {}
    for T in (1, 1024):
        vera[T], _ = single_layer_time(synth.vera_sweep(d_out=14336, tenants=T), torch)
    return {
        "prefill_q_proj_n1024": pre,
        "dora_expand_over_lora_expand": dora,
        "vera_4096x14336_n256": {"us_T1": vera[1] * 1e6, "us_T1024": vera[1024] * 1e6,
                                 "growth": vera[1024] / vera[1] - 1.0},
    }


def prefill_main(args):
    """The prefill q_proj layer alone (1024 rows, 16 segments of LoRA / DoRA
    r16, 4096 -> 4096, f16): `warmup` then `steps` graph-replayed forwards
    with the default kernels, then the same number of forwards of the same
    layer without adapters and with the expand in its own launch (the base
    GEMM alone).  One JSON line with both times."""
    import torch
    from tenant_peft_adapter_amd import binding as B
    from workloads import synth
    torch.cuda.set_device(0)
    # One 1 GiB device copy first: the reference that scales the hardware
    # byte counters of a profiled run.
    nb = 1 << 30
    src = torch.empty(nb, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    B.tpa_probe_copy(dst.data_ptr(), src.data_ptr(), nb, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    del src, dst
    n = 1024
    wl = synth.prefill_lora_dora(n=n, tenants=16)
    p = wl["projections"][0]
    x = torch.tensor(p["x"]).half().cuda()
    res = {"workload": "prefill_q_proj: 4096 -> 4096, n=1024 in 16 segments, 8 LoRA + 8 DoRA r16, f16"}
    for tag, pp, rows, opts in (("mixed", p, torch.tensor(wl["slot_of_row"]).cuda(), None),
                                ("base_gemm", {**p, "adapters": {}, "shared": None},
                                 torch.zeros(n, dtype=torch.int32, device="cuda"), {B.TPA_OPT_FUSE_EXPAND: 0})):
        L = load_layer(pp, torch, options=opts)
        call = layer_call([L], [x], rows, torch)
        g = capture(lambda: call(0), torch)
        t = time_graph(g, args.steps, args.warmup, torch)
        res[tag] = {"us_per_layer": t * 1e6, "config": L.config(n)}
        del g
        L.close()
        log("%s: %.1f us" % (tag, t * 1e6))
    print(json.dumps(res), flush=True)


def main():
    args = parse()
    ws = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or ws != 1:
        print("bench.py measures one GPU only (the library has no multi-GPU path); got --gpus %d" % args.gpus,
              file=sys.stderr)
        sys.exit(2)
    if args.workload == "stack":
        return stack_main(args)
    if args.workload == "prefill_q_proj":
        return prefill_main(args)
    import numpy as np
    import torch
    from tenant_peft_adapter_amd import bytemodel as bm
    from workloads import synth

    torch.cuda.set_device(0)
    if args.only_routes:
        cal = calibrate(torch, full=True)
        out = {"workload": "routes against the byte model", "calibration": {k: v for k, v in cal.items()},
               "routes_vs_byte_model": route_table(torch, cal)}
        print(json.dumps(out), flush=True)
        return
    log("generating the mixed decoder-layer workload")
    wl = synth.decoder_layer_mixed()
    n = wl["n"]
    log("loading 20 tenants into 7 projections, %d buffer sets" % args.sets)
    sets = [build_step(wl, torch) for _ in range(args.sets)]
    layers, step, units = sets[0]
    # Warm-up steps, then the timed region: exactly `steps` steps of
    # the captured graph, the chain rotating over the buffer sets (every
    # step reads W from HBM, as consecutive decoder layers do).
    chain = [st for _, st, _ in sets]
    graphs = [capture(c, torch) for c in chain]
    for i in range(args.warmup):
        graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    log("timing %d graph-replayed steps" % args.steps)
    t0 = time.perf_counter()
    for i in range(args.steps):
        graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    t_step = (time.perf_counter() - t0) / args.steps
    del graphs
    log("%.1f us per step (timed region)" % (t_step * 1e6))
    # Appendix "Kernel timing": chains of >= 2 ms, five rebuilds, median;
    # cold (rotating the buffer sets) and warm (one set).
    t_cold, cold_samples, cold_copies = time_chain(lambda i: chain[i % len(chain)](), torch)
    t_warm, warm_samples, warm_copies = time_chain(lambda i: step(), torch)
    log("%.1f us per step cold, %.1f warm (chained graphs)" % (t_cold * 1e6, t_warm * 1e6))

    # Eager (no graph) for reference.
    for _ in range(3):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(20):
        step()
    torch.cuda.synchronize()
    t_eager = (time.perf_counter() - t0) / 20

    log("per-stage event timing")
    stages = stage_times([layers[m[0]] for m in units], step, args.stage_reps, torch)
    log("calibration")
    cal = calibrate(torch, full=True)
    beta, lam, beta_mall = cal["beta_hbm"], cal["lambda"], cal["beta_mall"]

    # Byte model per projection; measured times per launch unit (a fused
    # group or a single projection), each kernel one launch per unit.
    names = [p["name"] for p in wl["projections"]]
    unit_names = ["+".join(names[i] for i in m) for m in units]
    shapes = [bm.shape_of(n, p["d_in"], p["d_out"], wl["slot_of_row"], p["adapters"], q=2, r_v=256,
                          vera_a_read=not (p["shared"] or {}).get("a_from"))
              for p in wl["projections"]]
    kb = [bm.kernel_bytes(s) for s in shapes]
    # Kernel times are the raw event intervals, which agree with rocprofv3's
    # per-dispatch durations.  An event pair with no kernel between (stage 3
    # on this path) is reported for reference: its interval overlaps a
    # kernel's start-up, so it is not taken off.
    pair_cost = sum(st[3] for st in stages) / len(stages) * 1e-6
    gemm_t = [max(st[2] * 1e-6, 1e-9) for st in stages]
    # Dominant kernel: the base-GEMM launch with the most algorithmic bytes.
    # A unit's decode GEMM instance takes the column-block width of its
    # widest projection.  A unit whose shrink runs in the GEMM's own launch
    # counts the shrink's bytes and time there, not in the adapter path.
    mb = 1 if n <= 16 else 2 if n <= 32 else 4
    sg = [all(layers[i].config(n)["shrink_in_gemm"] for i in m) for m in units]
    gemm_bytes = [sum(kb[i]["gemm"]["bytes"] for i in m) for m in units]
    side_bytes = [sum(kb[i]["shrink"]["bytes"] for i in m) if sg[u] else 0 for u, m in enumerate(units)]
    launch_bytes = [g + b for g, b in zip(gemm_bytes, side_bytes)]
    du = max(range(len(units)), key=lambda u: launch_bytes[u])
    widest = max(units[du], key=lambda i: wl["projections"][i]["d_out"])
    cfg = layers[widest].config(n)
    dom_name = {0: "gemm_skinny_kernel<f16,%d,%d,%d>" % (mb, cfg["gemm_nb"], cfg["gemm_groups"]),
                2: "gemm_stream_kernel<f16,%d,%d,%d,%d>" % (mb, cfg["gemm_nb"], cfg["gemm_groups"], cfg["gemm_stages"])
                }.get(cfg["gemm_path"], "gemm_tiled_kernel<f16>")
    dom_cfg = "nb=%d groups=%d stages=%d kc=%d split=%d shrink_in_launch=%d" % (
        cfg["gemm_nb"], cfg["gemm_groups"], cfg["gemm_stages"], cfg["gemm_kc"], cfg["gemm_split"], int(sg[du]))
    dom_bytes, dom_time = launch_bytes[du], gemm_t[du]
    gemm_bytes_all = sum(launch_bytes)
    gemm_time_all = sum(gemm_t)
    # A launch before the GEMM remains where the shrink runs there or OFT
    # tenants need their rotation.
    pre = [not sg[u] or any(kb[i]["oft"]["launches"] for i in m) for u, m in enumerate(units)]
    adapter_bytes = sum(bm.adapter_path_bytes(s) for s in shapes) - sum(side_bytes)
    adapter_time = sum((st[1] if pre[u] else 0.0) + st[4] for u, st in enumerate(stages)) * 1e-6
    adapter_launches = len(step.plans) + sum(pre) + len(units)
    predicted = bm.predict_time(gemm_time_all, adapter_bytes, adapter_launches, beta, lam)

    ratio = t_pure = None
    if not args.no_pure_lora:
        log("pure-LoRA batch")
        wl_pure = synth.decoder_layer_mixed(pure_lora=True)
        for ls, _, _ in sets:
            for L in ls:
                L.close()
        sets = chain = None
        torch.cuda.empty_cache()
        sets_p = [build_step(wl_pure, torch) for _ in range(args.sets)]
        chain_p = [st for _, st, _ in sets_p]
        t_pure = time_chain(lambda i: chain_p[i % len(chain_p)](), torch)[0]
        ratio = t_cold / t_pure
        for ls, _, _ in sets_p:
            for L in ls:
                L.close()
        sets_p = chain_p = None
        torch.cuda.empty_cache()

    side = None
    if not args.no_side_targets:
        log("prefill, DoRA-expand and VeRA-sweep layers")
        side = side_targets(torch, args)
    routes = None
    if args.routes:
        log("routes against the byte model")
        routes = route_table(torch, cal)

    out = {
        "metric": METRIC,
        "value": 7 * n / t_step,
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": t_step * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic (seeded; Llama-3.1-8B projection shapes, random-init weights and adapters)",
        "config": {"workload": "decoder_layer_mixed: one Llama-3.1-8B decoder layer, 7 adapted projections, "
                               "n=64 decode rows, 20 tenants (4 each LoRA r16, DoRA r16, (IA)3 k/v/up, "
                               "VeRA shared r256, OFT b32 q/k/v), rows shuffled",
                   "n": n, "projections": names, "graph": True},
        "us_per_adapted_layer": t_step * 1e6 / 7,
        "decoder_layer_rows_per_s": n / t_step,
        "timing": {"timed_region_us_per_step": t_step * 1e6, "buffer_sets": args.sets,
                   "cold_us_per_step": t_cold * 1e6, "cold_samples_us": [round(v * 1e6, 2) for v in cold_samples],
                   "warm_us_per_step": t_warm * 1e6, "warm_samples_us": [round(v * 1e6, 2) for v in warm_samples],
                   "steps_per_chain": [cold_copies, warm_copies],
                   "protocol": "graph chains of >= 2 ms, 5 rebuilds, median; cold rotates %d buffer sets "
                               "(%.0f MB of weights)" % (args.sets, args.sets * sum(gemm_bytes) / 1e6)},
        "eager_ms_per_step": t_eager * 1e3,
        "mixed_over_pure_lora": ratio,
        "pure_lora_us_per_step_cold": None if t_pure is None else t_pure * 1e6,
        "roofline": {
            "kernel": "%s (base GEMM of %s in one launch)" % (dom_name, ", ".join(names[i] for i in units[du])),
            "bound": "hbm", "achieved": dom_bytes / dom_time / 1e9, "peak": HBM_PEAK / 1e9, "unit": "GB/s",
            "frac": dom_bytes / dom_time / HBM_PEAK, "traffic": profiled_traffic(dom_name, dom_cfg),
            "frac_of_copy_rate": dom_bytes / dom_time / beta,
            "frac_of_read_rate": dom_bytes / dom_time / cal["read_hbm"],
            "bytes_per_launch": dom_bytes, "us_per_launch": dom_time * 1e6,
            "us_event_pair_cost": pair_cost * 1e6, "config": dom_cfg,
        },
        "base_gemm": {"bytes_per_step": gemm_bytes_all, "us_per_step": gemm_time_all * 1e6,
                      "GBps": gemm_bytes_all / gemm_time_all / 1e9, "shrink_bytes_in_gemm_launches": sum(side_bytes),
                      "units_with_shrink_in_gemm": [unit_names[u] for u in range(len(units)) if sg[u]]},
        "adapter_path": {"bytes_per_step": adapter_bytes, "us_per_step_shrink_oft_expand": adapter_time * 1e6,
                         "GBps": adapter_bytes / adapter_time / 1e9, "launches": adapter_launches,
                         "predicted_step_us": predicted * 1e6},
        "calibration": {"beta_hbm_GBps": beta / 1e9, "beta_mall_GBps": beta_mall / 1e9,
                        "beta_l2_GBps": cal["beta_l2"] / 1e9, "read_hbm_GBps": cal["read_hbm"] / 1e9,
                        "lambda_us": lam * 1e6},
        "side_targets": side,
        "routes_vs_byte_model": routes,
        "stages_us_raw_events": {nm: dict(zip(("plan", "shrink+oft", "gemm+reduce", "pre-expand", "expand"),
                                              [round(v, 2) for v in st]))
                                 for nm, st in zip(unit_names, stages)},
    }
    if not args.no_cpu_baseline:
        log("oracle on the CPU")
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
