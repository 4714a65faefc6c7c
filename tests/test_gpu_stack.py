"""GPU parity at the full adapter stack's sizes: one decoder layer of the
stack (seven Llama-3.1-8B projections, 1024 resident tenants, LoRA/DoRA at
rank 64, VeRA r256, (IA)3, OFT b32), a Zipf(1.1) batch run as the stack
benchmark runs it (one row plan, q/k/v and gate/up as groups), sampled rows
against the oracle row by row.  Every tenant holds values of its own
(workloads.stack.tenant_record), and the sample takes one row from each of
at least 64 distinct tenants, several of every method, so a row sent to
another tenant of its own method fails the check."""
import numpy as np
import pytest
import torch

from gpu_util import check, reference, say
from workloads import stack, synth

pytestmark = pytest.mark.gpu

T = 1024


@pytest.fixture(scope="module")
def stack_layer():
    """The last decoder layer of the stack with every tenant loaded."""
    from tenant_peft_adapter_amd.layer import AdaptedLayer
    protos = stack.prototypes()
    layers = []
    for name, d_in, d_out in synth.LLAMA8B_PROJECTIONS:
        say("stack layer: loading %d tenants into %s (%d -> %d)" % (T, name, d_in, d_out))
        W = stack.device_weight(torch, 31, name, d_out, d_in)
        L = AdaptedLayer(W, max_slots=T + 1, max_rank=256)
        L.set_vera_shared(protos[name]["shared"]["A"], protos[name]["shared"]["B"])
        for t in range(T):
            assert L.load(stack.tenant_record(protos[name], t)) == t + 1
        layers.append(L)
    yield protos, layers
    for L in layers:
        L.close()


@pytest.mark.parametrize("n", [256, 4096])
def test_stack_layer_sampled_rows(stack_layer, n):
    from tenant_peft_adapter_amd.layer import LayerGroup, RowPlan
    protos, layers = stack_layer
    shapes = synth.LLAMA8B_PROJECTIONS
    xs = [stack.device_input(torch, n, d_in, name) for name, d_in, _ in shapes]
    sor_np = stack.zipf_rows(n, T)
    sor = torch.tensor(sor_np).cuda()
    plan = RowPlan(layers[0], n).build(layers[0], sor)
    assert all(plan.accepts(L) for L in layers)
    outs = LayerGroup(layers[0:3], n).forward(plan, xs[0:3])
    outs.append(layers[3].forward_planned(plan, xs[3]))
    outs += LayerGroup(layers[4:6], n).forward(plan, xs[4:6])
    outs.append(layers[6].forward_planned(plan, xs[6]))
    torch.cuda.synchronize()
    # One row of each of up to `per` distinct tenants per method: the most
    # popular tenants first, then the rarest present, so rows of tenants far
    # apart in slot order (and in the plan's sort) are both checked.
    per = 14 if n >= 4096 else 3
    rows = []
    for m in stack.METHODS:
        first = {}
        for i, s in enumerate(sor_np.tolist()):
            if stack.method_of(s - 1) == m and s not in first:
                first[s] = i
        ids = sorted(first)
        pick = ids if len(ids) <= per else ids[:per // 2] + ids[-(per - per // 2):]
        rows += [first[s] for s in pick]
    rows = np.array(sorted(rows))
    tenants = sorted(set(sor_np[rows].tolist()))
    say("stack layer n=%d: %d sampled rows of %d tenants (%d distinct in the batch)"
        % (n, len(rows), len(tenants), len(set(sor_np.tolist()))))
    if n >= 4096:
        assert len(tenants) >= 64
    for (name, d_in, d_out), L, x, o in zip(shapes, layers, xs, outs):
        p = {"name": name, "d_in": d_in, "d_out": d_out, "dtype": "f16",
             "W": L.W.float().cpu().numpy(), "x": x.float().cpu().numpy(),
             "shared": protos[name]["shared"], "adapters": stack.adapters_of(protos[name], T)}
        y, h, xw = reference(p, sor_np, rows)
        check(o.float().cpu().numpy().astype(np.float64)[rows], y, h, xw, label="stack %s n=%d" % (name, n))
    plan.close()
