"""The no-allocation forward (tpa_layer_forward_noalloc), called through the
C ABI: on two calls in a row, the second with fewer rows, it gives the same
bits as tpa_layer_forward on the same layer and inputs, and both match the
oracle; a batch whose workspace exceeds the scratch array is refused with
-6 before anything is launched; and the calls take no device memory."""
import numpy as np
import pytest
import torch

from gpu_util import check, make_layer, reference, say
from tenant_peft_adapter_amd import binding as B
from workloads import synth

pytestmark = pytest.mark.gpu


def _noalloc(L, x, sor, out):
    B.tpa_layer_forward_noalloc(L.handle, x.data_ptr(), sor.data_ptr(), x.shape[0], out.data_ptr(),
                                torch.cuda.current_stream().cuda_stream)
    return out


def _pair(L, p, sor_np, rows, dtype, label, mean_tol=0.01, max_tol=2e-3):
    x = torch.tensor(p["x"][rows]).to({"f16": torch.float16, "f32": torch.float32}[dtype]).cuda()
    sor = torch.tensor(np.asarray(sor_np)[rows].astype(np.int32)).cuda()
    say("%s: %d rows, workspace %d bytes" % (label, len(rows), B.tpa_workspace_size(L.handle, len(rows))))
    want = L.forward(x, sor).clone()
    out = torch.full((x.shape[0], L.d_out), float("nan"), dtype=L.W.dtype, device="cuda")
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    got = _noalloc(L, x, sor, out)
    torch.cuda.synchronize()
    free1 = torch.cuda.mem_get_info()[0]
    assert free0 - free1 < (1 << 20), (free0, free1)
    assert torch.equal(got, want), label
    y, h, xw = reference(p, sor_np, rows)
    check(got.float().cpu().numpy().astype(np.float64), y, h, xw, mean_tol=mean_tol, max_tol=max_tol, label=label)


@pytest.mark.parametrize("dtype", ["f16", "f32"])
def test_noalloc_matches_forward_tiny(dtype):
    wl = synth.tiny_mixed(seed=21, n=300, dtype=dtype, with_identity=True)
    p = wl["projections"][0]
    L = make_layer(p, max_slots=8, max_rank=32)
    tol = dict(mean_tol=1e-4, max_tol=2e-5) if dtype == "f32" else {}
    _pair(L, p, wl["slot_of_row"], np.arange(300), dtype, "noalloc tiny %s n=300" % dtype, **tol)
    _pair(L, p, wl["slot_of_row"], np.arange(7, 47), dtype, "noalloc tiny %s n=40" % dtype, **tol)
    L.close()


def test_noalloc_matches_forward_decoder_projection():
    """The q projection of the mixed decoder layer (4096 -> 4096, 20 tenants
    of five methods, OFT rows rotated): all 64 decode rows, then 17."""
    wl = synth.decoder_layer_mixed(shapes=(("q", 4096, 4096),))
    p = wl["projections"][0]
    L = make_layer(p, max_slots=32, max_rank=256)
    _pair(L, p, wl["slot_of_row"], np.arange(64), "f16", "noalloc q n=64")
    _pair(L, p, wl["slot_of_row"], np.arange(3, 20), "f16", "noalloc q n=17")
    L.close()


def test_noalloc_refuses_batches_beyond_the_scratch():
    wl = synth.decoder_layer_mixed(shapes=(("q", 4096, 4096),))
    p = wl["projections"][0]
    L = make_layer(p, max_slots=32, max_rank=256)
    n = 8192
    need = B.tpa_workspace_size(L.handle, n)
    assert need > B.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((n, 4096), dtype=torch.float16, device="cuda")
    sor = torch.zeros(n, dtype=torch.int32, device="cuda")
    out = torch.zeros((n, 4096), dtype=torch.float16, device="cuda")
    with pytest.raises(B.TpaError) as e:
        B.tpa_layer_forward_noalloc(L.handle, x.data_ptr(), sor.data_ptr(), n, out.data_ptr(),
                                    torch.cuda.current_stream().cuda_stream)
    assert e.value.code == -6
    assert "scratch" in B.tpa_last_error()
    torch.cuda.synchronize()
    assert torch.count_nonzero(out).item() == 0      # nothing ran
    # n = 0 is a no-op; the layer still works afterwards.
    B.tpa_layer_forward_noalloc(L.handle, x.data_ptr(), sor.data_ptr(), 0, out.data_ptr(), 0)
    _pair(L, p, wl["slot_of_row"], np.arange(64), "f16", "noalloc q after refusal")
    L.close()
