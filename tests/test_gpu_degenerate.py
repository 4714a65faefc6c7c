"""Degenerate members and extreme ranks on the GPU.

Members whose parameters make them the identity -- (IA)3 with l = 1, SSF
with s = 1 and b = 0, OFT with Q = 0 (R = I exactly), VeRA with d = 0 (a
zero term) -- must give the base output bit for bit, on the decode and the
prefill paths.  DoRA with B = 0 is the base output rescaled by m ⊘ ‖W‖_c,
and LoRA at rank 1 and at the largest rank a layer takes (512) match the
oracle within the parity tolerance (1% mean relative, 2e-3 · max|h|)."""
import numpy as np
import pytest
import torch

from gpu_util import check, make_layer, reference, run, say
from workloads import synth

pytestmark = pytest.mark.gpu


def _layer_with_degenerate_slots(n, dtype="f16"):
    rng = np.random.default_rng(900 + n)
    d = 256
    p = synth.make_projection(rng, "degenerate", d, d, dtype, n)
    p["shared"] = synth._vera_shared(rng, d, d, 32, dtype)
    W = p["W"].astype(np.float64)
    norms = np.sqrt((W * W).sum(axis=1))  # column norms of the math-layout W
    zeros_B = np.zeros((8, d), np.float32)
    p["adapters"] = {
        1: {"method": "ia3", "l": np.ones(d, np.float32)},
        2: {"method": "ssf", "s": np.ones(d, np.float32), "b": np.zeros(d, np.float32)},
        3: {"method": "oft", "Q": np.zeros((d // 32, 32, 32), np.float32)},
        4: {"method": "vera", "d": np.zeros(32, np.float32), "e": (1 + 0.3 * rng.standard_normal(d)).astype(np.float32),
            "c": 1.0},
        5: {"method": "dora", "A": synth.round_to(rng.standard_normal((d, 8)) / 16, dtype), "B": zeros_B, "c": 2.0,
            "m": (norms * (1 + 0.1 * rng.standard_normal(d))).astype(np.float32)},
        6: synth._lora(rng, d, d, 1, dtype),
        7: synth._lora(rng, d, d, 512, dtype),
    }
    return p


@pytest.mark.parametrize("n", [48, 300])
def test_identity_members_are_bitwise_base(n):
    p = _layer_with_degenerate_slots(n)
    say("degenerate identity members n=%d" % n)
    L = make_layer(p, max_slots=8, max_rank=512)
    base = run(L, p["x"], np.zeros(n, np.int32), "f16")
    for slot in (1, 2, 3, 4):
        got = run(L, p["x"], np.full(n, slot, np.int32), "f16")
        np.testing.assert_array_equal(got, base, err_msg="slot %d" % slot)
    L.close()


@pytest.mark.parametrize("n", [48, 300])
def test_dora_without_update_and_extreme_ranks(n):
    p = _layer_with_degenerate_slots(n)
    say("DoRA B=0, LoRA ranks 1 and 512, n=%d" % n)
    L = make_layer(p, max_slots=8, max_rank=512)
    sor = (np.arange(n) % 3 + 5).astype(np.int32)  # slots 5, 6, 7 in turn
    y_gpu = run(L, p["x"], sor, "f16")
    y, h, xw = reference(p, sor)
    check(y_gpu, y, h, xw, label="degenerate n=%d" % n)
    L.close()
