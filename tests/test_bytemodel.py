"""The byte model against the numbers the pages print (Table 2, the Table A9
predicted column, the size of a rank-64 tenant)."""
import json
import os

import pytest

from tenant_peft_adapter_amd import bytemodel as bm

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "table2_bytes.json")))
# The printed (IA)3 route-one row (0.01 GB) does not match the count the page
# itself states (k·d_out per adapted projection gives 0.017 GB); that row is
# checked against the stated count instead and is left unpinned.
UNPINNED = {"ia3_route1"}


@pytest.mark.parametrize("row", sorted(GOLD["rows"]))
def test_table2_rows(row):
    got = bm.table2(tenants=GOLD["tenants"], beta=GOLD["beta_gb_s"] * 1e9)[row]
    want = GOLD["rows"][row]
    if row in UNPINNED:
        assert abs(got[0] / 1e9 - 0.0168) < 1e-3
        return
    assert abs(got[0] / 1e9 - want["gb"]) <= 0.005 + 1e-9, (row, got[0] / 1e9)
    assert abs(got[1] * 1e3 - want["ms"]) <= 0.005 + 1e-9, (row, got[1] * 1e3)


def test_table_a9_predicted_column():
    got = bm.per_tenant_decode(beta=GOLD["beta_gb_s"] * 1e9)
    for k, ms in GOLD["table_a9_predicted_ms"].items():
        assert abs(got[k] * 1e3 - ms) <= 0.005 + 1e-9, (k, got[k] * 1e3)


def test_rank64_tenant_size():
    assert abs(bm.lora_bytes(64, 1) / 1e9 - GOLD["rank64_tenant_gb"]) <= 0.005


def test_vera_factors_read_once_whatever_k():
    # Proposition 2(iv): the factor bytes do not depend on k; only vectors do.
    a = bm.vera_route2_bytes(256, 1)
    b = bm.vera_route2_bytes(256, 1024)
    per_tenant = (b - a) / 1023
    assert per_tenant == bm.vera_route2_bytes(256, 2) - a


def test_route_extras():
    assert bm.scale_route_extra(1024, 4096, 1) == (2 * 1024 * 4096 * 2, 1)
    assert bm.scale_route_extra(1024, 4096, 3)[1] == 2
    assert bm.predict_time(1.0, 680e9, 2, 680e9, 0.5) == 1.0 + 1.0 + 1.0


def test_kernel_bytes_counts():
    import numpy as np
    ad = {1: {"method": "lora", "A": np.zeros((64, 16)), "B": np.zeros((16, 128)), "c": 2.0},
          2: {"method": "ia3", "l": np.zeros(128)},
          3: {"method": "vera", "d": np.zeros(32), "e": np.zeros(128)},
          4: {"method": "oft", "Q": np.zeros((2, 32, 32))}}
    b = bm.shape_of(8, 64, 128, [1, 1, 2, 3, 3, 3, 4, 0], ad, q=2, r_v=32)
    assert (b.n_owned, b.v_elems, b.k_s, b.n_vera, b.k_vera, b.n_oft, b.k_oft) == (2, 32, 1, 3, 1, 1, 1)
    kb = bm.kernel_bytes(b)
    assert kb["gemm"]["bytes"] == 2 * (8 * 64 + 64 * 128 + 8 * 128)
    assert kb["oft"]["bytes"] == 2 * (2 * 64 + 64 * 32)
    assert kb["shrink"]["bytes"] == 2 * (2 * 64 + 16 * 64) + 2 * 32 + 2 * (3 * 64 + 32 * 64) + 2 * 3 * 32 + 4 * 32
    assert kb["expand"]["bytes"] == 2 * (2 * 8 * 128 + 16 * 128) + 2 * (32 + 3 * 32) + 4 * (1 + 1) * 128 + 2 * 32 * 128


def test_true_rank_counts_and_stored_padding():
    import numpy as np
    ad = {1: {"method": "lora", "A": np.zeros((64, 8)), "B": np.zeros((8, 128)), "c": 2.0}}
    b = bm.shape_of(4, 64, 128, [1, 1, 1, 1], ad, q=2)
    assert b.owned_ranks == [8] and b.owned_ranks_stored == [16] and b.v_elems == 32
    assert bm.kernel_bytes(b)["shrink"]["bytes"] == 2 * (4 * 64 + 8 * 64) + 2 * 32
    assert bm.stored_factor_bytes(b) == 2 * 16 * (64 + 128)


def test_vera_a_read_once_per_fused_input():
    """A projection that shares its input and VeRA's A with an earlier one of
    its fused layer reads neither x nor A_v for the VeRA rows: it reads the
    shared x·A_v product instead (appendix "Byte counts")."""
    import numpy as np
    ad = {1: {"method": "vera", "d": np.zeros(256), "e": np.zeros(1024)}}
    own = bm.kernel_bytes(bm.shape_of(8, 4096, 1024, [1] * 8, ad, q=2, r_v=256))["shrink"]["bytes"]
    shared = bm.kernel_bytes(bm.shape_of(8, 4096, 1024, [1] * 8, ad, q=2, r_v=256,
                                         vera_a_read=False))["shrink"]["bytes"]
    assert own - shared == 2 * (8 * 4096 + 256 * 4096) - 2 * 8 * 256
