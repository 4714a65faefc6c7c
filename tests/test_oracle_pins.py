"""Pins of the CPU oracle against what the pages and mathematics fix.

Each test checks the oracle against something other than itself: values
derived by hand from the definitions (tests/golden/hand_examples.json),
the printed Table 1 (tests/golden/table1_members.json), closed forms
(the 2x2 Cayley rotation, Pythagorean column norms), identities the pages
state (the fold identities, (IA)3 on the gated FFN, VeRA = its rank-r LoRA
conversion, stacking), and a pure-Python brute force on tiny inputs.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import normal_form as nf
from oracle import methods as om

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _arr(rec):
    out = {}
    for k, v in rec.items():
        out[k] = np.array(v, dtype=np.float64) if isinstance(v, list) else v
    return out


# ---------------------------------------------------------------- golden ----

@pytest.mark.parametrize("case", _load("hand_examples.json")["cases"], ids=lambda c: c["name"])
def test_hand_examples(case):
    gold = _load("hand_examples.json")
    x = np.array(gold["x"], dtype=np.float64)
    W = np.array(case["W"], dtype=np.float64)
    ad = _arr(case["adapter"])
    shared = _arr(case["shared"]) if "shared" in case else None
    want = np.array(case["y"], dtype=np.float64)
    got = oracle.direct_forward(x, W, ad, shared)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)
    slots = nf.unfolded_slots(ad, W, shared)
    np.testing.assert_allclose(nf.normal_form_eval(x, W, slots), want, rtol=0, atol=1e-12)
    folded, _ = nf.fold(slots)
    np.testing.assert_allclose(nf.normal_form_eval(x, W, folded), want, rtol=0, atol=1e-12)
    if "s" in case:
        np.testing.assert_allclose(slots["s"], case["s"], rtol=0, atol=1e-15)
    if "R" in case:
        np.testing.assert_allclose(om.oft_rotation(ad["Q"]), case["R"], rtol=0, atol=1e-15)


def test_stacking_order_matters():
    gold = _load("hand_examples.json")
    st = gold["stacking"]
    x = np.array(gold["x"], dtype=np.float64)
    W = np.array(st["W"], dtype=np.float64)
    lora = nf.unfolded_slots(_arr(st["lora"]), W)
    ia3 = nf.unfolded_slots(_arr(st["ia3"]), W)
    np.testing.assert_allclose(nf.normal_form_eval(x, W, nf.stack(lora, ia3)),
                               st["ia3_after_lora"], atol=1e-12, rtol=0)
    np.testing.assert_allclose(nf.normal_form_eval(x, W, nf.stack(ia3, lora)),
                               st["lora_after_ia3"], atol=1e-12, rtol=0)


def test_member_table_is_table1():
    table1 = _load("table1_members.json")["methods"]
    got = nf.member_table()
    for meth, row in table1.items():
        assert got[meth]["owned"] == sorted(row["owned"]), meth
        assert got[meth]["folds"] == sorted(row["folds"]), meth
        assert got[meth]["live"] == sorted(row["live"]), meth


def test_fold_rule_matches_folds_made():
    # The folds the converter makes on real slots are the ones the rule
    # allows (Table 1), and afterwards exactly the live slots remain.
    rng = np.random.default_rng(7)
    d_in, d_out = 12, 10
    W = rng.standard_normal((d_in, d_out))
    ads = {
        "lora": {"method": "lora", "A": rng.standard_normal((d_in, 3)), "B": rng.standard_normal((3, d_out)), "c": 2.0},
        "dora": {"method": "dora", "A": rng.standard_normal((d_in, 3)), "B": rng.standard_normal((3, d_out)), "c": 2.0,
                 "m": rng.uniform(1, 2, d_out)},
        "ia3": {"method": "ia3", "l": rng.uniform(0.5, 1.5, d_out)},
        "ssf": {"method": "ssf", "s": rng.uniform(0.5, 1.5, d_out), "b": rng.standard_normal(d_out)},
        "vera": {"method": "vera", "d": rng.uniform(0.5, 1.5, 4), "e": rng.uniform(0.5, 1.5, d_out), "c": 3.0},
        "oft": {"method": "oft", "Q": _skew(rng, 3, 4)},
    }
    shared = {"A": rng.standard_normal((d_in, 4)), "B": rng.standard_normal((4, d_out))}
    table1 = _load("table1_members.json")["methods"]
    for meth, ad in ads.items():
        slots = nf.unfolded_slots(ad, W, shared)
        folded, made = nf.fold(slots)
        assert sorted(made) == sorted(table1[meth]["folds"]), meth
        assert sorted(nf.live_slots(folded)) == sorted(table1[meth]["live"]), meth


# ------------------------------------------------------- identity slots ----

def test_identity_slots_reproduce_xW_exactly():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((9, 17))
    W = rng.standard_normal((17, 11))
    ref = x @ W
    slots = nf.unfolded_slots({"method": "identity"}, W)
    assert np.array_equal(nf.normal_form_eval(x, W, slots), ref)
    # Explicit identity values in every slot: x I W * 1 + 0 stays exact.
    full = {"R": np.eye(17), "s": np.ones(11), "b": np.zeros(11), "terms": [], "owned": set()}
    assert np.array_equal(nf.normal_form_eval(x, W, full), ref)
    y, h = oracle.layer_forward(x, W, np.zeros(9, dtype=np.int32), {})
    assert np.array_equal(y, ref) and np.array_equal(h, ref)


# ------------------------------------------------------ fold identities ----

def _ints(rng, shape, lo=-4, hi=5):
    return rng.integers(lo, hi, size=shape).astype(np.float64)


def test_fold_identities_exact_on_integers():
    rng = np.random.default_rng(2)
    x, A, B = _ints(rng, (5, 7)), _ints(rng, (7, 3)), _ints(rng, (3, 6))
    d, e = _ints(rng, 3), _ints(rng, 6)
    V = x @ A
    assert np.array_equal((x @ A) * d, x @ (A @ np.diag(d)))
    assert np.array_equal(((x @ A) * d) @ B, (x @ A) @ (np.diag(d) @ B))
    assert np.array_equal((V @ B) * e, V @ (B @ np.diag(e)))


@pytest.mark.parametrize("meth", ["lora", "vera", "ia3", "ssf"])
def test_folded_equals_unfolded_exactly_on_integers(meth):
    rng = np.random.default_rng(3)
    d_in, d_out, r = 8, 6, 3
    x, W = _ints(rng, (5, d_in)), _ints(rng, (d_in, d_out))
    shared = {"A": _ints(rng, (d_in, r)), "B": _ints(rng, (r, d_out))}
    ad = {
        "lora": {"method": "lora", "A": _ints(rng, (d_in, r)), "B": _ints(rng, (r, d_out)), "c": 3.0},
        "vera": {"method": "vera", "d": _ints(rng, r), "e": _ints(rng, d_out), "c": 2.0},
        "ia3": {"method": "ia3", "l": _ints(rng, d_out)},
        "ssf": {"method": "ssf", "s": _ints(rng, d_out), "b": _ints(rng, d_out)},
    }[meth]
    slots = nf.unfolded_slots(ad, W, shared)
    folded, _ = nf.fold(slots)
    direct = oracle.direct_forward(x, W, ad, shared)
    assert np.array_equal(nf.normal_form_eval(x, W, slots), direct)
    assert np.array_equal(nf.normal_form_eval(x, W, folded), direct)


def _skew(rng, nb, b, std=0.3):
    Q = rng.standard_normal((nb, b, b)) * std
    return Q - np.transpose(Q, (0, 2, 1))


@pytest.mark.parametrize("meth", ["dora", "oft", "lora", "vera", "ia3", "ssf"])
def test_normal_form_equals_direct_definition(meth):
    rng = np.random.default_rng(4)
    d_in, d_out, r = 32, 24, 4
    x = rng.standard_normal((7, d_in))
    W = rng.standard_normal((d_in, d_out)) / math.sqrt(d_in)
    shared = {"A": rng.standard_normal((d_in, 8)), "B": rng.standard_normal((8, d_out))}
    A, B = rng.standard_normal((d_in, r)), rng.standard_normal((r, d_out))
    ad = {
        "dora": {"method": "dora", "A": A, "B": B, "c": 2.0, "m": rng.uniform(0.5, 2.0, d_out)},
        "oft": {"method": "oft", "Q": _skew(rng, 4, 8)},
        "lora": {"method": "lora", "A": A, "B": B, "c": 2.0},
        "vera": {"method": "vera", "d": rng.standard_normal(8), "e": rng.standard_normal(d_out), "c": 0.5},
        "ia3": {"method": "ia3", "l": rng.standard_normal(d_out)},
        "ssf": {"method": "ssf", "s": rng.standard_normal(d_out), "b": rng.standard_normal(d_out)},
    }[meth]
    direct = oracle.direct_forward(x, W, ad, shared)
    slots = nf.unfolded_slots(ad, W, shared)
    folded, _ = nf.fold(slots)
    scale = np.max(np.abs(direct))
    for s in (slots, folded):
        np.testing.assert_allclose(nf.normal_form_eval(x, W, s), direct, rtol=0, atol=1e-13 * scale)


# ----------------------------------------------------------------- DoRA ----

def test_dora_pythagorean_column_norms():
    # W + cAB has columns (3e_0 + 4e_2) and (5e_1 + 12e_3): norms 5 and 13,
    # fixed by construction; the norm runs over d_in for each output column.
    W = np.zeros((4, 2))
    W[0, 0], W[1, 1] = 3.0, 5.0
    A = np.zeros((4, 2))
    A[2, 0], A[3, 1] = 1.0, 1.0
    B = np.array([[2.0, 0.0], [0.0, 6.0]])       # c = 2 -> cAB columns 4e_2, 12e_3
    np.testing.assert_array_equal(oracle.dora_column_norm(W, A, B, 2.0), [5.0, 13.0])
    np.testing.assert_allclose(oracle.dora_scale(W, A, B, 2.0, [10.0, 6.5]), [2.0, 0.5], rtol=0, atol=0)


def test_dora_scale_recovers_gain():
    rng = np.random.default_rng(5)
    d_in, d_out, r = 64, 40, 8
    W = rng.standard_normal((d_in, d_out))
    A, B = rng.standard_normal((d_in, r)), rng.standard_normal((r, d_out))
    # Column norms computed here by an explicit loop, not the oracle's call.
    col = np.array([math.sqrt(sum((W[i, j] + 2.0 * sum(A[i, k] * B[k, j] for k in range(r))) ** 2
                                   for i in range(d_in))) for j in range(d_out)])
    g = 1.0 + 0.1 * rng.standard_normal(d_out)
    s = oracle.dora_scale(W, A, B, 2.0, col * g)
    np.testing.assert_allclose(s, g, rtol=1e-14, atol=0)


def test_dora_at_init_is_lora_and_zero_B_is_base():
    rng = np.random.default_rng(6)
    d_in, d_out, r = 16, 12, 3
    x = rng.standard_normal((5, d_in))
    W = rng.standard_normal((d_in, d_out))
    A, B = rng.standard_normal((d_in, r)), rng.standard_normal((r, d_out))
    m = np.sqrt(np.sum((W + 2.0 * A @ B) ** 2, axis=0))
    dora = {"method": "dora", "A": A, "B": B, "c": 2.0, "m": m}
    lora = {"method": "lora", "A": A, "B": B, "c": 2.0}
    np.testing.assert_allclose(oracle.direct_forward(x, W, dora), oracle.direct_forward(x, W, lora),
                               rtol=1e-13, atol=1e-13)
    dora0 = {"method": "dora", "A": A, "B": np.zeros((r, d_out)), "c": 2.0,
             "m": np.sqrt(np.sum(W ** 2, axis=0))}
    np.testing.assert_allclose(oracle.direct_forward(x, W, dora0), x @ W, rtol=1e-13, atol=1e-13)


# ----------------------------------------------------------------- OFT -----

@pytest.mark.parametrize("q", [0.0, 0.5, -1.25, 3.0])
def test_cayley_2x2_closed_form(q):
    R = oracle.cayley(np.array([[0.0, q], [-q, 0.0]]))
    want = np.array([[1 - q * q, 2 * q], [-2 * q, 1 - q * q]]) / (1 + q * q)
    np.testing.assert_allclose(R, want, rtol=0, atol=1e-15)


def test_cayley_block_of_plane_rotations():
    # A 32x32 skew block made of 2x2 planes maps to the 2x2 closed form in
    # each plane: pins the full-size Cayley map, not just the 2x2 case.
    qs = np.linspace(-1.5, 1.5, 16)
    Q = np.zeros((32, 32))
    for p, q in enumerate(qs):
        Q[2 * p, 2 * p + 1], Q[2 * p + 1, 2 * p] = q, -q
    R = oracle.cayley(Q)
    want = np.zeros((32, 32))
    for p, q in enumerate(qs):
        want[2 * p:2 * p + 2, 2 * p:2 * p + 2] = np.array([[1 - q * q, 2 * q], [-2 * q, 1 - q * q]]) / (1 + q * q)
    np.testing.assert_allclose(R, want, rtol=0, atol=1e-14)


def test_cayley_orthogonal_det_one():
    rng = np.random.default_rng(8)
    Q = _skew(rng, 1, 32, 0.1)[0]
    R = oracle.cayley(Q)
    np.testing.assert_allclose(R.T @ R, np.eye(32), rtol=0, atol=1e-13)
    assert abs(np.linalg.det(R) - 1.0) < 1e-12
    np.testing.assert_allclose(oracle.cayley(-Q), R.T, rtol=0, atol=1e-13)
    np.testing.assert_array_equal(oracle.cayley(np.zeros((32, 32))), np.eye(32))


# ---------------------------------------------------------------- VeRA -----

def test_vera_equals_its_rank_r_lora_conversion():
    # §4.2 / §3.2: VeRA is exactly a rank-r LoRA with A_a = A diag(c d_a),
    # B_a = B diag(e_a) (each tenant then owns its own copy of the factors).
    rng = np.random.default_rng(9)
    d_in, d_out, r = 24, 20, 8
    x = rng.standard_normal((6, d_in))
    W = rng.standard_normal((d_in, d_out))
    Av, Bv = rng.standard_normal((d_in, r)), rng.standard_normal((r, d_out))
    d, e, c = rng.standard_normal(r), rng.standard_normal(d_out), 0.7
    vera = oracle.direct_forward(x, W, {"method": "vera", "d": d, "e": e, "c": c}, {"A": Av, "B": Bv})
    conv = {"method": "lora", "A": Av * (c * d)[None, :], "B": Bv * e[None, :], "c": 1.0}
    np.testing.assert_allclose(vera, oracle.direct_forward(x, W, conv), rtol=0, atol=1e-12)
    merged = x @ (W + c * Av @ np.diag(d) @ Bv @ np.diag(e))
    np.testing.assert_allclose(vera, merged, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- (IA)3 ----

def test_ia3_on_gated_ffn_is_scale_of_up():
    # §3.1: (σ(xWg) ⊙ xWu) ⊙ l = σ(xWg) ⊙ (xWu ⊙ l), so l is s of the up
    # projection.
    rng = np.random.default_rng(10)
    x = rng.standard_normal((5, 16))
    Wg, Wu = rng.standard_normal((16, 24)), rng.standard_normal((16, 24))
    l = 1.0 + 0.3 * rng.standard_normal(24)
    silu = lambda z: z / (1.0 + np.exp(-z))
    lhs = (silu(x @ Wg) * (x @ Wu)) * l
    rhs = silu(x @ Wg) * oracle.direct_forward(x, Wu, {"method": "ia3", "l": l})
    np.testing.assert_allclose(lhs, rhs, rtol=1e-15, atol=1e-15)


# ---------------------------------------------------------------- stack ----

def test_stacking_equals_sequential_application():
    rng = np.random.default_rng(11)
    d_in, d_out = 12, 10
    x = rng.standard_normal((4, d_in))
    W = rng.standard_normal((d_in, d_out))
    f1 = nf.unfolded_slots({"method": "ssf", "s": rng.standard_normal(d_out), "b": rng.standard_normal(d_out)}, W)
    f1["terms"].append({"c": 2.0, "A": rng.standard_normal((d_in, 2)), "d": None,
                        "B": rng.standard_normal((2, d_out)), "e": None})
    f2 = nf.unfolded_slots({"method": "ssf", "s": rng.standard_normal(d_out), "b": rng.standard_normal(d_out)}, W)
    f2["terms"].append({"c": 0.5, "A": rng.standard_normal((d_in, 3)), "d": rng.standard_normal(3),
                        "B": rng.standard_normal((3, d_out)), "e": rng.standard_normal(d_out)})
    h1 = nf.normal_form_eval(x, W, f1)
    # F2 applied to F1's output: its base path is h1 in place of xW.
    seq = h1 * f2["s"] + f2["b"]
    for t in f2["terms"]:
        seq = seq + t["c"] * ((((x @ t["A"]) * t["d"]) @ t["B"]) * t["e"])
    np.testing.assert_allclose(nf.normal_form_eval(x, W, nf.stack(f1, f2)), seq, rtol=0, atol=1e-12)


# ---------------------------------------------------------- brute force ----

def _py_matmul(a, b):
    n, k = len(a), len(a[0])
    m = len(b[0])
    return [[sum(a[i][t] * b[t][j] for t in range(k)) for j in range(m)] for i in range(n)]


def _py_cayley(Q):
    # Gauss-Jordan inverse of I - Q, then (I + Q) @ inv.
    b = len(Q)
    M = [[(1.0 if i == j else 0.0) - Q[i][j] for j in range(b)] + [1.0 if i == j else 0.0 for j in range(b)]
         for i in range(b)]
    for c in range(b):
        p = max(range(c, b), key=lambda r: abs(M[r][c]))
        M[c], M[p] = M[p], M[c]
        piv = M[c][c]
        M[c] = [v / piv for v in M[c]]
        for r in range(b):
            if r != c and M[r][c] != 0.0:
                f = M[r][c]
                M[r] = [vr - f * vc for vr, vc in zip(M[r], M[c])]
    inv = [row[b:] for row in M]
    IpQ = [[(1.0 if i == j else 0.0) + Q[i][j] for j in range(b)] for i in range(b)]
    return _py_matmul(IpQ, inv)


def _py_forward_row(xr, W, ad, shared):
    d_in, d_out = len(W), len(W[0])
    meth = ad["method"]
    if meth == "oft":
        Q = ad["Q"]
        b = len(Q[0])
        xr2 = [0.0] * d_in
        for j in range(len(Q)):
            R = _py_cayley([list(map(float, row)) for row in Q[j]])
            for c in range(b):
                xr2[j * b + c] = sum(xr[j * b + t] * R[t][c] for t in range(b))
        xr = xr2
    base = [sum(xr[i] * W[i][j] for i in range(d_in)) for j in range(d_out)]
    if meth in ("identity", "oft"):
        return base
    if meth == "ia3":
        return [base[j] * ad["l"][j] for j in range(d_out)]
    if meth == "ssf":
        return [base[j] * ad["s"][j] + ad["b"][j] for j in range(d_out)]
    if meth in ("lora", "dora"):
        A, B, c = ad["A"], ad["B"], ad["c"]
        r = len(B)
        if meth == "lora":
            v = [sum(xr[i] * A[i][k] for i in range(d_in)) for k in range(r)]
            return [base[j] + c * sum(v[k] * B[k][j] for k in range(r)) for j in range(d_out)]
        Wp = [[W[i][j] + c * sum(A[i][k] * B[k][j] for k in range(r)) for j in range(d_out)] for i in range(d_in)]
        out = []
        for j in range(d_out):
            nrm = math.sqrt(sum(Wp[i][j] ** 2 for i in range(d_in)))
            out.append(sum(xr[i] * Wp[i][j] for i in range(d_in)) * ad["m"][j] / nrm)
        return out
    if meth == "vera":
        Av, Bv = shared["A"], shared["B"]
        r = len(Bv)
        v = [sum(xr[i] * Av[i][k] for i in range(d_in)) * ad["d"][k] for k in range(r)]
        return [base[j] + ad["c"] * sum(v[k] * Bv[k][j] for k in range(r)) * ad["e"][j] for j in range(d_out)]
    raise ValueError(meth)


def test_layer_forward_matches_pure_python_brute_force():
    rng = np.random.default_rng(12)
    d_in, d_out, r, n = 8, 6, 2, 8
    W = rng.standard_normal((d_in, d_out))
    shared = {"A": rng.standard_normal((d_in, 3)), "B": rng.standard_normal((3, d_out))}
    adapters = {
        1: {"method": "lora", "A": rng.standard_normal((d_in, r)), "B": rng.standard_normal((r, d_out)), "c": 2.0},
        2: {"method": "dora", "A": rng.standard_normal((d_in, r)), "B": rng.standard_normal((r, d_out)), "c": 2.0,
            "m": rng.uniform(0.5, 2, d_out)},
        3: {"method": "ia3", "l": rng.standard_normal(d_out)},
        4: {"method": "vera", "d": rng.standard_normal(3), "e": rng.standard_normal(d_out), "c": 1.5},
        5: {"method": "oft", "Q": _skew(rng, 2, 4)},
        6: {"method": "ssf", "s": rng.standard_normal(d_out), "b": rng.standard_normal(d_out)},
    }
    x = rng.standard_normal((n, d_in))
    slot_of_row = np.array([0, 1, 2, 3, 4, 5, 6, 4], dtype=np.int32)
    y, h = oracle.layer_forward(x, W, slot_of_row, adapters, shared)
    Wl = W.tolist()
    sh = {k: v.tolist() for k, v in shared.items()}
    for i in range(n):
        ad = adapters.get(int(slot_of_row[i]), {"method": "identity"})
        adl = {k: (v.tolist() if isinstance(v, np.ndarray) else v) for k, v in ad.items()}
        want = _py_forward_row(x[i].tolist(), Wl, adl, sh)
        np.testing.assert_allclose(y[i], want, rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------- plan ------

def test_plan_canonical_small():
    # Slots 1, 2 own terms (class 0), 3 shared term (class 1), 4 none (2).
    cls = [2, 0, 0, 1, 2]
    sor = [3, 1, 4, 2, 1, 9, 3, 0, 2, 1]
    p = oracle.plan(sor, cls, tile_rows=2, has_R=[0, 0, 0, 0, 1])
    # row 5 (slot 9) is invalid -> slot 0.
    assert p["invalid"] == 1
    assert p["row_slot"] == [3, 1, 4, 2, 1, 0, 3, 0, 2, 1]
    assert p["perm"] == [1, 4, 9, 3, 8, 0, 6, 5, 7, 2]
    assert p["seg_ptr"] == [0, 3, 5, 7, 9, 10]
    assert p["seg_slot"] == [1, 2, 3, 0, 4]
    assert p["class_ptr"] == [0, 5, 7, 10]
    assert p["tiles"] == [(0, 2, 0, 1), (2, 3, 0, 1), (3, 5, 0, 2), (5, 7, 1, -1), (7, 9, 2, -1), (9, 10, 2, -1)]
    assert p["oft_tiles"] == [(9, 10, 4)]


def test_plan_properties_random():
    rng = np.random.default_rng(13)
    for trial in range(50):
        ns = int(rng.integers(1, 12))
        cls = [2] + [int(c) for c in rng.integers(-1, 3, size=ns - 1)]
        n = int(rng.integers(0, 40))
        sor = rng.integers(-2, ns + 2, size=n).tolist()
        tr = int(rng.choice([1, 2, 4, 16]))
        p = oracle.plan(sor, cls, tile_rows=tr)
        assert sorted(p["perm"]) == list(range(n))
        keys = [((cls[p["row_slot"][i]] if p["row_slot"][i] else 2), p["row_slot"][i], i) for i in p["perm"]]
        assert keys == sorted(keys)
        covered = []
        for (a, b, kind, slot) in p["tiles"]:
            assert 0 < b - a <= tr
            covered.extend(range(a, b))
            if kind == 0:
                assert all(p["row_slot"][p["perm"][q]] == slot for q in range(a, b))
        assert sorted(covered) == list(range(n))
        bad = any(s < 0 or s >= ns or cls[s] < 0 for s in sor)
        assert p["invalid"] == int(bad)


# -------------------------------------------------------------- metrics ----

def test_parity_metrics_simple():
    y_ref = np.array([[3.0, 4.0], [1.0, 1.0]])
    xw = np.array([[0.0, 0.0], [1.0, 1.0]])      # row 2 has no effect
    y = y_ref + np.array([[0.03, 0.04], [0.5, 0.0]])
    m = oracle.parity_metrics(y, y_ref, xw, xw)
    assert m["rows_with_effect"] == 1
    assert abs(m["mean_rel"] - 0.01) < 1e-15
    assert m["max_abs"] == 0.5


# ------------------------------------------------- the pins catch mistakes -

def test_pins_detect_planted_mistakes(monkeypatch):
    """Plant plausible mistakes in the oracle (on the CPU) and check that a
    pin fails for each: the other Cayley convention, the DoRA norm over the
    wrong axis, a dropped c, a transposed shared factor, a stacked scale
    that skips the previous member's update."""
    gold = _load("hand_examples.json")
    x = np.array(gold["x"], dtype=np.float64)
    cases = {c["name"]: c for c in gold["cases"]}

    def run(name):
        c = cases[name]
        shared = _arr(c["shared"]) if "shared" in c else None
        got = oracle.direct_forward(x, np.array(c["W"], float), _arr(c["adapter"]), shared)
        return np.allclose(got, c["y"], atol=1e-12)

    assert all(run(n) for n in cases)
    # 1. Cayley convention flipped.
    orig_cayley = om.cayley
    monkeypatch.setattr(om, "cayley", lambda Q: orig_cayley(Q).T)
    assert not run("oft")
    monkeypatch.setattr(om, "cayley", orig_cayley)
    # 2. DoRA norm taken over d_out instead of d_in.
    orig_dforward = om.direct_forward

    def bad_dora(x_, W_, ad, shared=None):
        if ad["method"] == "dora":
            Wp = W_ + ad["c"] * ad["A"] @ ad["B"]
            return (x_ @ Wp) * (ad["m"] / np.sqrt(np.sum(Wp * Wp, axis=1)))
        return orig_dforward(x_, W_, ad, shared)
    monkeypatch.setattr(oracle, "direct_forward", bad_dora)
    assert not run("dora")
    # 3. LoRA without c.
    def bad_lora(x_, W_, ad, shared=None):
        if ad["method"] == "lora":
            return x_ @ W_ + (x_ @ ad["A"]) @ ad["B"]
        return orig_dforward(x_, W_, ad, shared)
    monkeypatch.setattr(oracle, "direct_forward", bad_lora)
    assert not run("lora")
    # 4. VeRA with the shared B transposed.
    def bad_vera(x_, W_, ad, shared=None):
        if ad["method"] == "vera":
            return x_ @ W_ + ad["c"] * ((((x_ @ shared["A"]) * ad["d"]) @ shared["B"].T) * ad["e"])
        return orig_dforward(x_, W_, ad, shared)
    monkeypatch.setattr(oracle, "direct_forward", bad_vera)
    assert not run("vera")
    monkeypatch.setattr(oracle, "direct_forward", orig_dforward)
    # 5. A stacked scale applied to the base output only, not to the
    #    previous member's update (the order would then not matter).
    st = gold["stacking"]
    W2 = np.array(st["W"], dtype=np.float64)
    rec = {"method": "stack", "members": [_arr(st["lora"]), _arr(st["ia3"])]}
    assert np.array_equal(om.direct_forward(x, W2, rec), st["ia3_after_lora"])
    orig_applied = om.applied_to

    def bad_applied(y_, x_, W_, ad, shared=None):
        if ad["method"] == "ia3":
            return (x_ @ W_) * ad["l"] + (y_ - x_ @ W_)
        return orig_applied(y_, x_, W_, ad, shared)
    monkeypatch.setattr(om, "applied_to", bad_applied)
    assert not np.array_equal(om.direct_forward(x, W2, rec), st["ia3_after_lora"])


# ------------------------------------------------------ stacked records ----

def _member(rng, meth, d_in, d_out, r=2, r_v=3, bs=2):
    if meth == "lora":
        return {"method": "lora", "A": rng.standard_normal((d_in, r)), "B": rng.standard_normal((r, d_out)), "c": 1.5}
    if meth == "dora":
        return {"method": "dora", "A": rng.standard_normal((d_in, r)), "B": rng.standard_normal((r, d_out)), "c": 0.5,
                "m": rng.uniform(1, 2, d_out)}
    if meth == "ia3":
        return {"method": "ia3", "l": rng.uniform(0.5, 1.5, d_out)}
    if meth == "ssf":
        return {"method": "ssf", "s": rng.uniform(0.5, 1.5, d_out), "b": rng.standard_normal(d_out)}
    if meth == "vera":
        return {"method": "vera", "d": rng.uniform(0.5, 1.5, r_v), "e": rng.uniform(0.5, 1.5, d_out), "c": 2.0}
    if meth == "oft":
        return {"method": "oft", "Q": _skew(rng, d_in // bs, bs)}
    return {"method": "identity"}


STACKABLE = ("identity", "lora", "dora", "ia3", "ssf", "vera")


@pytest.mark.parametrize("first", STACKABLE + ("oft",))
def test_stack_record_equals_the_appendix_closed_form(first):
    # Sequential application (each member's definition on the previous
    # output) equals eq. (1) with the appendix's composed slots, for every
    # pair and a triple: s1⊙s2, b1⊙s2 + b2, F1's terms times s2.
    rng = np.random.default_rng(21)
    d_in, d_out = 8, 6
    x = rng.standard_normal((5, d_in))
    W = rng.standard_normal((d_in, d_out))
    shared = {"A": rng.standard_normal((d_in, 3)), "B": rng.standard_normal((3, d_out))}
    for second in STACKABLE:
        for third in (None, "ia3", "lora"):
            members = [_member(rng, first, d_in, d_out), _member(rng, second, d_in, d_out)]
            if third:
                members.append(_member(rng, third, d_in, d_out))
            rec = {"method": "stack", "members": members}
            direct = om.direct_forward(x, W, rec, shared)
            slots = nf.unfolded_slots(rec, W, shared)
            composed = nf.normal_form_eval(x, W, slots)
            scale = np.max(np.abs(direct))
            np.testing.assert_allclose(direct, composed, rtol=0, atol=1e-12 * scale)
            # folded slots (what a loader stores) give the same output
            folded, _ = nf.fold(slots)
            np.testing.assert_allclose(nf.normal_form_eval(x, W, folded), direct, rtol=0, atol=1e-12 * scale)


def test_stack_record_hand_example():
    gold = _load("hand_examples.json")
    st = gold["stacking"]
    x = np.array(gold["x"], dtype=np.float64)
    W = np.array(st["W"], dtype=np.float64)
    lora, ia3 = _arr(st["lora"]), _arr(st["ia3"])
    np.testing.assert_array_equal(om.direct_forward(x, W, {"method": "stack", "members": [lora, ia3]}),
                                  st["ia3_after_lora"])
    np.testing.assert_array_equal(om.direct_forward(x, W, {"method": "stack", "members": [ia3, lora]}),
                                  st["lora_after_ia3"])


def test_stack_integer_inputs_exact():
    # Integer values keep every product exact in float64: SSF then LoRA then
    # (IA)3 must equal ((xW⊙s + b) + c(xA)B)⊙l written out by hand.
    rng = np.random.default_rng(5)
    d_in, d_out = 6, 4
    ri = lambda *s: rng.integers(-3, 4, size=s).astype(np.float64)
    x, W = ri(3, d_in), ri(d_in, d_out)
    ssf = {"method": "ssf", "s": ri(d_out), "b": ri(d_out)}
    lora = {"method": "lora", "A": ri(d_in, 2), "B": ri(2, d_out), "c": 2.0}
    ia3 = {"method": "ia3", "l": ri(d_out)}
    want = ((x @ W) * ssf["s"] + ssf["b"] + 2.0 * ((x @ lora["A"]) @ lora["B"])) * ia3["l"]
    got = om.direct_forward(x, W, {"method": "stack", "members": [ssf, lora, ia3]})
    np.testing.assert_array_equal(got, want)


def test_stack_input_transform_only_first():
    rng = np.random.default_rng(6)
    d_in, d_out = 4, 3
    x, W = rng.standard_normal((2, d_in)), rng.standard_normal((d_in, d_out))
    oft = _member(rng, "oft", d_in, d_out)
    ia3 = _member(rng, "ia3", d_in, d_out)
    R = om.oft_rotation(oft["Q"])
    got = om.direct_forward(x, W, {"method": "stack", "members": [oft, ia3]})
    np.testing.assert_allclose(got, ((x @ R) @ W) * ia3["l"], rtol=0, atol=1e-13)
    np.testing.assert_allclose(om.input_transform({"method": "stack", "members": [oft, ia3]}, d_in), R)
    with pytest.raises(ValueError):
        om.direct_forward(x, W, {"method": "stack", "members": [ia3, oft]})


# ------------------------------------------------------- LoHa and LoKr ----

def _loha(rng, d_in, d_out, r1=2, r2=3, c=0.75, ints=False):
    f = (lambda *s: rng.integers(-2, 3, size=s).astype(np.float64)) if ints else (lambda *s: rng.standard_normal(s))
    return {"method": "loha", "A": f(d_in, r1), "B": f(r1, d_out), "A2": f(d_in, r2), "B2": f(r2, d_out), "c": c}


def _lokr(rng, d_in, d_out, p=2, q=3, r=2, c=0.75, ints=False):
    f = (lambda *s: rng.integers(-2, 3, size=s).astype(np.float64)) if ints else (lambda *s: rng.standard_normal(s))
    return {"method": "lokr", "C": f(p, q), "A": f(d_in // p, r), "B": f(r, d_out // q), "c": c}


def _py_delta(ad, d_in, d_out):
    """Pure-Python ΔW by each method's elementwise definition."""
    c = ad["c"]
    if ad["method"] == "loha":
        A1, B1, A2, B2 = (ad[k].tolist() for k in ("A", "B", "A2", "B2"))
        return [[c * sum(A1[i][k] * B1[k][j] for k in range(len(B1))) *
                 sum(A2[i][l] * B2[l][j] for l in range(len(B2))) for j in range(d_out)] for i in range(d_in)]
    C, A, B = (ad[k].tolist() for k in ("C", "A", "B"))
    p2, q2 = len(A), len(B[0])
    return [[c * C[i // p2][j // q2] * sum(A[i % p2][k] * B[k][j % q2] for k in range(len(B)))
             for j in range(d_out)] for i in range(d_in)]


@pytest.mark.parametrize("meth,shape", [("loha", {}), ("lokr", dict(p=2, q=3)), ("lokr", dict(p=3, q=2)),
                                        ("lokr", dict(p=1, q=1))])
def test_product_methods_brute_force(meth, shape):
    rng = np.random.default_rng(31)
    d_in, d_out = 6, 6
    ad = _loha(rng, d_in, d_out) if meth == "loha" else _lokr(rng, d_in, d_out, **shape)
    x, W = rng.standard_normal((3, d_in)), rng.standard_normal((d_in, d_out))
    dW = np.array(_py_delta(ad, d_in, d_out))
    np.testing.assert_allclose(om.product_update(ad), dW, rtol=0, atol=1e-13)
    np.testing.assert_allclose(om.direct_forward(x, W, ad), x @ W + x @ dW, rtol=0, atol=1e-12)


@pytest.mark.parametrize("meth", ["loha", "lokr"])
def test_product_expansion_exact_and_rank(meth):
    # The load-time expansion into one low-rank term reproduces the update
    # exactly on integer inputs; its rank is r1·r2 (LoHa) or min(p, q)·r
    # (LoKr), above the adapter's own rank.
    rng = np.random.default_rng(32)
    d_in, d_out = 12, 12
    ad = _loha(rng, d_in, d_out, ints=True, c=2.0) if meth == "loha" else _lokr(rng, d_in, d_out, p=3, q=2, r=2,
                                                                              ints=True, c=2.0)
    x = rng.integers(-3, 4, size=(4, d_in)).astype(np.float64)
    W = rng.integers(-3, 4, size=(d_in, d_out)).astype(np.float64)
    A, B = nf.expand_product(ad)
    assert A.shape[1] == (6 if meth == "loha" else 4)
    direct = om.direct_forward(x, W, ad)
    np.testing.assert_array_equal(nf.normal_form_eval(x, W, nf.unfolded_slots(ad, W)), direct)
    folded, made = nf.fold(nf.unfolded_slots(ad, W))
    assert made == ["c->A"]
    np.testing.assert_array_equal(nf.normal_form_eval(x, W, folded), direct)
    g = np.random.default_rng(33)
    gen = _loha(g, d_in, d_out) if meth == "loha" else _lokr(g, d_in, d_out, p=3, q=2, r=2)
    assert np.linalg.matrix_rank(om.product_update(gen)) == A.shape[1]


def test_product_methods_reduce_to_lora():
    rng = np.random.default_rng(34)
    d_in, d_out = 8, 6
    x, W = rng.standard_normal((3, d_in)), rng.standard_normal((d_in, d_out))
    lora = {"method": "lora", "A": rng.standard_normal((d_in, 2)), "B": rng.standard_normal((2, d_out)), "c": 1.5}
    want = om.direct_forward(x, W, lora)
    loha = {"method": "loha", "A": lora["A"], "B": lora["B"], "A2": np.ones((d_in, 1)), "B2": np.ones((1, d_out)),
            "c": 1.5}
    lokr = {"method": "lokr", "C": np.ones((1, 1)), "A": lora["A"], "B": lora["B"], "c": 1.5}
    np.testing.assert_allclose(om.direct_forward(x, W, loha), want, rtol=0, atol=1e-13)
    np.testing.assert_allclose(om.direct_forward(x, W, lokr), want, rtol=0, atol=1e-13)
    # C = I: block-diagonal update, each block of d_in/p inputs feeds its own outputs
    eye = {"method": "lokr", "C": np.eye(2), "A": rng.standard_normal((4, 2)), "B": rng.standard_normal((2, 3)),
           "c": 1.0}
    D = eye["A"] @ eye["B"]
    blocks = np.concatenate([x[:, :4] @ D, x[:, 4:] @ D], axis=1)
    np.testing.assert_allclose(om.direct_forward(x, W, eye) - x @ W, blocks, rtol=0, atol=1e-13)


def test_dora_magnitude_recipe_is_the_expected_norm():
    """The input generator sets DoRA's magnitude to m = sqrt(1 + c²) ·
    (1 + 0.1 z), a constant of its draws and no norm of the drawn values
    (it does none of the method's arithmetic).  Replaying its seeded draws
    gives exactly that m; and sqrt(1 + c²) is the expected column norm of
    W + cAB under the draws (W ~ N(0, 1/d_in), A ~ N(0, 1/d_in),
    B ~ N(0, 1/r)): the mean of the oracle's squared column norms over
    1024 columns is 1 + c² within a few standard errors, so the scale the
    oracle derives from m stays near the drawn gain on average."""
    from workloads import synth
    for d_in, d_out, r, dt in ((64, 96, 4, "f16"), (1024, 1024, 16, "f32")):
        rng = np.random.default_rng(d_in + d_out)
        W = synth.round_to(synth._normal(rng, (d_out, d_in), 1.0 / np.sqrt(d_in)), dt)
        state = rng.bit_generator.state
        rec = synth._dora(rng, W, r, dt)
        rng2 = np.random.default_rng()
        rng2.bit_generator.state = state
        lo = synth._lora(rng2, d_in, d_out, r, dt)
        g = 1.0 + 0.1 * rng2.standard_normal(d_out)
        c = rec["c"]
        assert c == 2.0
        assert np.array_equal(lo["A"], rec["A"]) and np.array_equal(lo["B"], rec["B"])
        assert np.array_equal(rec["m"], (np.sqrt(1.0 + c * c) * g).astype(np.float32))
        if d_in < 1024:
            continue
        norm = oracle.dora_column_norm(W.T.astype(np.float64), rec["A"], rec["B"], c)
        assert abs(np.mean(norm ** 2) / (1.0 + c * c) - 1.0) < 0.04
        s = oracle.dora_scale(W.T.astype(np.float64), rec["A"], rec["B"], c, rec["m"])
        assert abs(np.mean(s / g) - 1.0) < 0.06

