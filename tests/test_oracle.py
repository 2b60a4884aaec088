"""Pins for the CPU float64 oracle (no GPU needed).

Each check ties the oracle to something other than itself: hand-derived
closed forms (tests/golden), a 50-digit mpmath brute force of the
definition, central finite differences of the loss L = sum(dO * O), and
invariants the mathematics fixes.  The mutation tests at the end plant
plausible mistakes in copies of the oracle and require that some pin fails.
"""
import json
import math
import os
import types

import mpmath
import numpy as np
import pytest

import oracle
from oracle import attention as OA

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_softmax_cases.json")


def rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def rand_case(B, Hq, Hkv, Sq, Skv, D, seed):
    r = np.random.default_rng(seed)
    return (r.standard_normal((B, Hq, Sq, D)), r.standard_normal((B, Hkv, Skv, D)),
            r.standard_normal((B, Hkv, Skv, D)), r.standard_normal((B, Hq, Sq, D)))


REAL = types.SimpleNamespace(fwd=OA.attention_forward, bwd=OA.attention_backward)

# (B, Hq, Hkv, Sq, Skv, D, causal)
SHAPES = [
    (2, 4, 2, 5, 7, 3, False),
    (2, 4, 2, 5, 7, 3, True),
    (1, 2, 1, 4, 9, 3, True),
    (1, 2, 2, 6, 6, 4, True),
    (1, 3, 1, 3, 3, 2, False),
]


# ---------------------------------------------------------------- check functions
def check_golden(impl):
    with open(GOLDEN) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        q, k, v, do = (np.array(c[n], dtype=np.float64) for n in ("q", "k", "v", "do"))
        o, lse = impl.fwd(q, k, v, c["causal"], c["scale"])
        dq, dk, dv, _ = impl.bwd(q, k, v, do, c["causal"], c["scale"])
        for name, got in (("o", o), ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv)):
            np.testing.assert_allclose(got, np.array(c[name]), rtol=0, atol=1e-14,
                                       err_msg=f"{c['name']}:{name}")


def _mp_forward(q, k, v, causal, scale):
    """50-digit brute force of the definition: plain loops over every index."""
    mpmath.mp.dps = 50
    B, Hq, Sq, D = q.shape
    Hkv, Skv = k.shape[1], k.shape[2]
    G = Hq // Hkv
    o = np.zeros(q.shape[:3] + (v.shape[3],))
    lse = np.zeros(q.shape[:3])
    for b in range(B):
        for h in range(Hq):
            kv = h // G
            for i in range(Sq):
                sc = []
                for j in range(Skv):
                    if causal and j > i + Skv - Sq:
                        continue
                    acc = mpmath.mpf(0)
                    for d in range(D):
                        acc += mpmath.mpf(q[b, h, i, d]) * mpmath.mpf(k[b, kv, j, d])
                    sc.append((j, mpmath.mpf(scale) * acc))
                den = mpmath.fsum(mpmath.exp(s) for _, s in sc)
                lse[b, h, i] = float(mpmath.log(den))
                for d in range(v.shape[3]):
                    num = mpmath.fsum(mpmath.exp(s) * mpmath.mpf(v[b, kv, j, d]) for j, s in sc)
                    o[b, h, i, d] = float(num / den)
    return o, lse


def check_mpmath(impl):
    for n, (B, Hq, Hkv, Sq, Skv, D, causal) in enumerate(
            [(1, 1, 1, 3, 4, 2, False), (1, 2, 1, 3, 4, 2, True), (1, 2, 2, 4, 3, 3, False)]):
        q, k, v, _ = rand_case(B, Hq, Hkv, Sq, Skv, D, 100 + n)
        o, lse = impl.fwd(q, k, v, causal, 0.7)
        mo, mlse = _mp_forward(q, k, v, causal, 0.7)
        np.testing.assert_allclose(o, mo, rtol=0, atol=1e-14)
        np.testing.assert_allclose(lse, mlse, rtol=0, atol=1e-14)


def check_finite_differences(impl, shapes=SHAPES, h=1e-6):
    for n, (B, Hq, Hkv, Sq, Skv, D, causal) in enumerate(shapes):
        q, k, v, do = rand_case(B, Hq, Hkv, Sq, Skv, D, 200 + n)
        scale = 0.6
        dq, dk, dv, _ = impl.bwd(q, k, v, do, causal, scale)

        def loss(qq, kk, vv):
            o, _ = impl.fwd(qq, kk, vv, causal, scale)
            return float(np.sum(do * o))

        for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
            fd = np.zeros_like(x)
            it = np.nditer(x, flags=["multi_index"])
            for _ in it:
                idx = it.multi_index
                xp = x.copy(); xp[idx] += h
                xm = x.copy(); xm[idx] -= h
                ap = {"q": q, "k": k, "v": v}
                ap[name] = xp
                am = {"q": q, "k": k, "v": v}
                am[name] = xm
                fd[idx] = (loss(ap["q"], ap["k"], ap["v"]) - loss(am["q"], am["k"], am["v"])) / (2 * h)
            err = np.abs(fd - g) / (1 + np.abs(g))
            assert err.max() <= 1e-7, f"FD mismatch d{name} shape {(B, Hq, Hkv, Sq, Skv, D, causal)}: {err.max()}"


def check_row_sums(impl_probs):
    for causal in (False, True):
        q, k = rand((7, 4), 1), rand((9, 4), 2)
        p, _ = impl_probs(q, k, causal, 0.8)
        np.testing.assert_allclose(p.sum(1), 1.0, rtol=0, atol=1e-14 * 9)
        assert (p >= 0).all()
        vis = OA.visible(np.arange(7), 7, 9, causal)
        assert (p[~vis] == 0).all()


def check_kv_permutation(impl):
    q, k, v, do = rand_case(2, 4, 2, 5, 8, 3, 7)
    perm = np.random.default_rng(3).permutation(8)
    o, lse = impl.fwd(q, k, v, False, 0.5)
    dq, dk, dv, _ = impl.bwd(q, k, v, do, False, 0.5)
    o2, lse2 = impl.fwd(q, k[:, :, perm], v[:, :, perm], False, 0.5)
    dq2, dk2, dv2, _ = impl.bwd(q, k[:, :, perm], v[:, :, perm], do, False, 0.5)
    for a, b in ((o, o2), (lse, lse2), (dq, dq2), (dk[:, :, perm], dk2), (dv[:, :, perm], dv2)):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)


def check_constant_v(impl):
    for causal in (False, True):
        q, k, _, do = rand_case(1, 2, 1, 6, 6, 3, 11)
        c = np.array([0.5, -2.0, 3.0])
        v = np.broadcast_to(c, (1, 1, 6, 3)).copy()
        o, _ = impl.fwd(q, k, v, causal, 0.9)
        dq, dk, _, _ = impl.bwd(q, k, v, do, causal, 0.9)
        np.testing.assert_allclose(o, np.broadcast_to(c, o.shape), rtol=0, atol=1e-12)
        np.testing.assert_allclose(dq, 0, atol=1e-12)
        np.testing.assert_allclose(dk, 0, atol=1e-12)


def check_gqa_vs_repeat(impl):
    for causal in (False, True):
        G = 3
        q, k, v, do = rand_case(2, 6, 2, 5, 7, 4, 13)
        kr, vr = np.repeat(k, G, axis=1), np.repeat(v, G, axis=1)  # head h -> kv h // G
        o, lse = impl.fwd(q, k, v, causal, 0.4)
        o2, lse2 = impl.fwd(q, kr, vr, causal, 0.4)
        dq, dk, dv, _ = impl.bwd(q, k, v, do, causal, 0.4)
        dq2, dk2, dv2, _ = impl.bwd(q, kr, vr, do, causal, 0.4)
        np.testing.assert_allclose(o, o2, rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse, lse2, rtol=0, atol=1e-13)
        np.testing.assert_allclose(dq, dq2, rtol=0, atol=1e-13)
        np.testing.assert_allclose(dk, dk2.reshape(2, 2, G, 7, 4).sum(2), rtol=0, atol=1e-13)
        np.testing.assert_allclose(dv, dv2.reshape(2, 2, G, 7, 4).sum(2), rtol=0, atol=1e-13)


def check_closed_forms(impl):
    # one key: O = v0, LSE = scale*q.k0, dQ = dK = 0, dV0 = sum_i dO_i
    q, k, v, do = rand_case(1, 2, 2, 4, 1, 3, 17)
    o, lse = impl.fwd(q, k, v, False, 0.3)
    dq, dk, dv, _ = impl.bwd(q, k, v, do, False, 0.3)
    np.testing.assert_allclose(o, np.broadcast_to(v, o.shape), atol=1e-13)
    np.testing.assert_allclose(lse, 0.3 * np.einsum("bhid,bhd->bhi", q, k[:, :, 0]), atol=1e-13)
    np.testing.assert_allclose(dq, 0, atol=1e-13)
    np.testing.assert_allclose(dk, 0, atol=1e-13)
    np.testing.assert_allclose(dv[:, :, 0], do.sum(2), atol=1e-13)
    # zero queries: O_i is the mean of the visible V rows, LSE_i = ln(#visible)
    for causal in (False, True):
        _, k, v, _ = rand_case(1, 1, 1, 4, 6, 3, 19)
        q = np.zeros((1, 1, 4, 3))
        o, lse = impl.fwd(q, k, v, causal, 1.0)
        for i in range(4):
            nvis = 6 if not causal else i + 2 + 1
            np.testing.assert_allclose(o[0, 0, i], v[0, 0, :nvis].mean(0), atol=1e-13)
            np.testing.assert_allclose(lse[0, 0, i], math.log(nvis), atol=1e-13)
    # causal with Sq == Skv: the first query sees only the first key
    q, k, v, _ = rand_case(1, 1, 1, 5, 5, 3, 23)
    o, _ = impl.fwd(q, k, v, True, 0.7)
    np.testing.assert_allclose(o[0, 0, 0], v[0, 0, 0], atol=1e-14)


def check_sum_invariants(impl):
    for causal in (False, True):
        q, k, v, do = rand_case(2, 4, 2, 5, 7, 3, 29)
        dq, dk, dv, _ = impl.bwd(q, k, v, do, causal, 0.5)
        np.testing.assert_allclose(dk.sum(2), 0, atol=1e-12)
        np.testing.assert_allclose(dv.sum(2), do.reshape(2, 2, 2, 5, 3).sum((2, 3)), atol=1e-12)


def check_key_translation(impl):
    q, k, v, do = rand_case(1, 2, 1, 5, 6, 3, 31)
    c = np.array([0.3, -1.1, 0.7])
    o, lse = impl.fwd(q, k, v, False, 0.5)
    o2, lse2 = impl.fwd(q, k + c, v, False, 0.5)
    g = impl.bwd(q, k, v, do, False, 0.5)
    g2 = impl.bwd(q, k + c, v, do, False, 0.5)
    np.testing.assert_allclose(o, o2, atol=1e-12)
    np.testing.assert_allclose(lse2 - lse, 0.5 * (q @ c), atol=1e-12)
    for a, b in zip(g[:3], g2[:3]):
        np.testing.assert_allclose(a, b, atol=1e-12)


def check_decode_equivalence(impl):
    # Causal row i equals non-causal attention of q_i over keys 0..i+(Skv-Sq).
    for Sq, Skv in ((6, 6), (3, 8)):
        q, k, v, _ = rand_case(1, 1, 1, Sq, Skv, 4, 37)
        o, lse = impl.fwd(q, k, v, True, 0.6)
        for i in range(Sq):
            last = i + Skv - Sq
            oi, li = impl.fwd(q[:, :, i:i + 1], k[:, :, :last + 1], v[:, :, :last + 1], False, 0.6)
            np.testing.assert_allclose(o[0, 0, i], oi[0, 0, 0], atol=1e-14)
            np.testing.assert_allclose(lse[0, 0, i], li[0, 0, 0], atol=1e-14)


def check_dlt_identity(impl_bwd_head):
    q, k, v, do = rand((5, 3), 41), rand((7, 3), 42), rand((7, 3), 43), rand((5, 3), 44)
    for causal in (False, True):
        _, _, _, dlt = impl_bwd_head(q, k, v, do, causal, 0.5)
        p, _ = OA.probs_head(q, k, causal, 0.5)
        np.testing.assert_allclose(dlt, (p * (do @ v.T)).sum(1), atol=1e-12)


# ---------------------------------------------------------------- the pins on the real oracle
def test_golden_hand_cases():
    check_golden(REAL)


def test_mpmath_brute_force():
    check_mpmath(REAL)


def test_finite_differences():
    check_finite_differences(REAL)


def test_probability_rows():
    check_row_sums(OA.probs_head)


def test_kv_permutation_invariance():
    check_kv_permutation(REAL)


def test_constant_v():
    check_constant_v(REAL)


def test_gqa_equals_repeated_mha():
    check_gqa_vs_repeat(REAL)


def test_closed_forms():
    check_closed_forms(REAL)


def test_gradient_sum_invariants():
    check_sum_invariants(REAL)


def test_key_translation():
    check_key_translation(REAL)


def test_decode_row_equivalence():
    check_decode_equivalence(REAL)


def test_dlt_identity():
    check_dlt_identity(OA.backward_head)


def test_fully_masked_rows():
    # causal with Sq > Skv leaves the first Sq-Skv rows without any key
    q, k, v, do = rand_case(1, 1, 1, 5, 3, 2, 47)
    o, lse = OA.attention_forward(q, k, v, True, 1.0)
    dq, dk, dv, _ = OA.attention_backward(q, k, v, do, True, 1.0)
    assert np.all(o[0, 0, :2] == 0) and np.all(np.isneginf(lse[0, 0, :2]))
    assert np.all(dq[0, 0, :2] == 0)
    assert np.isfinite(dk).all() and np.isfinite(dv).all()


def test_dq_rows_matches_full():
    q, k, v, do = rand((9, 4), 51), rand((11, 4), 52), rand((11, 4), 53), rand((9, 4), 54)
    for causal in (False, True):
        dq, _, _, _ = OA.backward_head(q, k, v, do, causal, 0.5)
        rows = [0, 3, 8]
        np.testing.assert_allclose(OA.dq_rows(q, k, v, do, causal, 0.5, rows), dq[rows], atol=1e-13)


def test_forward_head_row_sampling():
    q, k, v = rand((2100, 4), 61), rand((50, 4), 62), rand((50, 4), 63)
    o, lse = OA.forward_head(q, k, v, False, 0.5)
    rows = [0, 1023, 1024, 2099]
    o2, lse2 = OA.forward_head(q, k, v, False, 0.5, rows)
    np.testing.assert_array_equal(o[rows], o2)
    np.testing.assert_array_equal(lse[rows], lse2)


# ---------------------------------------------------------------- planted mistakes must be caught
def _mutant_bwd(kind):
    def bwd_head(q, k, v, do, causal, scale):
        q, k, v, do = (np.asarray(a, dtype=np.float64) for a in (q, k, v, do))
        p, _ = OA.probs_head(q, k, causal, scale)
        o = p @ v
        dlt = np.sum(do * o, axis=1)
        dp = do @ v.T
        if kind == "drop_dlt":
            ds = p * dp
        elif kind == "sign":
            ds = p * (dlt[:, None] - dp)
        else:
            ds = p * (dp - dlt[:, None])
        dq = (1.0 if kind == "dq_no_scale" else scale) * (ds @ k)
        dk = scale * (ds.T @ q)
        dv = (p @ do[: p.shape[1]] if kind == "dv_transposed" and p.shape[0] == p.shape[1]
              else p.T @ do)
        return dq, dk, dv, dlt
    return bwd_head


@pytest.mark.parametrize("kind", ["drop_dlt", "sign", "dq_no_scale", "dv_transposed"])
def test_pins_catch_backward_mutants(kind, monkeypatch):
    monkeypatch.setattr(OA, "backward_head", _mutant_bwd(kind))
    impl = types.SimpleNamespace(fwd=OA.attention_forward, bwd=OA.attention_backward)
    shapes = [(1, 2, 2, 6, 6, 4, True), (1, 2, 1, 4, 4, 3, False)]
    with pytest.raises(AssertionError):
        check_finite_differences(impl, shapes)


def test_pins_catch_topleft_causal(monkeypatch):
    def topleft(rows, Sq, Skv, causal):
        rows = np.asarray(rows)
        if not causal:
            return np.ones((rows.shape[0], Skv), dtype=bool)
        return np.arange(Skv)[None, :] <= rows[:, None]
    monkeypatch.setattr(OA, "visible", topleft)
    with pytest.raises(AssertionError):
        check_mpmath(REAL)


def test_pins_catch_modulo_head_map():
    def fwd(q, k, v, causal, scale):
        B, Hq, Sq, D = q.shape
        Hkv = k.shape[1]
        o = np.zeros(q.shape[:3] + (v.shape[3],)); lse = np.zeros(q.shape[:3])
        for b in range(B):
            for h in range(Hq):
                o[b, h], lse[b, h] = OA.forward_head(q[b, h], k[b, h % Hkv], v[b, h % Hkv], causal, scale)
        return o, lse
    with pytest.raises(AssertionError):
        check_gqa_vs_repeat(types.SimpleNamespace(fwd=fwd, bwd=OA.attention_backward))


def test_pins_catch_log2_lse(monkeypatch):
    real = OA.probs_head

    def probs_log2(q, k, causal, scale, rows=None):
        p, lse = real(q, k, causal, scale, rows)
        return p, lse / math.log(2)
    monkeypatch.setattr(OA, "probs_head", probs_log2)
    with pytest.raises(AssertionError):
        check_golden(REAL)


def test_pins_catch_missing_scale_in_scores(monkeypatch):
    real = OA.probs_head

    def probs_noscale(q, k, causal, scale, rows=None):
        return real(q, k, causal, 1.0, rows)
    monkeypatch.setattr(OA, "probs_head", probs_noscale)
    with pytest.raises(AssertionError):
        check_mpmath(REAL)
