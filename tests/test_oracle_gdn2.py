"""Pins of the Gated Delta Rule-2 oracle (oracle.gdn2_fwd) against what the
aitrends.kr Gated DeltaNet-2 summary fixes (sections 핵심 기여 and 방법론)
and against the mathematics of the rule:

* the page's product form (I - k e^T) D S + k z^T, iterated with plain matrix
  algebra, equals the oracle's decay / erase-write loop;
* a hand-worked 2x2 example (tests/golden/gdn2_hand_worked.txt);
* with b = w = 0 the rule is pure decay: closed form diag(prod alpha) S0;
* with alpha = 1, b = w = 1 and orthonormal keys every pair is recalled
  exactly, immediately and after all later writes;
* with w = 0, b = 1, alpha = 1 and a unit key, the key's direction is erased;
* running a sequence in two pieces, the state carried, equals one run.
"""
import os

import numpy as np
import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


def rand_inputs(rng, B, T, H, dk, dv):
    q = rng.standard_normal((B, T, H, dk))
    k = rng.standard_normal((B, T, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, dv))
    a = rng.uniform(0.6, 1.0, (B, T, H, dk))
    b = rng.uniform(0.0, 1.0, (B, T, H, dk))
    w = rng.uniform(0.0, 1.0, (B, T, H, dv))
    S0 = rng.standard_normal((B, H, dk, dv)) * 0.3
    return q, k, v, a, b, w, S0


def test_hand_worked_fixture():
    rows = {}
    for line in open(os.path.join(HERE, "golden", "gdn2_hand_worked.txt")):
        if line.strip() and not line.startswith("#"):
            name, *vals = line.split()
            rows[name] = np.array([float(x) for x in vals])
    shp = (1, 2, 1, 2)
    o, ST = oracle.gdn2_fwd(rows["q"].reshape(shp), rows["k"].reshape(shp), rows["v"].reshape(shp),
                            rows["alpha"].reshape(shp), rows["b"].reshape(shp), rows["w"].reshape(shp))
    assert np.array_equal(o.reshape(-1), rows["o"])
    assert np.array_equal(ST.reshape(-1), rows["ST"])


def test_product_form_of_the_page():
    rng = np.random.default_rng(11)
    B, T, H, dk, dv = 2, 9, 3, 5, 4
    q, k, v, a, b, w, S0 = rand_inputs(rng, B, T, H, dk, dv)
    o, ST = oracle.gdn2_fwd(q, k, v, a, b, w, S0)
    for bb in range(B):
        for h in range(H):
            S = S0[bb, h].copy()
            for t in range(T):
                kt, e, z = k[bb, t, h], b[bb, t, h] * k[bb, t, h], w[bb, t, h] * v[bb, t, h]
                S = (np.eye(dk) - np.outer(kt, e)) @ np.diag(a[bb, t, h]) @ S + np.outer(kt, z)
                np.testing.assert_allclose(o[bb, t, h], S.T @ q[bb, t, h], rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(ST[bb, h], S, rtol=1e-12, atol=1e-12)


def test_decay_only_closed_form():
    rng = np.random.default_rng(12)
    B, T, H, dk, dv = 1, 20, 2, 6, 3
    q, k, v, a, b, w, S0 = rand_inputs(rng, B, T, H, dk, dv)
    o, ST = oracle.gdn2_fwd(q, k, v, a, np.zeros_like(b), np.zeros_like(w), S0)
    for h in range(H):
        g = np.ones(dk)
        for t in range(T):
            g = g * a[0, t, h]
            np.testing.assert_allclose(o[0, t, h], (g[:, None] * S0[0, h]).T @ q[0, t, h], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(ST[0, h], g[:, None] * S0[0, h], rtol=1e-12, atol=1e-14)


def test_exact_recall_with_orthonormal_keys():
    rng = np.random.default_rng(13)
    dk, dv, T = 8, 5, 6
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    k = Qm[:, :T].T.reshape(1, T, 1, dk)          # orthonormal keys
    v = rng.standard_normal((1, T, 1, dv))
    ones_k, ones_v = np.ones((1, T, 1, dk)), np.ones((1, T, 1, dv))
    S0 = rng.standard_normal((1, 1, dk, dv))
    o, ST = oracle.gdn2_fwd(k, k, v, ones_k, ones_k, ones_v, S0)   # query with the key itself
    np.testing.assert_allclose(o[0, :, 0], v[0, :, 0], rtol=0, atol=1e-12)   # immediate recall
    for i in range(T):                                               # recall after all writes
        np.testing.assert_allclose(ST[0, 0].T @ k[0, i, 0], v[0, i, 0], rtol=0, atol=1e-12)


def test_erase_only_wipes_the_key_direction():
    rng = np.random.default_rng(14)
    dk, dv = 6, 4
    k = rng.standard_normal((1, 1, 1, dk))
    k /= np.linalg.norm(k)
    S0 = rng.standard_normal((1, 1, dk, dv))
    q = rng.standard_normal((1, 1, 1, dk))
    o, ST = oracle.gdn2_fwd(q, k, rng.standard_normal((1, 1, 1, dv)), np.ones_like(k), np.ones_like(k),
                            np.zeros((1, 1, 1, dv)), S0)
    np.testing.assert_allclose(k[0, 0, 0] @ ST[0, 0], np.zeros(dv), atol=1e-13)
    # everything orthogonal to k is untouched
    P = np.eye(dk) - np.outer(k[0, 0, 0], k[0, 0, 0])
    np.testing.assert_allclose(P @ ST[0, 0], P @ S0[0, 0], atol=1e-13)


@pytest.mark.parametrize("T1", [0, 1, 7, 13])
def test_split_and_resume(T1):
    rng = np.random.default_rng(15)
    B, T, H, dk, dv = 2, 13, 2, 4, 3
    q, k, v, a, b, w, S0 = rand_inputs(rng, B, T, H, dk, dv)
    o, ST = oracle.gdn2_fwd(q, k, v, a, b, w, S0)
    sl = lambda x, lo, hi: x[:, lo:hi]
    o1, S1 = oracle.gdn2_fwd(*(sl(x, 0, T1) for x in (q, k, v, a, b, w)), S0)
    o2, S2 = oracle.gdn2_fwd(*(sl(x, T1, T) for x in (q, k, v, a, b, w)), S1)
    np.testing.assert_allclose(np.concatenate([o1, o2], axis=1), o, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(S2, ST, rtol=1e-13, atol=1e-13)
