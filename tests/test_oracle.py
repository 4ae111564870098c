"""Pins of the fp64 oracle against what the pages and the mathematics fix.

None of these tests re-types the oracle's loop.  Each checks the oracle
against a different statement of the method or a consequence of it:

* the lifted Widrow-Hoff form on a = k (x) v with an explicit generalised
  Householder transition (KronLSTM summary page, onedev.kr, section "how it
  differs");
* the exact non-expansiveness identity when beta |k|^2 |v|^2 = beta < 1 (same
  page, section "how it is used"), and for beta in (0, 2);
* immediate recall of the target after a step (section "how it works");
* capacity: orthogonal lifted features are stored exactly in one pass, one key
  can hold several orthogonal values; linearly independent features reach
  exact recall under repeated passes (section "how it differs");
* interference proportional to value overlap times key overlap (section
  "how it differs"; Figure 1 caption of the review of the same paper);
* closed forms: gated linear attention (beta = 0), causal linear attention
  (beta = 0, f = 1), NLMS (dv = 1, v = 1);
* split/resume through S0 -> S_T (bitwise);
* hand-worked fixtures under tests/golden/;
* gradients: central finite differences over every input element, and
  autograd of the lifted form.
"""
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_inputs(rng, B, T, H, dk, dv, unit=True, beta_range=(0.0, 1.0), f_range=(0.3, 1.0)):
    q = rng.standard_normal((B, T, H, dk))
    k = rng.standard_normal((B, T, H, dk))
    v = rng.standard_normal((B, T, H, dv))
    if unit:
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
        v /= np.linalg.norm(v, axis=-1, keepdims=True)
    f = rng.uniform(*f_range, (B, T, H, dk))
    beta = rng.uniform(*beta_range, (B, T, H))
    c = rng.uniform(-1.0, 1.0, (B, T, H))
    return q, k, v, f, beta, c


# ---------------------------------------------------------------- lifted form
def _lifted_forward(q, k, v, f, beta, c, S0):
    """x_t = (I - beta_t a_t a_t^T)(diag(f_t) (x) I_dv) x_{t-1} + c_t a_t,
    a_t = k_t (x) v_t, x = column-major vec(S); o_t = (q_t^T (x) I_dv) x_t."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    o = np.zeros((B, T, H, dv))
    ST = np.zeros((B, H, dv, dk))
    n = dk * dv
    for b in range(B):
        for h in range(H):
            x = S0[b, h].T.reshape(-1).copy()
            for t in range(T):
                a = np.kron(k[b, t, h], v[b, t, h])
                D = np.kron(np.diag(f[b, t, h]), np.eye(dv))
                A = np.eye(n) - beta[b, t, h] * np.outer(a, a)
                x = A @ (D @ x) + c[b, t, h] * a
                o[b, t, h] = np.kron(q[b, t, h][None, :], np.eye(dv)) @ x
            ST[b, h] = x.reshape(dk, dv).T
    return o, ST


@pytest.mark.parametrize("dk,dv", [(3, 5), (6, 4), (8, 8)])
def test_lifted_widrow_hoff_form(dk, dv):
    rng = np.random.default_rng(11 + dk)
    B, T, H = 1, 64, 2
    q, k, v, f, beta, c = _rand_inputs(rng, B, T, H, dk, dv, unit=False, beta_range=(0, 2))
    S0 = rng.standard_normal((B, H, dv, dk))
    o, ST, _ = oracle.fwd(q, k, v, f, beta, c, S0)
    o2, ST2 = _lifted_forward(q, k, v, f, beta, c, S0)
    scale = max(np.abs(o2).max(), 1.0)
    assert np.abs(o - o2).max() <= 1e-13 * scale
    assert np.abs(ST - ST2).max() <= 1e-13 * max(np.abs(ST2).max(), 1.0)


# ------------------------------------------------------ non-expansiveness
@pytest.mark.parametrize("beta_hi", [1.0, 2.0])
def test_non_expansive_identity(beta_hi):
    """Two runs from different S0 on the same unit-norm inputs.  Their
    difference D evolves by D_t = (I - beta a a^T)(F (x) I) D_{t-1}, so
    |D_t|^2 = |Dbar|^2 - beta (2 - beta) (v^T Dbar k)^2 with Dbar = D_{t-1} diag(f)."""
    rng = np.random.default_rng(5)
    dk, dv, T = 6, 5, 40
    q, k, v, f, beta, c = _rand_inputs(rng, 1, T, 1, dk, dv, unit=True, beta_range=(0.0, beta_hi))
    Sa = rng.standard_normal((1, 1, dv, dk))
    Sb = rng.standard_normal((1, 1, dv, dk))
    prev = np.linalg.norm(Sa - Sb)
    for t in range(T):
        sl = slice(t, t + 1)
        _, Sa_n, _ = oracle.fwd(q[:, sl], k[:, sl], v[:, sl], f[:, sl], beta[:, sl], c[:, sl], Sa)
        _, Sb_n, _ = oracle.fwd(q[:, sl], k[:, sl], v[:, sl], f[:, sl], beta[:, sl], c[:, sl], Sb)
        D = (Sa - Sb)[0, 0]
        Dbar = D * f[0, t, 0][None, :]
        proj = v[0, t, 0] @ Dbar @ k[0, t, 0]
        b = beta[0, t, 0]
        expect = np.sum(Dbar ** 2) - b * (2.0 - b) * proj ** 2
        got = np.sum((Sa_n - Sb_n) ** 2)
        # D is a difference of two O(1) states: its rounding error is
        # ~eps*|S|, so |D|^2 carries ~2|D| eps |S| absolute error.
        tol = 1e-12 * expect + 1e-14 * np.sqrt(expect) * (np.linalg.norm(Sa_n) + np.linalg.norm(Sb_n))
        assert abs(got - expect) <= tol
        now = np.sqrt(got)
        assert now <= prev * (1 + 1e-12)
        prev = now
        Sa, Sb = Sa_n, Sb_n


# ------------------------------------------------------ immediate recall
def test_immediate_recall_general_and_unit():
    """After step t: v_t^T S_t k_t = (1 - beta |a|^2) r_t + c_t |a|^2 with
    |a| = |k||v| and r_t = v_t^T S_{t-1} diag(f_t) k_t; for |a| = 1 and
    beta = 1 this is exactly c_t (the target)."""
    rng = np.random.default_rng(7)
    dk, dv, T = 5, 7, 30
    for unit, brange in ((False, (0, 2)), (True, (1.0, 1.0))):
        q, k, v, f, beta, c = _rand_inputs(rng, 1, T, 1, dk, dv, unit=unit, beta_range=brange)
        S = rng.standard_normal((1, 1, dv, dk))
        for t in range(T):
            sl = slice(t, t + 1)
            _, Sn, _ = oracle.fwd(q[:, sl], k[:, sl], v[:, sl], f[:, sl], beta[:, sl], c[:, sl], S)
            kt, vt = k[0, t, 0], v[0, t, 0]
            a2 = (kt @ kt) * (vt @ vt)
            r = vt @ (S[0, 0] * f[0, t, 0][None, :]) @ kt
            expect = (1 - beta[0, t, 0] * a2) * r + c[0, t, 0] * a2
            got = vt @ Sn[0, 0] @ kt
            assert abs(got - expect) <= 1e-13 * max(1.0, abs(expect))
            if unit:
                assert abs(got - c[0, t, 0]) <= 1e-14
            S = Sn


# ------------------------------------------------------ capacity / recall
def _orth(rng, n):
    Qm, _ = np.linalg.qr(rng.standard_normal((n, n)))
    return Qm


def test_capacity_orthogonal_pairs_one_pass():
    """f = 1, beta = 1: all dk*dv pairs of two orthonormal bases are stored
    exactly after one pass: v_b^T S_T k_a = c_ab for every pair."""
    rng = np.random.default_rng(3)
    dk, dv = 4, 3
    U, W = _orth(rng, dk), _orth(rng, dv)
    pairs = [(a, b) for a in range(dk) for b in range(dv)]
    rng.shuffle(pairs)
    T = len(pairs)
    k = np.stack([U[:, a] for a, _ in pairs])[None, :, None, :]
    v = np.stack([W[:, b] for _, b in pairs])[None, :, None, :]
    q = k.copy()
    f = np.ones_like(k)
    beta = np.ones((1, T, 1))
    c = rng.uniform(-2, 2, (1, T, 1))
    S0 = rng.standard_normal((1, 1, dv, dk))  # overwritten along every direction
    _, ST, _ = oracle.fwd(q, k, v, f, beta, c, S0)
    for idx, (a, b) in enumerate(pairs):
        assert abs(W[:, b] @ ST[0, 0] @ U[:, a] - c[0, idx, 0]) <= 1e-13


def test_capacity_one_key_many_values():
    rng = np.random.default_rng(4)
    dk, dv = 5, 6
    key = rng.standard_normal(dk)
    key /= np.linalg.norm(key)
    W = _orth(rng, dv)
    T = dv
    k = np.tile(key, (T, 1))[None, :, None, :]
    v = W.T[None, :, None, :]
    q = k.copy()
    f = np.ones_like(k)
    beta = np.ones((1, T, 1))
    c = rng.uniform(-1, 1, (1, T, 1))
    _, ST, _ = oracle.fwd(q, k, v, f, beta, c, None)
    for b in range(dv):
        assert abs(W[:, b] @ ST[0, 0] @ key - c[0, b, 0]) <= 1e-13


def test_capacity_linearly_independent_repeated_passes():
    """Non-orthogonal, linearly independent lifted features: one pass does not
    recall exactly, cyclic passes (Kaczmarz) converge to exact recall."""
    rng = np.random.default_rng(9)
    dk, dv, N = 3, 3, 6
    k = rng.standard_normal((N, dk))
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = rng.standard_normal((N, dv))
    v /= np.linalg.norm(v, axis=1, keepdims=True)
    A = np.stack([np.kron(k[i], v[i]) for i in range(N)])
    assert np.linalg.matrix_rank(A) == N
    c = rng.uniform(-1, 1, N)
    passes = 3000
    kk = np.tile(k, (passes, 1))[None, :, None, :]
    vv = np.tile(v, (passes, 1))[None, :, None, :]
    T = kk.shape[1]
    _, S1, _ = oracle.fwd(kk[:, :N], kk[:, :N], vv[:, :N], np.ones((1, N, 1, dk)),
                          np.ones((1, N, 1)), c[None, :, None], None)
    one_pass = max(abs(v[i] @ S1[0, 0] @ k[i] - c[i]) for i in range(N))
    assert one_pass > 1e-3
    _, ST, _ = oracle.fwd(kk, kk, vv, np.ones((1, T, 1, dk)), np.ones((1, T, 1)),
                          np.tile(c, passes)[None, :, None], None)
    resid = max(abs(v[i] @ ST[0, 0] @ k[i] - c[i]) for i in range(N))
    assert resid < 1e-10


# ------------------------------------------------------ interference
def test_interference_product_of_overlaps():
    """f = 1: a step changes another pair's association v_i^T S k_i by exactly
    u_t (v_i . v_t)(k_i . k_t), u_t = c_t - beta_t r_t; zero if either overlap is zero."""
    rng = np.random.default_rng(13)
    dk, dv = 6, 5
    S = rng.standard_normal((1, 1, dv, dk))
    kt = rng.standard_normal(dk); vt = rng.standard_normal(dv)
    qt = rng.standard_normal(dk)
    bt, ct = 0.7, 0.3
    _, Sn, r = oracle.fwd(qt[None, None, None], kt[None, None, None], vt[None, None, None],
                          np.ones((1, 1, 1, dk)), np.array([[[bt]]]), np.array([[[ct]]]), S)
    u = ct - bt * r[0, 0, 0]
    assert abs(r[0, 0, 0] - vt @ S[0, 0] @ kt) <= 1e-13
    for _ in range(20):
        ki = rng.standard_normal(dk); vi = rng.standard_normal(dv)
        delta = vi @ Sn[0, 0] @ ki - vi @ S[0, 0] @ ki
        assert abs(delta - u * (vi @ vt) * (ki @ kt)) <= 1e-13
    # value-orthogonal probe with overlapping key, and key-orthogonal probe
    vi = rng.standard_normal(dv); vi -= (vi @ vt) / (vt @ vt) * vt
    ki = kt + 0.1 * rng.standard_normal(dk)
    assert abs(vi @ Sn[0, 0] @ ki - vi @ S[0, 0] @ ki) <= 1e-13
    ki = rng.standard_normal(dk); ki -= (ki @ kt) / (kt @ kt) * kt
    vi = vt.copy()
    assert abs(vi @ Sn[0, 0] @ ki - vi @ S[0, 0] @ ki) <= 1e-13


# ------------------------------------------------------ closed forms
def test_beta_zero_is_gated_linear_attention():
    """beta = 0: o_t = S0 (gamma_t * q_t) + sum_{s<=t} c_s v_s ((k_s * gamma_t/gamma_s) . q_t)
    with gamma_t the cumulative product of f up to and including t."""
    rng = np.random.default_rng(17)
    B, T, H, dk, dv = 1, 37, 2, 5, 4
    q, k, v, f, beta, c = _rand_inputs(rng, B, T, H, dk, dv, unit=False)
    beta[:] = 0.0
    S0 = rng.standard_normal((B, H, dv, dk))
    o, ST, _ = oracle.fwd(q, k, v, f, beta, c, S0)
    for h in range(H):
        gam = np.cumprod(f[0, :, h], axis=0)  # [T, dk]
        for t in range(T):
            exp = S0[0, h] @ (gam[t] * q[0, t, h])
            for s in range(t + 1):
                exp = exp + c[0, s, h] * v[0, s, h] * np.sum(k[0, s, h] * gam[t] / gam[s] * q[0, t, h])
            assert np.abs(o[0, t, h] - exp).max() <= 1e-12 * max(1.0, np.abs(exp).max())
        expST = S0[0, h] * gam[-1][None, :] + sum(
            c[0, s, h] * np.outer(v[0, s, h], k[0, s, h] * gam[-1] / gam[s]) for s in range(T))
        assert np.abs(ST[0, h] - expST).max() <= 1e-12 * max(1.0, np.abs(expST).max())


def test_beta_zero_f_one_is_causal_linear_attention():
    rng = np.random.default_rng(19)
    B, T, H, dk, dv = 2, 50, 1, 6, 3
    q, k, v, f, beta, c = _rand_inputs(rng, B, T, H, dk, dv, unit=False)
    beta[:] = 0.0
    f[:] = 1.0
    o, _, _ = oracle.fwd(q, k, v, f, beta, c, None)
    for b in range(B):
        Q, K, V = q[b, :, 0], k[b, :, 0], v[b, :, 0]
        A = np.tril(Q @ K.T) * c[b, :, 0][None, :]
        assert np.abs(o[b, :, 0] - A @ V).max() <= 1e-12 * np.abs(A @ V).max()


def test_dv1_is_nlms():
    """dv = 1, v = 1, f = 1: the state is a row vector w and the rule is the
    normalised LMS filter w <- w + mu (d - w.x) x with step mu = beta and
    desired response d = c / beta for unit-norm inputs x = k."""
    rng = np.random.default_rng(23)
    dk, T = 7, 60
    k = rng.standard_normal((T, dk)); k /= np.linalg.norm(k, axis=1, keepdims=True)
    mu = rng.uniform(0.1, 1.0, T)
    d = rng.standard_normal(T)
    w = np.zeros(dk)
    preds = []
    for t in range(T):
        w = w + mu[t] * (d[t] - w @ k[t]) * k[t]
        preds.append(w @ k[t])
    o, ST, _ = oracle.fwd(k[None, :, None], k[None, :, None], np.ones((1, T, 1, 1)),
                          np.ones((1, T, 1, dk)), mu[None, :, None], (mu * d)[None, :, None], None)
    assert np.abs(ST[0, 0, 0] - w).max() <= 1e-13
    assert np.abs(o[0, :, 0, 0] - np.array(preds)).max() <= 1e-13


# ------------------------------------------------------ split / resume
def test_split_resume_bitwise():
    rng = np.random.default_rng(29)
    B, T, H, dk, dv = 2, 96, 3, 8, 6
    q, k, v, f, beta, c = _rand_inputs(rng, B, T, H, dk, dv, beta_range=(0, 2))
    S0 = rng.standard_normal((B, H, dv, dk))
    o, ST, _ = oracle.fwd(q, k, v, f, beta, c, S0)
    m = 41
    oa, Sm, _ = oracle.fwd(q[:, :m], k[:, :m], v[:, :m], f[:, :m], beta[:, :m], c[:, :m], S0)
    ob, ST2, _ = oracle.fwd(q[:, m:], k[:, m:], v[:, m:], f[:, m:], beta[:, m:], c[:, m:], Sm)
    assert np.array_equal(np.concatenate([oa, ob], axis=1), o)
    assert np.array_equal(ST2, ST)


def test_empty_sequence_returns_initial_state():
    rng = np.random.default_rng(31)
    S0 = rng.standard_normal((1, 2, 3, 4))
    z = np.zeros((1, 0, 2, 4))
    o, ST, _ = oracle.fwd(z, z, np.zeros((1, 0, 2, 3)), z, np.zeros((1, 0, 2)), np.zeros((1, 0, 2)), S0)
    assert o.shape == (1, 0, 2, 3)
    assert np.array_equal(ST, S0)


# ------------------------------------------------------ hand-worked fixtures
def _read_fixture(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, rest = line.split(":", 1)
            vals[key.strip()] = np.array([float(x) for x in rest.split()])
    return vals


def test_hand_worked_two_steps():
    g = _read_fixture("hand_worked_2x2.txt")
    T, d = 2, 2
    shp = (1, T, 1, d)
    o, ST, _ = oracle.fwd(g["q"].reshape(shp), g["k"].reshape(shp), g["v"].reshape(shp),
                          g["f"].reshape(shp), g["beta"].reshape(1, T, 1), g["c"].reshape(1, T, 1),
                          g["S0"].reshape(1, 1, d, d))
    assert np.abs(o.reshape(-1) - g["o"]).max() <= 1e-15
    assert np.abs(ST.reshape(-1) - g["ST"]).max() <= 1e-15


def test_hand_worked_scalar_gradient():
    g = _read_fixture("hand_worked_scalar_grad.txt")
    s = lambda x: x.reshape(1, 1, 1, 1)
    s3 = lambda x: x.reshape(1, 1, 1)
    o, ST, _ = oracle.fwd(s(g["q"]), s(g["k"]), s(g["v"]), s(g["f"]), s3(g["beta"]), s3(g["c"]), s(g["s"]))
    assert o.item() == g["o"].item() and ST.item() == g["ST"].item()
    gr = oracle.bwd(s(g["q"]), s(g["k"]), s(g["v"]), s(g["f"]), s3(g["beta"]), s3(g["c"]), s(g["s"]),
                    s(g["dO"]), None)
    for key in ("dq", "dk", "dv", "df", "dbeta", "dc", "dS0"):
        assert gr[key].item() == g[key].item(), key


# ------------------------------------------------------ gradients
def _loss(inp, dO, dST):
    o, ST, _ = oracle.fwd(inp["q"], inp["k"], inp["v"], inp["f"], inp["beta"], inp["c"], inp["S0"])
    return float(np.sum(o * dO) + np.sum(ST * dST))


def test_gradients_central_differences_every_element():
    rng = np.random.default_rng(37)
    B, T, H, dk, dv = 1, 64, 2, 8, 8
    q, k, v, f, beta, c = _rand_inputs(rng, B, T, H, dk, dv, beta_range=(0, 2), f_range=(0.6, 1.0))
    S0 = 0.3 * rng.standard_normal((B, H, dv, dk))
    dO = rng.standard_normal((B, T, H, dv))
    dST = rng.standard_normal((B, H, dv, dk))
    inp = dict(q=q, k=k, v=v, f=f, beta=beta, c=c, S0=S0)
    g = oracle.bwd(q, k, v, f, beta, c, S0, dO, dST)
    h = 1e-6
    names = dict(q="dq", k="dk", v="dv", f="df", beta="dbeta", c="dc", S0="dS0")
    for name, gname in names.items():
        base = inp[name]
        fd = np.zeros_like(base)
        flat = base.reshape(-1)
        for idx in range(flat.size):
            keep = flat[idx]
            flat[idx] = keep + h
            lp = _loss(inp, dO, dST)
            flat[idx] = keep - h
            lm = _loss(inp, dO, dST)
            flat[idx] = keep
            fd.reshape(-1)[idx] = (lp - lm) / (2 * h)
        err = np.abs(fd - g[gname]).max() / max(np.abs(g[gname]).max(), 1e-12)
        assert err <= 1e-7, (name, err)


def test_gradients_random_direction_vjp():
    rng = np.random.default_rng(41)
    B, T, H, dk, dv = 2, 130, 2, 5, 7  # two full 64-step segments and a ragged tail
    q, k, v, f, beta, c = _rand_inputs(rng, B, T, H, dk, dv, beta_range=(0, 2), f_range=(0.5, 1.0))
    S0 = 0.3 * rng.standard_normal((B, H, dv, dk))
    dO = rng.standard_normal((B, T, H, dv))
    dST = rng.standard_normal((B, H, dv, dk))
    inp = dict(q=q, k=k, v=v, f=f, beta=beta, c=c, S0=S0)
    g = oracle.bwd(q, k, v, f, beta, c, S0, dO, dST)
    names = dict(q="dq", k="dk", v="dv", f="df", beta="dbeta", c="dc", S0="dS0")
    dirs = {n: rng.standard_normal(inp[n].shape) for n in names}
    eps = 1e-6
    plus = {n: inp[n] + eps * dirs[n] for n in names}
    minus = {n: inp[n] - eps * dirs[n] for n in names}
    fd = (_loss(plus, dO, dST) - _loss(minus, dO, dST)) / (2 * eps)
    an = sum(np.sum(g[names[n]] * dirs[n]) for n in names)
    assert abs(fd - an) <= 1e-7 * max(1.0, abs(an))


def test_gradients_match_autograd_of_lifted_form():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(43)
    B, T, H, dk, dv = 1, 20, 2, 3, 4
    q, k, v, f, beta, c = _rand_inputs(rng, B, T, H, dk, dv, unit=False, beta_range=(0, 2))
    S0 = rng.standard_normal((B, H, dv, dk))
    dO = rng.standard_normal((B, T, H, dv))
    dST = rng.standard_normal((B, H, dv, dk))
    tens = {n: torch.tensor(x, dtype=torch.float64, requires_grad=True)
            for n, x in dict(q=q, k=k, v=v, f=f, beta=beta, c=c, S0=S0).items()}
    n = dk * dv
    loss = 0.0
    for h in range(H):
        x = tens["S0"][0, h].T.reshape(-1)
        for t in range(T):
            a = torch.kron(tens["k"][0, t, h], tens["v"][0, t, h])
            D = torch.kron(torch.diag(tens["f"][0, t, h]), torch.eye(dv, dtype=torch.float64))
            A = torch.eye(n, dtype=torch.float64) - tens["beta"][0, t, h] * torch.outer(a, a)
            x = A @ (D @ x) + tens["c"][0, t, h] * a
            ot = torch.kron(tens["q"][0, t, h][None, :], torch.eye(dv, dtype=torch.float64)) @ x
            loss = loss + (ot * torch.tensor(dO[0, t, h])).sum()
        loss = loss + (x.reshape(dk, dv).T * torch.tensor(dST[0, h])).sum()
    loss.backward()
    g = oracle.bwd(q, k, v, f, beta, c, S0, dO, dST)
    names = dict(q="dq", k="dk", v="dv", f="df", beta="dbeta", c="dc", S0="dS0")
    for name, gname in names.items():
        ref = tens[name].grad.numpy()
        assert np.abs(ref - g[gname]).max() <= 1e-12 * max(1.0, np.abs(ref).max()), name
