"""Pins of the mixer pre/post oracle (oracle/mixer.py) against the
definitions the KronLSTM summary page (onedev.kr, section "어떻게 쓰나")
names and against library routines:

* the causal depthwise convolution equals numpy.convolve of each channel with
  its reversed taps (first T outputs), is causal, reduces to the identity for
  a single unit tap, and matches a hand-worked example;
* sigmoid and SiLU agree with scipy.special.expit;
* L2 normalisation gives unit rows up to its eps, keeps directions and is
  scale invariant, and matches a hand-worked example;
* the forget gate is the sigmoid for a_log = 0 and follows
  log f = exp(a_log) log sigmoid(x);
* the gated RMSNorm has unit mean square for a unit weight and an open gate,
  is scale invariant, halves at a zero gate logit, and matches a hand-worked
  example;
* the whole pre-processing makes every update non-expansive, beta |k|^2 |v|^2
  < 1 (same page and section), and with identity settings reduces to the
  plain rule on L2-normalised SiLU inputs.
"""
import os

import numpy as np
import pytest
from scipy.special import expit

import oracle
from oracle import mixer as mx

HERE = os.path.dirname(os.path.abspath(__file__))


def golden():
    rows = {}
    for line in open(os.path.join(HERE, "golden", "mixer_hand_worked.txt")):
        if line.strip() and not line.startswith("#"):
            name, *vals = line.split()
            rows[name] = np.array([float(x) for x in vals])
    return rows


def test_conv_hand_worked():
    g = golden()
    T, K = len(g["conv_x"]), len(g["conv_w"])
    y = mx.causal_depthwise_conv(g["conv_x"].reshape(1, T, 1, 1), g["conv_w"].reshape(1, 1, K))
    assert np.array_equal(y.reshape(-1), g["conv_y"])


@pytest.mark.parametrize("K", [1, 2, 4, 7])
def test_conv_is_numpy_convolve_per_channel(K):
    rng = np.random.default_rng(30 + K)
    B, T, H, d = 2, 13, 3, 5
    x = rng.standard_normal((B, T, H, d))
    w = rng.standard_normal((H, d, K))
    y = mx.causal_depthwise_conv(x, w)
    for b in range(B):
        for h in range(H):
            for i in range(d):
                ref = np.convolve(x[b, :, h, i], w[h, i, ::-1])[:T]
                np.testing.assert_allclose(y[b, :, h, i], ref, rtol=1e-13, atol=1e-13)


def test_conv_is_causal_and_identity_for_one_unit_tap():
    rng = np.random.default_rng(40)
    x = rng.standard_normal((1, 20, 2, 4))
    w = rng.standard_normal((2, 4, 4))
    y = mx.causal_depthwise_conv(x, w)
    x2 = x.copy()
    x2[:, 9] += 1.0
    y2 = mx.causal_depthwise_conv(x2, w)
    assert np.array_equal(y[:, :9], y2[:, :9])
    assert not np.any(y[:, 9:13] == y2[:, 9:13])
    assert np.array_equal(y[:, 13:], y2[:, 13:])
    e = np.zeros((2, 4, 4))
    e[..., 3] = 1.0            # the tap on the current token
    assert np.array_equal(mx.causal_depthwise_conv(x, e), x)


def test_sigmoid_and_silu_against_expit():
    x = np.linspace(-30, 30, 601)
    np.testing.assert_allclose(mx.sigmoid(x), expit(x), rtol=1e-15, atol=1e-300)
    np.testing.assert_allclose(mx.silu(x), x * expit(x), rtol=1e-15, atol=1e-300)
    assert mx.silu(0.0) == 0.0 and mx.sigmoid(0.0) == 0.5


def test_l2_normalise():
    g = golden()
    assert np.array_equal(mx.l2_normalise(g["l2_x"], eps=0.0), g["l2_y"])
    rng = np.random.default_rng(50)
    x = rng.standard_normal((3, 7, 2, 16))
    y = mx.l2_normalise(x)
    s = np.sum(x * x, axis=-1)
    np.testing.assert_allclose(np.sum(y * y, axis=-1), s / (s + mx.EPS_L2), rtol=1e-13)
    np.testing.assert_allclose(y * np.linalg.norm(x, axis=-1, keepdims=True), x * np.sqrt(s / (s + mx.EPS_L2))[..., None],
                               rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(mx.l2_normalise(x * 7.5, eps=0.0), mx.l2_normalise(x, eps=0.0), rtol=1e-13)


def test_forget_gate_power_law():
    rng = np.random.default_rng(60)
    x = rng.normal(3.0, 2.0, (2, 5, 3, 4))
    a_log = np.array([0.0, -0.7, 0.9])
    f = mx.forget_gate(x, a_log)
    np.testing.assert_allclose(f[:, :, 0], expit(x[:, :, 0]), rtol=1e-15)
    np.testing.assert_allclose(np.log(f), np.exp(a_log)[None, None, :, None] * np.log(expit(x)), rtol=1e-12)
    assert np.all((f > 0) & (f < 1))


def test_rms_norm_gate():
    g = golden()
    y = mx.rms_norm_gate(g["rms_o"].reshape(1, 1, 1, 4), g["rms_g"].reshape(1, 1, 1, 4),
                         g["rms_w"].reshape(1, 4), eps=0.0)
    assert np.array_equal(y.reshape(-1), g["rms_y"])
    rng = np.random.default_rng(70)
    o = rng.standard_normal((2, 6, 3, 8))
    one = np.ones((3, 8))
    open_gate = np.full(o.shape, 40.0)      # sigmoid(40) = 1 - 4e-18
    y = mx.rms_norm_gate(o, open_gate, one, eps=0.0)
    np.testing.assert_allclose(np.mean(y * y, axis=-1), 1.0, rtol=1e-13)
    np.testing.assert_allclose(mx.rms_norm_gate(3.25 * o, open_gate, one, 0.0), y, rtol=1e-13)
    half = mx.rms_norm_gate(o, np.zeros(o.shape), one, 0.0)
    np.testing.assert_allclose(half, 0.5 * y, rtol=1e-13)
    w = rng.standard_normal((3, 8))
    np.testing.assert_allclose(mx.rms_norm_gate(o, open_gate, w, 0.0), y * w[None, None], rtol=1e-13)
    # eps enters the mean square only
    ms = np.mean(o * o, axis=-1, keepdims=True)
    np.testing.assert_allclose(mx.rms_norm_gate(o, open_gate, one, 0.3), y * np.sqrt(ms / (ms + 0.3)), rtol=1e-13)


def _raw(rng, B, T, H, d, K):
    return dict(q_raw=rng.standard_normal((B, T, H, d)), k_raw=rng.standard_normal((B, T, H, d)),
                v_raw=rng.standard_normal((B, T, H, d)), f_raw=rng.normal(3.0, 1.0, (B, T, H, d)),
                beta_raw=rng.standard_normal((B, T, H)), c_raw=rng.standard_normal((B, T, H)),
                conv_q=rng.standard_normal((H, d, K)) / K, conv_k=rng.standard_normal((H, d, K)) / K,
                conv_v=rng.standard_normal((H, d, K)) / K, a_log=rng.uniform(-1, 1, (H,)))


def test_pre_processing_makes_updates_non_expansive():
    rng = np.random.default_rng(80)
    r = _raw(rng, 2, 40, 3, 16, 4)
    q, k, v, f, beta, c = mx.mixer_pre(**r)
    nk = np.sum(k * k, axis=-1)
    nv = np.sum(v * v, axis=-1)
    assert np.all(beta * nk * nv < 1.0)
    assert np.all(nk <= 1.0) and np.all(nv <= 1.0)
    assert np.all((beta > 0) & (beta < 1) & (c > 0) & (c < 1))
    _, _, _, _, beta2, _ = mx.mixer_pre(**r, beta_scale=2.0)
    np.testing.assert_allclose(beta2, 2.0 * beta, rtol=1e-15)


def test_pre_with_identity_conv_is_silu_then_l2():
    rng = np.random.default_rng(90)
    r = _raw(rng, 1, 12, 2, 8, 4)
    e = np.zeros((2, 8, 4))
    e[..., 3] = 1.0
    r.update(conv_q=e, conv_k=e, conv_v=e, a_log=np.zeros(2))
    q, k, v, f, beta, c = mx.mixer_pre(**r)
    for got, raw in ((q, r["q_raw"]), (k, r["k_raw"]), (v, r["v_raw"])):
        s = raw * expit(raw)
        np.testing.assert_allclose(got, s / np.sqrt(np.sum(s * s, axis=-1, keepdims=True) + mx.EPS_L2),
                                   rtol=1e-13)
    np.testing.assert_allclose(f, expit(r["f_raw"]), rtol=1e-15)
    # the rule on these inputs is the plain oracle (nothing else is carried)
    o, ST, _ = oracle.fwd(q, k, v, f, beta, c)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(ST))
