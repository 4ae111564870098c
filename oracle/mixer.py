"""fp64 numpy oracle of the KronLSTM mixer's pre- and post-processing --
TEST INFRASTRUCTURE ONLY (imported by ``tests/``, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py``; never by the GPU library).

What the KronLSTM summary page (onedev.kr, section "어떻게 쓰나", how it is
used) says surrounds the Kronecker delta rule inside the mixer:
  * q, k and v each pass a short causal depthwise convolution, then SiLU,
    then L2 normalisation over the head dimension;
  * the erase gate beta and the write gate c are sigmoids of linear
    projections, one scalar per head;
  * the key-channel forget gate is a sigmoid raised to a learned positive
    per-head exponent a = exp(a_log);
  * the read-out passes a sigmoid output gate and a per-head RMSNorm before
    the output projection.
The review page (blog.secrett2633.cloud, KronLSTM review, section 3 and the
caption of its Figure 3) states the same q/k/v path.

Readings where the pages leave a step open (each also listed in the design
notes): the convolution has no bias, zero history before the first token and
a caller-chosen width (4 in the workloads); L2 normalisation divides by
sqrt(sum x^2 + eps_l2) with eps_l2 = 1e-6; the RMSNorm is
o / sqrt(mean o^2 + eps) times a per-head weight [H, dv], and the sigmoid
gate multiplies its result; beta may be scaled by beta_scale (2 gives the
(0, 2) range of the state-tracking extension, same page, section "전제와
한계").  The output projection is a plain matrix product and is not part of
the mixer.

Layouts: x_raw [B, T, H, d]; conv weights [H, d, K]; a_log [H];
beta_raw, c_raw [B, T, H]; norm_w [H, dv].  All arithmetic in fp64.
Parity status: pinned (tests/test_oracle_mixer.py: numpy.convolve per
channel, causality, the SiLU/sigmoid definitions against scipy's expit, unit
norms and scale invariance, the RMSNorm moments, the forget-gate power law,
the identity settings that reduce the pipeline to the plain rule).
"""
from __future__ import annotations

import numpy as np

EPS_L2 = 1e-6


def causal_depthwise_conv(x, w):
    """y[b, t, h, i] = sum_tau w[h, i, tau] * x[b, t - (K - 1) + tau, h, i],
    with x = 0 before the first token (no bias)."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    B, T, H, d = x.shape
    K = w.shape[-1]
    assert w.shape == (H, d, K)
    y = np.zeros_like(x)
    for tau in range(K):
        shift = K - 1 - tau                  # tap tau reads token t - shift
        if shift >= T:
            continue
        y[:, shift:] += w[None, None, :, :, tau] * x[:, :T - shift]
    return y


def sigmoid(x):
    return 1.0 / (1.0 + np.exp(-np.asarray(x, dtype=np.float64)))


def silu(x):
    x = np.asarray(x, dtype=np.float64)
    return x * sigmoid(x)


def l2_normalise(x, eps=EPS_L2):
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def forget_gate(f_raw, a_log):
    """f = sigmoid(f_raw) ** exp(a_log[h])."""
    a = np.exp(np.asarray(a_log, dtype=np.float64))
    return sigmoid(f_raw) ** a[None, None, :, None]


def mixer_pre(q_raw, k_raw, v_raw, f_raw, beta_raw, c_raw, conv_q, conv_k, conv_v, a_log,
              beta_scale=1.0):
    """The mixer's inputs from the projections: returns q, k, v, f, beta, c."""
    q = l2_normalise(silu(causal_depthwise_conv(q_raw, conv_q)))
    k = l2_normalise(silu(causal_depthwise_conv(k_raw, conv_k)))
    v = l2_normalise(silu(causal_depthwise_conv(v_raw, conv_v)))
    f = forget_gate(f_raw, a_log)
    beta = beta_scale * sigmoid(beta_raw)
    c = sigmoid(c_raw)
    return q, k, v, f, beta, c


def rms_norm_gate(o, g_raw, norm_w, eps):
    """y = o / sqrt(mean_i o_i^2 + eps) * norm_w[h] * sigmoid(g_raw), per (b, t, h)."""
    o = np.asarray(o, dtype=np.float64)
    ms = np.mean(o * o, axis=-1, keepdims=True)
    w = np.asarray(norm_w, dtype=np.float64)[None, None, :, :]
    return o / np.sqrt(ms + eps) * w * sigmoid(g_raw)
