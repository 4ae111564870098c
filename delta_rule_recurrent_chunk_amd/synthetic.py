"""Seeded synthetic inputs for the Kronecker delta rule mixer.

This module is shared by the tests, the benchmark and the smoke check.  It
draws inputs only; it holds none of the mixer's arithmetic.

Recipe (fixed draw order from one ``numpy.random.Generator(PCG64(seed))``):
  1. q, k, v ~ N(0, 1) of shape [B, T, H, d], each L2-normalised over d per
     (b, t, h) -- the mixer receives normalised q, k, v (KronLSTM summary page,
     onedev.kr, section "how it is used": short causal conv, SiLU, L2 norm).
  2. x ~ N(mu, 1) of shape [B, T, H, dk].
  3. a_log ~ U(-1, 1) of shape [H].
  4. f = sigmoid(x) ** exp(a_log[h])  -- the forget gate is a sigmoid raised to
     a learned positive per-head exponent (same section).
  5. beta = beta_scale * sigmoid(N(0, 1)) of shape [B, T, H]; beta_scale = 2
     gives the (0, 2) range of the state-tracking extension (same page,
     section "premises and limits").
  6. c = sigmoid(N(0, 1)) of shape [B, T, H].
  7. dO ~ N(0, 1) of shape [B, T, H, dv] (only when requested).
  8. S0 ~ N(0, s0_std^2) of shape [B, H, dv, dk] (only when s0_std is given).
  9. dS_T ~ N(0, dST_std^2) (only when dST_std is given).
  10. resets: that many (b, t, h) rows per (b, h), drawn uniformly, get f = 0
      on every key channel (an exact reset of the state; only when requested).
With a_log_value given, step 3 still draws (so every later draw is the same)
but every head takes exp(a_log_value) as its exponent: a_log_value = 1 with
mu = 0 gives the fast-decay gates sigmoid(N(0, 1))^e, whose decay over a
64-token chunk falls below 2^-100 on most key channels.
q, k, v, f (and dO) are then rounded to the workload's dtype with
round-to-nearest-even; beta, c and S0 stay fp32.  Both the GPU library and
the oracle consume the rounded values (the oracle upcasts them exactly).

Gated Delta Rule-2 inputs (``draw_gdn2``; aitrends.kr Gated DeltaNet-2
summary, sections 방법론 and 기술 상세), same generator and order:
  1. q, k, v as above.
  2. x ~ N(mu, 1) of shape [B, T, H, dk] and a_log ~ U(-1, 1) of shape [H];
     alpha = exp(-exp(a_log[h]) * softplus(-x)), the page's log-decay form
     (numerically the forget gate of the recipe above).
  3. b = sigmoid(N(0, 1)) of shape [B, T, H, dk] (erase gate, key axis).
  4. w = sigmoid(N(0, 1)) of shape [B, T, H, dv] (write gate, value axis).
  5. S0 ~ N(0, s0_std^2) of shape [B, H, dk, dv] (only when s0_std is given).
q, k, v, alpha, b, w are rounded to the workload's dtype.

Mixer inputs (``draw_mixer``: the projections and parameters that the
mixer's pre- and post-processing take; KronLSTM summary page, section "how it
is used"), same generator, this order:
  1. q_raw, k_raw, v_raw ~ N(0, 1) of shape [B, T, H, d].
  2. f_raw ~ N(mu, 1) of shape [B, T, H, dk]; a_log ~ U(-1, 1) of shape [H].
  3. beta_raw, c_raw ~ N(0, 1) of shape [B, T, H].
  4. g ~ N(0, 1) of shape [B, T, H, dv] (output-gate logits).
  5. conv_q, conv_k, conv_v ~ N(0, 1/K) of shape [H, d, K] (K = conv_size).
  6. norm_w = 1 + 0.1 N(0, 1) of shape [H, dv].
  7. S0 ~ N(0, s0_std^2) of shape [B, H, dv, dk] (only when s0_std is given).
The projections and g are rounded to the workload's dtype; the rest stays
fp32 (conv taps, a_log and norm_w are rounded to fp32).

These seeded draws stand in for real activations: the pages measure on
FineWeb-Edu language-model training, for which no data or weights exist here.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    T: int
    H: int
    dk: int
    dv: int
    dtype: str          # "fp32" or "bf16" for q, k, v, f, o (and dO, dq, ...)
    mu: float = 3.0     # mean of the forget-gate pre-activation
    beta_scale: float = 1.0
    seed: int = 1000
    backward: bool = False
    decode: bool = False   # token-by-token on a carried state (S0 drawn, N(0, 0.1^2))
    gdn2: bool = False     # the Gated Delta Rule-2 variant (decoupled erase and write)
    mixer: bool = False    # from the projections: pre-processing, the rule, gated RMSNorm
    a_log_value: float | None = None   # every head's gate exponent is exp(a_log_value)

    @property
    def tokens(self) -> int:
        return self.B * self.T


WORKLOADS = {
    # Tiny fp32 forward; the oracle finishes it in well under a second.
    "tiny_fp32": Workload("tiny_fp32", 1, 256, 2, 32, 32, "fp32", seed=1000),
    # One bf16 sequence at the 16-head, d=128 layer shape.
    "single_seq": Workload("single_seq", 1, 2048, 16, 128, 128, "bf16", seed=1001),
    # Training-step shape: 8 x 2048 = 16,384 tokens per step (headline).
    "train_step": Workload("train_step", 8, 2048, 16, 128, 128, "bf16", seed=1002),
    # Forward plus gate-aware backward.
    "fwd_bwd": Workload("fwd_bwd", 4, 2048, 16, 128, 128, "bf16", seed=1003, backward=True),
    # Long context, non-contractive erase gate in (0, 2), near-1 decay.
    "long_ctx": Workload("long_ctx", 1, 32768, 16, 128, 128, "bf16", mu=5.0,
                         beta_scale=2.0, seed=1004),
    # Serving: one new token for each of 32 sequences on their carried states.
    "decode_step": Workload("decode_step", 32, 1, 16, 128, 128, "bf16", seed=1005, decode=True),
    # Gated Delta Rule-2 at the training-step shape (decoupled erase and write).
    "gdn2_step": Workload("gdn2_step", 8, 2048, 16, 128, 128, "bf16", seed=1006, gdn2=True),
    # The whole mixer forward at the training-step shape, from the projections.
    "mixer_step": Workload("mixer_step", 8, 2048, 16, 128, 128, "bf16", seed=1007, mixer=True),
    # The training-step forward under fast-decay gates sigmoid(N(0,1))^e.
    "fast_decay": Workload("fast_decay", 8, 2048, 16, 128, 128, "bf16", mu=0.0, seed=1008,
                           a_log_value=1.0),
}

MIXER_CONV_SIZE = 4


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def _l2n(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def draw(B, T, H, dk, dv, seed, mu=3.0, beta_scale=1.0, with_dO=False,
         s0_std=None, dST_std=None, a_log_value=None, resets=0):
    """Draw fp64 inputs (before dtype rounding).  Returns a dict."""
    rng = np.random.Generator(np.random.PCG64(seed))
    q = _l2n(rng.standard_normal((B, T, H, dk)))
    k = _l2n(rng.standard_normal((B, T, H, dk)))
    v = _l2n(rng.standard_normal((B, T, H, dv)))
    x = rng.normal(mu, 1.0, (B, T, H, dk))
    a_log = rng.uniform(-1.0, 1.0, (H,))
    if a_log_value is not None:
        a_log = np.full((H,), float(a_log_value))
    f = _sigmoid(x) ** np.exp(a_log)[None, None, :, None]
    beta = beta_scale * _sigmoid(rng.standard_normal((B, T, H)))
    c = _sigmoid(rng.standard_normal((B, T, H)))
    out = dict(q=q, k=k, v=v, f=f, beta=beta, c=c, S0=None, dO=None, dST=None)
    if with_dO:
        out["dO"] = rng.standard_normal((B, T, H, dv))
    if s0_std is not None:
        out["S0"] = rng.normal(0.0, s0_std, (B, H, dv, dk))
    if dST_std is not None:
        out["dST"] = rng.normal(0.0, dST_std, (B, H, dv, dk))
    if resets and T > 0:
        for b in range(B):
            for h in range(H):
                out["f"][b, rng.integers(0, T, resets), h, :] = 0.0
    return out


def draw_gdn2(B, T, H, dk, dv, seed, mu=3.0, s0_std=None):
    """Gated Delta Rule-2 inputs (fp64, before dtype rounding): q, k, v,
    alpha, b, w and, when s0_std is given, S0 [B, H, dk, dv]."""
    rng = np.random.Generator(np.random.PCG64(seed))
    q = _l2n(rng.standard_normal((B, T, H, dk)))
    k = _l2n(rng.standard_normal((B, T, H, dk)))
    v = _l2n(rng.standard_normal((B, T, H, dv)))
    x = rng.normal(mu, 1.0, (B, T, H, dk))
    a_log = rng.uniform(-1.0, 1.0, (H,))
    alpha = np.exp(-np.exp(a_log)[None, None, :, None] * np.logaddexp(0.0, -x))
    b = _sigmoid(rng.standard_normal((B, T, H, dk)))
    w = _sigmoid(rng.standard_normal((B, T, H, dv)))
    out = dict(q=q, k=k, v=v, alpha=alpha, b=b, w=w, S0=None)
    if s0_std is not None:
        out["S0"] = rng.normal(0.0, s0_std, (B, H, dk, dv))
    return out


def draw_mixer(B, T, H, dk, dv, seed, mu=3.0, conv_size=MIXER_CONV_SIZE, s0_std=None):
    """Mixer inputs (fp64 projections before dtype rounding; fp32-exact parameters)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out = dict(q_raw=rng.standard_normal((B, T, H, dk)), k_raw=rng.standard_normal((B, T, H, dk)),
               v_raw=rng.standard_normal((B, T, H, dv)))
    out["f_raw"] = rng.normal(mu, 1.0, (B, T, H, dk))
    out["a_log"] = rng.uniform(-1.0, 1.0, (H,))
    out["beta_raw"] = rng.standard_normal((B, T, H))
    out["c_raw"] = rng.standard_normal((B, T, H))
    out["g"] = rng.standard_normal((B, T, H, dv))
    for n, d in (("conv_q", dk), ("conv_k", dk), ("conv_v", dv)):
        out[n] = rng.normal(0.0, 1.0 / np.sqrt(conv_size), (H, d, conv_size))
    out["norm_w"] = 1.0 + 0.1 * rng.standard_normal((H, dv))
    out["S0"] = rng.normal(0.0, s0_std, (B, H, dv, dk)) if s0_std is not None else None
    for n in ("a_log", "beta_raw", "c_raw", "conv_q", "conv_k", "conv_v", "norm_w", "S0"):
        if out[n] is not None:
            out[n] = out[n].astype(np.float32).astype(np.float64)
    return out


def draw_workload(w: Workload, with_dO=None, s0_std=None):
    if w.mixer:
        return draw_mixer(w.B, w.T, w.H, w.dk, w.dv, w.seed, mu=w.mu, s0_std=s0_std)
    if w.gdn2:
        return draw_gdn2(w.B, w.T, w.H, w.dk, w.dv, w.seed, mu=w.mu, s0_std=s0_std)
    if s0_std is None and w.decode:
        s0_std = 0.1
    return draw(w.B, w.T, w.H, w.dk, w.dv, w.seed, mu=w.mu, beta_scale=w.beta_scale,
                with_dO=w.backward if with_dO is None else with_dO, s0_std=s0_std,
                a_log_value=w.a_log_value)


def round_to(x, dtype: str):
    """Round an fp64 array to ``dtype`` ("fp32" or "bf16", round-to-nearest-even)
    and return the rounded values as fp64 (exact upcast)."""
    if x is None:
        return None
    if dtype == "fp32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        import torch
        t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64))
        return t.to(torch.bfloat16).to(torch.float64).numpy()
    raise ValueError(dtype)


def rounded(inputs: dict, dtype: str) -> dict:
    """Round the per-token tensors to ``dtype``; gates and states to fp32."""
    out = {}
    for key, val in inputs.items():
        if val is None:
            out[key] = None
        elif key in ("q", "k", "v", "f", "dO", "alpha", "b", "w", "q_raw", "k_raw", "v_raw", "f_raw", "g"):
            out[key] = round_to(val, dtype)
        else:
            out[key] = round_to(val, "fp32")
    return out
