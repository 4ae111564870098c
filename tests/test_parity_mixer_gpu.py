"""GPU parity of the mixer's pre-processing, post-processing and whole forward
(projections -> q, k, v, f, beta, c -> the rule -> gated per-head RMSNorm)
against the fp64 oracle (oracle/mixer.py and oracle.fwd).

Every case draws seeded projections and parameters (synthetic.draw_mixer),
rounds the projections to the dtype, runs the HIP path through the C ABI and
the oracle on the same values, and compares per tensor
    err(x) = max |x - x_ref| / max |x_ref|.
Bars: the pre/post outputs are rounded once to the dtype after fp32
arithmetic, so err <= 2^-8 for bf16 and <= 1e-5 for fp32.  The whole forward
feeds the rule with q, k, v, f in the dtype (its interface contract), so the
oracle chain rounds them the same way; the rule's bar then applies:
err <= 2e-2 for bf16 and 1e-5 for fp32.
"""
import numpy as np
import pytest

import oracle
from oracle import mixer as mx
from delta_rule_recurrent_chunk_amd import synthetic as sy

pytestmark = pytest.mark.gpu

PRE_TOL = {"bf16": 2.0 ** -8, "fp32": 1e-5}
FWD_TOL = {"bf16": 2e-2, "fp32": 1e-5}


def _torch():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def rel(a, b):
    den = np.abs(b).max()
    return float(np.abs(a - b).max() / den) if den > 0 else float(np.abs(a).max())


PROJ = ("q_raw", "k_raw", "v_raw", "f_raw", "g")


def to_dev(torch, x, dtype):
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    return {n: (None if a is None else
                torch.tensor(a, dtype=tdt if n in PROJ else torch.float32, device="cuda"))
            for n, a in x.items()}


def host(t):
    return t.double().cpu().numpy()


def draw(B, T, H, d, K, dtype, seed, s0_std=None):
    x = sy.draw_mixer(B, T, H, d, d, seed, conv_size=K, s0_std=s0_std)
    return sy.rounded(x, dtype)


def oracle_pre(x, beta_scale=1.0):
    return mx.mixer_pre(x["q_raw"], x["k_raw"], x["v_raw"], x["f_raw"], x["beta_raw"], x["c_raw"],
                        x["conv_q"], x["conv_k"], x["conv_v"], x["a_log"], beta_scale=beta_scale)


@pytest.mark.parametrize("dtype,d", [("bf16", 32), ("bf16", 64), ("bf16", 128), ("fp32", 32), ("fp32", 128)])
@pytest.mark.parametrize("T,K", [(1, 4), (3, 4), (100, 4), (100, 1), (65, 2)])
def test_pre_matches_oracle(dtype, d, T, K):
    torch = _torch()
    import delta_rule_recurrent_chunk_amd as kd
    x = draw(2, T, 3, d, K, dtype, seed=900 + T + d + K)
    t = to_dev(torch, x, dtype)
    print("case: pre B=2 T=%d H=3 d=%d K=%d %s" % (T, d, K, dtype), flush=True)
    got = kd.mixer_pre(t["q_raw"], t["k_raw"], t["v_raw"], t["f_raw"], t["beta_raw"], t["c_raw"],
                       t["conv_q"], t["conv_k"], t["conv_v"], t["a_log"], beta_scale=2.0 if K == 2 else 1.0)
    torch.cuda.synchronize()
    ref = oracle_pre(x, beta_scale=2.0 if K == 2 else 1.0)
    for name, g, r in zip(("q", "k", "v", "f", "beta", "c"), got, ref):
        e = rel(host(g), r)
        tol = PRE_TOL[dtype] if name not in ("beta", "c") else 1e-5
        assert e <= tol, (name, e)


@pytest.mark.parametrize("dtype,d", [("bf16", 64), ("bf16", 128), ("fp32", 32)])
def test_post_matches_oracle(dtype, d):
    torch = _torch()
    import delta_rule_recurrent_chunk_amd as kd
    rng = np.random.default_rng(950 + d)
    B, T, H = 2, 77, 5
    o = sy.round_to(rng.standard_normal((B, T, H, d)) * rng.uniform(0.01, 3.0, (B, T, H, 1)), dtype)
    g = sy.round_to(rng.standard_normal((B, T, H, d)), dtype)
    w = sy.round_to(1.0 + 0.1 * rng.standard_normal((H, d)), "fp32")
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    print("case: post B=%d T=%d H=%d d=%d %s" % (B, T, H, d, dtype), flush=True)
    y = kd.mixer_post(torch.tensor(o, dtype=tdt, device="cuda"), torch.tensor(g, dtype=tdt, device="cuda"),
                      torch.tensor(w, dtype=torch.float32, device="cuda"), norm_eps=1e-5)
    torch.cuda.synchronize()
    ref = mx.rms_norm_gate(o, g, w, 1e-5)
    assert rel(host(y), ref) <= PRE_TOL[dtype]


def oracle_mixer_fwd(x, dtype, norm_eps=1e-5):
    q, k, v, f, beta, c = oracle_pre(x)
    q, k, v, f = (sy.round_to(a, dtype) for a in (q, k, v, f))
    beta, c = sy.round_to(beta, "fp32"), sy.round_to(c, "fp32")
    o, ST, _ = oracle.fwd(q, k, v, f, beta, c, x["S0"])
    return mx.rms_norm_gate(o, x["g"], x["norm_w"], norm_eps), ST


def run_mixer_fwd(torch, kd, t, norm_eps=1e-5):
    return kd.mixer_fwd(t["q_raw"], t["k_raw"], t["v_raw"], t["f_raw"], t["beta_raw"], t["c_raw"], t["g"],
                        t["conv_q"], t["conv_k"], t["conv_v"], t["a_log"], t["norm_w"], t["S0"],
                        norm_eps=norm_eps)


@pytest.mark.parametrize("dtype,d,T", [("bf16", 128, 200), ("bf16", 64, 130), ("bf16", 32, 64),
                                       ("fp32", 32, 150), ("bf16", 128, 1)])
def test_mixer_fwd_matches_oracle(dtype, d, T):
    torch = _torch()
    import delta_rule_recurrent_chunk_amd as kd
    x = draw(2, T, 2, d, 4, dtype, seed=970 + d + T, s0_std=0.05)
    t = to_dev(torch, x, dtype)
    print("case: mixer_fwd B=2 T=%d H=2 d=%d %s" % (T, d, dtype), flush=True)
    y, ST = run_mixer_fwd(torch, kd, t)
    torch.cuda.synchronize()
    ry, rST = oracle_mixer_fwd(x, dtype)
    ey, es = rel(host(y), ry), rel(host(ST), rST)
    print("  y=%.2e ST=%.2e" % (ey, es), flush=True)
    assert np.isfinite(host(y)).all()
    assert ey <= FWD_TOL[dtype] and es <= FWD_TOL[dtype], (ey, es)


def test_mixer_fwd_equals_its_three_steps_bitwise():
    """kron_delta_mixer_fwd is kron_delta_mixer_pre, kron_delta_fwd and
    kron_delta_mixer_post in sequence: the same bits."""
    torch = _torch()
    import delta_rule_recurrent_chunk_amd as kd
    x = draw(2, 150, 3, 128, 4, "bf16", seed=990, s0_std=0.05)
    t = to_dev(torch, x, "bf16")
    y, ST = run_mixer_fwd(torch, kd, t)
    q, k, v, f, beta, c = kd.mixer_pre(t["q_raw"], t["k_raw"], t["v_raw"], t["f_raw"], t["beta_raw"], t["c_raw"],
                                       t["conv_q"], t["conv_k"], t["conv_v"], t["a_log"])
    # the mixer runs the rule's one-launch kernel (an empty workspace keeps
    # kron_delta_fwd off the few-heads path)
    o, ST2 = kd.fwd(q, k, v, f, beta, c, t["S0"], workspace=torch.empty(0, dtype=torch.uint8, device="cuda"))
    y2 = kd.mixer_post(o, t["g"], t["norm_w"], norm_eps=1e-5)
    torch.cuda.synchronize()
    assert torch.equal(y, y2) and torch.equal(ST, ST2)


def draw_fast_forget(B, T, H, d, dtype, seed):
    """Mixer inputs whose forget gates run fast on some channels: logits
    N(-8, 1) on channels 0-15 (sub-block decays below 2^-100: the diagonal
    tiles' exact pass), N(-2, 1) on 16-47 (chunk decays below 2^-100: the
    sub-block references), the usual draw elsewhere."""
    x = sy.draw_mixer(B, T, H, d, d, seed, conv_size=4, s0_std=0.05)
    x["f_raw"] = np.array(x["f_raw"])
    x["f_raw"][..., :16] -= 8.0
    x["f_raw"][..., 16:48] -= 2.0
    return sy.rounded(x, dtype)


def test_mixer_fwd_fast_forget_matches_oracle():
    """The gates made inside the forward on chunks that take the sub-block
    references and the exact pass (which makes its decay again from the
    logit, with the producers' function)."""
    torch = _torch()
    import delta_rule_recurrent_chunk_amd as kd
    x = draw_fast_forget(2, 300, 3, 128, "bf16", seed=995)
    t = to_dev(torch, x, "bf16")
    y, ST = run_mixer_fwd(torch, kd, t)
    torch.cuda.synchronize()
    ry, rST = oracle_mixer_fwd(x, "bf16")
    ey, es = rel(host(y), ry), rel(host(ST), rST)
    print("  y=%.2e ST=%.2e" % (ey, es), flush=True)
    assert np.isfinite(host(y)).all()
    assert ey <= FWD_TOL["bf16"] and es <= FWD_TOL["bf16"], (ey, es)


def test_mixer_fwd_fast_forget_equals_its_three_steps_bitwise():
    """With fast-forget gates, the fused mixer forward (gates made from their
    logits inside the forward, including its exact pass) equals the gate
    kernel + the one-launch forward + the post-processing kernel, bit for
    bit."""
    torch = _torch()
    import delta_rule_recurrent_chunk_amd as kd
    x = draw_fast_forget(2, 300, 3, 128, "bf16", seed=996)
    t = to_dev(torch, x, "bf16")
    y, ST = run_mixer_fwd(torch, kd, t)
    q, k, v, f, beta, c = kd.mixer_pre(t["q_raw"], t["k_raw"], t["v_raw"], t["f_raw"], t["beta_raw"], t["c_raw"],
                                       t["conv_q"], t["conv_k"], t["conv_v"], t["a_log"])
    o, ST2 = kd.fwd(q, k, v, f, beta, c, t["S0"], workspace=torch.empty(0, dtype=torch.uint8, device="cuda"))
    y2 = kd.mixer_post(o, t["g"], t["norm_w"], norm_eps=1e-5)
    torch.cuda.synchronize()
    assert torch.equal(y, y2) and torch.equal(ST, ST2)


def test_mixer_step_workload_sampled():
    """The full mixer_step shape (B=8, T=2048, H=16, d=128, bf16) as bench.py
    runs it; the oracle checks two sampled sequences end to end."""
    torch = _torch()
    import delta_rule_recurrent_chunk_amd as kd
    w = sy.WORKLOADS["mixer_step"]
    x = sy.rounded(sy.draw_workload(w), w.dtype)
    t = to_dev(torch, x, w.dtype)
    print("case: mixer_step full size", flush=True)
    y, ST = run_mixer_fwd(torch, kd, t)
    torch.cuda.synchronize()
    yh, sh = host(y), host(ST)
    assert np.isfinite(yh).all() and np.isfinite(sh).all()
    for b, h in ((0, 0), (5, 11)):
        xs = {n: (None if a is None else
                  a[b:b + 1, :, h:h + 1] if n in PROJ or n in ("beta_raw", "c_raw") else
                  a[h:h + 1] if n in ("conv_q", "conv_k", "conv_v", "a_log", "norm_w") else a)
              for n, a in x.items()}
        ry, rST = oracle_mixer_fwd(xs, w.dtype)
        ey, es = rel(yh[b:b + 1, :, h:h + 1], ry), rel(sh[b:b + 1, h:h + 1], rST)
        print("  (b,h)=(%d,%d) y=%.2e ST=%.2e" % (b, h, ey, es), flush=True)
        assert ey <= FWD_TOL["bf16"] and es <= FWD_TOL["bf16"]


def test_mixer_fwd_replays_under_graph_capture():
    """The mixer forward with its convolution on workers beside the rule
    (one launch, hand-off words cleared by a kernel ahead of it) captured in
    a graph and replayed with new inputs: every replay equals an eager call
    on the same inputs, bit for bit, with eager work between the replays."""
    torch = _torch()
    import delta_rule_recurrent_chunk_amd as kd
    xs = [draw(2, 200, 3, 128, 4, "bf16", seed=995 + i, s0_std=0.05) for i in range(2)]
    t = to_dev(torch, xs[0], "bf16")
    ws = torch.empty(64 << 20, dtype=torch.uint8, device="cuda")
    ws_eager = torch.empty(64 << 20, dtype=torch.uint8, device="cuda")

    def call(w):
        return kd.mixer_fwd(t["q_raw"], t["k_raw"], t["v_raw"], t["f_raw"], t["beta_raw"], t["c_raw"], t["g"],
                            t["conv_q"], t["conv_k"], t["conv_v"], t["a_log"], t["norm_w"], t["S0"],
                            norm_eps=1e-5, workspace=w)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):
            call(ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        y, ST = call(ws)
    for rep, i in enumerate((1, 0, 1, 1, 0)):
        src = to_dev(torch, xs[i], "bf16")
        for n in t:
            if t[n] is not None and n in src and src[n] is not None:
                t[n].copy_(src[n])
        graph.replay()
        torch.cuda.synchronize()
        y_ref, ST_ref = call(ws_eager)
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref) and torch.equal(ST, ST_ref), rep
