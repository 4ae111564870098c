"""GPU parity of the gate-aware backward against the fp64 oracle's reverse mode.

Each case draws seeded inputs (with an upstream dO ~ N(0,1), and a non-zero
S0 and dS_T where stated), rounds the per-token tensors to the workload
dtype, runs kron_delta_bwd through the binding, runs the oracle's
hand-derived backward on the same rounded values, and compares all seven
gradients element by element with
    err(x) = max |x - x_ref| / max |x_ref|      (per gradient tensor)
Bar: err <= 2e-2 for bf16 inputs (fp32 state), err <= 1e-5 for fp32 inputs.
"""
import numpy as np
import pytest

import oracle
from delta_rule_recurrent_chunk_amd import synthetic as sy

pytestmark = pytest.mark.gpu

TOL = {"fp32": 1e-5, "bf16": 2e-2}
GRADS = ("dq", "dk", "dv", "df", "dbeta", "dc", "dS0")


def _torch():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def rel(a, b):
    den = np.abs(b).max()
    return float(np.abs(a - b).max() / den) if den > 0 else float(np.abs(a).max())


def to_dev(torch, x, dtype):
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    out = {}
    for n, a in x.items():
        if a is None:
            out[n] = None
        elif n in ("q", "k", "v", "f", "dO"):
            out[n] = torch.tensor(a, dtype=tdt, device="cuda")
        else:
            out[n] = torch.tensor(a, dtype=torch.float32, device="cuda")
    return out


def run_bwd(x, dtype):
    torch = _torch()
    import delta_rule_recurrent_chunk_amd as kd
    t = to_dev(torch, x, dtype)
    print("case: B,T,H,d =", tuple(x["q"].shape), dtype, "S0" if x["S0"] is not None else "",
          "dST" if x["dST"] is not None else "", flush=True)
    g = kd.bwd(t["q"], t["k"], t["v"], t["f"], t["beta"], t["c"], t["S0"], t["dO"], t["dST"])
    torch.cuda.synchronize()
    return {n: g[n].double().cpu().numpy() for n in GRADS}


def oracle_bwd(xr):
    return oracle.bwd(xr["q"], xr["k"], xr["v"], xr["f"], xr["beta"], xr["c"], xr["S0"],
                      xr["dO"], xr["dST"])


def check(x, dtype, tol=None):
    xr = sy.rounded(x, dtype)
    got = run_bwd(xr, dtype)
    ref = oracle_bwd(xr)
    tol = TOL[dtype] if tol is None else tol
    errs = {n: rel(got[n], ref[n]) for n in GRADS}
    print("  " + "  ".join("%s=%.2e" % (n, e) for n, e in errs.items()), flush=True)
    for n in GRADS:
        assert np.isfinite(got[n]).all(), n
    bad = {n: e for n, e in errs.items() if not e <= tol}
    assert not bad, bad
    return errs


# ------------------------------------------------------------ named workloads
def test_fwd_bwd_workload_full_size():
    """B=4, T=2048, H=16, d=128, bf16, dO ~ N(0,1), S0 = 0."""
    w = sy.WORKLOADS["fwd_bwd"]
    check(sy.draw_workload(w), w.dtype)


def test_fwd_bwd_shape_fast_decay_with_resets():
    """The fwd_bwd shape (B=4, T=2048, H=16, d=128, bf16) under fast-decay gates
    sigmoid(N(0,1))^e, with exact resets (f = 0 on every key channel) at a few
    random tokens of each (b, h), S0 and dS_T non-zero: every gradient finite
    and within the bar."""
    x = sy.draw(4, 2048, 16, 128, 128, seed=1013, mu=0.0, a_log_value=1.0, with_dO=True,
                s0_std=0.1, dST_std=0.1, resets=3)
    check(x, "bf16")


def test_tiny_fp32_with_state_gradients():
    w = sy.WORKLOADS["tiny_fp32"]
    x = sy.draw(w.B, w.T, w.H, w.dk, w.dv, w.seed, with_dO=True, s0_std=0.1, dST_std=0.1)
    check(x, "fp32")


# ------------------------------------------------------------ shapes and tails
@pytest.mark.parametrize("dtype,d", [("bf16", 32), ("bf16", 64), ("bf16", 128), ("fp32", 32), ("fp32", 64),
                                     ("fp32", 128)])
@pytest.mark.parametrize("T", [1, 63, 64, 65, 200])
def test_shapes_ragged_tails_nonzero_states(dtype, d, T):
    x = sy.draw(2, T, 3, d, d, seed=300 + T + d, beta_scale=2.0, with_dO=True,
                s0_std=0.1, dST_std=0.1)
    check(x, dtype)


def test_long_context_shape_near_one_decay():
    """mu = 5 (many f round to exactly 1 in bf16), beta in (0, 2), 16 chunks."""
    x = sy.draw(1, 1024, 4, 128, 128, seed=310, mu=5.0, beta_scale=2.0, with_dO=True)
    check(x, "bf16")


def test_long_context_workload_backward_full_size():
    """The backward at the long_ctx workload's full shape and distributions
    (B=1, T=32768, H=16, d=128, bf16, beta = 2 sigmoid(N(0,1)) in (0, 2),
    f = sigmoid(N(5,1))^e): 512 chunks of state gradient carried in fp32,
    all seven gradients against the oracle at the bf16 bar."""
    w = sy.WORKLOADS["long_ctx"]
    check(sy.draw_workload(w, with_dO=True), w.dtype)


def test_empty_sequence_passes_state_gradient_through():
    torch = _torch()
    import delta_rule_recurrent_chunk_amd as kd
    x = sy.rounded(sy.draw(2, 0, 2, 64, 64, seed=311, with_dO=True, s0_std=0.2, dST_std=0.3), "bf16")
    t = to_dev(torch, x, "bf16")
    g = kd.bwd(t["q"], t["k"], t["v"], t["f"], t["beta"], t["c"], t["S0"], t["dO"], t["dST"])
    torch.cuda.synchronize()
    assert g["dq"].shape == (2, 0, 2, 64)
    assert torch.equal(g["dS0"], t["dST"])
    g = kd.bwd(t["q"], t["k"], t["v"], t["f"], t["beta"], t["c"], t["S0"], t["dO"], None)
    torch.cuda.synchronize()
    assert float(g["dS0"].abs().max()) == 0.0


# ------------------------------------------------------------ structured inputs
@pytest.mark.parametrize("T", [256, 2048])
def test_clustered_repeated_keys_beta_near_two(T):
    """Clustered keys and values with beta ~ 1.95-1.99: (I + M) far from identity."""
    rng = np.random.default_rng(312)
    B, H, d = 1, 4, 128
    x = sy.draw(B, T, H, d, d, seed=312, mu=5.0, beta_scale=2.0, with_dO=True)
    base_k = rng.standard_normal((H, 4, d))
    base_v = rng.standard_normal((H, 4, d))
    for h in range(H):
        idx = rng.integers(0, 4, T)
        k = base_k[h, idx] + 0.05 * rng.standard_normal((T, d))
        v = base_v[h, idx] + 0.05 * rng.standard_normal((T, d))
        x["k"][0, :, h] = k / np.linalg.norm(k, axis=1, keepdims=True)
        x["v"][0, :, h] = v / np.linalg.norm(v, axis=1, keepdims=True)
    x["beta"][:] = 1.95 + 0.04 * rng.random(x["beta"].shape)
    check(x, "bf16")


def test_no_decay_no_erase():
    """f = 1, beta = 0 (causal linear attention): the decay and solve paths are trivial."""
    x = sy.draw(2, 130, 2, 64, 64, seed=313, with_dO=True, s0_std=0.1)
    x["f"][:] = 1.0
    x["beta"][:] = 0.0
    check(x, "bf16")


FAST = [("bf16", 128), ("bf16", 64), ("bf16", 32), ("fp32", 32), ("fp32", 64), ("fp32", 128)]


@pytest.mark.parametrize("dtype,d", FAST)
@pytest.mark.parametrize("mu", [0.0, 1.0])
def test_fast_decay_gates(dtype, d, mu):
    """Gates sigmoid(N(mu, 1))^e: most (mu = 0) or about half (mu = 1) of the
    key channels decay below 2^-100 over a chunk; a ragged tail, non-zero S0
    and dS_T."""
    x = sy.draw(2, 600 + 37, 3, d, d, seed=320 + d + int(4 * mu), mu=mu, a_log_value=1.0,
                beta_scale=2.0, with_dO=True, s0_std=0.1, dST_std=0.1)
    check(x, dtype)


@pytest.mark.parametrize("dtype,d", FAST)
def test_resets_under_fast_decay(dtype, d):
    """Exact resets (f = 0 on every key channel) at random tokens: their
    sub-blocks leave the diagonal Gram tiles' matrix products and take the
    exact pass, whose df needs no division by f."""
    x = sy.draw(2, 500, 3, d, d, seed=340 + d, mu=0.0, a_log_value=1.0, with_dO=True,
                s0_std=0.1, dST_std=0.1, resets=5)
    check(x, dtype)


def test_extreme_decay_matches_oracle():
    """A chunk where three key channels decay to about 1e-90 (below 2^-100
    over a 16-token sub-block) and a partial reset: every gradient, of every
    chunk and head, matches the oracle."""
    x = sy.draw(1, 256, 2, 64, 64, seed=314, with_dO=True, s0_std=0.1, dST_std=0.1)
    x["f"][0, 70:100, 0, :3] = 1e-3      # head 0, chunk 1: three channels decay to ~1e-90
    x["f"][0, 140:143, 1, 5:9] = 0.0     # head 1, chunk 2: a partial reset
    check(x, "bf16")


# ------------------------------------------------------------ run properties
def test_backward_deterministic_bitwise():
    torch = _torch()
    import delta_rule_recurrent_chunk_amd as kd
    x = sy.rounded(sy.draw(2, 200, 2, 128, 128, seed=315, with_dO=True, s0_std=0.1), "bf16")
    t = to_dev(torch, x, "bf16")
    g1 = kd.bwd(t["q"], t["k"], t["v"], t["f"], t["beta"], t["c"], t["S0"], t["dO"])
    g2 = kd.bwd(t["q"], t["k"], t["v"], t["f"], t["beta"], t["c"], t["S0"], t["dO"])
    torch.cuda.synchronize()
    for n in GRADS:
        assert torch.equal(g1[n], g2[n]), n


def test_fp32_d128_fwd_bwd_shape():
    """fp32 inputs at the fwd_bwd shape (B=4, T=2048, H=16, d=128), S0 and
    dS_T non-zero: the per-token backward against the oracle at the 1e-5 bar
    on every gradient (the fp32 diagnostic of the training pair)."""
    x = sy.draw(4, 2048, 16, 128, 128, seed=1017, with_dO=True, s0_std=0.1, dST_std=0.1)
    check(x, "fp32")


@pytest.mark.parametrize("dtype,d,T", [("bf16", 128, 150), ("bf16", 64, 200), ("fp32", 32, 130), ("fp32", 64, 130),
                                       ("fp32", 128, 130)])
def test_training_pair_equals_forward_and_backward_bitwise(dtype, d, T):
    """kron_delta_fwd_train gives the one-launch kron_delta_fwd's o and S_T,
    and kron_delta_bwd_saved from its records gives kron_delta_bwd's
    gradients, bit for bit (the same kernels, the records kept instead of
    recomputed).  kron_delta_fwd is held to its one-launch form here (an
    empty workspace): with few heads it would otherwise take the
    preparation + state-pass form, which rounds differently."""
    torch = _torch()
    import delta_rule_recurrent_chunk_amd as kd
    x = sy.rounded(sy.draw(2, T, 2, d, d, seed=800 + d, s0_std=0.1, with_dO=True, dST_std=0.1), dtype)
    t = to_dev(torch, x, dtype)
    args = (t["q"], t["k"], t["v"], t["f"], t["beta"], t["c"], t["S0"])
    o1, S1 = kd.fwd(*args, workspace=torch.empty(0, dtype=torch.uint8, device="cuda"))
    o2, S2, ws = kd.fwd_train(*args)
    g2 = kd.bwd(*args, t["dO"], t["dST"], workspace=ws, saved=True)
    g1 = kd.bwd(*args, t["dO"], t["dST"])
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)
    for n in GRADS:
        assert torch.equal(g1[n], g2[n]), n


def test_fused_backward_replays_under_graph_capture():
    """The fused backward captured in a graph and replayed with new inputs: a
    clearing kernel ahead of each launch keeps the hand-off flags of the
    previous replay (same frozen epoch) from matching.  Every replay equals an
    eager call on the same inputs, bit for bit, with eager work between the
    replays."""
    torch = _torch()
    import delta_rule_recurrent_chunk_amd as kd
    xs = [sy.rounded(sy.draw(1, 200, 8, 64, 64, seed=830 + i, s0_std=0.1, with_dO=True, dST_std=0.1), "bf16")
          for i in range(2)]
    t = to_dev(torch, xs[0], "bf16")
    args = lambda: (t["q"], t["k"], t["v"], t["f"], t["beta"], t["c"], t["S0"], t["dO"], t["dST"])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):
            kd.bwd(*args())
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        out = kd.bwd(*args())
    for rep, i in enumerate((0, 1, 0, 1, 1)):
        src = to_dev(torch, xs[i], "bf16")
        for n in t:
            if t[n] is not None:
                t[n].copy_(src[n])
        graph.replay()
        torch.cuda.synchronize()
        ref = kd.bwd(*args())
        torch.cuda.synchronize()
        for n in GRADS:
            assert torch.equal(out[n], ref[n]), (rep, n)


def test_fused_and_two_kernel_backward_agree_bitwise():
    """With few (b, h) the sweep and the chunk gradients share one launch;
    with more (b, h) than leave 64 compute units free they run as two
    kernels.  Both run the same per-unit arithmetic, so the heads of a wide
    run equal, bit for bit, the same heads run on their own."""
    torch = _torch()
    import delta_rule_recurrent_chunk_amd as kd
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    H = max(8, ((cus - 64) // 8 + 1) * 8)   # (B*H + 7) / 8 * 8 > cus - 64: two kernels
    x = sy.rounded(sy.draw(1, 130, H, 64, 64, seed=817, s0_std=0.1, with_dO=True, dST_std=0.1), "bf16")
    t = to_dev(torch, x, "bf16")
    wide = kd.bwd(t["q"], t["k"], t["v"], t["f"], t["beta"], t["c"], t["S0"], t["dO"], t["dST"])
    for lo in (0, H - 8):
        sl = {n: (a[:, lo:lo + 8] if n in ("S0", "dST") else a[:, :, lo:lo + 8]).contiguous()
              for n, a in t.items() if a is not None}
        few = kd.bwd(sl["q"], sl["k"], sl["v"], sl["f"], sl["beta"], sl["c"], sl["S0"], sl["dO"], sl["dST"])
        torch.cuda.synchronize()
        for n in GRADS:
            w = wide[n][:, lo:lo + 8] if n == "dS0" else wide[n][:, :, lo:lo + 8]
            assert torch.equal(w, few[n]), (n, lo)


def test_wait_timeout_is_reported():
    """A chunk worker of the fused backward that gives up waiting for the
    reverse sweep writes its unit's gradients as NaN and sets the status word:
    kron_delta_bwd_status returns KD_ERR_TIMEOUT.  The condition is forced
    from the host with a one-poll wait limit (every wait still ends); the next
    backward with the default limit reads KD_OK and gives the oracle's values."""
    torch = _torch()
    import delta_rule_recurrent_chunk_amd as kd
    x = sy.rounded(sy.draw(2, 1024, 4, 64, 64, seed=850, s0_std=0.1, with_dO=True), "bf16")
    t = to_dev(torch, x, "bf16")
    args = (t["q"], t["k"], t["v"], t["f"], t["beta"], t["c"], t["S0"], t["dO"])
    need = kd.workspace_bytes(2, 1024, 4, 64, 1, with_backward=True)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    try:
        kd.bwd_set_wait_limit(1)
        g = kd.bwd(*args, workspace=ws)
        st = kd.bwd_status(t["q"], ws)
    finally:
        kd.bwd_set_wait_limit(0)
    assert st == kd.KD_ERR_TIMEOUT
    assert not torch.isfinite(g["dk"].float()).all()
    g = kd.bwd(*args, workspace=ws)
    assert kd.bwd_status(t["q"], ws) == 0
    ref = oracle.bwd(x["q"], x["k"], x["v"], x["f"], x["beta"], x["c"], x["S0"], x["dO"])
    for n in ("dq", "dk", "df"):
        assert rel(g[n].double().cpu().numpy(), ref[n]) <= 2e-2, n

