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


def test_tiny_fp32_with_state_gradients():
    w = sy.WORKLOADS["tiny_fp32"]
    x = sy.draw(w.B, w.T, w.H, w.dk, w.dv, w.seed, with_dO=True, s0_std=0.1, dST_std=0.1)
    check(x, "fp32")


# ------------------------------------------------------------ shapes and tails
@pytest.mark.parametrize("dtype,d", [("bf16", 32), ("bf16", 64), ("bf16", 128), ("fp32", 32)])
@pytest.mark.parametrize("T", [1, 63, 64, 65, 200])
def test_shapes_ragged_tails_nonzero_states(dtype, d, T):
    x = sy.draw(2, T, 3, d, d, seed=300 + T + d, beta_scale=2.0, with_dO=True,
                s0_std=0.1, dST_std=0.1)
    check(x, dtype)


def test_long_context_shape_near_one_decay():
    """mu = 5 (many f round to exactly 1 in bf16), beta in (0, 2), 16 chunks."""
    x = sy.draw(1, 1024, 4, 128, 128, seed=310, mu=5.0, beta_scale=2.0, with_dO=True)
    check(x, "bf16")


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
def test_clustered_repeated_keys_beta_near_two():
    """Clustered keys and values with beta ~ 1.95-1.99: (I + M) far from identity."""
    rng = np.random.default_rng(312)
    B, T, H, d = 1, 256, 4, 128
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


def test_extreme_decay_marks_prefix_nan():
    """A chunk where a key channel decays below 2^-100 is outside the backward's
    domain: all of its gradients are NaN, and so is everything that flows
    through the state gradient into earlier chunks (dk, dv, df, dbeta, dc and
    dS0 of that head).  dq_t = S_t^T dO_t of an earlier chunk does not depend on
    it and stays exact, as do later chunks and the other heads."""
    torch = _torch()
    import delta_rule_recurrent_chunk_amd as kd
    x = sy.draw(1, 256, 2, 64, 64, seed=314, with_dO=True, s0_std=0.1, dST_std=0.1)
    x["f"][0, 70:100, 0, :3] = 1e-3      # head 0, chunk 1: three channels decay to ~1e-90
    xr = sy.rounded(x, "bf16")
    t = to_dev(torch, xr, "bf16")
    g = kd.bwd(t["q"], t["k"], t["v"], t["f"], t["beta"], t["c"], t["S0"], t["dO"], t["dST"])
    torch.cuda.synchronize()
    got = {n: g[n].double().cpu().numpy() for n in GRADS}
    ref = oracle_bwd(xr)
    for n in ("dq", "dk", "dv", "df", "dbeta", "dc"):
        first = 64 if n == "dq" else 0
        assert np.isnan(got[n][0, first:128, 0]).all(), n
        assert np.isfinite(got[n][0, 128:, 0]).all(), n
        if first:
            assert rel(got[n][0, :first, 0], ref[n][0, :first, 0]) <= TOL["bf16"], n
        assert rel(got[n][0, 128:, 0], ref[n][0, 128:, 0]) <= TOL["bf16"], n
        assert rel(got[n][0, :, 1], ref[n][0, :, 1]) <= TOL["bf16"], n
    assert np.isnan(got["dS0"][0, 0]).all()
    assert rel(got["dS0"][0, 1], ref["dS0"][0, 1]) <= TOL["bf16"]


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


def test_backward_rejects_fp32_d64():
    torch = _torch()
    import delta_rule_recurrent_chunk_amd as kd
    x = sy.rounded(sy.draw(1, 64, 1, 64, 64, seed=316, with_dO=True), "fp32")
    t = to_dev(torch, x, "fp32")
    with pytest.raises(kd.KronDeltaError):
        kd.bwd(t["q"], t["k"], t["v"], t["f"], t["beta"], t["c"], None, t["dO"])


@pytest.mark.parametrize("dtype,d,T", [("bf16", 128, 150), ("bf16", 64, 200), ("fp32", 32, 130)])
def test_training_pair_equals_forward_and_backward_bitwise(dtype, d, T):
    """kron_delta_fwd_train gives kron_delta_fwd's o and S_T, and
    kron_delta_bwd_saved from its records gives kron_delta_bwd's gradients,
    bit for bit (the same kernels, the records kept instead of recomputed)."""
    torch = _torch()
    import delta_rule_recurrent_chunk_amd as kd
    x = sy.rounded(sy.draw(2, T, 2, d, d, seed=800 + d, s0_std=0.1, with_dO=True, dST_std=0.1), dtype)
    t = to_dev(torch, x, dtype)
    args = (t["q"], t["k"], t["v"], t["f"], t["beta"], t["c"], t["S0"])
    o1, S1 = kd.fwd(*args)
    o2, S2, ws = kd.fwd_train(*args)
    g2 = kd.bwd(*args, t["dO"], t["dST"], workspace=ws, saved=True)
    g1 = kd.bwd(*args, t["dO"], t["dST"])
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)
    for n in GRADS:
        assert torch.equal(g1[n], g2[n]), n


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
