"""GPU parity of the chunkwise forward against the fp64 oracle.

Every case draws seeded inputs, rounds q, k, v, f to the workload dtype, runs
the HIP path through the C ABI (via the binding) and the oracle on the same
rounded values, and compares element by element with
    err(x) = max |x - x_ref| / max |x_ref|      (per output tensor)
Bar: err <= 1e-5 for fp32 inputs, err <= 2e-2 for bf16 inputs (fp32 state).
"""
import numpy as np
import pytest

import oracle
from delta_rule_recurrent_chunk_amd import synthetic as sy

pytestmark = pytest.mark.gpu

TOL = {"fp32": 1e-5, "bf16": 2e-2}


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


def run_fwd(x, dtype):
    torch = _torch()
    import delta_rule_recurrent_chunk_amd as kd
    t = to_dev(torch, x, dtype)
    print("case: B,T,H,d =", tuple(x["q"].shape), dtype, flush=True)
    o, ST = kd.fwd(t["q"], t["k"], t["v"], t["f"], t["beta"], t["c"], t["S0"])
    torch.cuda.synchronize()
    return o.double().cpu().numpy(), ST.double().cpu().numpy()


def check(x, dtype, tol=None):
    xr = sy.rounded(x, dtype)
    o, ST = run_fwd(xr, dtype)
    o_ref, ST_ref, _ = oracle.fwd(xr["q"], xr["k"], xr["v"], xr["f"], xr["beta"], xr["c"], xr["S0"])
    tol = TOL[dtype] if tol is None else tol
    e_o, e_s = rel(o, o_ref), rel(ST, ST_ref)
    print("  err o=%.3e  S_T=%.3e" % (e_o, e_s), flush=True)
    assert np.isfinite(o).all() and np.isfinite(ST).all()
    assert e_o <= tol and e_s <= tol, (e_o, e_s)
    return e_o, e_s


# ------------------------------------------------------------ named workloads
@pytest.mark.parametrize("name", ["tiny_fp32", "single_seq", "train_step", "long_ctx"])
def test_workload_full_size(name):
    w = sy.WORKLOADS[name]
    x = sy.draw_workload(w, with_dO=False)
    check(x, w.dtype)


# ------------------------------------------------------------ shapes and tails
@pytest.mark.parametrize("dtype,d", [("bf16", 32), ("bf16", 64), ("bf16", 128), ("fp32", 32), ("fp32", 64)])
@pytest.mark.parametrize("T", [1, 63, 64, 65, 200, 384])
def test_shapes_ragged_tails_nonzero_state(dtype, d, T):
    x = sy.draw(2, T, 3, d, d, seed=100 + T + d, beta_scale=2.0, s0_std=0.1)
    check(x, dtype)


def test_empty_sequence_returns_initial_state():
    torch = _torch()
    import delta_rule_recurrent_chunk_amd as kd
    x = sy.rounded(sy.draw(2, 0, 2, 64, 64, seed=5, s0_std=0.3), "bf16")
    t = to_dev(torch, x, "bf16")
    o, ST = kd.fwd(t["q"], t["k"], t["v"], t["f"], t["beta"], t["c"], t["S0"])
    torch.cuda.synchronize()
    assert o.shape == (2, 0, 2, 64)
    assert torch.equal(ST, t["S0"])
    o, ST = kd.fwd(t["q"], t["k"], t["v"], t["f"], t["beta"], t["c"], None)
    torch.cuda.synchronize()
    assert float(ST.abs().max()) == 0.0


# ------------------------------------------------------------ structured inputs
def test_clustered_repeated_keys_beta_near_two():
    """Repeated / clustered keys and values make (I + M) far from identity."""
    rng = np.random.default_rng(77)
    B, T, H, d = 1, 256, 4, 128
    x = sy.draw(B, T, H, d, d, seed=77, mu=5.0, beta_scale=2.0)
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


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_extreme_decay_takes_exact_fallback(dtype):
    """Sub-blocks whose decay product drops below 2^-100 (tiny f, and exact
    zeros = full reset) go through the exact scalar fallback."""
    rng = np.random.default_rng(78)
    B, T, H, d = 1, 192, 2, 64 if dtype == "bf16" else 32
    x = sy.draw(B, T, H, d, d, seed=78, s0_std=0.2)
    x["f"][0, 10:30, 0, :7] = 1e-3          # 16-step products ~1e-48
    x["f"][0, 70:74, 1, 5:9] = 0.0          # hard reset of some channels
    x["f"][0, 130:150, :, -3:] = 1e-2
    x["f"][0, 160:176, 1, :] = 1.0          # no decay at all
    check(x, dtype)


def test_no_decay_no_erase_is_linear_attention():
    """f = 1, beta = 0: the method reduces to causal linear attention."""
    x = sy.draw(2, 130, 2, 64, 64, seed=79)
    x["f"][:] = 1.0
    x["beta"][:] = 0.0
    check(x, "bf16")


# ------------------------------------------------------------ run properties
def test_deterministic_bitwise():
    torch = _torch()
    import delta_rule_recurrent_chunk_amd as kd
    x = sy.rounded(sy.draw(2, 320, 4, 128, 128, seed=80, s0_std=0.1), "bf16")
    t = to_dev(torch, x, "bf16")
    o1, S1 = kd.fwd(t["q"], t["k"], t["v"], t["f"], t["beta"], t["c"], t["S0"])
    o2, S2 = kd.fwd(t["q"], t["k"], t["v"], t["f"], t["beta"], t["c"], t["S0"])
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


def test_split_resume_at_chunk_boundary_bitwise():
    torch = _torch()
    import delta_rule_recurrent_chunk_amd as kd
    x = sy.rounded(sy.draw(1, 384, 2, 128, 128, seed=81, s0_std=0.1), "bf16")
    t = to_dev(torch, x, "bf16")
    o, S = kd.fwd(t["q"], t["k"], t["v"], t["f"], t["beta"], t["c"], t["S0"])
    m = 192
    sl = lambda a: a[:, :m].contiguous()
    sr = lambda a: a[:, m:].contiguous()
    oa, Sm = kd.fwd(sl(t["q"]), sl(t["k"]), sl(t["v"]), sl(t["f"]), sl(t["beta"]), sl(t["c"]), t["S0"])
    ob, S2 = kd.fwd(sr(t["q"]), sr(t["k"]), sr(t["v"]), sr(t["f"]), sr(t["beta"]), sr(t["c"]), Sm)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat([oa, ob], dim=1), o)
    assert torch.equal(S2, S)


def test_bad_arguments_raise_without_launch():
    torch = _torch()
    import delta_rule_recurrent_chunk_amd as kd
    x = sy.rounded(sy.draw(1, 64, 2, 48, 48, seed=82), "bf16")
    t = to_dev(torch, x, "bf16")
    with pytest.raises(kd.KronDeltaError):
        kd.fwd(t["q"], t["k"], t["v"], t["f"], t["beta"], t["c"])
