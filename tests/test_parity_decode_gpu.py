"""GPU parity of kron_delta_decode (token-by-token recurrence on a carried
state) against the fp64 oracle's sequential loop.

The oracle runs R1-R4 over the same tokens from the same entering state S0
(oracle.fwd with S0 given); the decode calls run them one call at a time, the
state carried between calls in place.  Errors are
    err(x) = max |x - x_ref| / max |x_ref|
per tensor, with the bar of the forward: <= 1e-5 for fp32 inputs, <= 2e-2 for
bf16 inputs (fp32 state).
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


def to_dev(torch, a, dtype, per_token):
    if per_token:
        tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
        return torch.tensor(a, dtype=tdt, device="cuda")
    return torch.tensor(a, dtype=torch.float32, device="cuda")


def run_decode(x, dtype, steps):
    """Feed the sequence to decode in `steps` calls (token slices), S in place."""
    torch = _torch()
    import delta_rule_recurrent_chunk_amd as kd
    T = x["q"].shape[1]
    S = to_dev(torch, x["S0"], dtype, False).contiguous()
    outs = []
    bounds = np.linspace(0, T, steps + 1).astype(int)
    for a, b in zip(bounds[:-1], bounds[1:]):
        t = {n: to_dev(torch, np.ascontiguousarray(x[n][:, a:b]), dtype, n in ("q", "k", "v", "f"))
             for n in ("q", "k", "v", "f", "beta", "c")}
        outs.append(kd.decode(t["q"], t["k"], t["v"], t["f"], t["beta"], t["c"], S))
    torch.cuda.synchronize()
    o = torch.cat(outs, dim=1).double().cpu().numpy()
    return o, S.double().cpu().numpy()


def check(x, dtype, steps):
    xr = sy.rounded(x, dtype)
    print("case: B,T,H,d =", tuple(xr["q"].shape), dtype, "calls", steps, flush=True)
    o, S = run_decode(xr, dtype, steps)
    o_ref, S_ref, _ = oracle.fwd(xr["q"], xr["k"], xr["v"], xr["f"], xr["beta"], xr["c"], xr["S0"])
    e_o, e_s = rel(o, o_ref), rel(S, S_ref)
    print("  err o=%.3e  S=%.3e" % (e_o, e_s), flush=True)
    assert np.isfinite(o).all() and np.isfinite(S).all()
    assert e_o <= TOL[dtype] and e_s <= TOL[dtype], (e_o, e_s)


@pytest.mark.parametrize("dtype,d", [("bf16", 32), ("bf16", 64), ("bf16", 128),
                                     ("fp32", 32), ("fp32", 64), ("fp32", 128)])
def test_single_token_steps(dtype, d):
    """Eight decode calls of one token each from a non-zero state."""
    x = sy.draw(2, 8, 3, d, d, seed=400 + d, s0_std=0.1)
    check(x, dtype, steps=8)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_multi_token_calls_long_sequence(dtype):
    """A 200-token sequence in calls of 1 to 64 tokens, beta in (0, 2)."""
    x = sy.draw(1, 200, 4, 128 if dtype == "bf16" else 64, 128 if dtype == "bf16" else 64,
                seed=410, beta_scale=2.0, s0_std=0.1)
    check(x, dtype, steps=7)


def test_decode_continues_a_chunked_forward():
    """Prefill T tokens with kron_delta_fwd, then decode the next ones: the same
    as one oracle run over the whole sequence."""
    torch = _torch()
    import delta_rule_recurrent_chunk_amd as kd
    x = sy.rounded(sy.draw(2, 140, 2, 128, 128, seed=411, s0_std=0.1), "bf16")
    pre = 130
    t = {n: to_dev(torch, np.ascontiguousarray(x[n][:, :pre]), "bf16", n in ("q", "k", "v", "f"))
         for n in ("q", "k", "v", "f", "beta", "c")}
    S0 = to_dev(torch, x["S0"], "bf16", False)
    o1, S = kd.fwd(t["q"], t["k"], t["v"], t["f"], t["beta"], t["c"], S0)
    outs = [o1]
    for a in range(pre, 140):
        u = {n: to_dev(torch, np.ascontiguousarray(x[n][:, a:a + 1]), "bf16", n in ("q", "k", "v", "f"))
             for n in ("q", "k", "v", "f", "beta", "c")}
        outs.append(kd.decode(u["q"], u["k"], u["v"], u["f"], u["beta"], u["c"], S))
    torch.cuda.synchronize()
    o = torch.cat(outs, dim=1).double().cpu().numpy()
    o_ref, S_ref, _ = oracle.fwd(x["q"], x["k"], x["v"], x["f"], x["beta"], x["c"], x["S0"])
    assert rel(o, o_ref) <= TOL["bf16"]
    assert rel(S.double().cpu().numpy(), S_ref) <= TOL["bf16"]


def test_in_place_and_separate_output_agree_bitwise():
    torch = _torch()
    import delta_rule_recurrent_chunk_amd as kd
    x = sy.rounded(sy.draw(2, 3, 2, 128, 128, seed=412, s0_std=0.1), "bf16")
    t = {n: to_dev(torch, x[n], "bf16", n in ("q", "k", "v", "f")) for n in ("q", "k", "v", "f", "beta", "c")}
    S_a = to_dev(torch, x["S0"], "bf16", False)
    S_in = S_a.clone()
    S_b = torch.empty_like(S_a)
    o_a = kd.decode(t["q"], t["k"], t["v"], t["f"], t["beta"], t["c"], S_a)
    o_b = kd.decode(t["q"], t["k"], t["v"], t["f"], t["beta"], t["c"], S_in, S_out=S_b)
    torch.cuda.synchronize()
    assert torch.equal(o_a, o_b)
    assert torch.equal(S_a, S_b)
    assert torch.equal(S_in, to_dev(torch, x["S0"], "bf16", False))   # input state untouched


def test_zero_tokens_copies_the_state():
    torch = _torch()
    import delta_rule_recurrent_chunk_amd as kd
    x = sy.rounded(sy.draw(1, 0, 2, 64, 64, seed=413, s0_std=0.2), "bf16")
    t = {n: to_dev(torch, x[n], "bf16", n in ("q", "k", "v", "f")) for n in ("q", "k", "v", "f", "beta", "c")}
    S_in = to_dev(torch, x["S0"], "bf16", False)
    S_out = torch.full_like(S_in, 7.0)
    o = kd.decode(t["q"], t["k"], t["v"], t["f"], t["beta"], t["c"], S_in, S_out=S_out)
    torch.cuda.synchronize()
    assert o.shape == (1, 0, 2, 64)
    assert torch.equal(S_out, S_in)
