"""The allocation-free backward, kron_delta_bwd_noalloc, through the C ABI.

It runs kron_delta_bwd's kernels with the library's fixed scratch as the
workspace, so on the same inputs its seven gradients must equal
kron_delta_bwd's bit for bit; they are also checked against the fp64 oracle
at the bf16 bar (max |x - ref| / max |ref| <= 2e-2).  Two calls in a row, the
second on a smaller problem, so that the second starts from the scratch the
first one left.
"""
import numpy as np
import pytest

import oracle
from delta_rule_recurrent_chunk_amd import synthetic as sy

pytestmark = pytest.mark.gpu

GRADS = ("dq", "dk", "dv", "df", "dbeta", "dc", "dS0")


def _torch():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def rel(a, b):
    den = np.abs(b).max()
    return float(np.abs(a - b).max() / den) if den > 0 else float(np.abs(a).max())


def test_noalloc_backward_equals_backward_on_two_calls():
    torch = _torch()
    import delta_rule_recurrent_chunk_amd as kd
    for B, T, H, d, seed in ((2, 300, 4, 128, 900), (1, 130, 2, 64, 901)):
        x = sy.rounded(sy.draw(B, T, H, d, d, seed=seed, mu=1.0, a_log_value=1.0, with_dO=True,
                               s0_std=0.1, dST_std=0.1, resets=1), "bf16")
        t = {n: (torch.tensor(a, dtype=torch.bfloat16 if n in ("q", "k", "v", "f", "dO") else torch.float32,
                              device="cuda") if a is not None else None) for n, a in x.items()}
        args = (t["q"], t["k"], t["v"], t["f"], t["beta"], t["c"], t["S0"], t["dO"], t["dST"])
        print("case: B,T,H,d =", (B, T, H, d), flush=True)
        a = kd.bwd_noalloc(*args)
        b = kd.bwd(*args)
        torch.cuda.synchronize()
        for n in GRADS:
            assert torch.equal(a[n], b[n]), n
        ref = oracle.bwd(x["q"], x["k"], x["v"], x["f"], x["beta"], x["c"], x["S0"], x["dO"], x["dST"])
        errs = {n: rel(a[n].double().cpu().numpy(), ref[n]) for n in GRADS}
        print("  " + "  ".join("%s=%.2e" % kv for kv in errs.items()), flush=True)
        assert all(e <= 2e-2 for e in errs.values()), errs


def test_noalloc_backward_rejects_a_problem_beyond_its_scratch():
    torch = _torch()
    import delta_rule_recurrent_chunk_amd as kd
    x = sy.rounded(sy.draw(2, 2048, 16, 128, 128, seed=902, with_dO=True), "bf16")
    t = {n: (torch.tensor(a, dtype=torch.bfloat16 if n in ("q", "k", "v", "f", "dO") else torch.float32,
                          device="cuda") if a is not None else None) for n, a in x.items()}
    with pytest.raises(kd.KronDeltaError) as err:
        kd.bwd_noalloc(t["q"], t["k"], t["v"], t["f"], t["beta"], t["c"], None, t["dO"])
    assert err.value.status == kd.KD_ERR_SCRATCH
