"""GPU parity of kron_delta_gdn2_fwd (Gated Delta Rule-2, decoupled erase and
write) against the fp64 oracle (oracle.gdn2_fwd).

Inputs follow the gdn2 recipe of delta_rule_recurrent_chunk_amd.synthetic,
rounded to bf16; errors per tensor, err(x) = max|x - x_ref| / max|x_ref|,
with the bf16 bar of the forward: <= 2e-2 (fp32 state).
"""
import numpy as np
import pytest

import oracle
from delta_rule_recurrent_chunk_amd import synthetic as sy

pytestmark = pytest.mark.gpu

TOL = 2e-2
NAMES = ("q", "k", "v", "alpha", "b", "w")


def _torch():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def rel(a, b):
    den = np.abs(b).max()
    return float(np.abs(a - b).max() / den) if den > 0 else float(np.abs(a).max())


def run(x, with_s0=True):
    torch = _torch()
    import delta_rule_recurrent_chunk_amd as kd
    t = {n: torch.tensor(x[n], dtype=torch.bfloat16, device="cuda") for n in NAMES}
    S0 = torch.tensor(x["S0"], dtype=torch.float32, device="cuda") if with_s0 and x["S0"] is not None else None
    o, ST = kd.gdn2_fwd(t["q"], t["k"], t["v"], t["alpha"], t["b"], t["w"], S0)
    torch.cuda.synchronize()
    return o.double().cpu().numpy(), ST.double().cpu().numpy()


def check(x, label):
    print("case:", label, tuple(x["q"].shape), flush=True)
    o, ST = run(x)
    o_ref, S_ref = oracle.gdn2_fwd(*(x[n] for n in NAMES), x["S0"])
    e_o, e_s = rel(o, o_ref), rel(ST, S_ref)
    print("  err o=%.3e  S=%.3e" % (e_o, e_s), flush=True)
    assert np.isfinite(o).all() and np.isfinite(ST).all()
    assert e_o <= TOL and e_s <= TOL, (e_o, e_s)


@pytest.mark.parametrize("B,T,H", [(1, 64, 1), (1, 130, 3), (2, 256, 4), (1, 1, 2), (1, 63, 2)])
def test_against_oracle(B, T, H):
    x = sy.rounded(sy.draw_gdn2(B, T, H, 128, 128, seed=700 + T, s0_std=0.1), "bf16")
    check(x, "B,T,H=%d,%d,%d" % (B, T, H))


def test_zero_initial_state_long_sequence():
    x = sy.rounded(sy.draw_gdn2(1, 1024, 2, 128, 128, seed=710), "bf16")
    check(x, "S0=0, T=1024")


def test_strong_decay_takes_the_exact_path():
    """alpha = 0.25 on every 17th key channel: its decay over a chunk falls
    below 2^-100, so those channels' T and P terms take the exact path."""
    x = sy.draw_gdn2(1, 200, 2, 128, 128, seed=720, s0_std=0.1)
    x["alpha"][:, :, :, ::17] = 0.25
    x["alpha"][:, 5::64, :, 3] = 0.0
    check(sy.rounded(x, "bf16"), "strong decay")


def test_kda_special_case_and_no_erase():
    """b = w = beta 1 (the KDA special case named on the page) and b = 0 (no
    erase: the rule becomes a decayed linear attention write)."""
    x = sy.draw_gdn2(1, 150, 2, 128, 128, seed=730, s0_std=0.1)
    beta = np.random.default_rng(1).uniform(0.2, 1.0, (1, 150, 2, 1))
    y = dict(x)
    y["b"] = np.broadcast_to(beta, x["b"].shape).copy()
    y["w"] = np.broadcast_to(beta, x["w"].shape).copy()
    check(sy.rounded(y, "bf16"), "KDA gates")
    z = dict(x)
    z["b"] = np.zeros_like(x["b"])
    check(sy.rounded(z, "bf16"), "no erase")


def test_training_shape_sampled_heads():
    """The bench workload (B=8, T=2048, H=16) in one launch; four (b, h) of it
    against the oracle run on those heads alone."""
    torch = _torch()
    w = sy.WORKLOADS["gdn2_step"]
    x = sy.rounded(sy.draw_workload(w), "bf16")
    o, ST = run(x)
    assert np.isfinite(o).all() and np.isfinite(ST).all()
    for (b, h) in [(0, 0), (3, 7), (5, 11), (7, 15)]:
        sl = {n: x[n][b:b + 1, :, h:h + 1] for n in NAMES}
        o_ref, S_ref = oracle.gdn2_fwd(*(sl[n] for n in NAMES), None)
        e_o, e_s = rel(o[b:b + 1, :, h:h + 1], o_ref), rel(ST[b:b + 1, h:h + 1], S_ref)
        print("  (b,h)=(%d,%d) err o=%.3e S=%.3e" % (b, h, e_o, e_s), flush=True)
        assert e_o <= TOL and e_s <= TOL, (b, h, e_o, e_s)
