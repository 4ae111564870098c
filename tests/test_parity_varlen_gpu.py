"""GPU parity of kron_delta_fwd_varlen (packed variable-length sequences).

Each sequence of the packed batch is checked against the fp64 oracle run on
that sequence alone with its own entering state (errors per tensor,
max|x - ref| / max|ref|; bars 1e-5 fp32, 2e-2 bf16), and equal-length packs
must match the batched kron_delta_fwd bit for bit.
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


def packed(lengths, H, d, dtype, seed):
    """Draw one long sequence and cut it into the given lengths."""
    T = int(sum(lengths))
    x = sy.rounded(sy.draw(1, T, H, d, d, seed=seed, beta_scale=2.0, s0_std=0.1), dtype)
    rng = np.random.default_rng(seed)
    S0 = rng.standard_normal((len(lengths), H, d, d)) * 0.1
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    return x, S0, cu


def run(x, S0, cu, dtype):
    torch = _torch()
    import delta_rule_recurrent_chunk_amd as kd
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    t = {n: torch.tensor(x[n][0], dtype=tdt if n in ("q", "k", "v", "f") else torch.float32,
                         device="cuda") for n in ("q", "k", "v", "f", "beta", "c")}
    o, ST = kd.fwd_varlen(t["q"], t["k"], t["v"], t["f"], t["beta"], t["c"],
                          torch.tensor(cu, device="cuda"),
                          torch.tensor(S0, dtype=torch.float32, device="cuda"))
    torch.cuda.synchronize()
    return o.double().cpu().numpy(), ST.double().cpu().numpy()


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("fp32", 32), ("fp32", 128)])
def test_mixed_lengths_match_each_sequence_alone(dtype, d):
    lengths = [130, 0, 1, 64, 63, 65, 200]
    x, S0, cu = packed(lengths, 3, d, dtype, seed=500 + d)
    print("case: lengths", lengths, dtype, "d", d, flush=True)
    o, ST = run(x, S0, cu, dtype)
    for s in range(len(lengths)):
        a, b = cu[s], cu[s + 1]
        sl = {n: x[n][:, a:b] for n in ("q", "k", "v", "f", "beta", "c")}
        o_ref, S_ref, _ = oracle.fwd(sl["q"], sl["k"], sl["v"], sl["f"], sl["beta"], sl["c"], S0[s:s + 1])
        e_s = rel(ST[s], S_ref[0])
        assert e_s <= TOL[dtype], (s, e_s)
        if b > a:
            e_o = rel(o[a:b], o_ref[0])
            assert e_o <= TOL[dtype], (s, e_o)
    assert np.isfinite(o).all()


@pytest.mark.parametrize("d", [128, 64])
def test_equal_lengths_match_batched_forward_bitwise(d):
    torch = _torch()
    import delta_rule_recurrent_chunk_amd as kd
    B, T, H = 3, 150, 2
    x = sy.rounded(sy.draw(B, T, H, d, d, seed=510, s0_std=0.1), "bf16")
    t = {n: torch.tensor(x[n], dtype=torch.bfloat16 if n in ("q", "k", "v", "f") else torch.float32,
                         device="cuda") for n in ("q", "k", "v", "f", "beta", "c", "S0")}
    # the packed forward runs the one-launch kernel: compare with that form
    # of the batched forward (an empty workspace keeps it off the few-heads path)
    o1, S1 = kd.fwd(t["q"], t["k"], t["v"], t["f"], t["beta"], t["c"], t["S0"],
                    workspace=torch.empty(0, dtype=torch.uint8, device="cuda"))
    cu = torch.tensor([0, T, 2 * T, 3 * T], dtype=torch.int32, device="cuda")
    flat = {n: t[n].reshape((B * T,) + tuple(t[n].shape[2:])) for n in ("q", "k", "v", "f", "beta", "c")}
    o2, S2 = kd.fwd_varlen(flat["q"], flat["k"], flat["v"], flat["f"], flat["beta"], flat["c"], cu, t["S0"])
    torch.cuda.synchronize()
    assert torch.equal(o1.reshape(B * T, H, d), o2)
    assert torch.equal(S1, S2)


def test_offsets_past_the_end_are_clamped():
    """cu = [0, 5, T + 100]: the second sequence covers tokens 5 .. T-1 only."""
    torch = _torch()
    import delta_rule_recurrent_chunk_amd as kd
    x, S0, _ = packed([40, 60], 2, 64, "bf16", seed=520)
    T = 100
    cu = np.array([0, 5, T + 100], dtype=np.int32)
    o, ST = run(x, S0, cu, "bf16")
    sl = {n: x[n][:, 5:T] for n in ("q", "k", "v", "f", "beta", "c")}
    o_ref, S_ref, _ = oracle.fwd(sl["q"], sl["k"], sl["v"], sl["f"], sl["beta"], sl["c"], S0[1:2])
    assert rel(o[5:T], o_ref[0]) <= TOL["bf16"]
    assert rel(ST[1], S_ref[0]) <= TOL["bf16"]
