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
@pytest.mark.parametrize("name", ["tiny_fp32", "single_seq", "train_step", "long_ctx", "fast_decay"])
def test_workload_full_size(name):
    w = sy.WORKLOADS[name]
    x = sy.draw_workload(w, with_dO=False)
    check(x, w.dtype)


def test_long_context_fp32_diagnostic():
    """fp32 inputs at the long-context shape (B=1, T=32768, H=16, d=128, near-1
    decay, beta in (0, 2)): the whole launch on the GPU (the per-token path
    of fp32 at d = 128), two heads against the oracle run on those heads."""
    torch = _torch()
    w = sy.WORKLOADS["long_ctx"]
    xr = sy.rounded(sy.draw_workload(w, with_dO=False), "fp32")
    o, ST = run_fwd(xr, "fp32")
    for h in (0, 9):
        sl = {n: (xr[n][:, :, h:h + 1] if xr[n] is not None else None) for n in ("q", "k", "v", "f", "beta", "c")}
        o_ref, ST_ref, _ = oracle.fwd(sl["q"], sl["k"], sl["v"], sl["f"], sl["beta"], sl["c"], None)
        e_o, e_s = rel(o[:, :, h:h + 1], o_ref), rel(ST[:, h:h + 1], ST_ref)
        print("  head %d: err o=%.3e  S_T=%.3e" % (h, e_o, e_s), flush=True)
        assert e_o <= TOL["fp32"] and e_s <= TOL["fp32"], (h, e_o, e_s)


# ------------------------------------------------------------ shapes and tails
@pytest.mark.parametrize("dtype,d", [("bf16", 32), ("bf16", 64), ("bf16", 128), ("fp32", 32), ("fp32", 64),
                                     ("fp32", 128)])
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
@pytest.mark.parametrize("T", [256, 2048])
def test_clustered_repeated_keys_beta_near_two(T):
    """Repeated / clustered keys and values make (I + M) far from identity."""
    rng = np.random.default_rng(77)
    B, H, d = 1, 4, 128
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


FAST = [("bf16", 128), ("bf16", 64), ("bf16", 32), ("fp32", 32), ("fp32", 64), ("fp32", 128)]


@pytest.mark.parametrize("dtype,d", FAST)
@pytest.mark.parametrize("mu", [0.0, 1.0])
def test_fast_decay_gates(dtype, d, mu):
    """Gates sigmoid(N(mu, 1))^e: over a 64-token chunk most key channels
    (mu = 0) or about half of them (mu = 1) decay below 2^-100, while over a
    16-token sub-block none does.  Several chunks and a ragged tail."""
    x = sy.draw(2, 1024 + 37, 3, d, d, seed=120 + d + int(4 * mu), mu=mu, a_log_value=1.0,
                beta_scale=2.0, s0_std=0.1)
    check(x, dtype)


@pytest.mark.parametrize("dtype,d", FAST)
def test_resets_under_fast_decay(dtype, d):
    """Exact resets (f = 0 on every key channel at random tokens) on top of
    fast-decay gates: the sub-blocks that hold a reset take the exact path of
    their diagonal Gram tile."""
    x = sy.draw(2, 700, 3, d, d, seed=140 + d, mu=0.0, a_log_value=1.0, s0_std=0.1, resets=6)
    check(x, dtype)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_extreme_decay_takes_exact_fallback(dtype):
    """Sub-blocks whose decay product drops below 2^-100 (tiny f, and exact
    zeros = partial and full resets) take the exact path of their diagonal
    Gram tile; sub-blocks without decay next to them do not."""
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


# ------------------------------------------------------------ few-heads path
def run_fwd_path(x, dtype, split):
    """kd.fwd with the library's few-heads path (split=True: the workspace the
    binding allocates) or forced onto the one-launch kernel (an empty
    workspace)."""
    torch = _torch()
    import delta_rule_recurrent_chunk_amd as kd
    t = to_dev(torch, x, dtype)
    ws = None if split else torch.empty(0, dtype=torch.uint8, device="cuda")
    print("case: B,T,H,d =", tuple(x["q"].shape), dtype, "split" if split else "one-launch", flush=True)
    o, ST = kd.fwd(t["q"], t["k"], t["v"], t["f"], t["beta"], t["c"], t["S0"], workspace=ws)
    torch.cuda.synchronize()
    return o.double().cpu().numpy(), ST.double().cpu().numpy()


# workgroup shapes of the bf16 forward: waves per workgroup for each path
WAVE_FORMS = [(32, False, 2), (64, False, 4), (128, True, 8), (128, False, 16)]


@pytest.mark.parametrize("d,split,waves", WAVE_FORMS)
def test_lds_barriers_across_wave_counts(d, split, waves):
    """One ragged problem (three chunks and a tail, a non-zero state) through
    every workgroup shape of the bf16 forward (2, 4, 8 and 16 waves): a
    missing barrier or a stage that reads another wave's LDS early shows up
    as a mismatch with the oracle in the shape where it happens."""
    xr = sy.rounded(sy.draw(2, 200, 3, d, d, seed=330 + d, beta_scale=2.0, s0_std=0.1), "bf16")
    print("waves per workgroup:", waves, flush=True)
    o, ST = run_fwd_path(xr, "bf16", split)
    o_ref, ST_ref, _ = oracle.fwd(xr["q"], xr["k"], xr["v"], xr["f"], xr["beta"], xr["c"], xr["S0"])
    e_o, e_s = rel(o, o_ref), rel(ST, ST_ref)
    print("  err o=%.3e  S_T=%.3e" % (e_o, e_s), flush=True)
    assert e_o <= TOL["bf16"] and e_s <= TOL["bf16"], (waves, e_o, e_s)


def _clustered(B, T, H, d, seed):
    rng = np.random.default_rng(seed)
    x = sy.draw(B, T, H, d, d, seed=seed, mu=5.0, beta_scale=2.0)
    base_k = rng.standard_normal((H, 4, d))
    base_v = rng.standard_normal((H, 4, d))
    for b in range(B):
        for h in range(H):
            idx = rng.integers(0, 4, T)
            k = base_k[h, idx] + 0.05 * rng.standard_normal((T, d))
            v = base_v[h, idx] + 0.05 * rng.standard_normal((T, d))
            x["k"][b, :, h] = k / np.linalg.norm(k, axis=1, keepdims=True)
            x["v"][b, :, h] = v / np.linalg.norm(v, axis=1, keepdims=True)
    x["beta"][:] = 1.95 + 0.04 * rng.random(x["beta"].shape)
    return x


FEW = {
    "ragged_state": lambda: sy.draw(2, 200, 3, 128, 128, seed=301, beta_scale=2.0, s0_std=0.1),
    "fast_decay_resets": lambda: sy.draw(1, 700, 3, 128, 128, seed=302, mu=0.0, a_log_value=1.0,
                                         s0_std=0.1, resets=6),
    "clustered_beta2": lambda: _clustered(1, 512, 4, 128, 303),
    "single_token": lambda: sy.draw(1, 1, 2, 128, 128, seed=304, s0_std=0.2),
    "max_heads": lambda: sy.draw(3, 130, 16, 128, 128, seed=305, s0_std=0.05),
}


@pytest.mark.parametrize("split", [True, False])
@pytest.mark.parametrize("name", list(FEW))
def test_few_heads_paths_match_oracle(name, split):
    """Both forms of the bf16 d = 128 forward against the oracle: the
    chunk-parallel preparation + streaming state pass (u = A b with
    A = (I + M)^-1 by 16-blocks) and the one-launch substitution form."""
    xr = sy.rounded(FEW[name](), "bf16")
    o, ST = run_fwd_path(xr, "bf16", split)
    o_ref, ST_ref, _ = oracle.fwd(xr["q"], xr["k"], xr["v"], xr["f"], xr["beta"], xr["c"], xr["S0"])
    e_o, e_s = rel(o, o_ref), rel(ST, ST_ref)
    print("  err o=%.3e  S_T=%.3e" % (e_o, e_s), flush=True)
    assert np.isfinite(o).all() and np.isfinite(ST).all()
    assert e_o <= TOL["bf16"] and e_s <= TOL["bf16"], (e_o, e_s)


def test_few_heads_forward_replays_under_graph_capture():
    """The few-heads forward (preparation workers and per-head passes in one
    launch) captured in a graph and replayed with new inputs: the clearing
    kernel ahead of the launch keeps the previous replay's hand-off words
    (same frozen epoch) from matching.  Every replay equals an eager call on
    the same inputs, bit for bit, with eager work between the replays."""
    torch = _torch()
    import ctypes
    import delta_rule_recurrent_chunk_amd as kd
    xs = [sy.rounded(sy.draw(1, 300, 8, 128, 128, seed=840 + i, s0_std=0.1), "bf16") for i in range(2)]
    t = to_dev(torch, xs[0], "bf16")
    need = int(kd.lib().kron_delta_workspace_bytes(ctypes.byref(kd.KdDesc(1, 300, 8, 128, 128, 1)), 0))
    assert need > 0
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    ws_eager = torch.empty(need, dtype=torch.uint8, device="cuda")
    args = lambda: (t["q"], t["k"], t["v"], t["f"], t["beta"], t["c"], t["S0"])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):
            kd.fwd(*args(), workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        o, ST = kd.fwd(*args(), workspace=ws)
    for rep, i in enumerate((1, 0, 1, 1, 0)):
        src = to_dev(torch, xs[i], "bf16")
        for n in t:
            if t[n] is not None:
                t[n].copy_(src[n])
        graph.replay()
        torch.cuda.synchronize()
        o_ref, ST_ref = kd.fwd(*args(), workspace=ws_eager)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(ST, ST_ref), rep


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
