"""C-ABI boundary tests that need no GPU.

The library loads, exports every function include/kron_delta.h declares, and
rejects bad arguments with the documented status codes before any launch
(the pointers below are never dereferenced: every call fails its checks, or
has nothing to compute, before touching the device).
"""
import ctypes
import os
import re

import pytest

import delta_rule_recurrent_chunk_amd as kd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kron_delta.h")

OK, NULL, SHAPE, DTYPE, ALIGN, WORKSPACE, LAUNCH, ALIAS, SCRATCH = 0, -1, -2, -3, -4, -5, -6, -7, -8


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"KD_API\s+[\w\s\*]+?\b(kron_delta_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(kd.LIB_PATH):
        from delta_rule_recurrent_chunk_amd import build
        build.build()
    return kd.lib()


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert set(names) == set(kd.EXPORTED)
    for n in names:
        assert hasattr(L, n), n


def test_abi_version_and_strings(L):
    assert L.kron_delta_abi_version() == 1
    for s in (OK, NULL, SHAPE, DTYPE, ALIGN, WORKSPACE, LAUNCH, ALIAS, SCRATCH, 12345):
        assert isinstance(kd.status_string(s), str) and kd.status_string(s)


def _desc(B=1, T=128, H=2, dk=64, dv=64, dtype=kd.KD_BF16):
    return kd.KdDesc(B, T, H, dk, dv, dtype)


# fake, 256-byte aligned, far-apart device addresses (never dereferenced)
BASE = 0x7F0000000000
STEP = 1 << 32


def P(i, misalign=0):
    return ctypes.c_void_p(BASE + i * STEP + misalign)


def fwd(L, desc, ptrs=None, **over):
    names = ["q", "k", "v", "f", "beta", "c", "S0", "o", "ST"]
    p = {n: P(i) for i, n in enumerate(names)}
    if ptrs:
        p.update(ptrs)
    p.update(over)
    d = ctypes.byref(desc) if desc is not None else None
    return L.kron_delta_fwd(d, *[p[n] for n in names], None, 0, None)


def bwd(L, desc, ws_bytes=None, **over):
    names = ["q", "k", "v", "f", "beta", "c", "S0", "dO", "dST", "dq", "dk", "dv", "df",
             "dbeta", "dc", "dS0"]
    p = {n: P(i) for i, n in enumerate(names)}
    p["ws"] = P(40)
    p.update(over)
    need = L.kron_delta_workspace_bytes(ctypes.byref(desc), 1)
    wsb = need if ws_bytes is None else ws_bytes
    return L.kron_delta_bwd(ctypes.byref(desc), *[p[n] for n in names], p["ws"], wsb, None)


def test_fwd_argument_checks(L):
    assert fwd(L, None) == NULL
    assert fwd(L, _desc(dtype=7)) == DTYPE
    assert fwd(L, _desc(B=0)) == SHAPE
    assert fwd(L, _desc(H=0)) == SHAPE
    assert fwd(L, _desc(T=-1)) == SHAPE
    assert fwd(L, _desc(dk=64, dv=32)) == SHAPE
    assert fwd(L, _desc(dk=48, dv=48)) == SHAPE
    # fp32 at d = 128 is accepted (the per-token path); its checks still run first
    assert fwd(L, _desc(dk=128, dv=128, dtype=kd.KD_F32), q=None) == NULL
    assert fwd(L, _desc(dk=96, dv=96, dtype=kd.KD_F32)) == SHAPE
    assert fwd(L, _desc(T=1 << 20, H=16, dk=128, dv=128)) == SHAPE   # > 2^31 bytes per batch element
    assert fwd(L, _desc(), q=None) == NULL
    assert fwd(L, _desc(), o=None) == NULL
    assert fwd(L, _desc(), beta=None) == NULL
    assert fwd(L, _desc(), k=P(1, misalign=8)) == ALIGN
    assert fwd(L, _desc(), ST=P(8, misalign=4)) == ALIGN
    assert fwd(L, _desc(), o=P(0)) == ALIAS          # o == q
    assert fwd(L, _desc(), ST=P(6)) == ALIAS         # ST == S0
    assert fwd(L, _desc(), ST=P(7)) == ALIAS         # ST == o
    # nothing to compute: T = 0 and no final state requested
    assert fwd(L, _desc(T=0), ST=None) == OK


def test_bwd_argument_checks(L):
    d = _desc()
    assert L.kron_delta_workspace_bytes(ctypes.byref(d), 0) == 0
    need = L.kron_delta_workspace_bytes(ctypes.byref(d), 1)
    assert need >= 2 * 2 * 64 * 64 * 4   # one fp32 state per (b, h, chunk)
    assert bwd(L, _desc(dtype=3)) == DTYPE
    assert bwd(L, d, ws_bytes=need - 1) == WORKSPACE
    assert bwd(L, d, ws=None) == WORKSPACE
    assert bwd(L, d, dO=None) == NULL
    assert bwd(L, d, dq=P(2)) == ALIAS               # dq == v
    assert bwd(L, d, dS0=P(9)) == ALIAS              # dS0 == dq
    assert bwd(L, d, ws=P(13)) == ALIAS              # workspace == dbeta (an output)
    assert bwd(L, d, df=P(12, misalign=2)) == ALIGN
    assert bwd(L, _desc(T=0), dS0=None) == OK


def bwd_noalloc(L, desc, **over):
    names = ["q", "k", "v", "f", "beta", "c", "S0", "dO", "dST", "dq", "dk", "dv", "df",
             "dbeta", "dc", "dS0"]
    p = {n: P(i) for i, n in enumerate(names)}
    p.update(over)
    return L.kron_delta_bwd_noalloc(ctypes.byref(desc), *[p[n] for n in names], None)


def test_bwd_noalloc_rejects_before_any_device_call(L):
    """Checks that return before the scratch is looked up or anything is
    launched: a problem larger than the fixed scratch, bad descriptors, and an
    empty call."""
    assert "64 MiB" in kd.status_string(SCRATCH)
    big = _desc(B=2, T=2048, H=16, dk=128, dv=128)   # 32 heads of 2048 tokens
    assert L.kron_delta_workspace_bytes(ctypes.byref(big), 1) > kd.NOALLOC_SCRATCH_BYTES
    assert bwd_noalloc(L, big) == SCRATCH
    fits = _desc(B=1, T=2048, H=16, dk=128, dv=128)
    assert L.kron_delta_workspace_bytes(ctypes.byref(fits), 1) <= kd.NOALLOC_SCRATCH_BYTES
    assert bwd_noalloc(L, _desc(dtype=3)) == DTYPE
    assert bwd_noalloc(L, _desc(dk=48, dv=48)) == SHAPE
    assert bwd_noalloc(L, _desc(T=0), dS0=None) == OK


def test_workspace_scales_with_chunks(L):
    a = L.kron_delta_workspace_bytes(ctypes.byref(_desc(T=64)), 1)
    b = L.kron_delta_workspace_bytes(ctypes.byref(_desc(T=65)), 1)
    # two more (b, h, chunk) units, each at least: S0 and dS (d*d bf16 each),
    # u, r0, rho (C fp32 each), M (C*C fp32), P (C*C bf16); the 8-byte flags
    # of a few units fit in the padding of their part
    per_unit = 2 * 64 * 64 * 2 + 3 * 64 * 4 + 64 * 64 * 4 + 64 * 64 * 2
    assert 2 * per_unit <= b - a and b <= 2 * a
    assert L.kron_delta_workspace_bytes(ctypes.byref(_desc(dk=48, dv=48)), 1) == 0


def decode(L, desc, **over):
    names = ["q", "k", "v", "f", "beta", "c", "S_in", "o", "S_out"]
    p = {n: P(i) for i, n in enumerate(names)}
    p.update(over)
    d = ctypes.byref(desc) if desc is not None else None
    return L.kron_delta_decode(d, *[p[n] for n in names], None)


def test_decode_argument_checks(L):
    # every case fails its checks before a launch
    assert decode(L, None) == NULL
    assert decode(L, _desc(T=1, dtype=5)) == DTYPE
    assert decode(L, _desc(T=1, dk=48, dv=48)) == SHAPE
    assert decode(L, _desc(T=-1)) == SHAPE
    assert decode(L, _desc(T=1), S_out=None) == NULL
    assert decode(L, _desc(T=1), q=None) == NULL
    assert decode(L, _desc(T=1), beta=None) == NULL
    assert decode(L, _desc(T=1), v=P(2, misalign=4)) == ALIGN
    assert decode(L, _desc(T=1), S_out=P(8, misalign=8)) == ALIGN
    assert decode(L, _desc(T=1), o=P(0)) == ALIAS            # o == q
    assert decode(L, _desc(T=1), S_out=P(1)) == ALIAS        # S_out == k
    assert decode(L, _desc(T=1), S_out=P(7)) == ALIAS        # S_out == o
    assert decode(L, _desc(T=1), o=P(6)) == ALIAS            # o == S_in


def fwd_varlen(L, desc, **over):
    names = ["cu", "q", "k", "v", "f", "beta", "c", "S0", "o", "ST"]
    p = {n: P(i) for i, n in enumerate(names)}
    p.update(over)
    d = ctypes.byref(desc) if desc is not None else None
    return L.kron_delta_fwd_varlen(d, *[p[n] for n in names], None)


def test_fwd_varlen_argument_checks(L):
    d = _desc(B=3, T=200)   # 3 sequences, 200 packed tokens
    assert fwd_varlen(L, None) == NULL
    assert fwd_varlen(L, d, cu=None) == NULL
    assert fwd_varlen(L, d, cu=P(0, misalign=2)) == ALIGN
    assert fwd_varlen(L, _desc(B=3, T=200, dk=64, dv=32)) == SHAPE
    assert fwd_varlen(L, d, q=None) == NULL
    assert fwd_varlen(L, d, o=P(1)) == ALIAS          # o == q
    assert fwd_varlen(L, d, ST=P(7)) == ALIAS         # ST == S0
    assert fwd_varlen(L, d, o=P(0)) == ALIAS          # o == cu_seqlens
    assert fwd_varlen(L, _desc(B=3, T=0), ST=None) == OK


def test_gdn2_argument_checks(L):
    names = ["q", "k", "v", "alpha", "b", "w", "S0", "o", "ST"]

    def call(desc, **over):
        p = {n: P(i) for i, n in enumerate(names)}
        p.update(over)
        d = ctypes.byref(desc) if desc is not None else None
        return L.kron_delta_gdn2_fwd(d, *[p[n] for n in names], None)

    d = _desc(B=2, T=100, H=3, dk=128, dv=128)
    assert call(None) == NULL
    assert call(_desc(dk=64, dv=64)) == SHAPE                  # d = 128 only
    assert call(_desc(dk=32, dv=32, dtype=kd.KD_F32)) == DTYPE  # bf16 only
    assert call(d, alpha=None) == NULL
    assert call(d, w=P(5, misalign=4)) == ALIGN
    assert call(d, o=P(3)) == ALIAS                            # o == alpha
    assert call(d, ST=P(6)) == ALIAS                           # ST == S0
    assert call(_desc(B=2, T=0, H=3, dk=128, dv=128), ST=None) == OK


def test_training_pair_argument_checks(L):
    d = _desc()
    need = L.kron_delta_workspace_bytes(ctypes.byref(d), 1)
    names = ["q", "k", "v", "f", "beta", "c", "S0", "o", "ST"]

    def ftrain(desc, ws=P(40), ws_bytes=None, **over):
        p = {n: P(i) for i, n in enumerate(names)}
        p.update(over)
        wsb = need if ws_bytes is None else ws_bytes
        return L.kron_delta_fwd_train(ctypes.byref(desc), *[p[n] for n in names], ws, wsb, None)

    assert ftrain(d, ws=None) == WORKSPACE
    assert ftrain(d, ws_bytes=need - 1) == WORKSPACE
    assert ftrain(d, ws=P(2)) == ALIAS                     # workspace == v
    assert ftrain(d, o=P(40)) == ALIAS                     # o == workspace
    # fp32 at d = 128 is accepted (the per-token forward); its checks still run first
    assert ftrain(_desc(dk=128, dv=128, dtype=kd.KD_F32), f=None) == NULL
    assert ftrain(d, f=None) == NULL
    # the saved backward takes the same checks as kron_delta_bwd
    bn = ["q", "k", "v", "f", "beta", "c", "S0", "dO", "dST", "dq", "dk", "dv", "df",
          "dbeta", "dc", "dS0"]
    pb = [P(i) for i in range(len(bn))]
    assert L.kron_delta_bwd_saved(ctypes.byref(d), *pb, None, need, None) == WORKSPACE
    assert L.kron_delta_bwd_saved(ctypes.byref(d), *pb, P(40), need - 1, None) == WORKSPACE
    assert L.kron_delta_bwd_saved(ctypes.byref(d), *pb, P(9), need, None) == ALIAS   # ws == dq


def _mixer_params(conv_size=4, **over):
    p = dict(conv_q=P(50), conv_k=P(51), conv_v=P(52), conv_size=conv_size, a_log=P(53), beta_scale=1.0,
             norm_w=P(54), norm_eps=1e-5)
    p.update(over)
    return kd.KdMixerParams(**p)


def test_mixer_argument_checks(L):
    d = _desc(B=2, T=100, H=3, dk=128, dv=128)
    pre_names = ["q_raw", "k_raw", "v_raw", "f_raw", "beta_raw", "c_raw", "q", "k", "v", "f", "beta", "c"]

    def pre(desc, params=None, **over):
        p = {n: P(i) for i, n in enumerate(pre_names)}
        p.update(over)
        prm = ctypes.byref(params if params is not None else _mixer_params())
        return L.kron_delta_mixer_pre(ctypes.byref(desc), prm, *[p[n] for n in pre_names], None)

    assert L.kron_delta_mixer_pre(ctypes.byref(d), None, *[P(i) for i in range(12)], None) == NULL
    assert pre(d, _mixer_params(conv_size=5)) == SHAPE
    assert pre(d, _mixer_params(conv_size=0)) == SHAPE
    assert pre(d, _mixer_params(conv_k=None)) == NULL
    assert pre(d, _mixer_params(a_log=P(53, misalign=4))) == ALIGN
    assert pre(_desc(B=2, T=100, H=3, dk=48, dv=48)) == SHAPE
    assert pre(_desc(B=21846, T=1, H=1, dk=32, dv=32)) == SHAPE     # past the grid's batch limit
    assert pre(d, q=None) == NULL
    assert pre(d, c=P(5, misalign=8)) == ALIGN
    assert pre(d, q=P(0)) == ALIAS                        # q == q_raw
    assert pre(d, beta=P(50)) == ALIAS                    # beta == conv_q
    assert pre(d, k=P(6)) == ALIAS                        # k == q (two outputs)
    assert pre(_desc(B=2, T=0, H=3, dk=128, dv=128)) == OK

    def post(desc, params=None, **over):
        p = {"o": P(0), "g": P(1), "y": P(2)}
        p.update(over)
        prm = ctypes.byref(params if params is not None else _mixer_params())
        return L.kron_delta_mixer_post(ctypes.byref(desc), prm, p["o"], p["g"], p["y"], None)

    assert post(d, _mixer_params(norm_w=None)) == NULL
    assert post(d, _mixer_params(norm_eps=-1.0)) == SHAPE
    assert post(d, y=P(0)) == ALIAS
    assert post(d, y=P(54)) == ALIAS                      # y == norm_w
    assert post(d, g=P(1, misalign=2)) == ALIGN
    assert post(_desc(B=2, T=0, H=3, dk=128, dv=128)) == OK

    need = L.kron_delta_workspace_bytes(ctypes.byref(d), kd.KD_WS_MIXER)
    ntok = 2 * 100 * 3
    assert need >= ntok * 128 * 2 * 5 + ntok * 4 * 2      # q, k, v, f, o and beta, c
    assert L.kron_delta_workspace_bytes(ctypes.byref(d), 7) == 0
    fwd_names = ["q_raw", "k_raw", "v_raw", "f_raw", "beta_raw", "c_raw", "g", "S0", "y", "ST"]

    def mfwd(desc, params=None, ws=P(40), ws_bytes=None, **over):
        p = {n: P(i) for i, n in enumerate(fwd_names)}
        p.update(over)
        prm = ctypes.byref(params if params is not None else _mixer_params())
        return L.kron_delta_mixer_fwd(ctypes.byref(desc), prm, *[p[n] for n in fwd_names], ws,
                                      need if ws_bytes is None else ws_bytes, None)

    assert mfwd(d, ws=None) == WORKSPACE
    assert mfwd(d, ws_bytes=need - 1) == WORKSPACE
    assert mfwd(d, y=P(6)) == ALIAS                      # y == g
    assert mfwd(d, ST=P(40)) == ALIAS                    # ST == workspace
    assert mfwd(d, ws=P(3)) == ALIAS                     # workspace == f_raw
    assert mfwd(d, _mixer_params(norm_w=None)) == NULL
    assert mfwd(_desc(B=2, T=100, H=3, dk=128, dv=128, dtype=kd.KD_F32)) == DTYPE
    assert mfwd(_desc(B=2, T=0, H=3, dk=128, dv=128), ST=None) == OK


def test_few_heads_workspace_query():
    """The workspace that selects the few-heads path: one image per (b, h,
    64-token chunk) and the hand-off words, up to the head limit; none past it
    or for other shapes."""
    import ctypes
    import delta_rule_recurrent_chunk_amd as kd
    L = kd.lib()

    def ws(B, T, H, d=128, dt=1):
        return int(L.kron_delta_workspace_bytes(ctypes.byref(kd.KdDesc(B, T, H, d, d, dt)), 0))
    # per head and chunk an image, plus one 8-byte hand-off word per head and
    # per (head, chunk) for the fused launch
    img = ws(1, 64, 1) - 16
    assert img > 0 and img % 256 == 0
    assert ws(1, 65, 1) == 2 * img + 8 * (1 + 2) and ws(3, 130, 16) == 48 * 3 * img + 8 * (48 + 48 * 3)
    assert kd.lib() and ws(4, 130, 16) == 0   # 64 heads: past KRON_DELTA_FWD_SPLIT_MAX_HEADS (48)
    assert ws(5, 130, 13) == 0 and ws(1, 64, 1, d=64) == 0 and ws(1, 64, 1, dt=0) == 0


def test_fp32_d128_backward_workspace():
    """fp32 at d = 128 (the per-token backward): the state entering every
    64-token chunk and the states entering one chunk's tokens, per head, plus
    the status block; the 64 MiB fixed scratch of the allocation-free backward
    covers one head of 2048 tokens."""
    import ctypes
    L = kd.lib()

    def ws(B, T, H):
        return int(L.kron_delta_workspace_bytes(ctypes.byref(kd.KdDesc(B, T, H, 128, 128, 0)), 1))
    st = 128 * 128 * 4
    assert ws(1, 64, 1) == st * (1 + 64) + 256
    assert ws(2, 130, 3) == 6 * st * (3 + 64) + 256
    assert ws(1, 0, 1) == 256
    assert ws(1, 2048, 1) <= 64 << 20


def test_status_check_and_sync_switch(monkeypatch):
    """The binding raises KronDeltaError for a failed call; with
    KRON_DELTA_SYNC_CHECK=1 and no device it has nothing to wait for."""
    with pytest.raises(kd.KronDeltaError) as e:
        kd._done(-3, "kron_delta_fwd")
    assert e.value.status == -3 and "kron_delta_fwd" in str(e.value)
    monkeypatch.setenv(kd.SYNC_CHECK_ENV, "1")
    import torch
    if not torch.cuda.is_available():
        assert kd._done(0, "kron_delta_fwd") is None
