"""fp64 CPU oracle of the Kronecker delta rule mixer -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It wraps ``kron_delta_oracle.c`` (plain
C, fp64, sequential in time, OpenMP across independent heads) through ctypes.
It shares nothing with the GPU library; the GPU library never imports it.

Functions
---------
``fwd(q, k, v, f, beta, c, S0=None) -> (o, S_T, r)``
    The sequential recurrence, decay-read-update-readout per step: the
    Kronecker delta rule of the KronLSTM summary page (onedev.kr, sections
    "how it works" and "how it is used").
``bwd(q, k, v, f, beta, c, S0, dO, dST) -> dict``
    Hand-derived reverse mode of the same loop (gradients w.r.t. q, k, v, f,
    beta, c, S0).
``gdn2_fwd(q, k, v, alpha, b, w, S0=None) -> (o, S_T)``
    The Gated Delta Rule-2 recurrence (decoupled erase gate b on the key axis,
    write gate w on the value axis, key-channel decay alpha) of the aitrends.kr
    Gated DeltaNet-2 summary (sections 핵심 기여 and 방법론); state [B,H,dk,dv],
    o_t = S_t^T q_t.  Pinned in tests/test_oracle_gdn2.py (the page's product
    form, decay-only closed form, exact recall, erase-only annihilation,
    split/resume, hand-worked fixture).

``oracle.mixer`` (numpy, fp64): the mixer's pre-processing (short causal
    depthwise convolution, SiLU, L2 normalisation, sigmoid gates, the
    power-law forget gate) and post-processing (per-head RMSNorm with a
    sigmoid output gate) around the rule; pinned in
    tests/test_oracle_mixer.py.

All arrays are numpy fp64 in the layouts q,k,f:[B,T,H,dk], v:[B,T,H,dv],
beta,c:[B,T,H], S:[B,H,dv,dk].  Parity status: pinned (see tests/test_oracle.py
for the pins: lifted Widrow-Hoff form, non-expansiveness identity, immediate
recall, capacity, interference, closed-form special cases, split/resume,
finite differences, autograd of the lifted form, hand-worked fixtures).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kron_delta_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libkron_delta_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (IEEE fp64, no fast-math, OpenMP)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp",
               "-fno-fast-math", "-ffp-contract=off", _SRC, "-o", tmp]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        lib = ctypes.CDLL(_LIB_PATH)
        dp = ctypes.POINTER(ctypes.c_double)
        i = ctypes.c_int
        lib.kdo_fwd.argtypes = [i, i, i, i, i] + [dp] * 10
        lib.kdo_fwd.restype = i
        lib.kdo_bwd.argtypes = [i, i, i, i, i] + [dp] * 16
        lib.kdo_bwd.restype = i
        lib.gdo_fwd.argtypes = [i, i, i, i, i] + [dp] * 9
        lib.gdo_fwd.restype = i
        lib.kdo_num_threads.restype = i
        lib.kdo_set_num_threads.argtypes = [i]
        _lib = lib
    return _lib


def num_threads() -> int:
    return int(_load().kdo_num_threads())


def set_num_threads(n: int) -> None:
    _load().kdo_set_num_threads(int(n))


def _p(a):
    if a is None:
        return ctypes.POINTER(ctypes.c_double)()
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _f64(a):
    if a is None:
        return None
    return np.ascontiguousarray(a, dtype=np.float64)


def _dims(q, v):
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    return B, T, H, dk, dv


def fwd(q, k, v, f, beta, c, S0=None):
    q, k, v, f, beta, c, S0 = map(_f64, (q, k, v, f, beta, c, S0))
    B, T, H, dk, dv = _dims(q, v)
    assert k.shape == q.shape and f.shape == q.shape
    assert v.shape == (B, T, H, dv) and beta.shape == (B, T, H) and c.shape == (B, T, H)
    if S0 is not None:
        assert S0.shape == (B, H, dv, dk)
    o = np.zeros((B, T, H, dv))
    ST = np.zeros((B, H, dv, dk))
    r = np.zeros((B, T, H))
    rc = _load().kdo_fwd(B, T, H, dk, dv, _p(q), _p(k), _p(v), _p(f), _p(beta),
                         _p(c), _p(S0), _p(o), _p(ST), _p(r))
    if rc != 0:
        raise RuntimeError("oracle kdo_fwd failed: %d" % rc)
    return o, ST, r


def bwd(q, k, v, f, beta, c, S0, dO, dST=None):
    q, k, v, f, beta, c, S0, dO, dST = map(_f64, (q, k, v, f, beta, c, S0, dO, dST))
    B, T, H, dk, dv = _dims(q, v)
    assert dO.shape == (B, T, H, dv)
    out = dict(dq=np.zeros_like(q), dk=np.zeros_like(k), dv=np.zeros_like(v),
               df=np.zeros_like(f), dbeta=np.zeros_like(beta), dc=np.zeros_like(c),
               dS0=np.zeros((B, H, dv, dk)))
    rc = _load().kdo_bwd(B, T, H, dk, dv, _p(q), _p(k), _p(v), _p(f), _p(beta), _p(c),
                         _p(S0), _p(dO), _p(dST), _p(out["dq"]), _p(out["dk"]),
                         _p(out["dv"]), _p(out["df"]), _p(out["dbeta"]), _p(out["dc"]),
                         _p(out["dS0"]))
    if rc != 0:
        raise RuntimeError("oracle kdo_bwd failed: %d" % rc)
    return out


def gdn2_fwd(q, k, v, alpha, b, w, S0=None):
    q, k, v, alpha, b, w, S0 = map(_f64, (q, k, v, alpha, b, w, S0))
    B, T, H, dk, dv = _dims(q, v)
    assert k.shape == q.shape and alpha.shape == q.shape and b.shape == q.shape
    assert v.shape == (B, T, H, dv) and w.shape == (B, T, H, dv)
    if S0 is not None:
        assert S0.shape == (B, H, dk, dv)
    o = np.zeros((B, T, H, dv))
    ST = np.zeros((B, H, dk, dv))
    rc = _load().gdo_fwd(B, T, H, dk, dv, _p(q), _p(k), _p(v), _p(alpha), _p(b), _p(w),
                         _p(S0), _p(o), _p(ST))
    if rc != 0:
        raise RuntimeError("oracle gdo_fwd failed: %d" % rc)
    return o, ST
