"""MI355X (gfx950) Kronecker delta rule mixer -- thin Python binding.

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libkrondelta.so`` through its C ABI (``include/kron_delta.h``).
PyTorch supplies device memory and the current stream.  If the library is
missing, every entry point raises; there is no CPU fallback.

    o, S_T = fwd(q, k, v, f, beta, c, S0=None)
    grads  = bwd(q, k, v, f, beta, c, S0, dO, dST=None)
    o      = decode(q, k, v, f, beta, c, S)        (S updated in place)
    o, S_T = fwd_varlen(q, k, v, f, beta, c, cu_seqlens, S0=None)   (packed sequences)
    y, S_T = mixer_fwd(raw, params, g, S0=None)      (projections -> gated, normalised read-out)

Shapes: q, k, f [B, T, H, d]; v [B, T, H, d]; beta, c [B, T, H] fp32;
S0 / S_T [B, H, d, d] fp32 (S[i][j], i over values, j over keys).
Dtypes: q, k, v, f (and o, dO, dq, ...) all bfloat16 or all float32.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkrondelta.so")

KD_F32, KD_BF16 = 0, 1
ABI_VERSION = 1
EXPORTED = ("kron_delta_abi_version", "kron_delta_status_string",
            "kron_delta_workspace_bytes", "kron_delta_fwd", "kron_delta_bwd",
            "kron_delta_decode", "kron_delta_fwd_varlen", "kron_delta_gdn2_fwd",
            "kron_delta_fwd_train", "kron_delta_bwd_saved", "kron_delta_mixer_pre",
            "kron_delta_mixer_post", "kron_delta_mixer_fwd", "kron_delta_bwd_noalloc",
            "kron_delta_bwd_status", "kron_delta_bwd_set_wait_limit")
KD_WS_FWD, KD_WS_BWD, KD_WS_MIXER = 0, 1, 2
KD_ERR_SCRATCH = -8     # kron_delta_bwd_noalloc: the problem needs more than its fixed scratch
KD_ERR_TIMEOUT = -9     # kron_delta_bwd_status: a bounded wait of the backward ran out
NOALLOC_SCRATCH_BYTES = 64 << 20


class KronDeltaError(RuntimeError):
    def __init__(self, status: int, what: str, detail: str = ""):
        self.status = status
        super().__init__("%s failed: %s (status %d)%s" % (what, status_string(status), status, detail))


KD_ERR_LAUNCH = -6
SYNC_CHECK_ENV = "KRON_DELTA_SYNC_CHECK"


def _done(st: int, what: str, device=None):
    """Raise for a failed call.  With KRON_DELTA_SYNC_CHECK=1 in the
    environment, also wait for the enqueued work and report a device error
    (a fault in a kernel of this call) against this entry point; skipped while
    the current stream is being captured into a graph."""
    if st != 0:
        raise KronDeltaError(st, what)
    if os.environ.get(SYNC_CHECK_ENV) == "1":
        import torch
        if torch.cuda.is_available() and not torch.cuda.is_current_stream_capturing():
            try:
                torch.cuda.synchronize(device)
            except RuntimeError as e:   # the device reported an error for the enqueued work
                raise KronDeltaError(KD_ERR_LAUNCH, what, " after the launch: %s" % e) from e


class KdDesc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("T", ctypes.c_int32), ("H", ctypes.c_int32),
                ("dk", ctypes.c_int32), ("dv", ctypes.c_int32), ("dtype", ctypes.c_int32)]


class KdMixerParams(ctypes.Structure):
    _fields_ = [("conv_q", ctypes.c_void_p), ("conv_k", ctypes.c_void_p), ("conv_v", ctypes.c_void_p),
                ("conv_size", ctypes.c_int32), ("a_log", ctypes.c_void_p), ("beta_scale", ctypes.c_float),
                ("norm_w", ctypes.c_void_p), ("norm_eps", ctypes.c_float)]


_lib = None


def lib():
    """Load libkrondelta.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libkrondelta.so is not built (run __graft_entry__.build() "
                              "or python delta_rule_recurrent_chunk_amd/build.py)")
        L = ctypes.CDLL(LIB_PATH)
        vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
        dp = ctypes.POINTER(KdDesc)
        L.kron_delta_abi_version.restype = i32
        L.kron_delta_status_string.restype = ctypes.c_char_p
        L.kron_delta_status_string.argtypes = [i32]
        L.kron_delta_workspace_bytes.restype = sz
        L.kron_delta_workspace_bytes.argtypes = [dp, i32]
        L.kron_delta_fwd.restype = i32
        L.kron_delta_fwd.argtypes = [dp] + [vp] * 9 + [vp, sz, vp]
        L.kron_delta_bwd.restype = i32
        L.kron_delta_bwd.argtypes = [dp] + [vp] * 16 + [vp, sz, vp]
        L.kron_delta_bwd_saved.restype = i32
        L.kron_delta_bwd_saved.argtypes = [dp] + [vp] * 16 + [vp, sz, vp]
        L.kron_delta_bwd_noalloc.restype = i32
        L.kron_delta_bwd_noalloc.argtypes = [dp] + [vp] * 16 + [vp]
        L.kron_delta_bwd_status.restype = i32
        L.kron_delta_bwd_status.argtypes = [dp, vp, sz, vp]
        L.kron_delta_bwd_set_wait_limit.restype = None
        L.kron_delta_bwd_set_wait_limit.argtypes = [ctypes.c_uint32]
        L.kron_delta_fwd_train.restype = i32
        L.kron_delta_fwd_train.argtypes = [dp] + [vp] * 9 + [vp, sz, vp]
        L.kron_delta_decode.restype = i32
        L.kron_delta_fwd_varlen.restype = i32
        L.kron_delta_fwd_varlen.argtypes = [dp, vp] + [vp] * 9 + [vp]
        L.kron_delta_decode.argtypes = [dp] + [vp] * 9 + [vp]
        L.kron_delta_gdn2_fwd.restype = i32
        L.kron_delta_gdn2_fwd.argtypes = [dp] + [vp] * 9 + [vp]
        mp = ctypes.POINTER(KdMixerParams)
        L.kron_delta_mixer_pre.restype = i32
        L.kron_delta_mixer_pre.argtypes = [dp, mp] + [vp] * 12 + [vp]
        L.kron_delta_mixer_post.restype = i32
        L.kron_delta_mixer_post.argtypes = [dp, mp] + [vp] * 3 + [vp]
        L.kron_delta_mixer_fwd.restype = i32
        L.kron_delta_mixer_fwd.argtypes = [dp, mp] + [vp] * 10 + [vp, sz, vp]
        if L.kron_delta_abi_version() != ABI_VERSION:
            raise ImportError("libkrondelta.so ABI version mismatch")
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().kron_delta_status_string(int(status)).decode()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dtype_code(torch, dt):
    if dt == torch.bfloat16:
        return KD_BF16
    if dt == torch.float32:
        return KD_F32
    raise TypeError("q, k, v, f must be bfloat16 or float32, got %s" % dt)


def _prep(torch, q, k, v, f, beta, c, S0):
    if not (q.is_cuda and k.is_cuda and v.is_cuda and f.is_cuda):
        raise ValueError("inputs must be device tensors")
    dt = q.dtype
    for name, t in (("k", k), ("v", v), ("f", f)):
        if t.dtype != dt:
            raise TypeError("%s has dtype %s, q has %s" % (name, t.dtype, dt))
    if q.dim() != 4:
        raise ValueError("q must be [B, T, H, d]")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if tuple(k.shape) != (B, T, H, dk) or tuple(f.shape) != (B, T, H, dk) or tuple(v.shape) != (B, T, H, dv):
        raise ValueError("q, k, f must be [B, T, H, dk] and v [B, T, H, dv]")
    if tuple(beta.shape) != (B, T, H) or tuple(c.shape) != (B, T, H):
        raise ValueError("beta and c must be [B, T, H]")
    if beta.dtype != torch.float32 or c.dtype != torch.float32:
        raise TypeError("beta and c must be float32")
    if S0 is not None:
        if tuple(S0.shape) != (B, H, dv, dk) or S0.dtype != torch.float32:
            raise ValueError("S0 must be float32 [B, H, dv, dk]")
        S0 = S0.contiguous()
    desc = KdDesc(B, T, H, dk, dv, _dtype_code(torch, dt))
    return desc, q.contiguous(), k.contiguous(), v.contiguous(), f.contiguous(), \
        beta.contiguous(), c.contiguous(), S0


def fwd(q, k, v, f, beta, c, S0=None, *, return_state=True, workspace=None):
    """Chunkwise forward.  Returns (o, S_T); S_T is None if return_state=False.
    workspace: None (allocated when the shape takes the few-heads path), or a
    uint8 device tensor passed through (an empty one forces the one-launch
    path)."""
    import torch
    L = lib()
    desc, q, k, v, f, beta, c, S0 = _prep(torch, q, k, v, f, beta, c, S0)
    o = torch.empty((desc.B, desc.T, desc.H, desc.dv), dtype=q.dtype, device=q.device)
    ST = torch.empty((desc.B, desc.H, desc.dv, desc.dk), dtype=torch.float32,
                     device=q.device) if return_state else None
    stream = torch.cuda.current_stream(q.device).cuda_stream
    # few heads: the library runs the chunk-parallel preparation when given
    # its workspace (one hand-off image per head and chunk)
    need = int(L.kron_delta_workspace_bytes(ctypes.byref(desc), 0)) if workspace is None else 0
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    wsp = _ptr(workspace) if workspace is not None else None
    wsb = workspace.numel() if workspace is not None else 0
    st = L.kron_delta_fwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(f), _ptr(beta),
                          _ptr(c), _ptr(S0), _ptr(o), _ptr(ST), wsp, wsb, ctypes.c_void_p(stream))
    _done(st, "kron_delta_fwd")
    return o, ST


def fwd_varlen(q, k, v, f, beta, c, cu_seqlens, S0=None, *, return_state=True):
    """Forward over packed sequences: q, k, f [T, H, dk], v [T, H, dv], beta, c
    [T, H] (all sequences concatenated along T); cu_seqlens int32 [N + 1] on
    the device.  Returns (o [T, H, dv], S_T [N, H, dv, dk] or None)."""
    import torch
    L = lib()
    if q.dim() != 3:
        raise ValueError("packed q must be [T, H, d]")
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or not cu_seqlens.is_cuda:
        raise ValueError("cu_seqlens must be an int32 device vector [N + 1]")
    N = cu_seqlens.numel() - 1
    if N < 1:
        raise ValueError("cu_seqlens needs at least two entries")
    S0b = None
    if S0 is not None:
        S0b = S0
    desc, q4, k4, v4, f4, b4, c4, _ = _prep(torch, q[None], k[None], v[None], f[None], beta[None],
                                            c[None], None)
    T, H, dk, dv = desc.T, desc.H, desc.dk, desc.dv
    desc = KdDesc(N, T, H, dk, dv, desc.dtype)
    if S0b is not None:
        if tuple(S0b.shape) != (N, H, dv, dk) or S0b.dtype != torch.float32:
            raise ValueError("S0 must be float32 [N, H, dv, dk]")
        S0b = S0b.contiguous()
    cu = cu_seqlens.contiguous()
    o = torch.empty((T, H, dv), dtype=q.dtype, device=q.device)
    ST = torch.empty((N, H, dv, dk), dtype=torch.float32, device=q.device) if return_state else None
    stream = torch.cuda.current_stream(q.device).cuda_stream
    st = L.kron_delta_fwd_varlen(ctypes.byref(desc), _ptr(cu), _ptr(q4), _ptr(k4), _ptr(v4), _ptr(f4),
                                 _ptr(b4), _ptr(c4), _ptr(S0b), _ptr(o), _ptr(ST), ctypes.c_void_p(stream))
    _done(st, "kron_delta_fwd_varlen")
    return o, ST


def decode(q, k, v, f, beta, c, S, *, S_out=None):
    """Token-by-token recurrence on a carried state (serving).  q, k, v, f are
    [B, T, H, d] for the T new tokens (typically T = 1); S [B, H, d, d] fp32 is
    the state before them.  Returns o; the state after the last token goes to
    S_out, or into S itself (in place) when S_out is None."""
    import torch
    L = lib()
    desc, q, k, v, f, beta, c, S = _prep(torch, q, k, v, f, beta, c, S)
    if S is None:
        raise ValueError("decode needs the carried state S")
    out = S if S_out is None else S_out
    if tuple(out.shape) != tuple(S.shape) or out.dtype != torch.float32 or not out.is_contiguous():
        raise ValueError("S_out must be a contiguous float32 tensor shaped like S")
    o = torch.empty((desc.B, desc.T, desc.H, desc.dv), dtype=q.dtype, device=q.device)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    st = L.kron_delta_decode(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(f), _ptr(beta),
                             _ptr(c), _ptr(S), _ptr(o), _ptr(out), ctypes.c_void_p(stream))
    _done(st, "kron_delta_decode")
    return o


def workspace_bytes(B, T, H, d, dtype_code, with_backward=True) -> int:
    desc = KdDesc(B, T, H, d, d, dtype_code)
    return int(lib().kron_delta_workspace_bytes(ctypes.byref(desc), 1 if with_backward else 0))


def fwd_train(q, k, v, f, beta, c, S0=None, *, return_state=True, workspace=None):
    """Forward for training: returns (o, S_T, workspace), the workspace holding
    the per-chunk records that bwd(..., workspace=workspace, saved=True) reads
    instead of recomputing the forward."""
    import torch
    L = lib()
    desc, q, k, v, f, beta, c, S0 = _prep(torch, q, k, v, f, beta, c, S0)
    o = torch.empty((desc.B, desc.T, desc.H, desc.dv), dtype=q.dtype, device=q.device)
    ST = torch.empty((desc.B, desc.H, desc.dv, desc.dk), dtype=torch.float32,
                     device=q.device) if return_state else None
    need = int(L.kron_delta_workspace_bytes(ctypes.byref(desc), 1))
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    st = L.kron_delta_fwd_train(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(f), _ptr(beta),
                                _ptr(c), _ptr(S0), _ptr(o), _ptr(ST), _ptr(workspace),
                                workspace.numel() * workspace.element_size(), ctypes.c_void_p(stream))
    _done(st, "kron_delta_fwd_train")
    return o, ST, workspace


def bwd(q, k, v, f, beta, c, S0, dO, dST=None, *, want_dS0=True, workspace=None, saved=False):
    """Gate-aware backward.  Returns a dict with dq, dk, dv, df, dbeta, dc, dS0.

    saved=True starts from the records that fwd_train left in `workspace`
    (same inputs, same workspace) instead of recomputing the forward."""
    import torch
    L = lib()
    desc, q, k, v, f, beta, c, S0 = _prep(torch, q, k, v, f, beta, c, S0)
    if dO.dtype != q.dtype or tuple(dO.shape) != (desc.B, desc.T, desc.H, desc.dv):
        raise ValueError("dO must match o's shape and dtype")
    dO = dO.contiguous()
    if dST is not None:
        if tuple(dST.shape) != (desc.B, desc.H, desc.dv, desc.dk) or dST.dtype != torch.float32:
            raise ValueError("dST must be float32 [B, H, dv, dk]")
        dST = dST.contiguous()
    dev = q.device
    out = dict(dq=torch.empty_like(q), dk=torch.empty_like(k), dv=torch.empty_like(v),
               df=torch.empty_like(f), dbeta=torch.empty_like(beta), dc=torch.empty_like(c),
               dS0=torch.empty((desc.B, desc.H, desc.dv, desc.dk), dtype=torch.float32, device=dev)
               if want_dS0 else None)
    need = int(L.kron_delta_workspace_bytes(ctypes.byref(desc), 1))
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        if saved:
            raise ValueError("saved=True needs the workspace filled by fwd_train")
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    fn = L.kron_delta_bwd_saved if saved else L.kron_delta_bwd
    st = fn(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(f), _ptr(beta),
            _ptr(c), _ptr(S0), _ptr(dO), _ptr(dST), _ptr(out["dq"]), _ptr(out["dk"]),
            _ptr(out["dv"]), _ptr(out["df"]), _ptr(out["dbeta"]), _ptr(out["dc"]),
            _ptr(out["dS0"]), _ptr(workspace), need, ctypes.c_void_p(stream))
    _done(st, "kron_delta_bwd_saved" if saved else "kron_delta_bwd")
    return out


def bwd_status(q, workspace=None):
    """kron_delta_bwd_status for the backward that ran on `workspace` (None:
    kron_delta_bwd_noalloc's scratch) with inputs shaped like q [B, T, H, d]:
    0 or KD_ERR_TIMEOUT.  Waits for the current stream."""
    import torch
    L = lib()
    B, T, Hq, dq_ = q.shape
    desc = KdDesc(B, T, Hq, dq_, dq_, _dtype_code(torch, q.dtype))
    stream = torch.cuda.current_stream(q.device).cuda_stream
    wsp = _ptr(workspace) if workspace is not None else None
    wsb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    return int(L.kron_delta_bwd_status(ctypes.byref(desc), wsp, wsb, ctypes.c_void_p(stream)))


def bwd_set_wait_limit(polls: int) -> None:
    """kron_delta_bwd_set_wait_limit (0: the default bound)."""
    lib().kron_delta_bwd_set_wait_limit(int(polls))


def bwd_noalloc(q, k, v, f, beta, c, S0, dO, dST=None, *, want_dS0=True, out=None):
    """kron_delta_bwd_noalloc: the gate-aware backward with the library's
    fixed scratch as its workspace (no workspace argument; raises
    KronDeltaError with KD_ERR_SCRATCH when the problem needs more).  `out`
    may hold preallocated gradient tensors (dict as returned by bwd)."""
    import torch
    L = lib()
    desc, q, k, v, f, beta, c, S0 = _prep(torch, q, k, v, f, beta, c, S0)
    if dO.dtype != q.dtype or tuple(dO.shape) != (desc.B, desc.T, desc.H, desc.dv):
        raise ValueError("dO must match o's shape and dtype")
    dO = dO.contiguous()
    if dST is not None:
        if tuple(dST.shape) != (desc.B, desc.H, desc.dv, desc.dk) or dST.dtype != torch.float32:
            raise ValueError("dST must be float32 [B, H, dv, dk]")
        dST = dST.contiguous()
    dev = q.device
    if out is None:
        out = dict(dq=torch.empty_like(q), dk=torch.empty_like(k), dv=torch.empty_like(v),
                   df=torch.empty_like(f), dbeta=torch.empty_like(beta), dc=torch.empty_like(c),
                   dS0=torch.empty((desc.B, desc.H, desc.dv, desc.dk), dtype=torch.float32, device=dev)
                   if want_dS0 else None)
    stream = torch.cuda.current_stream(dev).cuda_stream
    st = L.kron_delta_bwd_noalloc(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(f), _ptr(beta),
                                  _ptr(c), _ptr(S0), _ptr(dO), _ptr(dST), _ptr(out["dq"]), _ptr(out["dk"]),
                                  _ptr(out["dv"]), _ptr(out["df"]), _ptr(out["dbeta"]), _ptr(out["dc"]),
                                  _ptr(out["dS0"]), ctypes.c_void_p(stream))
    _done(st, "kron_delta_bwd_noalloc")
    return out


def gdn2_fwd(q, k, v, alpha, b, w, S0=None, *, return_state=True):
    """Gated Delta Rule-2 forward (bf16, d = 128): q, k, alpha, b [B, T, H, dk],
    v, w [B, T, H, dv]; S0 fp32 [B, H, dk, dv] or None.  Returns (o, S_T)."""
    import torch
    L = lib()
    dt = q.dtype
    for name, t in (("k", k), ("v", v), ("alpha", alpha), ("b", b), ("w", w)):
        if t.dtype != dt:
            raise TypeError("%s has dtype %s, q has %s" % (name, t.dtype, dt))
    if q.dim() != 4:
        raise ValueError("q must be [B, T, H, d]")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    for name, t in (("k", k), ("alpha", alpha), ("b", b)):
        if tuple(t.shape) != (B, T, H, dk):
            raise ValueError("%s must be [B, T, H, dk]" % name)
    if tuple(w.shape) != (B, T, H, dv) or tuple(v.shape) != (B, T, H, dv):
        raise ValueError("v and w must be [B, T, H, dv]")
    if S0 is not None:
        if tuple(S0.shape) != (B, H, dk, dv) or S0.dtype != torch.float32:
            raise ValueError("S0 must be float32 [B, H, dk, dv]")
        S0 = S0.contiguous()
    desc = KdDesc(B, T, H, dk, dv, _dtype_code(torch, dt))
    q, k, v, alpha, b, w = (t.contiguous() for t in (q, k, v, alpha, b, w))
    o = torch.empty((B, T, H, dv), dtype=dt, device=q.device)
    ST = torch.empty((B, H, dk, dv), dtype=torch.float32, device=q.device) if return_state else None
    stream = torch.cuda.current_stream(q.device).cuda_stream
    st = L.kron_delta_gdn2_fwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(b),
                               _ptr(w), _ptr(S0), _ptr(o), _ptr(ST), ctypes.c_void_p(stream))
    _done(st, "kron_delta_gdn2_fwd")
    return o, ST


def _mixer_params(torch, H, dk, dv, conv_q=None, conv_k=None, conv_v=None, a_log=None, norm_w=None,
                  beta_scale=1.0, norm_eps=1e-5):
    """KdMixerParams for the given fp32 device tensors (kept alive by the caller)."""
    K = 0
    for name, t, d in (("conv_q", conv_q, dk), ("conv_k", conv_k, dk), ("conv_v", conv_v, dv)):
        if t is None:
            continue
        if t.dtype != torch.float32 or t.dim() != 3 or tuple(t.shape[:2]) != (H, d) or not t.is_contiguous():
            raise ValueError("%s must be a contiguous float32 [H, d, conv_size] tensor" % name)
        if K and t.shape[2] != K:
            raise ValueError("conv_q, conv_k and conv_v must have the same width")
        K = t.shape[2]
    if a_log is not None and (a_log.dtype != torch.float32 or tuple(a_log.shape) != (H,)):
        raise ValueError("a_log must be float32 [H]")
    if norm_w is not None and (norm_w.dtype != torch.float32 or tuple(norm_w.shape) != (H, dv)
                               or not norm_w.is_contiguous()):
        raise ValueError("norm_w must be a contiguous float32 [H, dv] tensor")
    return KdMixerParams(_ptr(conv_q), _ptr(conv_k), _ptr(conv_v), K, _ptr(a_log), float(beta_scale),
                         _ptr(norm_w), float(norm_eps))


def _raw_desc(torch, q_raw, k_raw, v_raw, f_raw, beta_raw, c_raw):
    dt = q_raw.dtype
    for name, t in (("k_raw", k_raw), ("v_raw", v_raw), ("f_raw", f_raw)):
        if t.dtype != dt or not t.is_cuda:
            raise TypeError("%s must be a device tensor of q_raw's dtype" % name)
    B, T, H, dk = q_raw.shape
    dv = v_raw.shape[-1]
    if tuple(k_raw.shape) != (B, T, H, dk) or tuple(f_raw.shape) != (B, T, H, dk):
        raise ValueError("q_raw, k_raw, f_raw must be [B, T, H, dk]")
    for name, t in (("beta_raw", beta_raw), ("c_raw", c_raw)):
        if t.dtype != torch.float32 or tuple(t.shape) != (B, T, H):
            raise ValueError("%s must be float32 [B, T, H]" % name)
    return KdDesc(B, T, H, dk, dv, _dtype_code(torch, dt))


def mixer_pre(q_raw, k_raw, v_raw, f_raw, beta_raw, c_raw, conv_q, conv_k, conv_v, a_log, *,
              beta_scale=1.0):
    """The rule's inputs from the projections (conv, SiLU, L2 norm; gates).
    Returns q, k, v, f (dtype of the projections) and beta, c (float32)."""
    import torch
    L = lib()
    desc = _raw_desc(torch, q_raw, k_raw, v_raw, f_raw, beta_raw, c_raw)
    p = _mixer_params(torch, desc.H, desc.dk, desc.dv, conv_q, conv_k, conv_v, a_log, beta_scale=beta_scale)
    ins = [t.contiguous() for t in (q_raw, k_raw, v_raw, f_raw, beta_raw, c_raw)]
    q, k, v, f = (torch.empty_like(t) for t in ins[:4])
    beta, c = torch.empty_like(ins[4]), torch.empty_like(ins[5])
    stream = torch.cuda.current_stream(q_raw.device).cuda_stream
    st = L.kron_delta_mixer_pre(ctypes.byref(desc), ctypes.byref(p), *[_ptr(t) for t in ins],
                                _ptr(q), _ptr(k), _ptr(v), _ptr(f), _ptr(beta), _ptr(c), ctypes.c_void_p(stream))
    _done(st, "kron_delta_mixer_pre")
    return q, k, v, f, beta, c


def mixer_post(o, g, norm_w, *, norm_eps=1e-5):
    """Gated per-head RMSNorm of the read-out: o / rms(o) * norm_w[h] * sigmoid(g)."""
    import torch
    L = lib()
    if g.dtype != o.dtype or tuple(g.shape) != tuple(o.shape) or o.dim() != 4:
        raise ValueError("o and g must be [B, T, H, dv] of one dtype")
    B, T, H, dv = o.shape
    desc = KdDesc(B, T, H, dv, dv, _dtype_code(torch, o.dtype))
    p = _mixer_params(torch, H, dv, dv, norm_w=norm_w, norm_eps=norm_eps)
    o, g = o.contiguous(), g.contiguous()
    y = torch.empty_like(o)
    stream = torch.cuda.current_stream(o.device).cuda_stream
    st = L.kron_delta_mixer_post(ctypes.byref(desc), ctypes.byref(p), _ptr(o), _ptr(g), _ptr(y),
                                 ctypes.c_void_p(stream))
    _done(st, "kron_delta_mixer_post")
    return y


def mixer_fwd(q_raw, k_raw, v_raw, f_raw, beta_raw, c_raw, g, conv_q, conv_k, conv_v, a_log, norm_w,
              S0=None, *, beta_scale=1.0, norm_eps=1e-5, return_state=True, workspace=None):
    """The mixer forward from the projections: pre-processing, the rule, and the
    gated RMSNorm of the read-out.  Returns (y, S_T)."""
    import torch
    L = lib()
    desc = _raw_desc(torch, q_raw, k_raw, v_raw, f_raw, beta_raw, c_raw)
    B, T, H, dk, dv = desc.B, desc.T, desc.H, desc.dk, desc.dv
    if g.dtype != q_raw.dtype or tuple(g.shape) != (B, T, H, dv):
        raise ValueError("g must be [B, T, H, dv] of the projections' dtype")
    if S0 is not None:
        if tuple(S0.shape) != (B, H, dv, dk) or S0.dtype != torch.float32:
            raise ValueError("S0 must be float32 [B, H, dv, dk]")
        S0 = S0.contiguous()
    p = _mixer_params(torch, H, dk, dv, conv_q, conv_k, conv_v, a_log, norm_w, beta_scale, norm_eps)
    ins = [t.contiguous() for t in (q_raw, k_raw, v_raw, f_raw, beta_raw, c_raw, g)]
    y = torch.empty((B, T, H, dv), dtype=q_raw.dtype, device=q_raw.device)
    ST = torch.empty((B, H, dv, dk), dtype=torch.float32, device=q_raw.device) if return_state else None
    need = int(L.kron_delta_workspace_bytes(ctypes.byref(desc), KD_WS_MIXER))
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q_raw.device)
    stream = torch.cuda.current_stream(q_raw.device).cuda_stream
    st = L.kron_delta_mixer_fwd(ctypes.byref(desc), ctypes.byref(p), *[_ptr(t) for t in ins], _ptr(S0), _ptr(y),
                                _ptr(ST), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                ctypes.c_void_p(stream))
    _done(st, "kron_delta_mixer_fwd")
    return y, ST

