"""Python binding of the MI355X exact-attention library (libfa_mi355x.so).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in include/fa.h.  PyTorch provides device
memory and the current stream.  If the shared library is missing, every call
raises; there is no fallback implementation.

Low level: one function per exported symbol (fa_fwd, fa_bwd, the three
backward stages, fa_fwd_dropout, fa_bwd_dropout, fa_fwd_decode,
fa_decode_workspace_bytes, fa_fwd_f32, fa_bwd_f32, fa_bwd_workspace_bytes,
fa_fwd_query_rows, fa_strerror, fa_version) takes the C arguments as they are (pointers as
integers).  High level: fwd, bwd, bwd_stages, fwd_dropout, bwd_dropout,
decode, fwd_f32 and bwd_f32 take torch tensors, allocate the outputs and
raise FAError on a nonzero status.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfa_mi355x.so")

FA_OK = 0
STATUS_NAMES = {
    0: "FA_OK", -1: "FA_ERR_NULL", -2: "FA_ERR_SHAPE", -3: "FA_ERR_HEADDIM",
    -4: "FA_ERR_ALIGN", -5: "FA_ERR_ALIAS", -6: "FA_ERR_WORKSPACE", -7: "FA_ERR_FLAG",
    -8: "FA_ERR_LAUNCH", -9: "FA_ERR_UNSUPPORTED", -10: "FA_ERR_SCALE", -11: "FA_ERR_DROPOUT",
}
EXPORTED = ("fa_fwd", "fa_bwd", "fa_bwd_preprocess", "fa_bwd_dkdv", "fa_bwd_dq",
            "fa_fwd_dropout", "fa_bwd_dropout", "fa_fwd_decode", "fa_decode_workspace_bytes",
            "fa_bwd_workspace_bytes", "fa_fwd_query_rows", "fa_fwd_f32",
            "fa_bwd_f32", "fa_strerror", "fa_version")

_lib = None


class FAError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)} ({fa_strerror(status)})")


def lib() -> ctypes.CDLL:
    """Load the shared library once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing; build it with exact_io_aware_18_amd.build.build()")
        L = ctypes.CDLL(LIB_PATH)
        P, I, F, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        U64 = ctypes.c_ulonglong
        L.fa_fwd.argtypes = [P, P, P, P, P, I, I, I, I, F, I, P, P]
        L.fa_fwd.restype = I
        L.fa_bwd.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, F, I, P, P, Z, P]
        L.fa_bwd.restype = I
        L.fa_bwd_preprocess.argtypes = [P, P, I, I, I, I, P, Z, P]
        L.fa_bwd_preprocess.restype = I
        L.fa_bwd_dkdv.argtypes = [P, P, P, P, P, P, P, I, I, I, I, F, I, P, P, Z, P]
        L.fa_bwd_dkdv.restype = I
        L.fa_bwd_dq.argtypes = [P, P, P, P, P, P, I, I, I, I, F, I, P, P, Z, P]
        L.fa_bwd_dq.restype = I
        L.fa_fwd_dropout.argtypes = [P, P, P, P, P, I, I, I, I, F, I, P, F, U64, P]
        L.fa_fwd_dropout.restype = I
        L.fa_bwd_dropout.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, F, I, P, F, U64, P, Z, P]
        L.fa_bwd_dropout.restype = I
        L.fa_fwd_decode.argtypes = [P, P, P, P, P, I, I, I, I, I, F, I, P, Z, P]
        L.fa_fwd_decode.restype = I
        L.fa_decode_workspace_bytes.argtypes = [I, I, I, I, I]
        L.fa_decode_workspace_bytes.restype = Z
        L.fa_fwd_f32.argtypes = L.fa_fwd.argtypes
        L.fa_fwd_f32.restype = I
        L.fa_bwd_f32.argtypes = L.fa_bwd.argtypes
        L.fa_bwd_f32.restype = I
        L.fa_bwd_workspace_bytes.argtypes = [I, I, I, I]
        L.fa_fwd_query_rows.argtypes = [I, I, I, I, I, I, I]
        L.fa_fwd_query_rows.restype = I
        L.fa_bwd_workspace_bytes.restype = Z
        L.fa_strerror.argtypes = [I]
        L.fa_strerror.restype = ctypes.c_char_p
        L.fa_version.argtypes = []
        L.fa_version.restype = I
        _lib = L
    return _lib


# ---- the C ABI, one Python function per exported symbol ----------------------
def fa_fwd(q, k, v, o, lse, B, H, N, d, scale, causal, blockmask, stream) -> int:
    return lib().fa_fwd(q, k, v, o, lse, B, H, N, d, scale, causal, blockmask, stream)


def fa_bwd(q, k, v, o, lse, dout, dq, dk, dv, B, H, N, d, scale, causal, blockmask,
           workspace, workspace_bytes, stream) -> int:
    return lib().fa_bwd(q, k, v, o, lse, dout, dq, dk, dv, B, H, N, d, scale, causal,
                        blockmask, workspace, workspace_bytes, stream)


def fa_bwd_preprocess(o, dout, B, H, N, d, workspace, workspace_bytes, stream) -> int:
    return lib().fa_bwd_preprocess(o, dout, B, H, N, d, workspace, workspace_bytes, stream)


def fa_bwd_dkdv(q, k, v, lse, dout, dk, dv, B, H, N, d, scale, causal, blockmask, workspace,
                workspace_bytes, stream) -> int:
    return lib().fa_bwd_dkdv(q, k, v, lse, dout, dk, dv, B, H, N, d, scale, causal, blockmask,
                             workspace, workspace_bytes, stream)


def fa_bwd_dq(q, k, v, lse, dout, dq, B, H, N, d, scale, causal, blockmask, workspace,
              workspace_bytes, stream) -> int:
    return lib().fa_bwd_dq(q, k, v, lse, dout, dq, B, H, N, d, scale, causal, blockmask,
                           workspace, workspace_bytes, stream)


def fa_fwd_dropout(q, k, v, o, lse, B, H, N, d, scale, causal, blockmask, p_drop, seed,
                   stream) -> int:
    return lib().fa_fwd_dropout(q, k, v, o, lse, B, H, N, d, scale, causal, blockmask, p_drop,
                                seed, stream)


def fa_bwd_dropout(q, k, v, o, lse, dout, dq, dk, dv, B, H, N, d, scale, causal, blockmask,
                   p_drop, seed, workspace, workspace_bytes, stream) -> int:
    return lib().fa_bwd_dropout(q, k, v, o, lse, dout, dq, dk, dv, B, H, N, d, scale, causal,
                                blockmask, p_drop, seed, workspace, workspace_bytes, stream)


def fa_fwd_decode(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, workspace, workspace_bytes,
                  stream) -> int:
    return lib().fa_fwd_decode(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, workspace,
                               workspace_bytes, stream)


def fa_decode_workspace_bytes(B, H, Nq, Nk, d) -> int:
    return lib().fa_decode_workspace_bytes(B, H, Nq, Nk, d)


def fa_fwd_f32(q, k, v, o, lse, B, H, N, d, scale, causal, blockmask, stream) -> int:
    return lib().fa_fwd_f32(q, k, v, o, lse, B, H, N, d, scale, causal, blockmask, stream)


def fa_bwd_f32(q, k, v, o, lse, dout, dq, dk, dv, B, H, N, d, scale, causal, blockmask,
               workspace, workspace_bytes, stream) -> int:
    return lib().fa_bwd_f32(q, k, v, o, lse, dout, dq, dk, dv, B, H, N, d, scale, causal,
                            blockmask, workspace, workspace_bytes, stream)


def fa_bwd_workspace_bytes(B, H, N, d) -> int:
    return lib().fa_bwd_workspace_bytes(B, H, N, d)


def fa_fwd_query_rows(B, H, N, d, causal, has_blockmask, dropout) -> int:
    return lib().fa_fwd_query_rows(B, H, N, d, int(causal), int(has_blockmask), int(dropout))


def fa_strerror(status: int) -> str:
    return lib().fa_strerror(status).decode()


def fa_version() -> int:
    return lib().fa_version()


# ---- tensor-level wrappers ---------------------------------------------------
def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    import torch

    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _check(status: int, where: str):
    if status != FA_OK:
        raise FAError(status, where)


def _shape(q):
    if q.dim() != 4:
        raise ValueError("tensors must be [B, H, N, d]")
    return tuple(int(x) for x in q.shape)


def fwd(q, k, v, scale, causal=False, blockmask=None, out=None, lse=None, stream=None):
    """bf16 forward: returns (O bf16 [B,H,N,d], lse fp32 [B,H,N])."""
    import torch

    B, H, N, d = _shape(q)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _check(fa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, N, d, float(scale),
                  int(causal), _ptr(blockmask), _stream(stream)), "fa_fwd")
    return out, lse


def bwd(q, k, v, o, lse, dout, scale, causal=False, blockmask=None, grads=None,
        workspace=None, stream=None):
    """bf16 backward: returns (dQ, dK, dV), fp32 [B,H,N,d]."""
    import torch

    B, H, N, d = _shape(q)
    if grads is None:
        grads = tuple(torch.empty(q.shape, dtype=torch.float32, device=q.device) for _ in range(3))
    dq, dk, dv = grads
    wsb = fa_bwd_workspace_bytes(B, H, N, d)
    if workspace is None:
        workspace = torch.empty(max(wsb, 1), dtype=torch.uint8, device=q.device)
    _check(fa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk),
                  _ptr(dv), B, H, N, d, float(scale), int(causal), _ptr(blockmask),
                  _ptr(workspace), workspace.numel() * workspace.element_size(),
                  _stream(stream)), "fa_bwd")
    return dq, dk, dv


def bwd_stages(q, k, v, o, lse, dout, scale, causal=False, blockmask=None, grads=None,
               workspace=None, stream=None):
    """The same backward as bwd() through its three stage calls, in order."""
    import torch

    B, H, N, d = _shape(q)
    if grads is None:
        grads = tuple(torch.empty(q.shape, dtype=torch.float32, device=q.device) for _ in range(3))
    dq, dk, dv = grads
    wsb = fa_bwd_workspace_bytes(B, H, N, d)
    if workspace is None:
        workspace = torch.empty(max(wsb, 1), dtype=torch.uint8, device=q.device)
    wn = workspace.numel() * workspace.element_size()
    s = _stream(stream)
    _check(fa_bwd_preprocess(_ptr(o), _ptr(dout), B, H, N, d, _ptr(workspace), wn, s),
           "fa_bwd_preprocess")
    _check(fa_bwd_dkdv(_ptr(q), _ptr(k), _ptr(v), _ptr(lse), _ptr(dout), _ptr(dk), _ptr(dv), B, H,
                       N, d, float(scale), int(causal), _ptr(blockmask), _ptr(workspace), wn, s),
           "fa_bwd_dkdv")
    _check(fa_bwd_dq(_ptr(q), _ptr(k), _ptr(v), _ptr(lse), _ptr(dout), _ptr(dq), B, H, N, d,
                     float(scale), int(causal), _ptr(blockmask), _ptr(workspace), wn, s),
           "fa_bwd_dq")
    return dq, dk, dv


def fwd_dropout(q, k, v, scale, p_drop, seed, causal=False, blockmask=None, out=None, lse=None,
                stream=None):
    """bf16 forward with dropout on P: returns (O bf16, lse fp32)."""
    import torch

    B, H, N, d = _shape(q)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _check(fa_fwd_dropout(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, N, d, float(scale),
                          int(causal), _ptr(blockmask), float(p_drop), int(seed), _stream(stream)),
           "fa_fwd_dropout")
    return out, lse


def bwd_dropout(q, k, v, o, lse, dout, scale, p_drop, seed, causal=False, blockmask=None,
                grads=None, workspace=None, stream=None):
    """bf16 backward of fwd_dropout (same p_drop and seed): returns (dQ, dK, dV), fp32."""
    import torch

    B, H, N, d = _shape(q)
    if grads is None:
        grads = tuple(torch.empty(q.shape, dtype=torch.float32, device=q.device) for _ in range(3))
    dq, dk, dv = grads
    wsb = fa_bwd_workspace_bytes(B, H, N, d)
    if workspace is None:
        workspace = torch.empty(max(wsb, 1), dtype=torch.uint8, device=q.device)
    _check(fa_bwd_dropout(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq),
                          _ptr(dk), _ptr(dv), B, H, N, d, float(scale), int(causal),
                          _ptr(blockmask), float(p_drop), int(seed), _ptr(workspace),
                          workspace.numel() * workspace.element_size(), _stream(stream)),
           "fa_bwd_dropout")
    return dq, dk, dv


def decode(q, k, v, scale, causal=False, out=None, lse=None, workspace=None, stream=None):
    """bf16 decode: q [B,H,Nq,d] against k, v [B,H,Nk,d]; returns (O bf16, lse fp32)."""
    import torch

    B, H, Nq, d = _shape(q)
    Nk = int(k.shape[2])
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = torch.empty(max(fa_decode_workspace_bytes(B, H, Nq, Nk, d), 1), dtype=torch.uint8,
                                device=q.device)
    _check(fa_fwd_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, Nq, Nk, d,
                         float(scale), int(causal), _ptr(workspace),
                         workspace.numel() * workspace.element_size(), _stream(stream)),
           "fa_fwd_decode")
    return out, lse


def fwd_f32(q, k, v, scale, causal=False, blockmask=None, out=None, lse=None, stream=None):
    """fp32 forward: returns (O fp32, lse fp32)."""
    import torch

    B, H, N, d = _shape(q)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _check(fa_fwd_f32(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, N, d, float(scale),
                      int(causal), _ptr(blockmask), _stream(stream)), "fa_fwd_f32")
    return out, lse


def bwd_f32(q, k, v, o, lse, dout, scale, causal=False, blockmask=None, grads=None,
            workspace=None, stream=None):
    """fp32 backward: returns (dQ, dK, dV), fp32."""
    import torch

    B, H, N, d = _shape(q)
    if grads is None:
        grads = tuple(torch.empty_like(q) for _ in range(3))
    dq, dk, dv = grads
    wsb = fa_bwd_workspace_bytes(B, H, N, d)
    if workspace is None:
        workspace = torch.empty(max(wsb, 1), dtype=torch.uint8, device=q.device)
    _check(fa_bwd_f32(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq),
                      _ptr(dk), _ptr(dv), B, H, N, d, float(scale), int(causal), _ptr(blockmask),
                      _ptr(workspace), workspace.numel() * workspace.element_size(),
                      _stream(stream)), "fa_bwd_f32")
    return dq, dk, dv
