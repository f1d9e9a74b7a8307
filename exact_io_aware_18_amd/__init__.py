"""Python binding of the MI355X exact-attention library (libfa_mi355x.so).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in include/fa.h.  PyTorch provides device
memory and the current stream.  If the shared library is missing, every call
raises; there is no fallback implementation.

Low level: one function per exported symbol (fa_fwd, fa_bwd, the three
backward stages, fa_bwd_noalloc, fa_bwd_noalloc_max_rows, fa_fwd_dropout, fa_bwd_dropout, fa_fwd_decode,
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
    -12: "FA_ERR_SCRATCH",
}
EXPORTED = ("fa_fwd", "fa_bwd", "fa_bwd_noalloc", "fa_bwd_noalloc_max_rows", "fa_bwd_preprocess", "fa_bwd_dkdv", "fa_bwd_dq",
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
        L.fa_bwd_noalloc.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, F, I, P, P]
        L.fa_bwd_noalloc.restype = I
        L.fa_bwd_noalloc_max_rows.argtypes = []
        L.fa_bwd_noalloc_max_rows.restype = Z
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


def fa_bwd_noalloc(q, k, v, o, lse, dout, dq, dk, dv, B, H, N, d, scale, causal, blockmask,
                   stream) -> int:
    return lib().fa_bwd_noalloc(q, k, v, o, lse, dout, dq, dk, dv, B, H, N, d, scale, causal,
                                blockmask, stream)


def fa_bwd_noalloc_max_rows() -> int:
    return lib().fa_bwd_noalloc_max_rows()


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
# The C ABI reads raw pointers as contiguous [B, H, N, d] tensors of a fixed
# dtype, so the wrappers check every tensor before a call: rank and shape
# agreement, dtype, contiguity, then device.  Device placement is checked last
# so that every other rejection can be exercised with CPU tensors.
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


class _Args:
    """Collects the tensors of one call and validates them together."""

    def __init__(self, where: str):
        self.where = where
        self.tensors = []  # (name, tensor)

    def tensor(self, name, t, shape, dtypes):
        import torch

        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{self.where}: {name} must be a torch.Tensor")
        if tuple(t.shape) != tuple(shape):
            raise ValueError(f"{self.where}: {name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
        if t.dtype not in dtypes:
            names = " or ".join(str(d).replace("torch.", "") for d in dtypes)
            raise ValueError(f"{self.where}: {name} has dtype {str(t.dtype).replace('torch.', '')}, "
                             f"expected {names}")
        if not t.is_contiguous():
            raise ValueError(f"{self.where}: {name} must be contiguous ([B, H, N, d] row-major)")
        self.tensors.append((name, t))
        return t

    def devices(self):
        """Every tensor on one GPU; returns that device."""
        dev = None
        for name, t in self.tensors:
            if not t.is_cuda:
                raise ValueError(f"{self.where}: {name} must be on a GPU device, got {t.device}")
            if dev is None:
                dev = t.device
            elif t.device != dev:
                raise ValueError(f"{self.where}: {name} is on {t.device}, the other tensors on {dev}")
        return dev


def _dt(kind):
    import torch

    return {"bf16": (torch.bfloat16,), "f32": (torch.float32,),
            "mask": (torch.uint8, torch.bool)}[kind]


def _mask_shape(N):
    nb = (N + 127) // 128
    return (nb, nb)


def _fwd_args(where, q, k, v, blockmask, out, lse, kind):
    """Validate a forward call; allocate out / lse when not given."""
    import torch

    a = _Args(where)
    shp = _shape(q)
    B, H, N, d = shp
    a.tensor("q", q, shp, _dt(kind))
    a.tensor("k", k, shp, _dt(kind))
    a.tensor("v", v, shp, _dt(kind))
    if blockmask is not None:
        a.tensor("blockmask", blockmask, _mask_shape(N), _dt("mask"))
    if out is not None:
        a.tensor("out", out, shp, _dt(kind))
    if lse is not None:
        a.tensor("lse", lse, (B, H, N), _dt("f32"))
    dev = a.devices()
    if out is None:
        out = torch.empty(shp, dtype=q.dtype, device=dev)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    return shp, out, lse


def _bwd_args(where, q, k, v, o, lse, dout, blockmask, grads, workspace, kind, ws_bytes,
              need_ws=True):
    """Validate a backward call; allocate the gradients and the workspace
    when not given."""
    import torch

    a = _Args(where)
    shp = _shape(q)
    B, H, N, d = shp
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout)):
        a.tensor(name, t, shp, _dt(kind))
    a.tensor("lse", lse, (B, H, N), _dt("f32"))
    if blockmask is not None:
        a.tensor("blockmask", blockmask, _mask_shape(N), _dt("mask"))
    if grads is not None:
        if len(grads) != 3:
            raise ValueError(f"{where}: grads must be (dq, dk, dv)")
        for name, t in zip(("dq", "dk", "dv"), grads):
            a.tensor(name, t, shp, _dt("f32"))
    if workspace is not None:
        a.tensor("workspace", workspace, tuple(workspace.shape), (workspace.dtype,))
        if workspace.numel() * workspace.element_size() < ws_bytes:
            raise ValueError(f"{where}: workspace holds {workspace.numel() * workspace.element_size()} "
                             f"bytes, {ws_bytes} needed")
    dev = a.devices()
    if grads is None:
        grads = tuple(torch.empty(shp, dtype=torch.float32, device=dev) for _ in range(3))
    if workspace is None and need_ws:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    return shp, grads, workspace


def _nbytes(t):
    return t.numel() * t.element_size()


def fwd(q, k, v, scale, causal=False, blockmask=None, out=None, lse=None, stream=None):
    """bf16 forward: returns (O bf16 [B,H,N,d], lse fp32 [B,H,N])."""
    (B, H, N, d), out, lse = _fwd_args("fwd", q, k, v, blockmask, out, lse, "bf16")
    _check(fa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, N, d, float(scale),
                  int(causal), _ptr(blockmask), _stream(stream)), "fa_fwd")
    return out, lse


def bwd(q, k, v, o, lse, dout, scale, causal=False, blockmask=None, grads=None,
        workspace=None, stream=None):
    """bf16 backward: returns (dQ, dK, dV), fp32 [B,H,N,d]."""
    B, H, N, d = _shape(q)
    (B, H, N, d), (dq, dk, dv), workspace = _bwd_args(
        "bwd", q, k, v, o, lse, dout, blockmask, grads, workspace, "bf16",
        fa_bwd_workspace_bytes(B, H, N, d))
    _check(fa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk),
                  _ptr(dv), B, H, N, d, float(scale), int(causal), _ptr(blockmask),
                  _ptr(workspace), _nbytes(workspace), _stream(stream)), "fa_bwd")
    return dq, dk, dv


def bwd_noalloc(q, k, v, o, lse, dout, scale, causal=False, blockmask=None, grads=None,
                stream=None):
    """bf16 backward through fa_bwd_noalloc (no workspace; D in the library's
    fixed per-GPU array).  Returns (dQ, dK, dV), fp32 [B,H,N,d]; with grads
    given, nothing is allocated here either."""
    B, H, N, d = _shape(q)
    (B, H, N, d), (dq, dk, dv), _ = _bwd_args(
        "bwd_noalloc", q, k, v, o, lse, dout, blockmask, grads, None, "bf16", 0, need_ws=False)
    _check(fa_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq),
                          _ptr(dk), _ptr(dv), B, H, N, d, float(scale), int(causal),
                          _ptr(blockmask), _stream(stream)), "fa_bwd_noalloc")
    return dq, dk, dv


def bwd_stages(q, k, v, o, lse, dout, scale, causal=False, blockmask=None, grads=None,
               workspace=None, stream=None):
    """The same backward as bwd() through its three stage calls, in order."""
    B, H, N, d = _shape(q)
    (B, H, N, d), (dq, dk, dv), workspace = _bwd_args(
        "bwd_stages", q, k, v, o, lse, dout, blockmask, grads, workspace, "bf16",
        fa_bwd_workspace_bytes(B, H, N, d))
    wn = _nbytes(workspace)
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
    (B, H, N, d), out, lse = _fwd_args("fwd_dropout", q, k, v, blockmask, out, lse, "bf16")
    _check(fa_fwd_dropout(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, N, d, float(scale),
                          int(causal), _ptr(blockmask), float(p_drop), int(seed), _stream(stream)),
           "fa_fwd_dropout")
    return out, lse


def bwd_dropout(q, k, v, o, lse, dout, scale, p_drop, seed, causal=False, blockmask=None,
                grads=None, workspace=None, stream=None):
    """bf16 backward of fwd_dropout (same p_drop and seed): returns (dQ, dK, dV), fp32."""
    B, H, N, d = _shape(q)
    (B, H, N, d), (dq, dk, dv), workspace = _bwd_args(
        "bwd_dropout", q, k, v, o, lse, dout, blockmask, grads, workspace, "bf16",
        fa_bwd_workspace_bytes(B, H, N, d))
    _check(fa_bwd_dropout(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq),
                          _ptr(dk), _ptr(dv), B, H, N, d, float(scale), int(causal),
                          _ptr(blockmask), float(p_drop), int(seed), _ptr(workspace),
                          _nbytes(workspace), _stream(stream)),
           "fa_bwd_dropout")
    return dq, dk, dv


def decode(q, k, v, scale, causal=False, out=None, lse=None, workspace=None, stream=None):
    """bf16 decode: q [B,H,Nq,d] against k, v [B,H,Nk,d]; returns (O bf16, lse fp32)."""
    import torch

    B, H, Nq, d = _shape(q)
    kshape = _shape(k)
    a = _Args("decode")
    a.tensor("q", q, (B, H, Nq, d), _dt("bf16"))
    if kshape[0] != B or kshape[1] != H or kshape[3] != d:
        raise ValueError(f"decode: k has shape {kshape}, expected ({B}, {H}, Nk, {d})")
    Nk = kshape[2]
    a.tensor("k", k, kshape, _dt("bf16"))
    a.tensor("v", v, kshape, _dt("bf16"))
    if out is not None:
        a.tensor("out", out, (B, H, Nq, d), _dt("bf16"))
    if lse is not None:
        a.tensor("lse", lse, (B, H, Nq), _dt("f32"))
    wsb = fa_decode_workspace_bytes(B, H, Nq, Nk, d)
    if workspace is not None:
        a.tensor("workspace", workspace, tuple(workspace.shape), (workspace.dtype,))
        if _nbytes(workspace) < wsb:
            raise ValueError(f"decode: workspace holds {_nbytes(workspace)} bytes, {wsb} needed")
    dev = a.devices()
    if out is None:
        out = torch.empty((B, H, Nq, d), dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
    _check(fa_fwd_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, Nq, Nk, d,
                         float(scale), int(causal), _ptr(workspace), _nbytes(workspace),
                         _stream(stream)),
           "fa_fwd_decode")
    return out, lse


def fwd_f32(q, k, v, scale, causal=False, blockmask=None, out=None, lse=None, stream=None):
    """fp32 forward: returns (O fp32, lse fp32)."""
    (B, H, N, d), out, lse = _fwd_args("fwd_f32", q, k, v, blockmask, out, lse, "f32")
    _check(fa_fwd_f32(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, N, d, float(scale),
                      int(causal), _ptr(blockmask), _stream(stream)), "fa_fwd_f32")
    return out, lse


def bwd_f32(q, k, v, o, lse, dout, scale, causal=False, blockmask=None, grads=None,
            workspace=None, stream=None):
    """fp32 backward: returns (dQ, dK, dV), fp32."""
    B, H, N, d = _shape(q)
    (B, H, N, d), (dq, dk, dv), workspace = _bwd_args(
        "bwd_f32", q, k, v, o, lse, dout, blockmask, grads, workspace, "f32",
        fa_bwd_workspace_bytes(B, H, N, d))
    _check(fa_bwd_f32(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq),
                      _ptr(dk), _ptr(dv), B, H, N, d, float(scale), int(causal), _ptr(blockmask),
                      _ptr(workspace), _nbytes(workspace), _stream(stream)), "fa_bwd_f32")
    return dq, dk, dv
