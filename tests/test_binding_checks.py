"""The tensor wrappers of the Python binding reject tensors the C ABI would
misread (it takes raw pointers to contiguous [B, H, N, d] data of a fixed
dtype).  Every rejection is raised before any call into the library, so these
tests run on the CPU: shape, dtype and contiguity are checked before device
placement, and correctly formed CPU tensors are rejected for their device."""
import os

import pytest
import torch

import exact_io_aware_18_amd as fa

B, H, N, D = 1, 2, 200, 64


@pytest.fixture(scope="module", autouse=True)
def lib():
    if not os.path.exists(fa.LIB_PATH):
        from exact_io_aware_18_amd import build

        build.build()
    return fa.lib()


def bf(*shape):
    return torch.zeros(shape, dtype=torch.bfloat16)


def f32(*shape):
    return torch.zeros(shape, dtype=torch.float32)


def qkv(dtype=torch.bfloat16):
    return tuple(torch.zeros((B, H, N, D), dtype=dtype) for _ in range(3))


def mask_ok():
    nb = (N + 127) // 128
    return torch.ones((nb, nb), dtype=torch.uint8)


# ---- forward -------------------------------------------------------------------
def test_fwd_rejects_rank():
    q, k, v = qkv()
    with pytest.raises(ValueError, match=r"\[B, H, N, d\]"):
        fa.fwd(q[0], k, v, 0.125)


@pytest.mark.parametrize("which", [1, 2])
def test_fwd_rejects_shape_mismatch(which):
    t = list(qkv())
    t[which] = bf(B, H, N + 1, D)
    with pytest.raises(ValueError, match="shape"):
        fa.fwd(*t, 0.125)


@pytest.mark.parametrize("dtype", [torch.float16, torch.float32])
def test_fwd_rejects_dtype(dtype):
    q, k, v = qkv()
    with pytest.raises(ValueError, match="dtype"):
        fa.fwd(q, k.to(dtype), v, 0.125)


def test_fwd_rejects_permuted_view():
    q, k, v = qkv()
    kp = bf(B, N, H, D).permute(0, 2, 1, 3)  # [B,H,N,d] shape, [B,N,H,d] storage
    assert kp.shape == q.shape
    with pytest.raises(ValueError, match="contiguous"):
        fa.fwd(q, kp, v, 0.125)


def test_fwd_rejects_bad_outputs():
    q, k, v = qkv()
    with pytest.raises(ValueError, match="out"):
        fa.fwd(q, k, v, 0.125, out=bf(B, H, N, D).transpose(2, 3).contiguous())
    with pytest.raises(ValueError, match="out"):
        fa.fwd(q, k, v, 0.125, out=f32(B, H, N, D))
    with pytest.raises(ValueError, match="lse"):
        fa.fwd(q, k, v, 0.125, lse=f32(B, H, N, 1))
    with pytest.raises(ValueError, match="lse"):
        fa.fwd(q, k, v, 0.125, lse=bf(B, H, N))


def test_fwd_rejects_bad_blockmask():
    q, k, v = qkv()
    nb = (N + 127) // 128
    with pytest.raises(ValueError, match="blockmask"):
        fa.fwd(q, k, v, 0.125, blockmask=torch.ones((nb, nb), dtype=torch.int64))
    with pytest.raises(ValueError, match="blockmask"):
        fa.fwd(q, k, v, 0.125, blockmask=torch.ones((nb + 1, nb), dtype=torch.uint8))
    with pytest.raises(ValueError, match="blockmask"):
        fa.fwd(q, k, v, 0.125, blockmask=torch.ones((nb, 2 * nb), dtype=torch.uint8)[:, ::2])


def test_fwd_rejects_cpu_tensors():
    q, k, v = qkv()
    with pytest.raises(ValueError, match="GPU"):
        fa.fwd(q, k, v, 0.125, blockmask=mask_ok())


def test_f32_paths_check_their_dtype():
    q, k, v = qkv()
    with pytest.raises(ValueError, match="dtype"):
        fa.fwd_f32(q, k, v, 0.125)
    q32, k32, v32 = qkv(torch.float32)
    with pytest.raises(ValueError, match="GPU"):
        fa.fwd_f32(q32, k32, v32, 0.125)
    with pytest.raises(ValueError, match="dtype"):
        fa.bwd_f32(q32, k32, v32, bf(B, H, N, D), f32(B, H, N), q32, 0.125)


def test_fwd_dropout_checks_like_fwd():
    q, k, v = qkv()
    with pytest.raises(ValueError, match="contiguous"):
        fa.fwd_dropout(q, k.transpose(2, 3).contiguous().transpose(2, 3), v, 0.125, 0.1, 1)
    with pytest.raises(ValueError, match="GPU"):
        fa.fwd_dropout(q, k, v, 0.125, 0.1, 1)


# ---- backward ------------------------------------------------------------------
def bwd_args():
    q, k, v = qkv()
    return dict(q=q, k=k, v=v, o=bf(B, H, N, D), lse=f32(B, H, N), dout=bf(B, H, N, D))


@pytest.mark.parametrize("fn", ["bwd", "bwd_stages", "bwd_dropout"])
@pytest.mark.parametrize("field,bad,match", [
    ("o", bf(B, H, N, D + 1), "shape"),
    ("dout", torch.zeros((B, H, N, D), dtype=torch.float16), "dtype"),
    ("lse", f32(B, H, N + 1), "lse"),
    ("lse", bf(B, H, N), "lse"),
    ("v", bf(B, H, D, N).transpose(2, 3), "contiguous"),
])
def test_bwd_rejects(fn, field, bad, match):
    a = bwd_args()
    a[field] = bad
    extra = (0.1, 7) if fn == "bwd_dropout" else ()
    with pytest.raises(ValueError, match=match):
        getattr(fa, fn)(a["q"], a["k"], a["v"], a["o"], a["lse"], a["dout"], 0.125, *extra)


def test_bwd_rejects_bad_grads_and_workspace():
    a = bwd_args()
    args = (a["q"], a["k"], a["v"], a["o"], a["lse"], a["dout"], 0.125)
    good = tuple(f32(B, H, N, D) for _ in range(3))
    with pytest.raises(ValueError, match="grads"):
        fa.bwd(*args, grads=good[:2])
    with pytest.raises(ValueError, match="dk"):
        fa.bwd(*args, grads=(good[0], bf(B, H, N, D), good[2]))
    with pytest.raises(ValueError, match="dv"):
        fa.bwd(*args, grads=(good[0], good[1], f32(B, H, N, D).transpose(0, 1)))
    with pytest.raises(ValueError, match="workspace"):
        fa.bwd(*args, workspace=torch.zeros(16, dtype=torch.uint8))
    with pytest.raises(ValueError, match="GPU"):
        fa.bwd(*args, grads=good)


# ---- decode --------------------------------------------------------------------
def test_decode_rejects():
    q = bf(B, H, 4, D)
    k = bf(B, H, 300, D)
    with pytest.raises(ValueError, match="shape"):
        fa.decode(q, k, bf(B, H, 299, D), 0.125)  # v shorter than k
    with pytest.raises(ValueError, match="k has shape"):
        fa.decode(q, bf(B, H + 1, 300, D), bf(B, H + 1, 300, D), 0.125)
    with pytest.raises(ValueError, match="k has shape"):
        fa.decode(q, bf(B, H, 300, 128), bf(B, H, 300, 128), 0.125)
    with pytest.raises(ValueError, match="dtype"):
        fa.decode(q.float(), k, k.clone(), 0.125)
    with pytest.raises(ValueError, match="contiguous"):
        fa.decode(q, k, bf(B, 300, H, D).transpose(1, 2), 0.125)
    with pytest.raises(ValueError, match="lse"):
        fa.decode(q, k, k.clone(), 0.125, lse=f32(B, H, 5))
    with pytest.raises(ValueError, match="GPU"):
        fa.decode(q, k, k.clone(), 0.125)
