"""Decode (fa_fwd_decode through the C ABI) against the fp64 decode oracle:
few queries, long caches, several key chunks merged, both causal modes."""
import numpy as np
import pytest
import torch

from exact_io_aware_18_amd.inputs import default_scale, make_qkvdo
from oracle.decode import attention_fwd_decode
from tests.gpu_helpers import Guarded, check, device, guarded_workspace, to64

pytestmark = pytest.mark.gpu


def qkv(B, H, Nq, Nk, d, seed):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn((B, H, Nq, d), generator=g).to(torch.bfloat16)
    k = torch.randn((B, H, Nk, d), generator=g).to(torch.bfloat16)
    v = torch.randn((B, H, Nk, d), generator=g).to(torch.bfloat16)
    return q, k, v


def parity(B, H, Nq, Nk, d, causal, seed=0, scale=None):
    import exact_io_aware_18_amd as fa

    dev = device()
    scale = default_scale(d) if scale is None else scale
    q, k, v = qkv(B, H, Nq, Nk, d, seed)
    print(f"\n[decode] B={B} H={H} Nq={Nq} Nk={Nk} d={d} causal={causal} "
          f"workspace={fa.fa_decode_workspace_bytes(B, H, Nq, Nk, d)}", flush=True)
    og = Guarded(q.shape, torch.bfloat16, dev)
    lg = Guarded((B, H, Nq), torch.float32, dev)
    ws = guarded_workspace(fa.fa_decode_workspace_bytes(B, H, Nq, Nk, d), dev)
    fa.decode(q.to(dev), k.to(dev), v.to(dev), scale, causal, out=og.view, lse=lg.view,
              workspace=ws.view)
    torch.cuda.synchronize()
    og.check("o")
    lg.check("lse")
    ws.check("workspace", interior=False)
    o, lse = og.view, lg.view
    o_ref, lse_ref = attention_fwd_decode(to64(q), to64(k), to64(v), scale, causal)
    rep = {}
    check("o", to64(o), o_ref, "bf16", rep)
    check("lse", to64(lse), lse_ref, "bf16", rep)
    print("[decode] max-abs:", {k_: f"{v_:.2e}" for k_, v_ in rep.items()}, flush=True)
    return o.cpu(), lse.cpu()


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Nq,Nk", [(1, 1), (1, 63), (5, 1000), (32, 5000), (40, 3001)])
def test_decode_parity(d, causal, Nq, Nk):
    parity(2, 3, Nq, Nk, d, causal, seed=Nq * 7 + Nk)


@pytest.mark.parametrize("d", [64, 128])
def test_decode_long_cache(d):
    parity(1, 8, 1, 100000, d, True, seed=3)
    parity(1, 4, 16, 65536, d, False, seed=4)


def test_decode_more_queries_than_keys():
    o, lse = parity(1, 2, 20, 7, 64, True, seed=5)
    assert torch.all(o[:, :, :13] == 0) and torch.all(torch.isneginf(lse[:, :, :13]))


def test_decode_other_scales():
    parity(1, 2, 4, 777, 64, True, seed=6, scale=-0.2)
    parity(1, 2, 4, 777, 128, False, seed=7, scale=0.0)


def test_decode_agrees_with_forward_at_equal_lengths():
    import exact_io_aware_18_amd as fa

    dev = device()
    q, k, v, _ = (t.to(dev) for t in make_qkvdo(1, 4, 700, 64, "bf16", seed=8))
    o1, l1 = fa.fwd(q, k, v, 0.125, True)
    o2, l2 = fa.decode(q, k, v, 0.125, True)
    torch.cuda.synchronize()
    assert (o1.float() - o2.float()).abs().max().item() < 2e-2
    assert (l1 - l2).abs().max().item() < 1e-3
