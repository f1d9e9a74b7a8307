"""The C-ABI calls inside a captured HIP graph (torch.cuda.CUDAGraph over the
stream the calls are given).  fa_fwd + fa_bwd, and fa_fwd + fa_bwd_noalloc,
are captured once and replayed several times, with eager work (refilling the
outputs with NaN) and synchronisations between the replays; every replay must
give the eager outputs bit for bit.  The calls allocate nothing, record no
memset and never synchronise, so nothing else enters the graph."""
import pytest
import torch

from exact_io_aware_18_amd.inputs import default_scale, make_blockmask, make_qkvdo
from tests.gpu_helpers import device

pytestmark = pytest.mark.gpu


def _capture(fn):
    side = torch.cuda.Stream()  # default priority
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up outside the capture
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("d,causal,masked,noalloc", [(64, True, False, False), (128, False, False, False),
                                                     (64, False, True, False), (128, True, False, True)])
def test_graph_replays_match_eager(d, causal, masked, noalloc):
    import exact_io_aware_18_amd as fa

    dev = device()
    B, H, N = 2, 4, 1000
    print(f"\n[graph] B={B} H={H} N={N} d={d} causal={causal} mask={masked} noalloc={noalloc}", flush=True)
    q, k, v, do = (t.to(dev) for t in make_qkvdo(B, H, N, d, "bf16", seed=81))
    mask = make_blockmask(N, 0.4, seed=9).to(dev) if masked else None
    scale = default_scale(d)
    o_ref, lse_ref = fa.fwd(q, k, v, scale, causal, mask)
    g_ref = fa.bwd(q, k, v, o_ref, lse_ref, do, scale, causal, mask)
    torch.cuda.synchronize()

    o, lse = torch.empty_like(o_ref), torch.empty_like(lse_ref)
    grads = tuple(torch.empty(q.shape, dtype=torch.float32, device=dev) for _ in range(3))
    ws = torch.empty(fa.fa_bwd_workspace_bytes(B, H, N, d), dtype=torch.uint8, device=dev)

    def step():
        fa.fwd(q, k, v, scale, causal, mask, out=o, lse=lse)
        if noalloc:
            fa.bwd_noalloc(q, k, v, o, lse, do, scale, causal, mask, grads=grads)
        else:
            fa.bwd(q, k, v, o, lse, do, scale, causal, mask, grads=grads, workspace=ws)

    g = _capture(step)
    for rep in range(3):
        for t in (o, lse, *grads):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref), f"replay {rep}: O differs from the eager call"
        assert torch.equal(lse, lse_ref), f"replay {rep}: lse differs from the eager call"
        for name, a, b in zip(("dq", "dk", "dv"), grads, g_ref):
            assert torch.equal(a, b), f"replay {rep}: {name} differs from the eager call"
