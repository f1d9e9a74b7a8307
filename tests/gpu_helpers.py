"""Shared helpers for the GPU parity tests (HIP path through the C ABI versus
the fp64 CPU oracle on the same seeded inputs)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

# Tolerances: max-abs over every compared element, per tensor.
TOL = {
    "bf16": {"o": 2e-2, "lse": 1e-3, "dq": 2e-2, "dk": 2e-2, "dv": 2e-2},
    "f32": {"o": 1e-5, "lse": 1e-3, "dq": 1e-5, "dk": 1e-5, "dv": 1e-5},
}


def device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_io_aware_18_amd as fa

    fa.lib()  # raises if the HIP library is missing: no fallback
    return torch.device("cuda:0")


def to64(t):
    return t.detach().to("cpu").double().numpy()


def maxerr(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    both_ninf = np.isneginf(got) & np.isneginf(ref)
    if not np.all(np.isfinite(got) | both_ninf):
        return float("inf")
    diff = np.where(both_ninf, 0.0, np.abs(np.where(both_ninf, 0.0, got) - np.where(both_ninf, 0.0, ref)))
    return float(diff.max()) if diff.size else 0.0


def check(name, got, ref, dtype, report):
    e = maxerr(got, ref)
    report[name] = e
    assert e <= TOL[dtype][name], f"{name}: max-abs error {e:.3e} > {TOL[dtype][name]:.1e} ({report})"


def run_gpu(q, k, v, do, scale, causal, mask, dtype, dev, backward=True):
    """Forward (+ backward) on the GPU; returns CPU tensors."""
    import exact_io_aware_18_amd as fa

    qg, kg, vg, dog = (t.to(dev) for t in (q, k, v, do))
    mg = None if mask is None else mask.to(dev)
    if dtype == "bf16":
        o, lse = fa.fwd(qg, kg, vg, scale, causal, mg)
        grads = fa.bwd(qg, kg, vg, o, lse, dog, scale, causal, mg) if backward else None
    else:
        o, lse = fa.fwd_f32(qg, kg, vg, scale, causal, mg)
        grads = fa.bwd_f32(qg, kg, vg, o, lse, dog, scale, causal, mg) if backward else None
    torch.cuda.synchronize()
    out = {"o": o.cpu(), "lse": lse.cpu()}
    if grads is not None:
        out.update(dq=grads[0].cpu(), dk=grads[1].cpu(), dv=grads[2].cpu())
    return out
