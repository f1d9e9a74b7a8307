"""Shared helpers for the GPU parity tests (HIP path through the C ABI versus
the fp64 CPU oracle on the same seeded inputs)."""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

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


# Accuracy envelope away from the workloads' scale (the C header states it):
# the bf16 path rounds O, P and dS to bf16 (unit roundoff 2^-8), so its errors
# grow with the outputs themselves; measured max-abs error / max |x| <= 0.85%.
# Outside the workloads, O, dQ, dK and dV are held to the larger of the fixed
# tolerance and REL[dtype] times the largest |element| of the reference tensor
# (about twice the measured ratio).  lse keeps its absolute tolerance.
REL = {"bf16": 2.0 ** -6, "f32": 2.0 ** -17}


def check_envelope(name, got, ref, dtype, report):
    ref = np.asarray(ref, dtype=np.float64)
    fin = ref[np.isfinite(ref)]
    mag = float(np.abs(fin).max()) if fin.size else 0.0
    tol = TOL[dtype][name] if name == "lse" else max(TOL[dtype][name], REL[dtype] * mag)
    e = maxerr(got, ref)
    report[name] = e
    report[name + "/max|x|"] = e / mag if mag else 0.0
    assert e <= tol, f"{name}: max-abs error {e:.3e} > {tol:.2e} (max|x| {mag:.3g}; {report})"


# ---- outputs with guard bands ---------------------------------------------------
# Every output and workspace the tests hand to the library is a view into a
# larger buffer: GUARD elements before and after it, all of it filled with a
# NaN bit pattern first.  After the call every guard element must still hold
# that exact pattern (no store outside the tensor) and no element of the
# tensor may be NaN (every element written; the inputs are finite, so a
# correct kernel never produces NaN).
GUARD = 128 * 128
_NAN_BITS = {torch.bfloat16: (torch.int16, 0x7FC1), torch.float32: (torch.int32, 0x7FC00001)}


class Guarded:
    def __init__(self, shape, dtype, dev):
        self.shape = tuple(int(s) for s in shape)
        self.n = int(np.prod(self.shape)) if self.shape else 1
        self.dtype = dtype
        ity, bits = _NAN_BITS[dtype]
        self.full = torch.empty(self.n + 2 * GUARD, dtype=dtype, device=dev)
        self.full.view(ity).fill_(bits)
        self.view = self.full[GUARD:GUARD + self.n].view(self.shape)

    def check(self, name, interior=True):
        """Guards untouched; with interior=True, no NaN left in the tensor."""
        ity, bits = _NAN_BITS[self.dtype]
        raw = self.full.view(ity)
        front, back = raw[:GUARD], raw[GUARD + self.n:]
        assert bool((front == bits).all()), f"{name}: a store landed in the guard before the tensor"
        assert bool((back == bits).all()), f"{name}: a store landed in the guard after the tensor"
        if interior:
            nan = torch.isnan(self.view)
            assert not bool(nan.any()), (f"{name}: {int(nan.sum())} elements not written (or NaN), "
                                         f"first at {tuple(torch.nonzero(nan)[0].tolist())}")


def guarded_workspace(nbytes, dev):
    return Guarded(((max(int(nbytes), 4) + 3) // 4,), torch.float32, dev)


def run_gpu(q, k, v, do, scale, causal, mask, dtype, dev, backward=True):
    """Forward (+ backward) on the GPU into guarded, NaN-prefilled outputs;
    checks the guards and that every output element was written; returns CPU
    tensors."""
    import exact_io_aware_18_amd as fa

    qg, kg, vg, dog = (t.to(dev) for t in (q, k, v, do))
    mg = None if mask is None else mask.to(dev)
    B, H, N, d = q.shape
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    o = Guarded(q.shape, tdt, dev)
    lse = Guarded((B, H, N), torch.float32, dev)
    grads = None
    if dtype == "bf16":
        fa.fwd(qg, kg, vg, scale, causal, mg, out=o.view, lse=lse.view)
    else:
        fa.fwd_f32(qg, kg, vg, scale, causal, mg, out=o.view, lse=lse.view)
    if backward:
        grads = [Guarded(q.shape, torch.float32, dev) for _ in range(3)]
        ws = guarded_workspace(fa.fa_bwd_workspace_bytes(B, H, N, d), dev)
        bwd = fa.bwd if dtype == "bf16" else fa.bwd_f32
        bwd(qg, kg, vg, o.view, lse.view, dog, scale, causal, mg,
            grads=tuple(g.view for g in grads), workspace=ws.view)
    torch.cuda.synchronize()
    o.check("o")
    lse.check("lse")
    out = {"o": o.view.cpu(), "lse": lse.view.cpu()}
    if grads is not None:
        ws.check("workspace", interior=False)
        for name, g in zip(("dq", "dk", "dv"), grads):
            g.check(name)
            out[name] = g.view.cpu()
    return out


# ---- the oracle over many heads ------------------------------------------------
def oracle_threads():
    """Worker threads for per-head oracle work: the CPUs this process may use,
    at most 16 (the host share of one GPU)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def per_head(fn, heads, progress=None):
    """fn(b, h) for every (b, h) in `heads` on a thread pool (numpy releases
    the GIL in its array loops); BLAS is held to one thread per worker.
    Returns {(b, h): result}."""
    from threadpoolctl import threadpool_limits

    out = {}
    with threadpool_limits(limits=1):
        with ThreadPoolExecutor(oracle_threads()) as ex:
            futs = {ex.submit(fn, b, h): (b, h) for b, h in heads}
            for n_done, f in enumerate(futs, 1):
                out[futs[f]] = f.result()
                if progress:
                    print(f"[{progress}] oracle head {futs[f]} done ({n_done}/{len(heads)})", flush=True)
    return out
