#!/usr/bin/env python3
"""Throughput of exact tiled attention (forward + backward) on one MI355X.

One step is the whole hot path over one batch of synthetic input: for each
sub-workload, fa_fwd, then the three backward stages (fa_bwd_preprocess,
fa_bwd_dkdv, fa_bwd_dq).  The default workload is long-context causal
attention, B=1, H=16, N=16384, with both head dimensions d=64 and d=128 (the
sequence length at which the forward target of half the bf16 MFMA peak is
set).  The timed steps replay one HIP graph holding a step's calls (the host's
launch gaps then leave the step time; --no-graph launches them call by call);
the same number of steps launched call by call, with HIP events recorded
between consecutive launches on the launch stream, give each kernel's average
duration.

FLOP convention: 4*d per unmasked (query, key) pair for the forward and 10*d
for the backward (its five products, including the recomputation of S);
masked or skipped pairs are not counted.  Per kernel the algorithmic share is
fwd 4d, dkdv 8d (S, dP, dV, dK), dq 2d (dQ only: its recomputation of S and dP
is extra work and is not counted).

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0
METRIC = "attention TFLOP/s fwd and fwd+bwd, % of MI355X bf16 MFMA peak, 1 GPU"

BENCH_WORKLOADS = {
    "long_causal_16k": ["long_d64", "long_d128"],
    "long_d64": ["long_d64"],
    "long_d128": ["long_d128"],
    "bert_large": ["bert_large"],
    "gpt2_small": ["gpt2_small"],
    "blocksparse_64k": ["blocksparse_64k"],
}

KERNEL_SOURCES = ["fa_device.h", "fa_sched.h", "fa_dropout.h", "fa_fwd.h", "fa_bwd.h", "fa_decode.h", "fa_api.hip"]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "exact_io_aware_18_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def pairs_per_head(N, causal, mask):
    """Unmasked (query, key) pairs of one head."""
    import torch

    if mask is None:
        return N * (N + 1) // 2 if causal else N * N
    nb = mask.shape[0]
    sizes = torch.full((nb,), 128, dtype=torch.int64)
    sizes[-1] = N - 128 * (nb - 1)
    m = (mask != 0).to(torch.int64)
    total = int((sizes[:, None] * m * sizes[None, :]).sum())
    if causal:
        # diagonal blocks keep their lower triangle; blocks above it vanish
        diag = int(((sizes * (sizes + 1)) // 2 * m.diagonal()).sum())
        below = torch.tril(m, diagonal=-1)
        total = diag + int((sizes[:, None] * below * sizes[None, :]).sum())
    return total


def load_traffic(workload: str, kernel_key: str):
    """HBM bytes per launch of one kernel of a workload, from the committed
    counter summary, if it was taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_hash") != kernel_source_hash():
        return None
    ent = rec.get("workloads", {}).get(workload, {}).get("kernels", {}).get(kernel_key)
    return None if ent is None else ent.get("hbm_bytes_per_launch")


CPU_BUDGET_S = 15.0  # host time for the oracle sample
CPU_MAX_HEADS = 64
COLD_FLUSH_BYTES = 512 << 20  # written between cold steps: twice the 256 MB last-level cache


def percentiles(xs):
    """p10 / median / p90 of a list of per-step durations (nearest rank)."""
    ys = sorted(xs)
    pick = lambda f: ys[min(len(ys) - 1, max(0, int(round(f * (len(ys) - 1)))))]
    return {"p10": pick(0.1), "p50": pick(0.5), "p90": pick(0.9)}


class ClockSampler:
    """Polls the GPU's current shader clock (the DPM level marked '*' in the
    kernel driver's pp_dpm_sclk file) from a background thread while the timed
    steps run.  Reports None where the file is not readable."""

    def __init__(self, period_s=0.005):
        import glob

        self.files = [f for f in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
                      if os.access(f, os.R_OK)]
        self.period = period_s
        self.samples = []
        self._stop = False
        self._thread = None

    def _read(self):
        for f in self.files:
            try:
                with open(f) as fh:
                    for line in fh:
                        if line.rstrip().endswith("*"):
                            mhz = line.split(":")[1].strip().split()[0].lower().replace("mhz", "")
                            return float(mhz)
            except (OSError, ValueError, IndexError):
                continue
        return None

    def _run(self):
        while not self._stop:
            v = self._read()
            if v is not None:
                self.samples.append(v)
            time.sleep(self.period)

    def __enter__(self):
        import threading

        if self.files:
            self._thread = threading.Thread(target=self._run, daemon=True)
            self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop = True
        if self._thread is not None:
            self._thread.join()

    def summary(self):
        if not self.samples:
            return None
        ys = sorted(self.samples)
        return {"median_mhz": ys[len(ys) // 2], "min_mhz": ys[0], "max_mhz": ys[-1], "samples": len(ys),
                "source": "pp_dpm_sclk"}


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(sub_names, budget_s=CPU_BUDGET_S):
    """The fp64 oracle, as it stands, timed on this host's cores: full forward
    and backward of whole heads of each sub-workload, one head after another
    until the sub-workload's share of the time budget is spent (at least one
    head, at most CPU_MAX_HEADS)."""
    import numpy as np

    from exact_io_aware_18_amd.inputs import WORKLOADS, default_scale, make_blockmask, make_qkvdo
    from oracle import attention_bwd, attention_fwd

    try:
        from threadpoolctl import threadpool_info

        cores = max([x.get("num_threads", 1) for x in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = len(os.sched_getaffinity(0))
    flops = 0.0
    secs = 0.0
    desc = []
    for name in sub_names:
        w = WORKLOADS[name]
        N, d = w["N"], w["d"]
        heads = min(CPU_MAX_HEADS, w["B"] * w["H"])
        q, k, v, do = make_qkvdo(1, heads, N, d, w["dtype"], seed=0)
        mask = make_blockmask(N, w.get("frac", 0.125)) if w["mask"] else None
        m = None if mask is None else mask.numpy()
        q64, k64, v64, do64 = (t.double().numpy() for t in (q, k, v, do))
        used, t_sub = 0, 0.0
        while used < heads and (used == 0 or t_sub < budget_s / len(sub_names)):
            sl = (slice(0, 1), slice(used, used + 1))
            t0 = time.perf_counter()
            attention_fwd(q64[sl], k64[sl], v64[sl], default_scale(d), w["causal"], m)
            attention_bwd(q64[sl], k64[sl], v64[sl], do64[sl], default_scale(d), w["causal"], m)
            t_sub += time.perf_counter() - t0
            used += 1
        secs += t_sub
        flops += 14.0 * d * pairs_per_head(N, w["causal"], mask) * used
        desc.append(f"{name}: {used} head(s) of N={N} d={d}")
    return {
        "value": flops / secs / 1e12,
        "unit": "TFLOP/s",
        "cores": cores,
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": "full fp64 forward+backward of whole heads, one after another until about "
                  f"{budget_s:.0f} s are spent (" + "; ".join(desc) + f"), {secs:.1f} s; FLOP count "
                  "14d per unmasked pair (the forward's 4d and the backward's 10d)",
    }


SPARSITY_FRACS = [0.0, 1 / 64, 1 / 32, 1 / 16, 1 / 8, 1 / 4, 1 / 2, 1.0]
IO_SEQS = [2048, 4096, 8192, 16384]
DECODE_POINTS = [(8, 32, 1, 4096, 128), (8, 32, 1, 16384, 128), (8, 32, 1, 65536, 128),
                 (1, 32, 1, 1 << 20, 128), (8, 32, 8, 16384, 128), (8, 32, 1, 16384, 64),
                 (64, 8, 1, 8192, 128)]


def _time_calls(fn, reps):
    """Mean ms of `reps` back-to-back calls of fn(), HIP events on the current stream."""
    import torch

    fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def sweep(kind, reps):
    """Block-sparsity and IO sweeps: one JSON line per point.

    sparsity: B=1, H=16, N=16384, d=64, block masks keeping the diagonal plus a
      fraction f of the off-diagonal 128x128 blocks; forward and backward time
      against the number of unmasked pairs (runtime should follow density).
    io: non-causal, d=64 and 128, N in IO_SEQS with B*H = 16 * 16384 / N heads
      (the same number of query rows at every N, so every point fills the
      chip), forward only, twice per point: without a mask (the kernel the
      dispatch picks; its query-tile height Br, 256 or 384, from
      fa_fwd_query_rows) and with an all-ones block mask (Br = 128, the same
      result).
      Run under rocprofv3 --pmc to read the bytes each launch moves; the
      launches come in the printed order, `reps` + 1 per point.
    """
    import torch

    import exact_io_aware_18_amd as fa
    from exact_io_aware_18_amd.inputs import default_scale, make_blockmask, make_qkvdo

    fa.lib()
    dev = torch.device("cuda:0")
    if kind == "sparsity":
        B, H, N, d = 1, 16, 16384, 64
        q, k, v, do = (t.to(dev) for t in make_qkvdo(B, H, N, d, "bf16", seed=0))
        o = torch.empty_like(q)
        lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
        grads = tuple(torch.empty(q.shape, dtype=torch.float32, device=dev) for _ in range(3))
        ws = torch.empty(fa.fa_bwd_workspace_bytes(B, H, N, d), dtype=torch.uint8, device=dev)
        for f in SPARSITY_FRACS:
            mcpu = make_blockmask(N, f, seed=1)
            m = mcpu.to(dev)
            pairs = B * H * pairs_per_head(N, False, mcpu)
            tf = _time_calls(lambda: fa.fwd(q, k, v, default_scale(d), False, m, out=o, lse=lse), reps)
            tb = _time_calls(lambda: fa.bwd(q, k, v, o, lse, do, default_scale(d), False, m,
                                            grads=grads, workspace=ws), reps)
            print(json.dumps({"sweep": "sparsity", "B": B, "H": H, "N": N, "d": d, "frac": f,
                              "density": round(float(mcpu.float().mean()), 6), "pairs": pairs,
                              "fwd_ms": round(tf, 4), "bwd_ms": round(tb, 4),
                              "fwd_tflops": round(4.0 * d * pairs / tf / 1e9, 1),
                              "bwd_tflops": round(10.0 * d * pairs / tb / 1e9, 1)}), flush=True)
    elif kind == "io":
        for d in (64, 128):
            for N in IO_SEQS:
                B, H = 1, 16 * 16384 // N
                q, k, v, _ = (t.to(dev) for t in make_qkvdo(B, H, N, d, "bf16", seed=0))
                o = torch.empty_like(q)
                lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
                nb = (N + 127) // 128
                ones = torch.ones((nb, nb), dtype=torch.uint8, device=dev)
                for m in (None, ones):
                    br = fa.fa_fwd_query_rows(B, H, N, d, 0, m is not None, 0)
                    t = _time_calls(lambda: fa.fwd(q, k, v, default_scale(d), False, m, out=o, lse=lse), reps)
                    # bytes of the tiled algorithm without cache reuse: K and V
                    # read once per query tile, Q read and O, lse written once
                    ntq = (N + br - 1) // br
                    model = B * H * (ntq * 2 * N * d * 2 + 2 * N * d * 2 + N * 4)
                    print(json.dumps({"sweep": "io", "B": B, "H": H, "N": N, "d": d, "Br": br,
                                      "mask": m is not None, "fwd_ms": round(t, 4),
                                      "tflops": round(4.0 * d * B * H * N * N / t / 1e9, 1),
                                      "io_model_bytes": model,
                                      "compulsory_bytes": B * H * (4 * N * d * 2 + N * 4)}), flush=True)
                del q, k, v, o, lse
    elif kind == "decode":
        # few queries against a long cache: K and V are streamed once, so the
        # bound is HBM bandwidth (bytes = K + V + Q + O + lse per call)
        for (B, H, nq, nk, d) in DECODE_POINTS:
            g = torch.Generator().manual_seed(0)
            q = torch.randn((B, H, nq, d), generator=g).to(torch.bfloat16).to(dev)
            k = torch.randn((B, H, nk, d), generator=g).to(torch.bfloat16).to(dev)
            v = torch.randn((B, H, nk, d), generator=g).to(torch.bfloat16).to(dev)
            o = torch.empty_like(q)
            lse = torch.empty((B, H, nq), dtype=torch.float32, device=dev)
            ws = torch.empty(fa.fa_decode_workspace_bytes(B, H, nq, nk, d), dtype=torch.uint8, device=dev)
            t = _time_calls(lambda: fa.decode(q, k, v, default_scale(d), True, out=o, lse=lse,
                                              workspace=ws), reps)
            nbytes = B * H * (2 * nk * d * 2 + 2 * nq * d * 2 + nq * 4)
            print(json.dumps({"sweep": "decode", "B": B, "H": H, "Nq": nq, "Nk": nk, "d": d,
                              "causal": True, "ms": round(t, 4), "bytes": nbytes,
                              "gbs": round(nbytes / t / 1e6, 1),
                              "frac_hbm_peak": round(nbytes / t / 1e6 / PEAK_HBM_GBS, 4)}), flush=True)
            del q, k, v, o, lse, ws
    else:
        raise SystemExit(f"unknown sweep {kind}")


def standard_baseline(workload, reps):
    """The standard attention of the pages' comparison, built from vendor
    library calls through PyTorch (rocBLAS/hipBLASLt batched GEMMs and
    PyTorch's softmax kernel), against this library on the same workload:
    time of the forward and of forward+backward, and peak device memory
    allocated beyond the inputs.  S and P are materialised in bf16, as a
    bf16 model would; every GEMM gets contiguous operands.  One JSON line.
    """
    import torch

    import exact_io_aware_18_amd as fa
    from exact_io_aware_18_amd.inputs import WORKLOADS, default_scale, make_qkvdo

    fa.lib()
    dev = torch.device("cuda:0")
    w = WORKLOADS[workload]
    if w["mask"]:
        raise SystemExit("the standard baseline covers dense and causal workloads")
    B, H, N, d, causal = w["B"], w["H"], w["N"], w["d"], w["causal"]
    scale = default_scale(d)
    q, k, v, do = (t.to(dev) for t in make_qkvdo(B, H, N, d, "bf16", seed=0))
    q3, k3, v3, do3 = (t.reshape(B * H, N, d) for t in (q, k, v, do))
    kT = k3.transpose(1, 2).contiguous()
    vT = v3.transpose(1, 2).contiguous()
    neg = torch.triu(torch.ones(N, N, dtype=torch.bool, device=dev), diagonal=1) if causal else None

    def std_fwd():
        s_ = torch.bmm(q3, kT) * scale
        if neg is not None:
            s_ = s_.masked_fill(neg, float("-inf"))
        p_ = torch.softmax(s_, dim=-1)
        return torch.bmm(p_, v3), p_

    def std_fwd_bwd():
        o_, p_ = std_fwd()
        dv_ = torch.bmm(p_.transpose(1, 2).contiguous(), do3)
        dp_ = torch.bmm(do3, vT)
        ds_ = p_ * (dp_ - (dp_ * p_).sum(-1, keepdim=True))
        dq_ = torch.bmm(ds_, k3) * scale
        dk_ = torch.bmm(ds_.transpose(1, 2).contiguous(), q3) * scale
        return o_, dq_, dk_, dv_

    def ours_fwd():
        return fa.fwd(q, k, v, scale, causal)

    def ours_fwd_bwd():
        o_, l_ = fa.fwd(q, k, v, scale, causal)
        return fa.bwd(q, k, v, o_, l_, do, scale, causal)

    def peak(fn):
        torch.cuda.synchronize()
        torch.cuda.reset_peak_memory_stats()
        base = torch.cuda.memory_allocated()
        fn()
        torch.cuda.synchronize()
        return torch.cuda.max_memory_allocated() - base

    res = {}
    for name, fn in (("standard_fwd", std_fwd), ("standard_fwd_bwd", std_fwd_bwd),
                     ("ours_fwd", ours_fwd), ("ours_fwd_bwd", ours_fwd_bwd)):
        res[name] = {"ms": round(_time_calls(fn, reps), 4), "peak_bytes": int(peak(fn))}
    # the two paths agree (bf16 standard attention against this library)
    o_std = std_fwd()[0].float().reshape(B, H, N, d)
    o_ours = ours_fwd()[0].float()
    res["max_abs_diff_o"] = float((o_std - o_ours).abs().max())
    res["speedup_fwd"] = round(res["standard_fwd"]["ms"] / res["ours_fwd"]["ms"], 2)
    res["speedup_fwd_bwd"] = round(res["standard_fwd_bwd"]["ms"] / res["ours_fwd_bwd"]["ms"], 2)
    res["memory_ratio_fwd"] = round(res["standard_fwd"]["peak_bytes"] / max(1, res["ours_fwd"]["peak_bytes"]), 1)
    print(json.dumps({"baseline": "standard attention (torch bmm + softmax, bf16)", "workload": workload,
                      "B": B, "H": H, "N": N, "d": d, "causal": causal, **res}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="long_causal_16k", choices=sorted(BENCH_WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true",
                    help="time the steps launched call by call instead of as HIP graph replays")
    ap.add_argument("--sweep", choices=["sparsity", "io", "decode"],
                    help="run a block-sparsity or IO sweep instead of the step (one JSON line per point)")
    ap.add_argument("--sweep-reps", type=int, default=10)
    ap.add_argument("--baseline", choices=["standard"],
                    help="time standard attention from vendor GEMMs on --workload against this library")
    ap.add_argument("--dropout", type=float, default=0.0,
                    help="dropout probability on P: the step becomes fa_fwd_dropout + "
                         "fa_bwd_dropout per sub-workload, each timed as one call")
    ap.add_argument("--cold-steps", type=int, default=5,
                    help="extra steps, each after writing %d MiB of scratch (outside the timed "
                         "region), so that no input is cache-resident; reported per kernel as "
                         "cold_ms" % (COLD_FLUSH_BYTES >> 20))
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only copy MIB mebibytes device-to-device three times (the known-size "
                         "reference for the FETCH_SIZE / WRITE_SIZE counters) and exit")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: every (batch, head) is independent, so the kernel "
              "is benchmarked on one GPU's share; run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.sweep:
        sweep(args.sweep, args.sweep_reps)
        return
    if args.baseline:
        standard_baseline(args.workload if args.workload != "long_causal_16k" else "gpt2_small",
                          args.sweep_reps)
        return

    if args.copy_calibration:
        x = torch.empty(args.copy_calibration << 20, dtype=torch.uint8, device="cuda:0")
        y = torch.empty_like(x)
        for _ in range(3):
            y.copy_(x)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": x.numel(), "copies": 3}), flush=True)
        return

    import exact_io_aware_18_amd as fa
    from exact_io_aware_18_amd.inputs import WORKLOADS, default_scale, make_blockmask, make_qkvdo

    fa.lib()
    dev = torch.device("cuda:0")
    subs = []
    for name in BENCH_WORKLOADS[args.workload]:
        w = WORKLOADS[name]
        B, H, N, d = w["B"], w["H"], w["N"], w["d"]
        q, k, v, do = (t.to(dev) for t in make_qkvdo(B, H, N, d, "bf16", seed=0))
        mask = make_blockmask(N, w.get("frac", 0.125)) if w["mask"] else None
        pairs = B * H * pairs_per_head(N, w["causal"], mask)
        sub = dict(name=name, B=B, H=H, N=N, d=d, causal=w["causal"], pairs=pairs,
                   q=q, k=k, v=v, do=do, mask=None if mask is None else mask.to(dev),
                   scale=default_scale(d))
        sub["o"] = torch.empty_like(q)
        sub["lse"] = torch.empty((B, H, N), dtype=torch.float32, device=dev)
        sub["grads"] = tuple(torch.empty(q.shape, dtype=torch.float32, device=dev) for _ in range(3))
        sub["ws"] = torch.empty(fa.fa_bwd_workspace_bytes(B, H, N, d), dtype=torch.uint8, device=dev)
        subs.append(sub)

    drop = args.dropout
    nk = 2 if drop > 0 else 4  # timed calls per sub-workload per step
    seed = 0x5EED0000DEADBEEF

    def step_dropout(events=None):
        stream = torch.cuda.current_stream()  # the capture stream while a graph is captured
        for si, s in enumerate(subs):
            if events is not None:
                events[si * nk].record(stream)
            fa.fwd_dropout(s["q"], s["k"], s["v"], s["scale"], drop, seed, s["causal"], s["mask"],
                           out=s["o"], lse=s["lse"])
            if events is not None:
                events[si * nk + 1].record(stream)
            fa.bwd_dropout(s["q"], s["k"], s["v"], s["o"], s["lse"], s["do"], s["scale"], drop, seed,
                           s["causal"], s["mask"], grads=s["grads"], workspace=s["ws"])
        if events is not None:
            events[len(subs) * nk].record(stream)

    def step(events=None):
        if drop > 0:
            return step_dropout(events)
        stream = torch.cuda.current_stream()  # the capture stream while a graph is captured
        for si, s in enumerate(subs):
            base = si * nk
            if events is not None:
                events[base].record(stream)
            fa.fwd(s["q"], s["k"], s["v"], s["scale"], s["causal"], s["mask"], out=s["o"], lse=s["lse"])
            B, H, N, d = s["B"], s["H"], s["N"], s["d"]
            wsp, wsn = s["ws"].data_ptr(), s["ws"].numel()
            sp = stream.cuda_stream
            dq, dk, dv = s["grads"]
            mp = None if s["mask"] is None else s["mask"].data_ptr()
            if events is not None:
                events[base + 1].record(stream)
            fa._check(fa.fa_bwd_preprocess(s["o"].data_ptr(), s["do"].data_ptr(), B, H, N, d, wsp,
                                           wsn, sp), "fa_bwd_preprocess")
            if events is not None:
                events[base + 2].record(stream)
            fa._check(fa.fa_bwd_dkdv(s["q"].data_ptr(), s["k"].data_ptr(), s["v"].data_ptr(),
                                     s["lse"].data_ptr(), s["do"].data_ptr(), dk.data_ptr(),
                                     dv.data_ptr(), B, H, N, d, s["scale"], int(s["causal"]), mp,
                                     wsp, wsn, sp), "fa_bwd_dkdv")
            if events is not None:
                events[base + 3].record(stream)
            fa._check(fa.fa_bwd_dq(s["q"].data_ptr(), s["k"].data_ptr(), s["v"].data_ptr(),
                                   s["lse"].data_ptr(), s["do"].data_ptr(), dq.data_ptr(), B, H, N,
                                   d, s["scale"], int(s["causal"]), mp, wsp, wsn, sp), "fa_bwd_dq")
        if events is not None:
            events[len(subs) * nk].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # One step's calls captured in a HIP graph (they allocate nothing, record
    # no memset and never synchronise): replaying it takes the host's launch
    # gaps out of the step, which matters for the small workloads.
    graph, graph_note = None, "not used (--no-graph)"
    if not args.no_graph:
        try:
            side = torch.cuda.Stream()  # default priority
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                step()
            torch.cuda.current_stream().wait_stream(side)
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                step()
            torch.cuda.synchronize()
            graph_note = "captured"
        except Exception as e:  # capture refused: the eager steps are the measurement
            graph, graph_note = None, f"capture failed ({type(e).__name__}: {e}); eager steps timed"

    nev = len(subs) * nk + 1
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    with ClockSampler() as clk:
        t0 = time.perf_counter()
        for i in range(args.steps):
            step(evs[i])
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        ms_per_step_eager = (t1 - t0) * 1e3 / args.steps
        ms_per_step = ms_per_step_eager
        if graph is not None:
            torch.cuda.synchronize()
            t2 = time.perf_counter()
            for i in range(args.steps):
                graph.replay()
            torch.cuda.synchronize()
            t3 = time.perf_counter()
            ms_per_step = (t3 - t2) * 1e3 / args.steps

    # cold regime: the inputs are evicted from every cache before each step
    cold = []
    if args.cold_steps > 0:
        flush = torch.empty(COLD_FLUSH_BYTES, dtype=torch.uint8, device=dev)
        for i in range(args.cold_steps):
            flush.fill_(i & 0xFF)
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(nev)]
            step(ev)
            cold.append(ev)
        torch.cuda.synchronize()
        del flush

    kinds = ["fwd_dropout", "bwd_dropout"] if drop > 0 else ["fwd", "bwd_pre", "bwd_dkdv", "bwd_dq"]
    kernels = {}
    for si, s in enumerate(subs):
        for j, kind in enumerate(kinds):
            a = si * nk + j
            per_step = [evs[i][a].elapsed_time(evs[i][a + 1]) for i in range(args.steps)]
            ms = sum(per_step) / args.steps
            key = f"{kind}_d{s['d']}"
            kernels[key] = {"ms": ms}
            kernels[key].update({f"ms_{k_}": v_ for k_, v_ in percentiles(per_step).items()})
            if cold:
                kernels[key]["cold_ms"] = sorted(ev[a].elapsed_time(ev[a + 1]) for ev in cold)[len(cold) // 2]
            d, p, rows = s["d"], s["pairs"], s["B"] * s["H"] * s["N"]
            if kind in ("fwd", "fwd_dropout"):
                kernels[key]["flops"] = 4.0 * d * p
            elif kind == "bwd_dropout":  # one call: preprocess, dK/dV and dQ kernels
                kernels[key]["flops"] = 10.0 * d * p
            elif kind == "bwd_dkdv":
                kernels[key]["flops"] = 8.0 * d * p
            elif kind == "bwd_dq":
                kernels[key]["flops"] = 2.0 * d * p
            else:
                kernels[key]["bytes"] = rows * (2 * d * 2 + 4)
            if "flops" in kernels[key]:
                kernels[key]["tflops"] = kernels[key]["flops"] / (ms * 1e-3) / 1e12
            else:
                kernels[key]["gbs"] = kernels[key]["bytes"] / (ms * 1e-3) / 1e9

    fwd_flops = sum(4.0 * s["d"] * s["pairs"] for s in subs)
    bwd_flops = sum(10.0 * s["d"] * s["pairs"] for s in subs)
    fwd_ms = sum(kernels[f"{kinds[0]}_d{s['d']}"]["ms"] for s in subs)
    value = (fwd_flops + bwd_flops) / (ms_per_step * 1e-3) / 1e12

    dom = max(kernels, key=lambda k_: kernels[k_]["ms"])
    dk_ = kernels[dom]
    if "flops" in dk_:
        achieved, peak, unit, bound = dk_["tflops"], PEAK_BF16_TFLOPS, "TFLOP/s", "mfma"
    else:
        achieved, peak, unit, bound = dk_["gbs"], PEAK_HBM_GBS, "GB/s", "hbm"
    roofline = {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
                "frac": round(achieved / peak, 4),
                "traffic": load_traffic(args.workload, dom) if drop == 0 else None, "kernel": dom,
                "kernel_ms": round(dk_["ms"], 4)}

    # the same object for each forward kernel (the forward alone has its own
    # target: a fraction of the bf16 MFMA peak at N >= 4K)
    roofline_fwd = {}
    for key, kv in kernels.items():
        if key.startswith(kinds[0] + "_d") and "tflops" in kv:
            roofline_fwd[key] = {"bound": "mfma", "achieved": round(kv["tflops"], 2), "peak": PEAK_BF16_TFLOPS,
                                 "unit": "TFLOP/s", "frac": round(kv["tflops"] / PEAK_BF16_TFLOPS, 4),
                                 "traffic": load_traffic(args.workload, key) if drop == 0 else None,
                                 "kernel_ms": round(kv["ms"], 4)}

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "ms_per_step_eager": round(ms_per_step_eager, 4),
        "hip_graph": graph_note,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": args.workload,
            "subs": [f"{s['name']}: B={s['B']} H={s['H']} N={s['N']} d={s['d']} "
                     f"causal={int(s['causal'])} mask={int(s['mask'] is not None)}" for s in subs],
            "parallelism": "single GPU",
            "dropout": drop,
        },
        "fwd_tflops": round(fwd_flops / (fwd_ms * 1e-3) / 1e12, 2),
        "fwd_frac_peak": round(fwd_flops / (fwd_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "fwd_bwd_frac_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "kernels": {k_: {kk: (round(vv, 4) if isinstance(vv, float) else vv) for kk, vv in v_.items()}
                    for k_, v_ in kernels.items()},
        "roofline": roofline,
        "roofline_fwd": roofline_fwd,
        "timing": "ms_per_step: the timed steps as replays of one HIP graph holding a step's "
                  "calls (hip_graph), else launched call by call; ms_per_step_eager: the same number "
                  "of steps launched call by call with HIP events between the kernels, which give "
                  "the per-kernel mean (ms) and p10/p50/p90; cold: median over cold_steps steps, "
                  "each after writing %d MiB of scratch" % (COLD_FLUSH_BYTES >> 20),
        "sclk": clk.summary(),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline([s["name"] for s in subs])
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
