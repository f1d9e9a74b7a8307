"""Host-side logic of bench.py (CPU only): the unmasked-pair count behind
every FLOP figure it prints, the traffic record's source check, and the
percentile helper."""
import json

import numpy as np
import pytest
import torch

import bench
from exact_io_aware_18_amd.inputs import make_blockmask


def brute_pairs(N, causal, mask):
    """Allowed (query, key) pairs of one head, element by element: key j is
    allowed for query i iff j <= i (causal) and its 128-block is set in the
    mask row of i's block."""
    i = np.arange(N)[:, None]
    j = np.arange(N)[None, :]
    allowed = np.ones((N, N), dtype=bool)
    if causal:
        allowed &= j <= i
    if mask is not None:
        m = mask.numpy().astype(bool)
        allowed &= m[i // 128, j // 128]
    return int(allowed.sum())


@pytest.mark.parametrize("N", [1, 2, 127, 128, 129, 300, 640, 1000])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("masked", [False, True])
def test_pairs_per_head_matches_brute_force(N, causal, masked):
    mask = make_blockmask(N, 0.4, seed=3) if masked else None
    assert bench.pairs_per_head(N, causal, mask) == brute_pairs(N, causal, mask)


def test_pairs_per_head_asymmetric_mask():
    # a mask with blocks only above the diagonal: causal leaves just the diagonal blocks' triangles
    N = 1000
    nb = (N + 127) // 128
    mask = torch.zeros((nb, nb), dtype=torch.uint8)
    mask[0, 3] = mask[2, 5] = mask[1, 1] = 1
    for causal in (False, True):
        assert bench.pairs_per_head(N, causal, mask) == brute_pairs(N, causal, mask)


def test_traffic_record_follows_the_sources(tmp_path, monkeypatch):
    rec = {"source_hash": bench.kernel_source_hash(),
           "workloads": {"w": {"kernels": {"k": {"hbm_bytes_per_launch": 123.0}}}}}
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "traffic.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: rec["source_hash"])
    assert bench.load_traffic("w", "k") == 123.0
    assert bench.load_traffic("w", "other") is None
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0" * 16)  # sources changed since
    assert bench.load_traffic("w", "k") is None


def test_percentiles_nearest_rank():
    xs = [float(v) for v in range(1, 12)]  # 1 .. 11
    p = bench.percentiles(list(reversed(xs)))
    assert p == {"p10": 2.0, "p50": 6.0, "p90": 10.0}
    assert bench.percentiles([5.0]) == {"p10": 5.0, "p50": 5.0, "p90": 5.0}
