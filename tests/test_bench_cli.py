"""bench.py's host-side contract, without a GPU: one GPU only, the counter records it
quotes only while their kernel sources are unchanged, and the FLOP count of a
multi-token step."""

import json
import os
import subprocess
import sys
from types import SimpleNamespace

import numpy as np

REPO = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, REPO)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(REPO, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_kernel_sources_exist():
    csrc = os.path.join(REPO, "paged_kv_cache_reshape_amd", "csrc")
    for family, files in bench.KERNEL_SOURCES.items():
        for f in files:
            assert os.path.isfile(os.path.join(csrc, f)), (family, f)
        assert len(bench.kernel_source_hash(family)) == 16


def test_traffic_records_only_for_current_sources(tmp_path, monkeypatch):
    cur = bench.kernel_source_hash("decode")
    recs = {"same": {"bytes_per_launch": 123, "source_hash": cur},
            "stale": {"bytes_per_launch": 456, "source_hash": "0" * 16 if cur != "0" * 16 else "1" * 16}}
    p = tmp_path / "traffic.json"
    p.write_text(json.dumps(recs))
    monkeypatch.setattr(bench, "PROFILE_TRAFFIC", str(p))
    assert bench.stored_traffic("same") == 123
    assert bench.stored_traffic("stale") is None
    assert bench.stored_traffic("absent") is None
    monkeypatch.setattr(bench, "PROFILE_TRAFFIC", str(tmp_path / "missing.json"))
    assert bench.stored_traffic("same") is None


def test_varlen_flops_counts_visible_tokens():
    """Causal: query token i of n newest over a history of L sees L - n + i + 1 positions;
    otherwise all L.  Four FLOPs per (row, head, visible token, dim): q.k and P.V."""
    wl = SimpleNamespace(num_seqs=2, seq_lens=np.array([5, 3]), num_q_heads=3, head_size=8)
    causal = SimpleNamespace(query_start_loc=np.array([0, 2, 5]), causal=True)
    full = SimpleNamespace(query_start_loc=np.array([0, 2, 5]), causal=False)
    # request 0: L 5, n 2 -> 4 + 5; request 1: L 3, n 3 -> 1 + 2 + 3
    assert bench.varlen_flops(wl, causal) == (4 + 5 + 1 + 2 + 3) * 3 * 8 * 4
    assert bench.varlen_flops(wl, full) == (2 * 5 + 3 * 3) * 3 * 8 * 4
