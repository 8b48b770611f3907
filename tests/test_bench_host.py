"""Host-side checks of the benchmark's bookkeeping (no GPU): the useful-work figures the bench
line reports are the closed forms of the method's definitions on the workloads' windows, and a
multi-GPU request is refused before anything touches a GPU."""

import os
import subprocess
import sys

import numpy as np

import bench
import oracle
from sparse_attention_11_amd import inputs as I

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_cp_share_work_closed_forms():
    """cp2-rank1-32K: rows at positions 16384..32767 see windows 16385..32768, so the window
    sum is an arithmetic series; every window exceeds topk = 2048."""
    wl = I.workload(3)
    w = bench.work(wl)
    win = (16385 + 32768) * 16384 // 2
    assert w["window_keys"] == win
    assert w["selected"] == 16384 * 2048
    assert w["f_idx"] == 2 * 64 * 128 * win                       # 6.597 TF
    assert w["f_attn"] == 2 * 128 * (576 + 512) * 16384 * 2048    # 9.346 TF
    assert abs(w["f_idx"] / 1e12 - 6.597) < 5e-4 and abs(w["f_attn"] / 1e12 - 9.346) < 5e-4


def test_head_tail_work_is_one_eighth_of_the_windows():
    """cp8 head-tail rank 0: chunks 0..2047 and 30720..32767; its indexer window entries are
    1/8 of the full 32768-row causal triangle, as for every rank of the head-tail split."""
    wl = I.workload(4)
    w = bench.work(wl)
    full = 32768 * 32769 // 2
    assert w["window_keys"] * 8 == full == 8 * 67_110_912


def test_work_matches_oracle_windows():
    """The bench's window lengths agree with the oracle's own window rule on every workload."""
    for n in (1, 2, 3, 4, 5):
        wl = I.workload(n)
        _, L = oracle.row_windows(list(wl.segments), wl.n_q, wl.n_k)
        L = L[L >= 0].astype(np.int64)
        w = bench.work(wl)
        assert w["window_keys"] == int(L.sum()), wl.name
        assert w["selected"] == int(np.minimum(L, wl.topk).sum()), wl.name


def test_multi_gpu_request_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
