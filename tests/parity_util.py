"""Comparison helpers for the GPU parity tests (tolerances from the DSA acceptance rules).

* scores: |gpu - oracle| <= 1e-2 |oracle| + 1e-5 * mag inside each window and -inf outside
  it, where mag = sum_j |w_j| sum_d |q_jd k_d| is the sum of absolute products that the fp32
  (MFMA) accumulation rounds against: a head dot that cancels to ~0 can land on either side
  of the ReLU, so near-zero scores get this absolute floor instead of a relative bound;
* selected indices: per row the sets are equal, unless the oracle's gap between its n-th and
  (n+1)-th score is below 1e-3 relative; then every index in the symmetric difference must
  have an oracle score within 1e-3 |I_n| (+ the same absolute floor) of I_n;
* attention output within 2e-2 absolute, plus 2^-8 relative for outputs far above 1 (the
  output is rounded to bf16, half an ulp is 2^-9 relative); softmax max / sum within 1e-2
  relative.
"""

import numpy as np

SCORE_RTOL = 1e-2
SCORE_FLOOR = 1e-6
SCORE_MAG_FLOOR = 1e-5
GAP_RTOL = 1e-3
OUT_ATOL = 2e-2
OUT_RTOL = 2.0 ** -8
STAT_RTOL = 1e-2


def sample_rows(n_q, segments, k=48, seed=0):
    """Seeded row sample that includes the first/last row of every segment."""
    rng = np.random.default_rng(seed)
    rows = set()
    for (qs, ql, _, _, _) in segments:
        if ql:
            rows.update([qs, qs + ql - 1, qs + ql // 2])
    extra = rng.choice(n_q, size=min(n_q, k), replace=False)
    rows.update(int(r) for r in extra)
    return np.array(sorted(rows))


def check_scores(gpu_rows, ref_rows, k_lo, L, mag_rows):
    """gpu_rows / ref_rows: dense [n, n_k] for the same rows; k_lo, L per row; mag_rows the
    oracle's scores of |q|, |k|, |w| (sum of absolute products) for the same rows."""
    for o in range(gpu_rows.shape[0]):
        g, r = gpu_rows[o], ref_rows[o]
        lo, n = int(k_lo[o]), int(L[o])
        win = slice(lo, lo + n)
        assert np.all(np.isneginf(g[:lo])) and np.all(np.isneginf(g[lo + n:])), f"row {o}: outside"
        rw, gw = r[win], g[win].astype(np.float64)
        tol = SCORE_RTOL * np.abs(rw) + SCORE_MAG_FLOOR * mag_rows[o][win]
        bad = np.abs(gw - rw) > tol
        assert not bad.any(), (f"row {o}: {bad.sum()} scores off, worst "
                               f"{np.max(np.abs(gw - rw) - tol):.3e}")


def check_selection(gpu_idx, ref_scores_win, ref_idx, k_lo, topk):
    """One row: gpu_idx [topk] vs oracle; ref_scores_win = oracle scores of the window."""
    L = ref_scores_win.shape[0]
    n = min(topk, L)
    assert np.all(gpu_idx[n:] == -1), "padding"
    sel = gpu_idx[:n]
    assert np.all(np.diff(sel) > 0), "not ascending / duplicates"
    assert sel.min() >= k_lo and sel.max() < k_lo + L, "outside window"
    a, b = set(sel.tolist()), set(ref_idx[:n].tolist())
    if a == b:
        return 0
    s = np.sort(ref_scores_win)[::-1]
    In = s[n - 1]
    floor = SCORE_FLOOR * np.max(np.abs(ref_scores_win))
    gap = (s[n - 1] - s[n]) / max(abs(In), 1e-300) if n < L else np.inf
    assert gap < GAP_RTOL, f"sets differ with oracle gap {gap:.3e}"
    for key in a ^ b:
        v = ref_scores_win[key - k_lo]
        assert abs(v - In) <= GAP_RTOL * abs(In) + floor, \
            f"key {key}: score {v} too far from threshold {In}"
    return len(a ^ b) // 2


def check_attention(gpu_out, gpu_max, gpu_sum, ref_out, ref_max, ref_sum, atol=OUT_ATOL):
    """atol: absolute bound; the probabilities enter the output product as bf16, so the
    error grows like 2^-9 * max|value| -- callers with unusually large values widen it."""
    err = np.abs(gpu_out.astype(np.float64) - ref_out)
    over = err - (atol + OUT_RTOL * np.abs(ref_out))
    assert over.max() <= 0, f"out off by {err.max():.3e} (worst excess {over.max():.3e})"
    if gpu_max is not None:
        fin = np.isfinite(ref_max)
        assert np.array_equal(np.isfinite(gpu_max), fin)
        rm = np.abs(gpu_max[fin] - ref_max[fin]) <= STAT_RTOL * np.abs(ref_max[fin]) + 1e-6
        assert rm.all(), "softmax_max off"
        rs = np.abs(gpu_sum - ref_sum) <= STAT_RTOL * np.abs(ref_sum) + 1e-6
        assert rs.all(), f"softmax_sum off (worst {np.max(np.abs(gpu_sum - ref_sum)):.3e})"
    return float(err.max())
