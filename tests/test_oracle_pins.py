"""Pins of the CPU oracle against what the pages and the mathematics fix (no GPU).

Each test checks the oracle against something other than itself: exact rational brute force,
exhaustive enumeration, a library routine the oracle does not use (torch SDPA, torch autograd,
torch's float8 cast), closed forms, or invariants that a dropped term, a wrong sign, an
off-by-one window or a transposed operand would break.
"""

import itertools
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O
from sparse_attention_11_amd import inputs as I

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bf16_vals(rng, shape, scale=1.0):
    """Random float64 values that are exactly representable in bfloat16."""
    x = torch.from_numpy(rng.standard_normal(shape).astype(np.float32) * scale)
    return x.to(torch.bfloat16).double().numpy()


# ---------------------------------------------------------------------------------- formats


def test_bf16_decode_closed_forms():
    bits = np.array([0x3F80, 0xC000, 0x0001, 0x7F7F, 0x8000, 0x3E80], dtype=np.uint16)
    want = [1.0, -2.0, 2.0 ** -133, (2 - 2 ** -7) * 2.0 ** 127, -0.0, 0.25]
    got = O.bf16_bits_to_f64(bits)
    assert list(got) == want
    assert np.signbit(got[4])


def test_e4m3fn_decode_matches_torch_for_every_code():
    codes = np.arange(256, dtype=np.uint8)
    ours = O.e4m3fn_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


def _golden_e4m3():
    pts = []
    with open(os.path.join(GOLDEN, "e4m3fn_points.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                v, c = line.split()
                pts.append((float.fromhex(v) if v.startswith(("0x", "-0x")) else float(v),
                            int(c, 16)))
    return pts


def test_e4m3fn_format_points():
    for v, c in _golden_e4m3():
        assert int(O.e4m3fn_encode(np.array([v]))[0]) == c, (v, hex(c))
        assert O.e4m3fn_decode(np.array([c]))[0] == v


def test_e4m3fn_encode_matches_torch_rne():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.uniform(-448, 448, 20000),
        rng.standard_normal(20000) * 0.01,
        rng.standard_normal(5000) * 2.0 ** -8,          # subnormal range
        np.array([0.0, -0.0, 448.0, -448.0, 2.0 ** -6, 2.0 ** -9, 1.0625, 1.1875]),
    ]).astype(np.float32)
    ours = O.e4m3fn_encode(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_e4m3fn_rne_ties_and_saturation():
    # 1 + 1/16 lies halfway between 1.0 (mantissa 0) and 1.125 (mantissa 1): even -> 1.0
    assert O.e4m3fn_encode(np.array([1.0625]))[0] == 0x38
    # 1 + 3/16 lies halfway between 1.125 (m=1) and 1.25 (m=2): even -> 1.25
    assert O.e4m3fn_encode(np.array([1.1875]))[0] == 0x3A
    # saturation instead of NaN above the largest finite value
    assert O.e4m3fn_encode(np.array([1000.0, -1e6, 464.0]))[0] == 0x7E
    assert O.e4m3fn_encode(np.array([-1e6]))[0] == 0xFE
    assert O.e4m3fn_encode(np.array([np.nan]))[0] == 0x7F


def test_quantize_rows_properties():
    rng = np.random.default_rng(1)
    x = _bf16_vals(rng, (16, 256)).astype(np.float32)
    x[3] = 0.0
    codes, scale = O.quantize_fp8_rows(x)
    assert scale.dtype == np.float32 and scale[3] == 1.0 and np.all(codes[3] == 0)
    amax = np.abs(x).max(axis=1)
    for r in range(16):
        if r == 3:
            continue
        assert scale[r] == np.float32(amax[r]) / np.float32(448.0)
        dec = O.e4m3fn_decode(codes[r]) * float(scale[r])
        # the largest element lands on the top code, every element within half a step
        assert np.max(np.abs(O.e4m3fn_decode(codes[r]))) == 448.0
        big = np.abs(x[r]) >= 2.0 ** -6 * scale[r]
        assert np.all(np.abs(dec[big] - x[r][big]) <= np.abs(x[r][big]) / 16 * 1.0001)
        # the codes are exactly torch's RNE cast of the fp32 quotient
        y = (x[r] / scale[r]).astype(np.float32)
        ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(codes[r], ref)


# ---------------------------------------------------------------------------------- windows


def test_row_windows_closed_form():
    k_lo, L = O.row_windows([(2, 3, 10, 8, 4), (6, 2, 0, 2, 0)], 8, 20)
    assert list(k_lo) == [-1, -1, 10, 10, 10, -1, 0, 0]
    assert list(L) == [-1, -1, 5, 6, 7, -1, 1, 2]
    with pytest.raises(ValueError):
        O.row_windows([(0, 4, 0, 4, 1)], 4, 4)          # position 4 beyond 4 keys
    with pytest.raises(ValueError):
        O.row_windows([(0, 4, 0, 8, 0), (3, 1, 0, 8, 0)], 4, 8)   # overlap
    with pytest.raises(ValueError):
        O.row_windows([(0, 4, 6, 4, 0)], 4, 8)          # keys out of range


# ---------------------------------------------------------------------------------- indexer


def _fr(x):
    return Fraction(float(x))


def test_indexer_matches_exact_rational_brute_force():
    rng = np.random.default_rng(2)
    H, d, L = 3, 5, 7
    q = _bf16_vals(rng, (H, d))
    k = _bf16_vals(rng, (L, d))
    w = torch.from_numpy(rng.uniform(-1, 1, H).astype(np.float32)).to(torch.bfloat16).double().numpy()
    got = O.indexer_scores_row(q, k, w)
    for s in range(L):
        tot = Fraction(0)
        for j in range(H):
            dot = sum((_fr(q[j, t]) * _fr(k[s, t]) for t in range(d)), Fraction(0))
            tot += _fr(w[j]) * max(dot, Fraction(0))
        assert got[s] == float(tot)


def test_indexer_relu_is_per_head_before_weighting():
    # two heads, one key: head dots are +3 and -2
    q = np.array([[3.0], [-2.0]])
    k = np.array([[1.0]])
    assert O.indexer_scores_row(q, k, np.array([1.0, 1.0]))[0] == 3.0   # not 1 (ReLU of sum)
    assert O.indexer_scores_row(q, k, np.array([0.5, 2.0]))[0] == 1.5   # not -2.5 or 5.5
    assert O.indexer_scores_row(q, k, np.array([-1.0, 1.0]))[0] == -3.0  # weights may be negative


def test_indexer_linear_in_weights_and_head_permutation():
    rng = np.random.default_rng(3)
    q = _bf16_vals(rng, (6, 8))
    k = _bf16_vals(rng, (20, 8))
    w1, w2 = rng.uniform(0, 1, 6), rng.uniform(-1, 1, 6)
    a = O.indexer_scores_row(q, k, w1)
    np.testing.assert_allclose(O.indexer_scores_row(q, k, 3.0 * w1), 3.0 * a, rtol=1e-14)
    np.testing.assert_allclose(O.indexer_scores_row(q, k, w1 + w2),
                               a + O.indexer_scores_row(q, k, w2), rtol=1e-12, atol=1e-12)
    perm = rng.permutation(6)
    np.testing.assert_allclose(O.indexer_scores_row(q[perm], k, w1[perm]), a, rtol=1e-14)


def test_indexer_dense_windows():
    rng = np.random.default_rng(4)
    n_q, n_k = 5, 12
    q = _bf16_vals(rng, (n_q, 2, 4))
    k = _bf16_vals(rng, (n_k, 4))
    w = rng.uniform(0, 1, (n_q, 2))
    segs = [(0, 3, 2, 6, 1), (3, 2, 8, 4, 2)]
    sc = O.indexer_scores(q, k, w, segs)
    for i, (lo, L) in enumerate([(2, 2), (2, 3), (2, 4), (8, 3), (8, 4)]):
        assert np.all(np.isneginf(sc[i, :lo])) and np.all(np.isneginf(sc[i, lo + L:]))
        for s in range(lo, lo + L):
            want = sum(w[i, j] * max(0.0, float(q[i, j] @ k[s])) for j in range(2))
            assert abs(sc[i, s] - want) <= 1e-12 * max(1.0, abs(want))


def test_indexer_fp8_scales_are_dequantization():
    rng = np.random.default_rng(5)
    q = _bf16_vals(rng, (4, 3, 8))
    k = _bf16_vals(rng, (6, 8))
    w = rng.uniform(0, 1, (4, 3))
    qs = rng.uniform(0.01, 1, 4)
    ks = rng.uniform(0.01, 1, 6)
    segs = [(0, 4, 0, 6, 2)]
    a = O.indexer_scores(q, k, w, segs, q_scale=qs, k_scale=ks)
    b = O.indexer_scores(q * qs[:, None, None], k * ks[:, None], w, segs)
    np.testing.assert_allclose(a, b, rtol=1e-13)


# ---------------------------------------------------------------------------------- top-k


def _enum_topk(scores, k):
    """Exhaustive reference: among all k-subsets with the maximal score sum, the
    lexicographically smallest sorted index tuple (= ties to the lower index)."""
    L = len(scores)
    if k >= L:
        return list(range(L))
    best, best_t = None, None
    for t in itertools.combinations(range(L), k):
        s = sum(scores[i] for i in t)
        if best is None or s > best or (s == best and t < best_t):
            best, best_t = s, t
    return list(best_t)


def test_topk_exhaustive_enumeration_tiny():
    rng = np.random.default_rng(6)
    for trial in range(300):
        L = int(rng.integers(1, 9))
        s = rng.integers(0, 4, L).astype(np.float64)      # many exact ties
        if trial % 3 == 0:
            s = -s
        for k in range(1, L + 3):
            got = O.topk_row(s, 100, k)
            want = _enum_topk(list(s), k)
            n = min(k, L)
            assert list(got[:n]) == [100 + i for i in want]
            assert np.all(got[n:] == -1)


def test_topk_invariants_random_rows():
    rng = np.random.default_rng(7)
    for _ in range(50):
        L = int(rng.integers(50, 400))
        k = int(rng.integers(1, 300))
        s = np.round(rng.standard_normal(L), 1)           # ties at 0.1 resolution
        got = O.topk_row(s, 0, k)
        n = min(k, L)
        sel = got[:n]
        assert np.all(np.diff(sel) > 0) and np.all(got[n:] == -1)
        un = np.setdiff1d(np.arange(L), sel)
        if un.size:
            thr = s[sel].min()
            assert thr >= s[un].max()
            # at the threshold, every selected equal key precedes every unselected equal key
            eq_sel = sel[s[sel] == thr]
            eq_un = un[s[un] == thr]
            if eq_un.size:
                assert eq_sel.max() < eq_un.min()


def test_topk_negative_zero_ties_positive_zero():
    s = np.array([1.0, -0.0, 0.0, -0.0, 2.0])
    assert list(O.topk_row(s, 0, 3)) == [0, 1, 4]
    s = np.array([1.0, 0.0, -0.0, 0.0, 2.0])
    assert list(O.topk_row(s, 0, 3)) == [0, 1, 4]


def test_topk_whole_window_when_short():
    s = np.array([3.0, 1.0, 2.0])
    assert list(O.topk_row(s, 7, 5)) == [7, 8, 9, -1, -1]


def test_topk_select_hand_built_multi_segment_windows():
    """topk_select over a dense score matrix with two segments and an uncovered row, worked by
    hand: each row's window starts at its segment's first key and holds pos0 + r + 1 keys."""
    ninf = -np.inf
    # n_q = 5 rows, n_k = 8 keys; segment A: rows 0-1, keys 1.., pos0 1 (windows {1,2}, {1,2,3});
    # row 2 uncovered; segment B: rows 3-4, keys 5.., pos0 0 (windows {5}, {5,6})
    segs = [(0, 2, 1, 4, 1), (3, 2, 5, 3, 0)]
    S = np.array([
        [9.0, 1.0, 2.0, 7.0, 7.0, 7.0, 7.0, 7.0],     # window keys 1,2 -> scores 1, 2
        [9.0, 3.0, 3.0, 5.0, 9.0, 9.0, 9.0, 9.0],     # window keys 1,2,3 -> 3, 3, 5
        [ninf] * 8,                                    # uncovered
        [9.0, 9.0, 9.0, 9.0, 9.0, -4.0, 8.0, 8.0],    # window key 5 -> -4
        [0.0, 0.0, 0.0, 0.0, 0.0, -1.0, -0.0, 8.0],   # window keys 5,6 -> -1, -0
    ])
    full = O.topk_select(S, segs, 2)
    # row 1: keys 1 and 2 tie at 3 below key 3's 5, so the lower key 1 goes with key 3
    want = np.array([[1, 2], [1, 3], [-1, -1], [5, -1], [5, 6]])
    assert np.array_equal(full, want)
    # topk 1: the largest score of each window; row 4 picks -0 (key 6) over -1
    assert np.array_equal(O.topk_select(S, segs, 1)[:, 0], [2, 3, -1, 5, 6])
    # a row subset, out of order and with the uncovered row: score row o is local row rows[o]
    rows = np.array([4, 0, 2, 1])
    got = O.topk_select(S[rows], segs, 2, n_q=5, rows=rows)
    assert np.array_equal(got, want[rows])
    with pytest.raises(ValueError):
        O.topk_select(S[rows], segs, 2, rows=rows)          # n_q is required with rows


def test_row_subsets_equal_rows_of_full_call():
    """The rows= paths of indexer_scores, topk_select, sparse_attn and dsa_forward give exactly
    the matching rows of the full call, on a multi-segment share with uncovered rows, for a row
    subset in arbitrary order (a wrong map from output row o to local row rows[o] fails)."""
    n_q, n_k, topk, dv, scale = 30, 50, 6, 8, 0.3
    p = _small_problem(31, n_q, n_k=n_k)
    # rows 10..13 uncovered; two segments with different key ranges and positions
    segs = [(0, 10, 0, 30, 12), (14, 16, 30, 20, 3)]
    full = O.dsa_forward(p["q_idx"], p["k_idx"], p["w"], p["q"], p["kv"], segs, topk, scale, dv)
    rows = np.array([29, 3, 11, 14, 0, 21, 12, 9])
    sub = O.dsa_forward(p["q_idx"], p["k_idx"], p["w"], p["q"], p["kv"], segs, topk, scale, dv,
                        rows=rows)
    for key in ("scores", "idx", "out", "softmax_max", "softmax_sum"):
        assert np.array_equal(sub[key], full[key][rows]), key
    sc = O.indexer_scores(p["q_idx"], p["k_idx"], p["w"], segs, rows=rows)
    assert np.array_equal(sc, full["scores"][rows])
    # uncovered rows: all -inf scores, no selection, empty attention
    unc = np.isin(rows, [10, 11, 12, 13])
    assert np.all(np.isneginf(sc[unc])) and np.all(sub["idx"][unc] == -1)
    assert np.all(sub["out"][unc] == 0) and np.all(sub["softmax_sum"][unc] == 0)
    tk = O.topk_select(full["scores"][rows], segs, topk, n_q=n_q, rows=rows)
    assert np.array_equal(tk, full["idx"][rows])
    assert np.array_equal(O.topk_select(full["scores"], segs, topk), full["idx"])
    o, m, s_ = O.sparse_attn(p["q"], p["kv"], full["idx"], scale, dv, rows=rows)
    assert np.array_equal(o, full["out"][rows])
    assert np.array_equal(m, full["softmax_max"][rows]) and np.array_equal(s_, full["softmax_sum"][rows])
    # and each covered row's selection is topk_row over its own window
    k_lo, L = O.row_windows(segs, n_q, n_k)
    for o_, i in enumerate(rows):
        if L[i] > 0:
            win = full["scores"][i, k_lo[i]:k_lo[i] + L[i]]
            assert np.array_equal(sub["idx"][o_], O.topk_row(win, int(k_lo[i]), topk))


# ---------------------------------------------------------------------------------- attention


def test_attention_matches_pure_python_brute_force():
    rng = np.random.default_rng(8)
    H, D, dv = 2, 3, 2
    q = rng.standard_normal((H, D))
    kv = rng.standard_normal((6, D))
    idx = np.array([4, 1, 5, -1])
    scale = 0.7
    out, m, l = O.attention_row(q, kv, idx, scale, dv)
    for h in range(H):
        z = [scale * sum(q[h, t] * kv[s, t] for t in range(D)) for s in (4, 1, 5)]
        mm = max(z)
        e = [math.exp(x - mm) for x in z]
        ll = sum(e)
        assert abs(m[h] - mm) < 1e-14 and abs(l[h] - ll) < 1e-13
        for c in range(dv):
            want = sum(ei * kv[s, c] for ei, s in zip(e, (4, 1, 5))) / ll
            assert abs(out[h, c] - want) < 1e-13


def _dense_causal_sdpa(q, kv, segs, scale, dv):
    """torch scaled_dot_product_attention in float64 with the segments' causal masks."""
    n_q, H, D = q.shape
    n_k = kv.shape[0]
    mask = torch.zeros(n_q, n_k, dtype=torch.bool)
    for (qs, ql, ks, kl, p0) in segs:
        for r in range(ql):
            mask[qs + r, ks:ks + p0 + r + 1] = True
    Q = torch.from_numpy(q).permute(1, 0, 2).unsqueeze(0)                 # [1, H, n_q, D]
    K = torch.from_numpy(kv).expand(1, H, n_k, D)
    V = torch.from_numpy(kv[:, :dv]).contiguous().expand(1, H, n_k, dv)
    out = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=mask, scale=scale)
    return out[0].permute(1, 0, 2).numpy()


def test_topk_at_least_window_reduces_to_dense_causal_mqa():
    rng = np.random.default_rng(9)
    n_q, n_k, H, D, dv = 40, 64, 4, 12, 8
    hi, di = 3, 6
    q_idx = _bf16_vals(rng, (n_q, hi, di))
    k_idx = _bf16_vals(rng, (n_k, di))
    w = rng.uniform(0, 1, (n_q, hi))
    q = _bf16_vals(rng, (n_q, H, D))
    kv = _bf16_vals(rng, (n_k, D))
    segs = [(0, 24, 0, 40, 16), (24, 16, 40, 24, 3)]
    scale = 1 / math.sqrt(D)
    res = O.dsa_forward(q_idx, k_idx, w, q, kv, segs, topk=64, scale=scale, d_v=dv)
    ref = _dense_causal_sdpa(q, kv, segs, scale, dv)
    np.testing.assert_allclose(res["out"], ref, rtol=1e-10, atol=1e-12)


def test_attention_single_key_and_permutation_and_sum_bounds():
    rng = np.random.default_rng(10)
    q = rng.standard_normal((3, 10))
    kv = rng.standard_normal((30, 10))
    out, m, l = O.attention_row(q, kv, np.array([7, -1, -1]), 0.3, 6)
    assert np.array_equal(out, np.tile(kv[7, :6], (3, 1)))
    assert np.all(l == 1.0)
    np.testing.assert_allclose(m, 0.3 * (q @ kv[7]), rtol=1e-15)
    idx = rng.permutation(30)[:12]
    a = O.attention_row(q, kv, idx, 0.3, 6)
    b = O.attention_row(q, kv, idx[::-1].copy(), 0.3, 6)
    np.testing.assert_allclose(a[0], b[0], rtol=1e-12, atol=1e-14)
    assert np.all(a[2] >= 1.0) and np.all(a[2] <= 12.0)
    e_out, e_m, e_l = O.attention_row(q, kv, np.array([-1, -1]), 0.3, 6)
    assert np.all(e_out == 0) and np.all(np.isneginf(e_m)) and np.all(e_l == 0)


# ---------------------------------------------------------------------------------- CP shares


def _small_problem(seed, n, n_k=None, H=4, D=12, dv=8, hi=3, di=6):
    rng = np.random.default_rng(seed)
    n_k = n if n_k is None else n_k
    return dict(q_idx=_bf16_vals(rng, (n, hi, di)), k_idx=_bf16_vals(rng, (n_k, di)),
                w=rng.uniform(0, 1, (n, hi)), q=_bf16_vals(rng, (n, H, D)),
                kv=_bf16_vals(rng, (n_k, D)))


def test_cp_share_equals_rows_of_unsharded_run():
    S, topk, dv = 96, 16, 8
    p = _small_problem(11, S)
    full = O.dsa_forward(p["q_idx"], p["k_idx"], p["w"], p["q"], p["kv"], [(0, S, 0, S, 0)],
                         topk, 0.3, dv)
    for a, b in [(0, 48), (48, 96), (30, 61)]:
        part = O.dsa_forward(p["q_idx"][a:b], p["k_idx"], p["w"][a:b], p["q"][a:b], p["kv"],
                             [(0, b - a, 0, S, a)], topk, 0.3, dv)
        for key in ("idx", "out", "softmax_max", "softmax_sum"):
            assert np.array_equal(part[key], full[key][a:b]), key


def test_head_tail_shares_reassemble_and_balance_indexer_work():
    S, cp, topk, dv = 128, 4, 16, 8
    p = _small_problem(12, S)
    full = O.dsa_forward(p["q_idx"], p["k_idx"], p["w"], p["q"], p["kv"], [(0, S, 0, S, 0)],
                         topk, 0.3, dv)
    c = S // (2 * cp)
    got = np.zeros_like(full["out"])
    seen = np.zeros(S, dtype=int)
    work = []
    for r in range(cp):
        segs = I.head_tail_segments(S, cp, r)
        pos = np.concatenate([np.arange(s[4], s[4] + s[1]) for s in segs])
        part = O.dsa_forward(p["q_idx"][pos], p["k_idx"], p["w"][pos], p["q"][pos], p["kv"],
                             segs, topk, 0.3, dv)
        got[pos] = part["out"]
        seen[pos] += 1
        assert np.array_equal(part["idx"], full["idx"][pos])
        work.append(int(O.row_windows(segs, 2 * c, S)[1].sum()))
    assert np.all(seen == 1)
    assert np.array_equal(got, full["out"])
    assert len(set(work)) == 1 and work[0] == c * c * (2 * cp - 1) + c * (c + 1)


def test_varlen_equals_each_document_alone():
    lens = [20, 7, 33]
    T = sum(lens)
    p = _small_problem(13, T)
    cu = np.concatenate([[0], np.cumsum(lens)])
    segs = [(int(cu[g]), lens[g], int(cu[g]), lens[g], 0) for g in range(3)]
    packed = O.dsa_forward(p["q_idx"], p["k_idx"], p["w"], p["q"], p["kv"], segs, 8, 0.3, 8)
    for g in range(3):
        a, b = cu[g], cu[g + 1]
        alone = O.dsa_forward(p["q_idx"][a:b], p["k_idx"][a:b], p["w"][a:b], p["q"][a:b],
                              p["kv"][a:b], [(0, lens[g], 0, lens[g], 0)], 8, 0.3, 8)
        idx = packed["idx"][a:b]
        assert np.array_equal(np.where(idx >= 0, idx - a, -1), alone["idx"])
        assert np.array_equal(packed["out"][a:b], alone["out"])


def test_varlen_doc_lengths_recipe():
    lens = I.varlen_doc_lengths(1005)
    assert len(lens) == 8 and sum(lens) == 32768 and min(lens) >= 512


# ---------------------------------------------------------------------------------- backward


def test_backward_matches_autograd_and_finite_differences():
    rng = np.random.default_rng(14)
    n_q, n_k, H, D, dv, topk = 6, 20, 3, 10, 6, 5
    q = rng.standard_normal((n_q, H, D))
    kv = rng.standard_normal((n_k, D))
    dout = rng.standard_normal((n_q, H, dv))
    idx = np.full((n_q, topk), -1)
    for i in range(n_q):
        n = int(rng.integers(1, topk + 1))
        idx[i, :n] = np.sort(rng.choice(n_k, n, replace=False))
    idx[2, :] = [0, 1, 2, 3, 19]
    scale = 0.37
    dq, dkv = O.sparse_attn_bwd(q, kv, idx, dout, scale, dv)

    Q = torch.tensor(q, requires_grad=True)
    KV = torch.tensor(kv, requires_grad=True)
    outs = []
    for i in range(n_q):
        sel = torch.tensor(idx[i][idx[i] >= 0])
        K = KV.index_select(0, sel)
        p = torch.softmax(scale * Q[i] @ K.T, dim=-1)
        outs.append(p @ K[:, :dv])
    loss = sum((o * torch.tensor(dout[i])).sum() for i, o in enumerate(outs))
    loss.backward()
    np.testing.assert_allclose(dq, Q.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dkv, KV.grad.numpy(), rtol=1e-10, atol=1e-12)

    def f(qq, kk):
        o, _, _ = O.sparse_attn(qq, kk, idx, scale, dv)
        return float(np.sum(o * dout))

    eps = 1e-6
    for (i, h, d) in [(0, 0, 0), (2, 1, 7), (5, 2, 3)]:
        qp, qm = q.copy(), q.copy()
        qp[i, h, d] += eps
        qm[i, h, d] -= eps
        assert abs((f(qp, kv) - f(qm, kv)) / (2 * eps) - dq[i, h, d]) < 1e-6
    for (s, d) in [(0, 0), (19, 4), (2, 9)]:
        kp, km = kv.copy(), kv.copy()
        kp[s, d] += eps
        km[s, d] -= eps
        assert abs((f(q, kp) - f(q, km)) / (2 * eps) - dkv[s, d]) < 1e-6


# ---------------------------------------------------------------------------------- indexer KL loss


def _kl_case(seed, n_q=5, n_k=17, G=3, d=6, H=4, D=9, topk=6):
    rng = np.random.default_rng(seed)
    qi = rng.standard_normal((n_q, G, d))
    ki = rng.standard_normal((n_k, d))
    w = rng.uniform(-0.5, 1.0, (n_q, G))
    q = rng.standard_normal((n_q, H, D))
    kv = rng.standard_normal((n_k, D))
    idx = np.full((n_q, topk), -1)
    for i in range(n_q):
        n = int(rng.integers(2, topk + 1))
        idx[i, :n] = np.sort(rng.choice(n_k, n, replace=False))
    return qi, ki, w, q, kv, idx


def _sdpa_target(q_i, K, scale):
    """Head-summed, L1-normalised attention probabilities via torch's attention with the
    identity as values (each output row is then the probability row)."""
    import torch.nn.functional as F
    n = K.shape[0]
    Q = torch.tensor(q_i)[None]                       # [1, H, D] as (batch, seq=H, dim)
    Kt = torch.tensor(K)[None]
    P = F.scaled_dot_product_attention(Q, Kt, torch.eye(n, dtype=torch.float64)[None],
                                       scale=scale)[0]  # [H, n]
    p = P.sum(0)
    return (p / p.sum()).numpy()


def test_indexer_kl_loss_matches_library_kl_and_attention():
    """Loss value: scipy's relative entropy between the target (torch attention with identity
    values, head-summed and normalised) and the softmax of the already pinned indexer score."""
    from scipy.special import rel_entr, softmax
    qi, ki, w, q, kv, idx = _kl_case(21)
    scale = 0.41
    losses, _, _, _ = O.indexer_kl_loss_grad(qi, ki, w, q, kv, idx, scale)
    for i in range(qi.shape[0]):
        sel = idx[i][idx[i] >= 0]
        p = _sdpa_target(q[i], kv[sel], scale)
        r = softmax(O.indexer_scores_row(qi[i], ki[sel], w[i]))
        assert abs(losses[i] - float(np.sum(rel_entr(p, r)))) < 1e-12
        assert losses[i] >= 0


def test_indexer_kl_grads_match_autograd_and_finite_differences():
    """Gradients of the summed loss with respect to the index weights, queries and keys: torch
    autograd through its own KL divergence, and central differences of the oracle's loss.  The
    case has a repeated key in one row (its two slots add into one key row)."""
    import torch.nn.functional as F
    qi, ki, w, q, kv, idx = _kl_case(22)
    idx[3, :4] = [2, 2, 7, 11]
    idx[3, 4:] = -1
    scale, g = 0.33, 1.7
    losses, dq, dw, dk = O.indexer_kl_loss_grad(qi, ki, w, q, kv, idx, scale, g)

    QI = torch.tensor(qi, requires_grad=True)
    KI = torch.tensor(ki, requires_grad=True)
    W = torch.tensor(w, requires_grad=True)
    total = 0
    for i in range(qi.shape[0]):
        sel = idx[i][idx[i] >= 0]
        p = torch.tensor(_sdpa_target(q[i], kv[sel], scale))
        K = KI.index_select(0, torch.tensor(sel))
        I_ = (W[i][:, None] * torch.relu(QI[i] @ K.T)).sum(0)
        total = total + F.kl_div(torch.log_softmax(I_, -1), p, reduction="sum")
    assert abs(float(total.detach()) - float(losses.sum())) < 1e-12
    (g * total).backward()
    np.testing.assert_allclose(dq, QI.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dw, W.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dk, KI.grad.numpy(), rtol=1e-10, atol=1e-12)

    def f(qq, kk, ww):
        return g * float(O.indexer_kl_loss_grad(qq, kk, ww, q, kv, idx, scale)[0].sum())

    eps = 1e-6
    for (i, j, c) in [(0, 0, 0), (3, 2, 5), (4, 1, 3)]:
        a, b = qi.copy(), qi.copy()
        a[i, j, c] += eps
        b[i, j, c] -= eps
        assert abs((f(a, ki, w) - f(b, ki, w)) / (2 * eps) - dq[i, j, c]) < 1e-6
    for (i, j) in [(0, 1), (3, 0), (4, 2)]:
        a, b = w.copy(), w.copy()
        a[i, j] += eps
        b[i, j] -= eps
        assert abs((f(qi, ki, a) - f(qi, ki, b)) / (2 * eps) - dw[i, j]) < 1e-6
    for (s, c) in [(2, 0), (7, 4), (11, 5)]:
        a, b = ki.copy(), ki.copy()
        a[s, c] += eps
        b[s, c] -= eps
        assert abs((f(qi, a, w) - f(qi, b, w)) / (2 * eps) - dk[s, c]) < 1e-6


def test_indexer_kl_closed_forms():
    """Zero attention query: uniform target, loss = logsumexp(I) - mean(I) - log n.  Zero index
    query: uniform indexer distribution, loss = log n - entropy(target), and no gradient
    reaches the index queries, weights or keys (every ReLU input is 0).  One selected key:
    both distributions are the point mass, loss and gradients 0.  An empty row: all 0."""
    from scipy.special import logsumexp
    from scipy.stats import entropy
    qi, ki, w, q, kv, idx = _kl_case(23)
    scale = 0.5
    losses, _, _, _ = O.indexer_kl_loss_grad(qi, ki, w, np.zeros_like(q), kv, idx, scale)
    for i in range(qi.shape[0]):
        sel = idx[i][idx[i] >= 0]
        I_ = O.indexer_scores_row(qi[i], ki[sel], w[i])
        assert abs(losses[i] - (logsumexp(I_) - I_.mean() - math.log(len(sel)))) < 1e-12
    losses, dq, dw, dk = O.indexer_kl_loss_grad(np.zeros_like(qi), ki, w, q, kv, idx, scale)
    for i in range(qi.shape[0]):
        sel = idx[i][idx[i] >= 0]
        p = _sdpa_target(q[i], kv[sel], scale)
        assert abs(losses[i] - (math.log(len(sel)) - entropy(p))) < 1e-12
    assert not dq.any() and not dw.any() and not dk.any()
    idx1 = np.full_like(idx, -1)
    idx1[:, 0] = 4
    idx1[2, 0] = -1                    # an empty row
    losses, dq, dw, dk = O.indexer_kl_loss_grad(qi, ki, w, q, kv, idx1, scale)
    assert np.all(np.abs(losses) < 1e-15)
    assert np.abs(dq).max() < 1e-15 and np.abs(dw).max() < 1e-15 and np.abs(dk).max() < 1e-15


def test_indexer_kl_gradient_scale_and_slot_order():
    """The incoming loss gradient scales every gradient and not the loss; permuting a row's
    slots (holes included) changes nothing."""
    qi, ki, w, q, kv, idx = _kl_case(24)
    scale = 0.3
    l1, dq1, dw1, dk1 = O.indexer_kl_loss_grad(qi, ki, w, q, kv, idx, scale, 1.0)
    l2, dq2, dw2, dk2 = O.indexer_kl_loss_grad(qi, ki, w, q, kv, idx, scale, -2.5)
    np.testing.assert_array_equal(l1, l2)
    for a, b in [(dq1, dq2), (dw1, dw2), (dk1, dk2)]:
        np.testing.assert_allclose(b, -2.5 * a, rtol=1e-13, atol=1e-15)
    rng = np.random.default_rng(5)
    perm = np.stack([rng.permutation(idx.shape[1]) for _ in range(idx.shape[0])])
    idxp = np.take_along_axis(idx, perm, 1)
    l3, dq3, dw3, dk3 = O.indexer_kl_loss_grad(qi, ki, w, q, kv, idxp, scale)
    np.testing.assert_allclose(l3, l1, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(dq3, dq1, rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(dw3, dw1, rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(dk3, dk1, rtol=1e-10, atol=1e-13)


# ---------------------------------------------------------------------------------- inputs


def test_generator_is_deterministic_and_shaped():
    wl = I.workload(1)
    a = I.generate(wl)
    b = I.generate(wl)
    for k in a:
        assert torch.equal(a[k], b[k])
    assert a["q_idx"].shape == (256, 4, 32) and a["q_idx"].dtype == torch.bfloat16
    assert a["kv"].shape == (256, 80) and a["w_idx"].dtype == torch.float32
    assert torch.equal(a["w_idx"], a["w_idx"].to(torch.bfloat16).float())
    assert float(a["w_idx"].min()) >= 0 and float(a["w_idx"].max()) <= 0.5


# ---- dense causal attention (Ulysses head shard) -------------------------------------------


def _dense_inputs(n, H, D, Dv, seed):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(n, H, D, generator=g, dtype=torch.float64)
    k = torch.randn(n, H, D, generator=g, dtype=torch.float64)
    v = torch.randn(n, H, Dv, generator=g, dtype=torch.float64)
    return q, k, v


def test_dense_attn_matches_library_sdpa_causal():
    # plain causal SDPA of torch (float64, CPU) over [H, S, D] is the definition written out
    n, H, D, Dv = 37, 3, 192, 128
    q, k, v = _dense_inputs(n, H, D, Dv, 11)
    scale = 1.0 / math.sqrt(D)
    out, lse = O.dense_attn(q.numpy(), k.numpy(), v.numpy(), [(0, n, 0, n, 0)], scale)
    ref = torch.nn.functional.scaled_dot_product_attention(
        q.transpose(0, 1), k.transpose(0, 1), v.transpose(0, 1), is_causal=True, scale=scale)
    np.testing.assert_allclose(out, ref.transpose(0, 1).numpy(), rtol=0, atol=1e-12)
    z = scale * torch.einsum("qhd,khd->hqk", q, k)
    z = z.masked_fill(torch.ones(n, n, dtype=torch.bool).triu(1), -math.inf)
    np.testing.assert_allclose(lse, torch.logsumexp(z, dim=-1).T.numpy(), rtol=0, atol=1e-12)


def test_dense_attn_hybrid_shard_and_documents():
    # a query shard at positions 40.. of a 64-key sequence (Hybrid: Q sharded, K/V gathered)
    # is a masked SDPA with the mask from the global positions, and equals those rows of the
    # unsharded call; packed documents equal each document alone
    n, H, D, Dv = 64, 2, 192, 128
    q, k, v = _dense_inputs(n, H, D, Dv, 12)
    scale = 0.07
    full, lse_full = O.dense_attn(q.numpy(), k.numpy(), v.numpy(), [(0, n, 0, n, 0)], scale)
    sh, lse_sh = O.dense_attn(q[40:].numpy(), k.numpy(), v.numpy(), [(0, 24, 0, n, 40)], scale)
    np.testing.assert_array_equal(sh, full[40:])
    np.testing.assert_array_equal(lse_sh, lse_full[40:])
    pos = torch.arange(40, 64)[:, None]
    mask = torch.arange(n)[None, :] <= pos
    ref = torch.nn.functional.scaled_dot_product_attention(
        q[40:].transpose(0, 1), k.transpose(0, 1), v.transpose(0, 1), attn_mask=mask, scale=scale)
    np.testing.assert_allclose(sh, ref.transpose(0, 1).numpy(), rtol=0, atol=1e-12)
    segs = [(0, 20, 0, 20, 0), (20, 44, 20, 44, 0)]
    packed, lse_p = O.dense_attn(q.numpy(), k.numpy(), v.numpy(), segs, scale)
    a, la = O.dense_attn(q[:20].numpy(), k[:20].numpy(), v[:20].numpy(), [(0, 20, 0, 20, 0)], scale)
    b, lb = O.dense_attn(q[20:].numpy(), k[20:].numpy(), v[20:].numpy(), [(0, 44, 0, 44, 0)], scale)
    np.testing.assert_array_equal(packed, np.concatenate([a, b]))
    np.testing.assert_array_equal(lse_p, np.concatenate([la, lb]))
    sub, lsub = O.dense_attn(q.numpy(), k.numpy(), v.numpy(), segs, scale, rows=[43, 2, 20])
    np.testing.assert_array_equal(sub, packed[[43, 2, 20]])
    np.testing.assert_array_equal(lsub, lse_p[[43, 2, 20]])


def test_dense_attn_closed_forms():
    n, H, D, Dv = 9, 2, 192, 128
    q, k, v = _dense_inputs(n, H, D, Dv, 13)
    segs = [(0, n, 0, n, 0)]
    out, lse = O.dense_attn(q.numpy(), k.numpy(), v.numpy(), segs, 0.1)
    # the first row sees one key: out is that key's value row, lse its logit
    np.testing.assert_array_equal(out[0], v[0].numpy())
    np.testing.assert_allclose(lse[0], 0.1 * (q[0] * k[0]).sum(-1).numpy(), rtol=1e-13)
    # zero queries: every logit is 0, so out is the mean of the window's values and lse = log L
    out0, lse0 = O.dense_attn(np.zeros((n, H, D)), k.numpy(), v.numpy(), segs, 0.1)
    for i in range(n):
        np.testing.assert_allclose(out0[i], v[: i + 1].numpy().mean(axis=0), rtol=0, atol=1e-14)
        np.testing.assert_allclose(lse0[i], math.log(i + 1), rtol=0, atol=1e-15)
    # uncovered rows: zero output, lse -inf
    o2, l2 = O.dense_attn(q.numpy(), k.numpy(), v.numpy(), [(0, 4, 0, n, 0)], 0.1)
    assert np.all(o2[4:] == 0) and np.all(l2[4:] == -np.inf)
