"""GPU parity of the HIP path (through the C ABI) against the float64 CPU oracle.

Every case draws its inputs from the seeded generator; the oracle runs on the same inputs
(never on anything the GPU produced).  Full-size workloads are launched whole, exactly as the
bench launches them, and checked on a seeded sample of rows (first/last/middle row of every
segment included).
"""

import math

import numpy as np
import pytest
import torch

import oracle as O
from sparse_attention_11_amd import dsa, inputs as I
from parity_util import (check_attention, check_scores, check_selection, sample_rows)

pytestmark = pytest.mark.gpu

_CACHE = {}


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a GPU")


def _wl_inputs(n):
    """CPU inputs of workload n (cached) and their GPU copies (forward inputs only)."""
    _need_gpu()
    if n not in _CACHE:
        _CACHE.clear()
        torch.cuda.empty_cache()
        wl = I.workload(n).with_(with_dout=False)
        x = I.generate(wl)
        g = {k: v.cuda() for k, v in x.items()}
        _CACHE[n] = (wl, x, g)
    return _CACHE[n]


f64 = I.to_f64


def _windows(wl, rows):
    k_lo, L = O.row_windows(list(wl.segments), wl.n_q, wl.n_k)
    return k_lo[rows], L[rows]


# ----------------------------------------------------------------------------- indexer ----

@pytest.mark.parametrize("n", [1, 2, 3, 4])
def test_indexer_scores_bf16(n):
    wl, x, g = _wl_inputs(n)
    print(f"indexer bf16 {wl.name}", flush=True)
    sc = dsa.dsa_indexer_scores(g["q_idx"], g["k_idx"], g["w_idx"], wl.segments)
    torch.cuda.synchronize()
    rows = np.arange(wl.n_q) if n == 1 else sample_rows(wl.n_q, wl.segments, 24)
    ref = O.indexer_scores(f64(x["q_idx"]), f64(x["k_idx"]), f64(x["w_idx"]), list(wl.segments),
                           rows=rows)
    mag = O.indexer_scores(np.abs(f64(x["q_idx"])), np.abs(f64(x["k_idx"])),
                           np.abs(f64(x["w_idx"])), list(wl.segments), rows=rows)
    got = sc[torch.from_numpy(rows).cuda()].cpu().numpy()
    k_lo, L = _windows(wl, rows)
    check_scores(got, ref, k_lo, L, mag)


def test_quantize_fp8_bit_exact():
    wl, x, g = _wl_inputs(1)
    for name in ("q_idx", "k_idx"):
        codes, scale = dsa.dsa_quantize_fp8_rows(g[name])
        torch.cuda.synchronize()
        flat = x[name].reshape(x[name].shape[0], -1).float().numpy()
        rc, rs = O.quantize_fp8_rows(flat)
        assert np.array_equal(scale.cpu().numpy(), rs), name
        assert np.array_equal(codes.reshape(codes.shape[0], -1).cpu().numpy(), rc), name
    # an all-zero row and a row with a huge dynamic range
    z = torch.zeros(3, 40, dtype=torch.bfloat16)
    z[1, 0] = 3e38
    z[1, 1] = 1e-30
    z[2] = torch.linspace(-5, 5, 40).to(torch.bfloat16)
    codes, scale = dsa.dsa_quantize_fp8_rows(z.cuda())
    rc, rs = O.quantize_fp8_rows(z.float().numpy())
    assert np.array_equal(scale.cpu().numpy(), rs)
    assert np.array_equal(codes.cpu().numpy(), rc)


def _fp8_inputs(x, g):
    """GPU-quantized fp8 index tensors, and the oracle's own quantization of the same bf16."""
    qc, qs = dsa.dsa_quantize_fp8_rows(g["q_idx"])
    kc, ks = dsa.dsa_quantize_fp8_rows(g["k_idx"])
    n_q, hi, di = x["q_idx"].shape
    rqc, rqs = O.quantize_fp8_rows(x["q_idx"].reshape(n_q, -1).float().numpy())
    rkc, rks = O.quantize_fp8_rows(x["k_idx"].float().numpy())
    ref = dict(q=O.e4m3fn_decode(rqc).reshape(n_q, hi, di), qs=rqs.astype(np.float64),
               k=O.e4m3fn_decode(rkc), ks=rks.astype(np.float64))
    return (qc, qs, kc, ks), ref


@pytest.mark.parametrize("n", [1, 4])
def test_indexer_scores_fp8(n):
    wl, x, g = _wl_inputs(n)
    (qc, qs, kc, ks), ref = _fp8_inputs(x, g)
    sc = dsa.dsa_indexer_scores(qc, kc, g["w_idx"], wl.segments, q_scale=qs, k_scale=ks)
    torch.cuda.synchronize()
    rows = np.arange(wl.n_q) if n == 1 else sample_rows(wl.n_q, wl.segments, 24)
    r = O.indexer_scores(ref["q"], ref["k"], f64(x["w_idx"]), list(wl.segments), rows=rows,
                         q_scale=ref["qs"], k_scale=ref["ks"])
    mag = O.indexer_scores(np.abs(ref["q"]), np.abs(ref["k"]), np.abs(f64(x["w_idx"])),
                           list(wl.segments), rows=rows, q_scale=ref["qs"], k_scale=ref["ks"])
    got = sc[torch.from_numpy(rows).cuda()].cpu().numpy()
    k_lo, L = _windows(wl, rows)
    check_scores(got, r, k_lo, L, mag)


# ------------------------------------------------------------------------------- top-k ----

def test_topk_bit_exact_on_oracle_scores_tiny():
    """The top-k kernel alone on the oracle's scores rounded to fp32: bit-exact, exact-zero
    ties included (workload 1 has many rows whose window reaches the zero band)."""
    wl, x, g = _wl_inputs(1)
    ref = O.indexer_scores(f64(x["q_idx"]), f64(x["k_idx"]), f64(x["w_idx"]), list(wl.segments))
    s32 = ref.astype(np.float32)
    assert (s32 == 0).sum() > 100
    for topk in (64, 1, 17, 300):
        got = dsa.dsa_topk_select(torch.from_numpy(s32).cuda(), wl.segments, topk).cpu().numpy()
        want = O.topk_select(s32.astype(np.float64), list(wl.segments), topk)
        assert np.array_equal(got, want), topk


def _tie_heavy_scores(n_q, n_k, seed):
    gen = torch.Generator().manual_seed(seed)
    s = torch.randn(n_q, n_k, generator=gen)
    # quantize a third of the rows coarsely (many exact ties), put -0.0 / +0.0 mixes in others
    s[0::3] = torch.round(s[0::3] * 4) / 4
    z = torch.rand(n_q, n_k, generator=gen) < 0.3
    s[1::3] = torch.where(z[1::3], torch.where(torch.rand(z[1::3].shape, generator=gen) < 0.5,
                                               torch.tensor(-0.0), torch.tensor(0.0)), s[1::3])
    s[2::3] = s[2::3].abs() * -1.0          # all-negative rows
    return s


@pytest.mark.parametrize("n_q,n_k,segs,topk", [
    (300, 700, [(0, 300, 0, 700, 400)], 64),                 # 256-thread kernel
    (200, 8000, [(0, 200, 0, 8000, 7800)], 2048),            # 512-thread kernel
    (512, 32768, [(0, 512, 0, 32768, 32256)], 2048),         # 1024 x 32 kernel, full 32K
    (64, 65536, [(0, 64, 0, 65536, 65472)], 4096),           # 1024 x 64 kernel
    (100, 5000, [(0, 40, 0, 3000, 100), (40, 60, 3000, 2000, 1900)], 257),
])
def test_topk_bit_exact_synthetic(n_q, n_k, segs, topk):
    _need_gpu()
    s = _tie_heavy_scores(n_q, n_k, n_q + n_k)
    got = dsa.dsa_topk_select(s.cuda(), segs, topk).cpu().numpy()
    rows = sample_rows(n_q, segs, 40, seed=1)
    want = O.topk_select(s.numpy()[rows].astype(np.float64), segs, topk, n_q=n_q, rows=rows)
    assert np.array_equal(got[rows], want)


# --------------------------------------------------------------------------- attention ----

def _oracle_idx_rows(wl, x, rows):
    res = O.dsa_forward(f64(x["q_idx"]), f64(x["k_idx"]), f64(x["w_idx"]), f64(x["q"]),
                        f64(x["kv"]), list(wl.segments), wl.topk, wl.softmax_scale, wl.d_v,
                        rows=rows)
    return res


@pytest.mark.parametrize("n", [1, 2, 3])
def test_sparse_attn_on_oracle_indices(n):
    wl, x, g = _wl_inputs(n)
    rows = np.arange(wl.n_q) if n == 1 else sample_rows(wl.n_q, wl.segments, 16)
    res = _oracle_idx_rows(wl, x, rows)
    # rows not checked get arbitrary valid selections (rows are independent)
    gen = torch.Generator().manual_seed(7)
    idx = torch.randint(0, wl.n_k, (wl.n_q, wl.topk), generator=gen, dtype=torch.int32)
    idx[torch.from_numpy(rows)] = torch.from_numpy(res["idx"]).to(torch.int32)
    out, smax, ssum = dsa.dsa_sparse_attn(g["q"], g["kv"], idx.cuda(), wl.softmax_scale, wl.d_v)
    torch.cuda.synchronize()
    r = torch.from_numpy(rows).cuda()
    check_attention(out[r].float().cpu().numpy(), smax[r].cpu().numpy(), ssum[r].cpu().numpy(),
                    res["out"], res["softmax_max"], res["softmax_sum"])


def test_sparse_attn_holes_and_bad_indices():
    """-1 holes anywhere, out-of-range indices (skipped), all-empty rows, duplicates."""
    wl, x, g = _wl_inputs(1)
    gen = torch.Generator().manual_seed(3)
    idx = torch.randint(0, wl.n_k, (wl.n_q, wl.topk), generator=gen, dtype=torch.int32)
    holes = torch.rand(wl.n_q, wl.topk, generator=gen) < 0.3
    idx[holes] = -1
    idx[5] = -1                       # empty row
    idx[6, :40] = -1                  # leading holes
    idx[7, 3] = wl.n_k + 5            # out of range: skipped
    idx[8, 10] = -7
    idx[9] = 4                        # one key repeated
    out, smax, ssum = dsa.dsa_sparse_attn(g["q"], g["kv"], idx.cuda(), wl.softmax_scale, wl.d_v)
    torch.cuda.synchronize()
    ref_idx = idx.numpy().astype(np.int64)
    ref_idx[(ref_idx >= wl.n_k)] = -1
    ro, rm, rs = O.sparse_attn(f64(x["q"]), f64(x["kv"]), ref_idx, wl.softmax_scale, wl.d_v)
    check_attention(out.float().cpu().numpy(), smax.cpu().numpy(), ssum.cpu().numpy(), ro, rm, rs)
    assert torch.all(out[5] == 0) and torch.all(torch.isneginf(smax[5])) and torch.all(ssum[5] == 0)


def test_sparse_attn_large_logit_growth_takes_exact_path():
    """Logits that grow far past the first tile's max (beyond 2^64 in probability) are
    recomputed by the exact path; results still match the oracle."""
    wl, x, g = _wl_inputs(1)
    q = x["q"].clone()
    kv = x["kv"].clone()
    # key 200 is strongly aligned with every head of rows 0..3
    kv[200] = (q[0, 0].float() * 40).to(torch.bfloat16)
    idx = torch.full((wl.n_q, wl.topk), -1, dtype=torch.int32)
    for i in range(wl.n_q):
        idx[i, :40] = torch.arange(i % 50, i % 50 + 40)
    idx[0:4, 39] = 200                # in the second tile
    out, smax, ssum = dsa.dsa_sparse_attn(q.cuda(), kv.cuda(), idx.cuda(), wl.softmax_scale, wl.d_v)
    torch.cuda.synchronize()
    ro, rm, rs = O.sparse_attn(f64(q), f64(kv), idx.numpy().astype(np.int64), wl.softmax_scale,
                               wl.d_v)
    assert np.max(rm[0:4]) - np.median(rm[4:]) > 64 * math.log(2), "case does not overflow"
    # p is rounded to bf16 (2^-9 relative) before the value product: |dO| <= 2^-9 max|v|
    atol = 2e-2 + 2.0 ** -9 * float(kv[:, :wl.d_v].float().abs().max())
    check_attention(out.float().cpu().numpy(), smax.cpu().numpy(), ssum.cpu().numpy(), ro, rm, rs,
                    atol=atol)


def test_forward_large_logit_growth_exact_path_deepseek_dims():
    """DeepSeek-V3.2 dims, two segments, every window selected whole: latent row 200 is aligned
    with head 0 of row 0 and lies past the row's first tile, so the fast path gives the row up
    and the exact pass (which scans the rows' marks in parallel) recomputes it.  The fused
    forward and the standalone attention on its indices both match the oracle."""
    _need_gpu()
    wl = I.workload(2).with_(n_q=64, n_k=256, topk=256, seed=777, with_dout=False,
                             segments=((0, 32, 0, 256, 200), (32, 32, 0, 256, 224)))
    x = I.generate(wl)
    x["kv"][200] = (x["q"][0, 0].float() * 8).to(torch.bfloat16)
    g = {k: v.cuda() for k, v in x.items()}
    out, idx, smax, ssum = dsa.dsa_forward(g["q_idx"], g["k_idx"], g["w_idx"], g["q"], g["kv"],
                                           wl.segments, wl.topk, wl.softmax_scale, wl.d_v)
    out2, smax2, ssum2 = dsa.dsa_sparse_attn(g["q"], g["kv"], idx, wl.softmax_scale, wl.d_v)
    torch.cuda.synchronize()
    gi = idx.cpu().numpy().astype(np.int64)
    # topk covers every window: each row selects exactly its window
    k_lo, L = _windows(wl, np.arange(wl.n_q))
    for r in range(wl.n_q):
        assert np.array_equal(np.sort(gi[r][gi[r] >= 0]), np.arange(k_lo[r], k_lo[r] + L[r]))
    ro, rm, rs = O.sparse_attn(f64(x["q"]), f64(x["kv"]), gi, wl.softmax_scale, wl.d_v)
    assert rm[0, 0] - np.median(rm) > 64 * math.log(2), "case does not overflow"
    atol = 2e-2 + 2.0 ** -9 * float(x["kv"][:, :wl.d_v].float().abs().max())
    for o, m, s_ in ((out, smax, ssum), (out2, smax2, ssum2)):
        check_attention(o.float().cpu().numpy(), m.cpu().numpy(), s_.cpu().numpy(), ro, rm, rs,
                        atol=atol)


# ------------------------------------------------------------------------- fused forward ----

def _check_forward(wl, x, out, idx, smax, ssum, rows, ref, max_flip_frac=0.2):
    """Selection against the oracle's (near-tie rule), then attention on every sampled row
    against the oracle run on the GPU's own indices: rows whose selection equals the oracle's
    reuse its forward, rows that flipped at a near tie get the oracle attention recomputed on
    the GPU's selection, so no row escapes the output check."""
    k_lo, L = _windows(wl, rows)
    gi = idx[torch.from_numpy(rows).cuda()].cpu().numpy()
    flips = 0
    flipped = []
    for o, i in enumerate(rows):
        win = ref["scores"][o, k_lo[o]:k_lo[o] + L[o]]
        f = check_selection(gi[o], win, ref["idx"][o], int(k_lo[o]), wl.topk)
        flips += f > 0
        if f:
            flipped.append(o)
    assert flips <= max_flip_frac * len(rows) + 1, f"{flips} of {len(rows)} rows differ"
    want_out = ref["out"].copy()
    want_max = ref["softmax_max"].copy()
    want_sum = ref["softmax_sum"].copy()
    if flipped:
        fl = np.array(flipped, dtype=np.int64)
        fo, fm, fs = O.sparse_attn(f64(x["q"][torch.from_numpy(rows[fl])]), f64(x["kv"]),
                                   gi[fl].astype(np.int64), wl.softmax_scale, wl.d_v)
        want_out[fl], want_max[fl], want_sum[fl] = fo, fm, fs
    r = torch.from_numpy(rows).cuda()
    err = check_attention(out[r].float().cpu().numpy(), smax[r].cpu().numpy(),
                          ssum[r].cpu().numpy(), want_out, want_max, want_sum)
    print(f"{wl.name}: rows {len(rows)}, near-tie flips {flips} (rows {list(rows[flipped])}), "
          f"max |out err| {err:.2e}", flush=True)


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5])
def test_forward_bf16(n):
    wl, x, g = _wl_inputs(n)
    print(f"forward {wl.name}", flush=True)
    out, idx, smax, ssum = dsa.dsa_forward(g["q_idx"], g["k_idx"], g["w_idx"], g["q"], g["kv"],
                                           wl.segments, wl.topk, wl.softmax_scale, wl.d_v)
    torch.cuda.synchronize()
    rows = np.arange(wl.n_q) if n == 1 else sample_rows(wl.n_q, wl.segments, 24)
    ref = _oracle_idx_rows(wl, x, rows)
    _check_forward(wl, x, out, idx, smax, ssum, rows, ref)


@pytest.mark.parametrize("n", [1, 4])
def test_forward_fp8_indexer(n):
    wl, x, g = _wl_inputs(n)
    (qc, qs, kc, ks), r8 = _fp8_inputs(x, g)
    out, idx, smax, ssum = dsa.dsa_forward(qc, kc, g["w_idx"], g["q"], g["kv"], wl.segments,
                                           wl.topk, wl.softmax_scale, wl.d_v, q_scale=qs,
                                           k_scale=ks)
    torch.cuda.synchronize()
    rows = np.arange(wl.n_q) if n == 1 else sample_rows(wl.n_q, wl.segments, 24)
    ref = O.dsa_forward(r8["q"], r8["k"], f64(x["w_idx"]), f64(x["q"]), f64(x["kv"]),
                        list(wl.segments), wl.topk, wl.softmax_scale, wl.d_v, rows=rows,
                        q_scale=r8["qs"], k_scale=r8["ks"])
    _check_forward(wl, x, out, idx, smax, ssum, rows, ref)


def test_forward_cp_shares_match_unsharded_rows():
    """A CP share (pos0 offset) and head-tail shares equal the matching rows of the
    unsharded GPU run bit for bit (rows are independent given the full keys)."""
    wl, x, g = _wl_inputs(2)
    S = wl.n_q
    full = dsa.dsa_forward(g["q_idx"], g["k_idx"], g["w_idx"], g["q"], g["kv"], wl.segments,
                           wl.topk, wl.softmax_scale, wl.d_v)
    for segs, pos in [
        ([(0, 1024, 0, S, 3072)], np.arange(3072, 4096)),
        (list(I.head_tail_segments(S, 4, 1)), np.concatenate([np.arange(512, 1024),
                                                              np.arange(3072, 3584)])),
    ]:
        p = torch.from_numpy(pos).cuda()
        part = dsa.dsa_forward(g["q_idx"][p].contiguous(), g["k_idx"], g["w_idx"][p].contiguous(),
                               g["q"][p].contiguous(), g["kv"], segs, wl.topk, wl.softmax_scale,
                               wl.d_v)
        for a, b in zip(part, full):
            assert torch.equal(a, b[p])


def test_forward_edge_cases():
    """Uncovered rows untouched, ragged row counts, windows shorter than topk, topk = 1,
    empty segments, zero rows."""
    wl, x, g = _wl_inputs(1)
    n_q = 77
    q_idx, w, q = g["q_idx"][:n_q].contiguous(), g["w_idx"][:n_q].contiguous(), g["q"][:n_q].contiguous()
    # rows 30..39 uncovered; windows 101..130 and 1..37
    segs = [(0, 30, 0, 256, 100), (30, 0, 0, 10, 0), (40, 37, 100, 150, 0)]
    for topk in (64, 1, 100):
        out = torch.full((n_q, wl.h, wl.d_v), 7.0, dtype=torch.bfloat16, device="cuda")
        o, idx, smax, ssum = dsa.dsa_forward(q_idx, g["k_idx"], w, q, g["kv"], segs, topk,
                                             wl.softmax_scale, wl.d_v, out=out)
        torch.cuda.synchronize()
        assert torch.all(o[30:40] == 7.0)
        rows = np.concatenate([np.arange(0, 30), np.arange(40, 77)])
        ref = O.dsa_forward(f64(x["q_idx"][:n_q]), f64(x["k_idx"]), f64(x["w_idx"][:n_q]),
                            f64(x["q"][:n_q]), f64(x["kv"]), segs, topk, wl.softmax_scale,
                            wl.d_v, rows=rows)
        wl2 = wl.with_(n_q=n_q, topk=topk, segments=tuple(segs))
        _check_forward(wl2, x, o, idx, smax, ssum, rows, ref)
    # no rows at all
    e = dsa.dsa_forward(q_idx[:0], g["k_idx"], w[:0], q[:0], g["kv"], [], 8, 0.1, wl.d_v)
    assert e[0].shape[0] == 0


def test_determinism():
    wl, x, g = _wl_inputs(2)
    a = dsa.dsa_forward(g["q_idx"], g["k_idx"], g["w_idx"], g["q"], g["kv"], wl.segments,
                        wl.topk, wl.softmax_scale, wl.d_v)
    b = dsa.dsa_forward(g["q_idx"], g["k_idx"], g["w_idx"], g["q"], g["kv"], wl.segments,
                        wl.topk, wl.softmax_scale, wl.d_v)
    for u, v in zip(a, b):
        assert torch.equal(u, v)
