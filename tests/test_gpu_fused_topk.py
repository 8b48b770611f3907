"""GPU tests of the indexer fused with the top-k (dsa_indexer_topk, also the first half of
dsa_forward).

Each row has a fixed number of candidate slots (from the workspace size); a row whose
candidates would outgrow them is compacted in place to what can still be selected.  Workspaces
smaller than the default force that path on every workload shape, and scores that rise with
the key index force it at every window length.

The fused path computes the same fp32 scores with the same kernels and keeps every score that
can still be in a row's top-k, so its indices must equal those of dsa_indexer_scores followed by
dsa_topk_select bit for bit (ties to the lower key index included).  The unfused pair is itself
checked against the oracle in test_gpu_parity.py.  Besides every workload shape, the cases
force the filter's corner cases: scores rising with the key index (every key stays a candidate),
one score for every key (the whole row ties), negative scores (index weights of both signs) and
the exact zero scores of the 4-head workload.
"""

import pytest
import torch

from sparse_attention_11_amd import dsa, inputs as I

pytestmark = pytest.mark.gpu


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a GPU")


def _unfused(g, wl, q_scale=None, k_scale=None):
    sc = dsa.dsa_indexer_scores(g["q_idx"], g["k_idx"], g["w_idx"], wl.segments,
                                q_scale=q_scale, k_scale=k_scale)
    out = torch.full((wl.n_q, wl.topk), -1, dtype=torch.int32, device="cuda")
    dsa.dsa_topk_select(sc, wl.segments, wl.topk, out=out)
    del sc
    return out


def _ws_bytes(wl, cap):
    """Forward workspace giving each row `cap` candidate slots (counts, indices, fp32 scores,
    16-bit keys; regions rounded up to 256 bytes)."""
    def al(x):
        return (x + 255) // 256 * 256
    return al(wl.n_q * 4) + al(wl.n_q * wl.topk * 4) + al(wl.n_q * cap * 4) + al(wl.n_q * cap * 2)


def _check(g, wl, q_scale=None, k_scale=None, caps=(None,)):
    """Fused indices (default workspace, then each of `caps` slots per row) equal the unfused
    pair's bit for bit."""
    ref = _unfused(g, wl, q_scale, k_scale)
    for cap in caps:
        ws = None if cap is None else torch.empty(_ws_bytes(wl, cap), dtype=torch.uint8,
                                                  device="cuda")
        got = dsa.dsa_indexer_topk(g["q_idx"], g["k_idx"], g["w_idx"], wl.segments, wl.topk,
                                   q_scale=q_scale, k_scale=k_scale, workspace=ws)
        torch.cuda.synchronize()
        diff = int((got != ref).any(dim=1).sum())
        print(f"  {wl.name}: slots per row {cap or 'default'}: rows differing {diff} of "
              f"{wl.n_q}", flush=True)
        assert diff == 0, cap
    return ref


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5])
def test_fused_equals_unfused_on_every_workload(n):
    _need_gpu()
    wl = I.workload(n).with_(with_dout=False)
    print(f"fused indexer+top-k {wl.name}", flush=True)
    g = I.generate(wl, device="cuda", gen_device="cpu" if wl.n_q * wl.n_k <= 1 << 24 else "cuda")
    # the fewest slots a row may have (topk + 192), and a few more: rows compact repeatedly
    caps = (None,) if n == 1 else (None, wl.topk + 192, wl.topk + 1024)
    _check(g, wl, caps=caps)


def test_fused_fp8_indexer():
    _need_gpu()
    wl = I.workload(4).with_(with_dout=False)
    g = I.generate(wl, device="cuda", gen_device="cuda")
    q8, qs = dsa.dsa_quantize_fp8_rows(g["q_idx"])
    k8, ks = dsa.dsa_quantize_fp8_rows(g["k_idx"])
    g8 = dict(g, q_idx=q8, k_idx=k8)
    print(f"fused indexer+top-k fp8 {wl.name}", flush=True)
    _check(g8, wl, q_scale=qs, k_scale=ks, caps=(None, wl.topk + 192))


def _small(seed, n_q=300, n_k=3000, topk=256, pos0=2700):
    wl = I.workload(2).with_(n_q=n_q, n_k=n_k, topk=topk, segments=((0, n_q, 0, n_k, pos0),),
                             seed=seed, with_dout=False)
    return wl, I.generate(wl, device="cuda")


def _rising(g, wl):
    """Index keys whose scores grow with the key index: every key is above the running bound
    when it arrives, so every key becomes a candidate."""
    g["q_idx"] = g["q_idx"].abs()
    ramp = torch.linspace(0.5, 4.0, wl.n_k, device=g["k_idx"].device)[:, None]
    g["k_idx"] = (g["k_idx"].float().abs() * ramp).to(torch.bfloat16)


def test_fused_rising_scores_keep_every_key():
    _need_gpu()
    wl, g = _small(3301)
    _rising(g, wl)
    _check(g, wl, caps=(None, wl.topk + 192))


@pytest.mark.parametrize("n_k", [20000, 40000])
def test_fused_rising_scores_long_windows(n_k):
    """Rising scores over windows of 20000 and 40000 keys: the rows' candidates outgrow the
    default slots (4.5 topk) many times over and are compacted again and again.  The fused
    indices equal the unfused pair's, and the unfused selection matches the oracle's on sampled
    rows (near-tie rule; the oracle's own float64 scores)."""
    _need_gpu()
    import numpy as np
    import oracle as O
    from parity_util import check_selection
    n_q, topk = 16, 2048
    wl = I.workload(2).with_(n_q=n_q, n_k=n_k, topk=topk, seed=3310 + n_k,
                             segments=((0, n_q, 0, n_k, n_k - n_q),), with_dout=False)
    gc = I.generate(wl)
    _rising(gc, wl)                       # on the CPU: the oracle reads the same tensors
    g = {k: v.cuda() for k, v in gc.items()}
    print(f"rising scores, windows up to {n_k}", flush=True)
    ref = _check(g, wl, caps=(None, topk + 192))
    rows = np.array([0, 7, n_q - 1])
    f64 = I.to_f64
    sc = O.indexer_scores(f64(gc["q_idx"]), f64(gc["k_idx"]), f64(gc["w_idx"]),
                          list(wl.segments), rows=rows)
    k_lo, L = O.row_windows(list(wl.segments), n_q, n_k)
    gi = ref.cpu().numpy()
    for o, i in enumerate(rows):
        win = sc[o, k_lo[i]:k_lo[i] + L[i]]
        want = O.topk_row(win, int(k_lo[i]), topk)
        check_selection(gi[i], win, want, int(k_lo[i]), topk)


def test_fused_all_scores_equal():
    """Every key has the same score: the whole row ties and the lowest keys win."""
    _need_gpu()
    wl, g = _small(3302)
    g["k_idx"] = g["k_idx"][:1].expand(wl.n_k, -1).contiguous()
    _check(g, wl, caps=(None, wl.topk + 192))
    got = dsa.dsa_indexer_topk(g["q_idx"], g["k_idx"], g["w_idx"], wl.segments, wl.topk)
    torch.cuda.synchronize()
    want = torch.arange(wl.topk, dtype=torch.int32, device="cuda")
    assert torch.equal(got, want.expand(wl.n_q, -1))


def test_fused_negative_scores():
    """Index weights of both signs make many scores negative."""
    _need_gpu()
    wl, g = _small(3303)
    gen = torch.Generator(device="cpu").manual_seed(9)
    w = (torch.rand(wl.n_q, wl.h_idx, generator=gen) * 2 - 1) / 8
    g["w_idx"] = w.to(torch.bfloat16).float().cuda()
    _check(g, wl, caps=(None, wl.topk + 192))


def test_fused_short_windows_and_heavy_ties():
    """The 4-head workload: windows shorter than topk and exact zero scores (ties)."""
    _need_gpu()
    wl = I.workload(1).with_(with_dout=False)
    g = I.generate(wl, device="cuda")
    g["w_idx"] = torch.zeros_like(g["w_idx"]) + 0.25    # same weight: more exact ties
    _check(g, wl)
