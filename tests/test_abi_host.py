"""Host-side checks of the C ABI (no GPU): the library loads, exports every entry point the
header declares, and rejects bad arguments before launching anything.

Calls here never get past validation (fake device pointers are passed only where the call
is expected to fail first), so nothing touches a GPU.
"""

import ctypes
import os
import re

import pytest

from sparse_attention_11_amd import dsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsa.h")
FAKE = ctypes.c_void_p(0x1000)      # never dereferenced: validation fails before any launch


def _declared():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(dsa_[a-z0-9_]+)\s*\(", txt)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(dsa.LIB_PATH):
        pytest.fail("libdsa.so is not built (run __graft_entry__.build())")
    return dsa.load_library()


def test_exports_every_declared_symbol(lib):
    names = _declared()
    assert names, "no declarations parsed"
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(dsa.EXPORTED)


def test_abi_version_matches_header(lib):
    m = re.search(r"#define DSA_ABI_VERSION (\d+)", open(HEADER).read())
    assert dsa.dsa_abi_version() == int(m.group(1))


def _ws(n_q, n_k, topk, segs):
    sh = dsa._shape(n_q=n_q, n_k=n_k, topk=topk, segments=segs)
    out = ctypes.c_size_t(0)
    st = dsa.load_library().dsa_workspace_bytes(ctypes.byref(sh), ctypes.byref(out))
    return st, out.value


def _cand_ws(n_q, topk, cap):
    """Forward workspace for `cap` candidate slots per row: counts, indices, fp32 candidate
    scores, 16-bit candidate keys, each region rounded up to 256 bytes."""
    def al(x):
        return (x + 255) // 256 * 256
    return al(n_q * 4) + al(n_q * topk * 4) + al(n_q * cap * 4) + al(n_q * cap * 2)


def test_workspace_bytes_formula(lib):
    # default slots per row: 4.5 topk rounded up to 64 (at least topk + 192, at most the
    # longest window rounded up to 64)
    st, n = _ws(16384, 32768, 2048, [(0, 16384, 0, 32768, 16384)])
    assert st == dsa.DSA_OK
    assert n == _cand_ws(16384, 2048, 9216)
    assert n <= 1.1e9          # the 32K CP-degree-2 share fits in 1.1 GB
    st, n = _ws(100, 300, 7, [(0, 60, 0, 100, 3), (60, 40, 100, 200, 150)])
    assert st == dsa.DSA_OK
    assert n == _cand_ws(100, 7, 192)     # longest window 190 -> 192 slots
    st, n = _ws(8, 70000, 4096, [(0, 8, 0, 65536, 65528)])
    assert st == dsa.DSA_OK
    assert n == _cand_ws(8, 4096, 18432)


@pytest.mark.parametrize("segs,n_q,n_k,why", [
    ([(0, 4, 0, 4, 1)], 4, 4, "position beyond keys"),
    ([(0, 4, 0, 8, 0), (3, 1, 0, 8, 0)], 4, 8, "overlap"),
    ([(0, 5, 0, 8, 0)], 4, 8, "query rows past n_q"),
    ([(0, 4, 6, 4, 0)], 4, 8, "keys past n_k"),
    ([(0, 4, -1, 4, 0)], 4, 8, "negative field"),
])
def test_bad_segments_rejected(lib, segs, n_q, n_k, why):
    st, _ = _ws(n_q, n_k, 4, segs)
    assert st == dsa.DSA_ERR_INVALID_ARG, why
    assert dsa.dsa_last_error()


def test_null_shape_and_topk_limits(lib):
    out = ctypes.c_size_t(0)
    assert lib.dsa_workspace_bytes(None, ctypes.byref(out)) == dsa.DSA_ERR_INVALID_ARG
    assert _ws(4, 4, 0, [(0, 4, 0, 4, 0)])[0] == dsa.DSA_ERR_INVALID_ARG
    assert _ws(4, 4, 5000, [(0, 4, 0, 4, 0)])[0] == dsa.DSA_ERR_UNSUPPORTED
    assert _ws(1, 70000, 8, [(0, 1, 0, 70000, 69999)])[0] == dsa.DSA_ERR_UNSUPPORTED
    # success clears the message
    assert _ws(4, 4, 4, [(0, 4, 0, 4, 0)])[0] == dsa.DSA_OK
    assert dsa.dsa_last_error() == ""


def _idx_call(lib, h_idx, d_idx, idx_dtype, q_scale=None, k_scale=None, segs=((0, 4, 0, 4, 0),)):
    sh = dsa._shape(n_q=4, n_k=4, h_idx=h_idx, d_idx=d_idx, idx_dtype=idx_dtype, segments=segs)
    return lib.dsa_indexer_scores(ctypes.byref(sh), FAKE, q_scale, FAKE, k_scale, FAKE, FAKE, None)


def test_indexer_argument_checks(lib):
    assert _idx_call(lib, 64, 96, 0) == dsa.DSA_ERR_UNSUPPORTED
    assert _idx_call(lib, 64, 128, 7) == dsa.DSA_ERR_INVALID_ARG
    assert _idx_call(lib, 64, 128, 1) == dsa.DSA_ERR_INVALID_ARG            # fp8 without scales
    assert _idx_call(lib, 64, 128, 0, q_scale=FAKE, k_scale=FAKE) == dsa.DSA_ERR_INVALID_ARG
    sh = dsa._shape(n_q=4, n_k=4, h_idx=64, d_idx=128, segments=[(0, 4, 0, 4, 0)])
    assert lib.dsa_indexer_scores(ctypes.byref(sh), None, None, FAKE, None, FAKE, FAKE,
                                  None) == dsa.DSA_ERR_INVALID_ARG


def test_attention_argument_checks(lib):
    sh = dsa._shape(n_q=4, n_k=4, h=64, d_qk=576, d_v=512, topk=4, softmax_scale=0.1)
    assert lib.dsa_sparse_attn(ctypes.byref(sh), FAKE, FAKE, FAKE, FAKE, None, None,
                               None) == dsa.DSA_ERR_UNSUPPORTED
    sh = dsa._shape(n_q=4, n_k=4, h=128, d_qk=576, d_v=512, topk=4, softmax_scale=float("nan"))
    assert lib.dsa_sparse_attn(ctypes.byref(sh), FAKE, FAKE, FAKE, FAKE, None, None,
                               None) == dsa.DSA_ERR_INVALID_ARG
    sh = dsa._shape(n_q=4, n_k=4, h=128, d_qk=576, d_v=512, topk=4, softmax_scale=0.1)
    assert lib.dsa_sparse_attn(ctypes.byref(sh), FAKE, FAKE, None, FAKE, None, None,
                               None) == dsa.DSA_ERR_INVALID_ARG


def _fwd(lib, ws_bytes, segs=((0, 4, 0, 4, 0),), workspace=FAKE):
    sh = dsa._shape(n_q=4, n_k=4, h_idx=4, d_idx=32, h=8, d_qk=80, d_v=64, topk=2,
                    softmax_scale=0.1, segments=segs)
    return lib.dsa_forward(ctypes.byref(sh), FAKE, None, FAKE, None, FAKE, FAKE, FAKE, FAKE,
                           None, None, None, workspace, ctypes.c_size_t(ws_bytes), None)


def test_forward_workspace_checks(lib):
    need = _ws(4, 4, 2, [(0, 4, 0, 4, 0)])[1]
    assert _fwd(lib, need - 1) == dsa.DSA_ERR_WORKSPACE
    assert "workspace" in dsa.dsa_last_error()
    assert _fwd(lib, need, workspace=None) == dsa.DSA_ERR_WORKSPACE
    # a smaller workspace is accepted down to topk + 192 candidate slots per row (fewer slots
    # than the default only make rows compact more often); one byte less is refused
    segs = [(0, 4, 0, 4000, 3000)]
    assert _ws(4, 4000, 64, segs)[1] == _cand_ws(4, 64, 320)
    lo = _cand_ws(4, 64, 256)
    sh = dsa._shape(n_q=4, n_k=4000, h_idx=4, d_idx=32, topk=64, segments=segs)
    call = lambda nb, ws=ctypes.c_void_p(0x1001): lib.dsa_indexer_topk(  # noqa: E731
        ctypes.byref(sh), FAKE, None, FAKE, None, FAKE, FAKE, ws, ctypes.c_size_t(nb), None)
    assert call(lo - 1) == dsa.DSA_ERR_WORKSPACE
    # (the workspace size passes; the misaligned workspace pointer is what is refused)
    assert call(lo) == dsa.DSA_ERR_INVALID_ARG and "workspace" in dsa.dsa_last_error()
    # nothing to do: every segment is empty, returns OK without launching
    assert _fwd(lib, _ws(4, 4, 2, [(0, 0, 0, 4, 0)])[1], segs=((0, 0, 0, 4, 0),)) == dsa.DSA_OK


def test_fused_indexer_topk_checks(lib):
    def call(sh, ws_bytes, workspace=FAKE, idx=FAKE):
        return lib.dsa_indexer_topk(ctypes.byref(sh), FAKE, None, FAKE, None, FAKE, idx,
                                    workspace, ctypes.c_size_t(ws_bytes), None)
    segs = [(0, 4, 0, 4, 0)]
    sh = dsa._shape(n_q=4, n_k=4, h_idx=64, d_idx=128, topk=2, segments=segs)
    need = _ws(4, 4, 2, segs)[1]
    assert call(sh, need - 1) == dsa.DSA_ERR_WORKSPACE
    assert call(sh, need, workspace=None) == dsa.DSA_ERR_WORKSPACE
    assert call(sh, need, idx=None) == dsa.DSA_ERR_INVALID_ARG
    bad = dsa._shape(n_q=4, n_k=4, h_idx=16, d_idx=128, topk=2, segments=segs)
    assert call(bad, need) == dsa.DSA_ERR_UNSUPPORTED
    empty = dsa._shape(n_q=4, n_k=4, h_idx=64, d_idx=128, topk=2, segments=[(0, 0, 0, 4, 0)])
    assert call(empty, 0, workspace=None) == dsa.DSA_OK


def _bwd(lib, sh, ws_bytes, workspace=FAKE, null_dkv=False):
    return lib.dsa_sparse_attn_bwd(ctypes.byref(sh), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                   FAKE, None if null_dkv else FAKE, workspace,
                                   ctypes.c_size_t(ws_bytes), None)


def test_backward_argument_checks(lib):
    # workspace formula: per row two bf16 [topk rounded up to 96, h] arrays, the bf16
    # [topk rounded up to 96, d_qk] contributions and topk list entries; per call 3 n_k + 1
    # ints + slack
    def al(x):
        return (x + 255) // 256 * 256

    def row(topk, topkp):
        return 2 * topkp * 128 * 2 + topkp * 576 * 2 + topk * 4

    sh = dsa._shape(n_q=5000, n_k=8192, h=128, d_qk=576, d_v=512, topk=2048, softmax_scale=0.1)
    n = ctypes.c_size_t(0)
    assert lib.dsa_sparse_attn_bwd_workspace_bytes(ctypes.byref(sh), ctypes.byref(n)) == dsa.DSA_OK
    fixed = al((3 * 8192 + 1) * 4) + 8 * 256
    assert n.value == fixed + 2048 * row(2048, 2112)
    assert dsa.dsa_sparse_attn_bwd_workspace_bytes(10, 100, 100) == \
        al((3 * 100 + 1) * 4) + 8 * 256 + 10 * row(100, 192)
    per_row = fixed + row(2048, 2112)
    assert _bwd(lib, sh, per_row - 1) == dsa.DSA_ERR_WORKSPACE
    assert _bwd(lib, sh, per_row, workspace=None) == dsa.DSA_ERR_WORKSPACE
    assert _bwd(lib, sh, per_row, workspace=ctypes.c_void_p(0x1008)) == dsa.DSA_ERR_INVALID_ARG
    assert _bwd(lib, sh, per_row, null_dkv=True) == dsa.DSA_ERR_INVALID_ARG
    # only the DeepSeek-V3.2 attention dims are built for the backward
    small = dsa._shape(n_q=4, n_k=4, h=8, d_qk=80, d_v=64, topk=4, softmax_scale=0.1)
    assert _bwd(lib, small, 1 << 20) == dsa.DSA_ERR_UNSUPPORTED
    assert "backward" in dsa.dsa_last_error()
    # nothing to do for zero rows
    empty = dsa._shape(n_q=0, n_k=4, h=128, d_qk=576, d_v=512, topk=4, softmax_scale=0.1)
    assert _bwd(lib, empty, 0) == dsa.DSA_OK


def _kl(lib, sh, ws_bytes, workspace=FAKE, null=None, misalign=None, loss_grad=1.0):
    ptrs = {k: FAKE for k in ("q_idx", "k_idx", "w_idx", "q", "kv", "idx", "smax", "ssum",
                              "loss_rows", "dq_idx", "dw_idx", "dk_idx")}
    if null:
        ptrs[null] = None
    if misalign:
        ptrs[misalign] = ctypes.c_void_p(0x1008)
    return lib.dsa_indexer_kl_loss_grad(
        ctypes.byref(sh), ptrs["q_idx"], ptrs["k_idx"], ptrs["w_idx"], ptrs["q"], ptrs["kv"],
        ptrs["idx"], ptrs["smax"], ptrs["ssum"], ctypes.c_float(loss_grad), ptrs["loss_rows"],
        None, ptrs["dq_idx"], ptrs["dw_idx"], ptrs["dk_idx"], workspace,
        ctypes.c_size_t(ws_bytes), None)


def test_indexer_kl_argument_checks(lib):
    # workspace: per row the bf16 [topk rounded up to 96, 128] key gradients, the fp32 dI of
    # those slots and topk list entries; per call 3 n_k + 1 ints, 1 KiB and alignment slack
    def al(x):
        return (x + 255) // 256 * 256

    def shape(**kw):
        base = dict(n_q=5000, n_k=8192, h_idx=64, d_idx=128, h=128, d_qk=576, d_v=512, topk=2048,
                    softmax_scale=0.1)
        base.update(kw)
        return dsa._shape(**base)

    sh = shape()
    n = ctypes.c_size_t(0)
    assert lib.dsa_indexer_kl_workspace_bytes(ctypes.byref(sh), ctypes.byref(n)) == dsa.DSA_OK
    fixed = al((3 * 8192 + 1) * 4) + 1024 + 8 * 256
    assert n.value == fixed + 2048 * (2112 * 260 + 2048 * 4)
    assert dsa.dsa_indexer_kl_workspace_bytes(10, 100, 100) == \
        al((3 * 100 + 1) * 4) + 1024 + 8 * 256 + 10 * (192 * 260 + 100 * 4)
    per_row = fixed + 2112 * 260 + 2048 * 4
    assert _kl(lib, sh, per_row - 1) == dsa.DSA_ERR_WORKSPACE
    assert _kl(lib, sh, per_row, workspace=None) == dsa.DSA_ERR_WORKSPACE
    for name in ("q_idx", "kv", "smax", "dk_idx", "loss_rows"):
        assert _kl(lib, sh, per_row, null=name) == dsa.DSA_ERR_INVALID_ARG, name
    for name in ("q_idx", "w_idx", "ssum", "dk_idx"):
        assert _kl(lib, sh, per_row, misalign=name) == dsa.DSA_ERR_INVALID_ARG, name
    assert _kl(lib, sh, per_row, workspace=ctypes.c_void_p(0x1008)) == dsa.DSA_ERR_INVALID_ARG
    assert _kl(lib, sh, per_row, loss_grad=float("nan")) == dsa.DSA_ERR_INVALID_ARG
    # built only for the DeepSeek-V3.2 shapes, bf16 index tensors and topk <= 2048
    assert _kl(lib, shape(h_idx=4, d_idx=32), 1 << 30) == dsa.DSA_ERR_UNSUPPORTED
    assert _kl(lib, shape(h=8, d_qk=80, d_v=64), 1 << 30) == dsa.DSA_ERR_UNSUPPORTED
    assert _kl(lib, shape(topk=2049), 1 << 30) == dsa.DSA_ERR_UNSUPPORTED
    assert _kl(lib, shape(topk=0), 1 << 30) == dsa.DSA_ERR_INVALID_ARG
    fp8 = shape()
    fp8.idx_dtype = dsa.DSA_IDX_FP8_E4M3
    assert _kl(lib, fp8, 1 << 30) == dsa.DSA_ERR_UNSUPPORTED
    assert "bf16" in dsa.dsa_last_error()
    # nothing to do for zero rows (and no total requested)
    assert _kl(lib, shape(n_q=0), 0, workspace=None) == dsa.DSA_OK


def _bwdkl(lib, sh, ws_bytes, workspace=FAKE, null=None, misalign=None, loss_grad=1.0):
    names = ("q", "kv", "idx", "out", "dout", "smax", "ssum", "dq", "dkv", "q_idx", "k_idx",
             "w_idx", "loss_rows", "dq_idx", "dw_idx", "dk_idx")
    ptrs = {k: FAKE for k in names}
    if null:
        ptrs[null] = None
    if misalign:
        ptrs[misalign] = ctypes.c_void_p(0x1008)
    return lib.dsa_sparse_attn_bwd_indexer_kl(
        ctypes.byref(sh), ptrs["q"], ptrs["kv"], ptrs["idx"], ptrs["out"], ptrs["dout"],
        ptrs["smax"], ptrs["ssum"], ptrs["dq"], ptrs["dkv"], ptrs["q_idx"], ptrs["k_idx"],
        ptrs["w_idx"], ctypes.c_float(loss_grad), ptrs["loss_rows"], None, ptrs["dq_idx"],
        ptrs["dw_idx"], ptrs["dk_idx"], workspace, ctypes.c_size_t(ws_bytes), None)


def test_backward_with_indexer_loss_argument_checks(lib):
    # workspace: the attention backward's (per row two bf16 [topk_p, h] arrays, the bf16
    # [topk_p, d_qk] contributions, topk list entries) plus fp32 [topk_p] head sums per row;
    # per call 3 n_k + 1 ints and alignment slack
    def al(x):
        return (x + 255) // 256 * 256

    def row(topk, topkp):
        return 2 * topkp * 128 * 2 + topkp * 576 * 2 + topk * 4 + topkp * 4

    def shape(**kw):
        base = dict(n_q=5000, n_k=8192, h_idx=64, d_idx=128, h=128, d_qk=576, d_v=512, topk=2048,
                    softmax_scale=0.1)
        base.update(kw)
        return dsa._shape(**base)

    sh = shape()
    n = ctypes.c_size_t(0)
    assert lib.dsa_sparse_attn_bwd_indexer_kl_workspace_bytes(ctypes.byref(sh),
                                                              ctypes.byref(n)) == dsa.DSA_OK
    fixed = al((3 * 8192 + 1) * 4) + 8 * 256
    assert n.value == fixed + 2048 * row(2048, 2112)
    assert dsa.dsa_sparse_attn_bwd_indexer_kl_workspace_bytes(10, 100, 100) == \
        al((3 * 100 + 1) * 4) + 8 * 256 + 10 * row(100, 192)
    per_row = fixed + row(2048, 2112)
    assert _bwdkl(lib, sh, per_row - 1) == dsa.DSA_ERR_WORKSPACE
    assert _bwdkl(lib, sh, per_row, workspace=None) == dsa.DSA_ERR_WORKSPACE
    for name in ("q", "dout", "dkv", "q_idx", "w_idx", "loss_rows", "dk_idx"):
        assert _bwdkl(lib, sh, per_row, null=name) == dsa.DSA_ERR_INVALID_ARG, name
    for name in ("dkv", "q_idx", "w_idx", "dk_idx", "dout"):
        assert _bwdkl(lib, sh, per_row, misalign=name) == dsa.DSA_ERR_INVALID_ARG, name
    assert _bwdkl(lib, sh, per_row, workspace=ctypes.c_void_p(0x1008)) == dsa.DSA_ERR_INVALID_ARG
    assert _bwdkl(lib, sh, per_row, loss_grad=float("inf")) == dsa.DSA_ERR_INVALID_ARG
    # the union of the two calls' unsupported cases
    assert _bwdkl(lib, shape(h_idx=4, d_idx=32), 1 << 30) == dsa.DSA_ERR_UNSUPPORTED
    assert _bwdkl(lib, shape(h=8, d_qk=80, d_v=64), 1 << 30) == dsa.DSA_ERR_UNSUPPORTED
    assert _bwdkl(lib, shape(topk=2049), 1 << 30) == dsa.DSA_ERR_UNSUPPORTED
    fp8 = shape()
    fp8.idx_dtype = dsa.DSA_IDX_FP8_E4M3
    assert _bwdkl(lib, fp8, 1 << 30) == dsa.DSA_ERR_UNSUPPORTED
    # nothing to do for zero rows (and no total requested)
    assert _bwdkl(lib, shape(n_q=0), 0, workspace=None) == dsa.DSA_OK


def test_quantize_argument_checks(lib):
    assert lib.dsa_quantize_fp8_rows(FAKE, -1, 8, FAKE, FAKE, None) == dsa.DSA_ERR_INVALID_ARG
    assert lib.dsa_quantize_fp8_rows(FAKE, 0, 8, FAKE, FAKE, None) == dsa.DSA_OK
    assert lib.dsa_quantize_fp8_rows(None, 4, 8, FAKE, FAKE, None) == dsa.DSA_ERR_INVALID_ARG


def test_binding_rejects_host_tensors():
    import torch
    x = torch.zeros(4, 4, 32, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        dsa.dsa_indexer_scores(x, torch.zeros(4, 32, dtype=torch.bfloat16),
                               torch.zeros(4, 4), [(0, 4, 0, 4, 0)])


def test_misaligned_pointers_rejected(lib):
    """The kernels read q_idx / k_idx / q / kv and write out in 16-byte pieces, and the index
    lists, statistics and scores as 4-byte words: misaligned pointers are refused by every
    entry point before anything is launched, naming the argument."""
    M16 = ctypes.c_void_p(0x1008)     # 8-byte aligned, not 16
    M4 = ctypes.c_void_p(0x1002)      # 2-byte aligned, not 4
    segs = [(0, 4, 0, 4, 0)]
    big = 1 << 30

    def fwd(**bad):
        p = dict(q_idx=FAKE, k_idx=FAKE, w_idx=FAKE, q=FAKE, kv=FAKE, out=FAKE, idx=None,
                 smax=None, ssum=None, ws=FAKE)
        p.update(bad)
        sh = dsa._shape(n_q=4, n_k=4, h_idx=4, d_idx=32, h=8, d_qk=80, d_v=64, topk=2,
                        softmax_scale=0.1, segments=segs)
        return lib.dsa_forward(ctypes.byref(sh), p["q_idx"], None, p["k_idx"], None, p["w_idx"],
                               p["q"], p["kv"], p["out"], p["idx"], p["smax"], p["ssum"],
                               p["ws"], ctypes.c_size_t(big), None)

    for name, ptr in [("q_idx", M16), ("k_idx", M16), ("w_idx", M4), ("q", M16), ("kv", M16),
                      ("out", M16), ("idx", M4), ("smax", M4), ("ssum", M4), ("ws", M16)]:
        assert fwd(**{name: ptr}) == dsa.DSA_ERR_INVALID_ARG, name
        assert "aligned" in dsa.dsa_last_error(), name

    sh = dsa._shape(n_q=4, n_k=4, h=8, d_qk=80, d_v=64, topk=4, softmax_scale=0.1)
    for args in [(M16, FAKE, FAKE, FAKE), (FAKE, M16, FAKE, FAKE), (FAKE, FAKE, M4, FAKE),
                 (FAKE, FAKE, FAKE, M16)]:
        assert lib.dsa_sparse_attn(ctypes.byref(sh), *args, None, None,
                                   None) == dsa.DSA_ERR_INVALID_ARG
    assert lib.dsa_sparse_attn(ctypes.byref(sh), FAKE, FAKE, FAKE, FAKE, M4, None,
                               None) == dsa.DSA_ERR_INVALID_ARG

    ish = dsa._shape(n_q=4, n_k=4, h_idx=4, d_idx=32, segments=segs)
    assert lib.dsa_indexer_scores(ctypes.byref(ish), M16, None, FAKE, None, FAKE, FAKE,
                                  None) == dsa.DSA_ERR_INVALID_ARG
    assert lib.dsa_indexer_scores(ctypes.byref(ish), FAKE, None, FAKE, None, FAKE, M4,
                                  None) == dsa.DSA_ERR_INVALID_ARG
    tsh = dsa._shape(n_q=4, n_k=4, h_idx=4, d_idx=32, topk=2, segments=segs)
    assert lib.dsa_topk_select(ctypes.byref(tsh), M4, FAKE, None) == dsa.DSA_ERR_INVALID_ARG
    assert lib.dsa_topk_select(ctypes.byref(tsh), FAKE, M4, None) == dsa.DSA_ERR_INVALID_ARG
    assert lib.dsa_indexer_topk(ctypes.byref(tsh), FAKE, None, M16, None, FAKE, FAKE, FAKE,
                                ctypes.c_size_t(big), None) == dsa.DSA_ERR_INVALID_ARG
    assert lib.dsa_indexer_topk(ctypes.byref(tsh), FAKE, None, FAKE, None, FAKE, M4, FAKE,
                                ctypes.c_size_t(big), None) == dsa.DSA_ERR_INVALID_ARG

    bsh = dsa._shape(n_q=4, n_k=4, h=128, d_qk=576, d_v=512, topk=4, softmax_scale=0.1)
    for pos in range(8):   # q, kv, idx, out, dout, smax, ssum, dq
        ptrs = [FAKE] * 8
        ptrs[pos] = M4 if pos in (2, 5, 6) else M16
        assert lib.dsa_sparse_attn_bwd(ctypes.byref(bsh), *ptrs, FAKE, FAKE,
                                       ctypes.c_size_t(big), None) == dsa.DSA_ERR_INVALID_ARG, pos


def test_package_exposes_every_binding():
    """Every entry point of the binding is reachable from the package itself."""
    import sparse_attention_11_amd as pkg
    for name in dsa.EXPORTED:
        if name.endswith(("_workspace_bytes",)) or name.startswith("dsa_"):
            if hasattr(dsa, name):
                assert getattr(pkg, name) is getattr(dsa, name), name


def test_dense_attention_argument_checks(lib):
    def call(h=2, d_qk=192, d_v=128, scale=0.1, segs=((0, 4, 0, 4, 0),), n_k=4, q=FAKE, k=FAKE,
             v=FAKE, out=FAKE, lse=None):
        sh = dsa._shape(n_q=4, n_k=n_k, h=h, d_qk=d_qk, d_v=d_v, softmax_scale=scale,
                        segments=segs)
        return lib.dsa_dense_attn(ctypes.byref(sh), q, k, v, out, lse, None)
    assert call(d_qk=576, d_v=512) == dsa.DSA_ERR_UNSUPPORTED
    assert call(d_v=64) == dsa.DSA_ERR_UNSUPPORTED
    assert call(h=0) == dsa.DSA_ERR_INVALID_ARG
    for bad in (0.0, -0.1, float("nan"), float("inf")):
        assert call(scale=bad) == dsa.DSA_ERR_INVALID_ARG, bad
    assert call(segs=((0, 4, 0, 4, 1),)) == dsa.DSA_ERR_INVALID_ARG      # position past k_len
    assert call(segs=((0, 4, 0, 8, 0),)) == dsa.DSA_ERR_INVALID_ARG      # keys past n_k
    for name in ("q", "k", "v", "out"):
        assert call(**{name: None}) == dsa.DSA_ERR_INVALID_ARG, name
        assert call(**{name: ctypes.c_void_p(0x1008)}) == dsa.DSA_ERR_INVALID_ARG, name
    assert call(lse=ctypes.c_void_p(0x1002)) == dsa.DSA_ERR_INVALID_ARG
    # K over 4 GiB of 32-bit DMA offsets
    big = ((0, 4, 0, 4, 0),)
    assert call(h=128, n_k=90000, segs=big) == dsa.DSA_ERR_UNSUPPORTED
    # no covered row: nothing is read or launched, even with NULL tensors
    assert call(segs=(), q=None, k=None, v=None, out=None) == dsa.DSA_OK
