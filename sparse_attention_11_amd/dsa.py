"""ctypes binding of libdsa with the C ABI's entry-point names (include/dsa.h).

Argument marshalling only: tensors are checked for device, dtype, shape and contiguity,
outputs are allocated with torch when not given, and the call is enqueued on the current
torch stream.  Every computation runs in the HIP library; if ``libdsa.so`` is missing the
first call raises instead of falling back to anything else.
"""

from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdsa.so")

DSA_OK, DSA_ERR_INVALID_ARG, DSA_ERR_UNSUPPORTED, DSA_ERR_WORKSPACE, DSA_ERR_HIP = range(5)
DSA_IDX_BF16, DSA_IDX_FP8_E4M3 = 0, 1
_STATUS = {1: "DSA_ERR_INVALID_ARG", 2: "DSA_ERR_UNSUPPORTED", 3: "DSA_ERR_WORKSPACE",
           4: "DSA_ERR_HIP"}


class DsaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status


class Segment(ctypes.Structure):
    _fields_ = [("q_start", ctypes.c_int32), ("q_len", ctypes.c_int32),
                ("k_start", ctypes.c_int32), ("k_len", ctypes.c_int32),
                ("pos0", ctypes.c_int32)]


class Shape(ctypes.Structure):
    _fields_ = [("n_q", ctypes.c_int32), ("n_k", ctypes.c_int32),
                ("h_idx", ctypes.c_int32), ("d_idx", ctypes.c_int32),
                ("h", ctypes.c_int32), ("d_qk", ctypes.c_int32), ("d_v", ctypes.c_int32),
                ("topk", ctypes.c_int32), ("softmax_scale", ctypes.c_float),
                ("idx_dtype", ctypes.c_int32), ("segs", ctypes.POINTER(Segment)),
                ("n_segs", ctypes.c_int32)]


_P = ctypes.c_void_p
_SIGS = {
    "dsa_abi_version": (ctypes.c_int, []),
    "dsa_last_error": (ctypes.c_char_p, []),
    "dsa_workspace_bytes": (ctypes.c_int, [ctypes.POINTER(Shape), ctypes.POINTER(ctypes.c_size_t)]),
    "dsa_indexer_scores": (ctypes.c_int, [ctypes.POINTER(Shape), _P, _P, _P, _P, _P, _P, _P]),
    "dsa_topk_select": (ctypes.c_int, [ctypes.POINTER(Shape), _P, _P, _P]),
    "dsa_indexer_topk": (ctypes.c_int, [ctypes.POINTER(Shape), _P, _P, _P, _P, _P, _P, _P,
                                        ctypes.c_size_t, _P]),
    "dsa_sparse_attn": (ctypes.c_int, [ctypes.POINTER(Shape), _P, _P, _P, _P, _P, _P, _P]),
    "dsa_forward": (ctypes.c_int, [ctypes.POINTER(Shape), _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                   _P, _P, _P, ctypes.c_size_t, _P]),
    "dsa_forward_noalloc": (ctypes.c_int, [ctypes.POINTER(Shape), _P, _P, _P, _P, _P, _P, _P, _P,
                                           _P, _P, _P, _P]),
    "dsa_quantize_fp8_rows": (ctypes.c_int, [_P, ctypes.c_int64, ctypes.c_int32, _P, _P, _P]),
    "dsa_dense_attn": (ctypes.c_int, [ctypes.POINTER(Shape), _P, _P, _P, _P, _P, _P]),
    "dsa_sparse_attn_bwd": (ctypes.c_int, [ctypes.POINTER(Shape), _P, _P, _P, _P, _P, _P, _P,
                                           _P, _P, _P, ctypes.c_size_t, _P]),
    "dsa_sparse_attn_bwd_workspace_bytes": (ctypes.c_int, [ctypes.POINTER(Shape),
                                                           ctypes.POINTER(ctypes.c_size_t)]),
    "dsa_indexer_kl_loss_grad": (ctypes.c_int, [ctypes.POINTER(Shape), _P, _P, _P, _P, _P, _P,
                                                _P, _P, ctypes.c_float, _P, _P, _P, _P, _P, _P,
                                                ctypes.c_size_t, _P]),
    "dsa_indexer_kl_workspace_bytes": (ctypes.c_int, [ctypes.POINTER(Shape),
                                                      ctypes.POINTER(ctypes.c_size_t)]),
    "dsa_sparse_attn_bwd_indexer_kl": (ctypes.c_int, [ctypes.POINTER(Shape), _P, _P, _P, _P, _P,
                                                      _P, _P, _P, _P, _P, _P, _P,
                                                      ctypes.c_float, _P, _P, _P, _P, _P, _P,
                                                      ctypes.c_size_t, _P]),
    "dsa_sparse_attn_bwd_indexer_kl_workspace_bytes": (ctypes.c_int,
                                                       [ctypes.POINTER(Shape),
                                                        ctypes.POINTER(ctypes.c_size_t)]),
}
EXPORTED = tuple(_SIGS)

_lib = None


def load_library(path: str | None = None) -> ctypes.CDLL:
    """Load libdsa.so (once) and declare the C signatures."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise DsaError(DSA_ERR_UNSUPPORTED,
                       f"{p} not found: build the HIP library first (__graft_entry__.build())")
    lib = ctypes.CDLL(p)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path is None:
        _lib = lib
    return lib


def _check(status: int):
    if status != DSA_OK:
        msg = load_library().dsa_last_error().decode(errors="replace")
        raise DsaError(status, msg)


def dsa_abi_version() -> int:
    return load_library().dsa_abi_version()


def dsa_last_error() -> str:
    return load_library().dsa_last_error().decode(errors="replace")


# ------------------------------------------------------------------------- marshalling ----


def _segs(segments):
    segs = list(segments)
    arr = (Segment * max(1, len(segs)))()
    for i, s in enumerate(segs):
        arr[i] = Segment(*[int(x) for x in s])
    return arr, len(segs)


def _shape(n_q=0, n_k=0, h_idx=0, d_idx=0, h=0, d_qk=0, d_v=0, topk=0, softmax_scale=0.0,
           idx_dtype=DSA_IDX_BF16, segments=()):
    arr, n = _segs(segments)
    sh = Shape(int(n_q), int(n_k), int(h_idx), int(d_idx), int(h), int(d_qk), int(d_v),
               int(topk), float(softmax_scale), int(idx_dtype),
               ctypes.cast(arr, ctypes.POINTER(Segment)), n)
    sh._keep = arr  # keep the segment array alive with the struct
    return sh


def _dev(t, name, dtypes, ndim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor (got {t.device})")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims (got shape {tuple(t.shape)})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device, stream):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


_FP8 = (torch.uint8, torch.float8_e4m3fn)


def _idx_inputs(q_idx, k_idx, w_idx, q_scale, k_scale):
    fp8 = q_idx.dtype in _FP8
    dts = _FP8 if fp8 else (torch.bfloat16,)
    _dev(q_idx, "q_idx", dts, 3)
    _dev(k_idx, "k_idx", dts, 2)
    _dev(w_idx, "w_idx", (torch.float32,), 2)
    if fp8:
        if q_scale is None or k_scale is None:
            raise ValueError("fp8 index inputs need q_scale and k_scale")
        _dev(q_scale, "q_scale", (torch.float32,), 1)
        _dev(k_scale, "k_scale", (torch.float32,), 1)
        if q_scale.shape[0] != q_idx.shape[0] or k_scale.shape[0] != k_idx.shape[0]:
            raise ValueError("q_scale / k_scale must hold one scale per token row")
    n_q, h_idx, d_idx = q_idx.shape
    if k_idx.shape[1] != d_idx or tuple(w_idx.shape) != (n_q, h_idx):
        raise ValueError("q_idx [n_q,h_idx,d_idx], k_idx [n_k,d_idx], w_idx [n_q,h_idx] mismatch")
    return fp8, n_q, h_idx, d_idx


# ------------------------------------------------------------------------- entry points ----


def dsa_workspace_bytes(n_q: int, n_k: int, topk: int, segments) -> int:
    sh = _shape(n_q=n_q, n_k=n_k, topk=topk, segments=segments)
    out = ctypes.c_size_t(0)
    _check(load_library().dsa_workspace_bytes(ctypes.byref(sh), ctypes.byref(out)))
    return int(out.value)


def dsa_indexer_scores(q_idx, k_idx, w_idx, segments, q_scale=None, k_scale=None, out=None,
                       stream=None):
    """Indexer scores [n_q, n_k] fp32 (-inf outside each covered row's causal window)."""
    fp8, n_q, h_idx, d_idx = _idx_inputs(q_idx, k_idx, w_idx, q_scale, k_scale)
    n_k = k_idx.shape[0]
    if out is None:
        out = torch.empty(n_q, n_k, dtype=torch.float32, device=q_idx.device)
    _dev(out, "out", (torch.float32,), 2)
    sh = _shape(n_q=n_q, n_k=n_k, h_idx=h_idx, d_idx=d_idx,
                idx_dtype=DSA_IDX_FP8_E4M3 if fp8 else DSA_IDX_BF16, segments=segments)
    _check(load_library().dsa_indexer_scores(ctypes.byref(sh), _ptr(q_idx), _ptr(q_scale),
                                             _ptr(k_idx), _ptr(k_scale), _ptr(w_idx), _ptr(out),
                                             _stream(q_idx.device, stream)))
    return out


def dsa_topk_select(scores, segments, topk: int, out=None, stream=None):
    """Top-k key rows [n_q, topk] int32 (ascending, -1 padded) from dense indexer scores."""
    _dev(scores, "scores", (torch.float32,), 2)
    n_q, n_k = scores.shape
    if out is None:
        out = torch.empty(n_q, topk, dtype=torch.int32, device=scores.device)
    _dev(out, "out", (torch.int32,), 2)
    sh = _shape(n_q=n_q, n_k=n_k, topk=topk, segments=segments)
    _check(load_library().dsa_topk_select(ctypes.byref(sh), _ptr(scores), _ptr(out),
                                          _stream(scores.device, stream)))
    return out


def dsa_indexer_topk(q_idx, k_idx, w_idx, segments, topk: int, q_scale=None, k_scale=None,
                     out=None, workspace=None, stream=None):
    """The indexer fused with the top-k: int32 [n_q, topk] indices (ascending, -1 padded) of
    every covered row, the same as dsa_indexer_scores followed by dsa_topk_select."""
    fp8, n_q, h_idx, d_idx = _idx_inputs(q_idx, k_idx, w_idx, q_scale, k_scale)
    n_k = k_idx.shape[0]
    dev = q_idx.device
    if out is None:
        out = torch.full((n_q, topk), -1, dtype=torch.int32, device=dev)
    _dev(out, "out", (torch.int32,), 2)
    sh = _shape(n_q=n_q, n_k=n_k, h_idx=h_idx, d_idx=d_idx, topk=topk,
                idx_dtype=DSA_IDX_FP8_E4M3 if fp8 else DSA_IDX_BF16, segments=segments)
    lib = load_library()
    if workspace is None:
        nbytes = ctypes.c_size_t(0)
        _check(lib.dsa_workspace_bytes(ctypes.byref(sh), ctypes.byref(nbytes)))
        workspace = torch.empty(max(1, nbytes.value), dtype=torch.uint8, device=dev)
    _dev(workspace, "workspace", (torch.uint8,))
    _check(lib.dsa_indexer_topk(ctypes.byref(sh), _ptr(q_idx), _ptr(q_scale), _ptr(k_idx),
                                _ptr(k_scale), _ptr(w_idx), _ptr(out), _ptr(workspace),
                                ctypes.c_size_t(workspace.numel()), _stream(dev, stream)))
    return out


def dsa_sparse_attn(q, kv, topk_idx, softmax_scale: float, d_v: int, out=None, stats=True,
                    stream=None):
    """Sparse MQA over the selected latent rows.  Returns (out, softmax_max, softmax_sum);
    the statistics are None when ``stats`` is False."""
    _dev(q, "q", (torch.bfloat16,), 3)
    _dev(kv, "kv", (torch.bfloat16,), 2)
    _dev(topk_idx, "topk_idx", (torch.int32,), 2)
    n_q, h, d_qk = q.shape
    if kv.shape[1] != d_qk or topk_idx.shape[0] != n_q:
        raise ValueError("q [n_q,h,d_qk], kv [n_k,d_qk], topk_idx [n_q,topk] mismatch")
    if out is None:
        out = torch.empty(n_q, h, d_v, dtype=torch.bfloat16, device=q.device)
    _dev(out, "out", (torch.bfloat16,), 3)
    smax = ssum = None
    if stats:
        smax = torch.empty(n_q, h, dtype=torch.float32, device=q.device)
        ssum = torch.empty(n_q, h, dtype=torch.float32, device=q.device)
    sh = _shape(n_q=n_q, n_k=kv.shape[0], h=h, d_qk=d_qk, d_v=d_v, topk=topk_idx.shape[1],
                softmax_scale=softmax_scale)
    _check(load_library().dsa_sparse_attn(ctypes.byref(sh), _ptr(q), _ptr(kv), _ptr(topk_idx),
                                          _ptr(out), _ptr(smax), _ptr(ssum),
                                          _stream(q.device, stream)))
    return out, smax, ssum


def dsa_dense_attn(q, k, v, segments, softmax_scale: float, out=None, lse=True, stream=None):
    """Dense causal attention of a head shard: q [n_q,h,192], k [n_k,h,192], v [n_k,h,128]
    (bf16), rows windowed by ``segments`` as in the DSA calls.  Returns (out [n_q,h,128] bf16,
    lse [n_q,h] fp32 or None when ``lse`` is False)."""
    _dev(q, "q", (torch.bfloat16,), 3)
    _dev(k, "k", (torch.bfloat16,), 3)
    _dev(v, "v", (torch.bfloat16,), 3)
    n_q, h, d_qk = q.shape
    n_k, d_v = k.shape[0], v.shape[2]
    if k.shape[1:] != (h, d_qk) or v.shape[:2] != (n_k, h):
        raise ValueError("q [n_q,h,d_qk], k [n_k,h,d_qk], v [n_k,h,d_v] mismatch")
    if out is None:
        out = torch.empty(n_q, h, d_v, dtype=torch.bfloat16, device=q.device)
    _dev(out, "out", (torch.bfloat16,), 3)
    lse_t = torch.empty(n_q, h, dtype=torch.float32, device=q.device) if lse else None
    sh = _shape(n_q=n_q, n_k=n_k, h=h, d_qk=d_qk, d_v=d_v, softmax_scale=softmax_scale,
                segments=segments)
    _check(load_library().dsa_dense_attn(ctypes.byref(sh), _ptr(q), _ptr(k), _ptr(v), _ptr(out),
                                         _ptr(lse_t), _stream(q.device, stream)))
    return out, lse_t


def dsa_sparse_attn_bwd_workspace_bytes(n_q: int, n_k: int, topk: int, h: int = 128,
                                        d_qk: int = 576, d_v: int = 512) -> int:
    sh = _shape(n_q=n_q, n_k=n_k, h=h, d_qk=d_qk, d_v=d_v, topk=topk, softmax_scale=1.0)
    n = ctypes.c_size_t(0)
    _check(load_library().dsa_sparse_attn_bwd_workspace_bytes(ctypes.byref(sh), ctypes.byref(n)))
    return int(n.value)


def dsa_sparse_attn_bwd(q, kv, topk_idx, out, dout, softmax_max, softmax_sum,
                        softmax_scale: float, dq=None, dkv=None, workspace=None, stream=None):
    """Gradients of the sparse attention.  Returns (dq bf16 [n_q,h,d_qk], dkv fp32 [n_k,d_qk]);
    a given ``dkv`` is accumulated into, a new one starts at zero."""
    _dev(q, "q", (torch.bfloat16,), 3)
    _dev(kv, "kv", (torch.bfloat16,), 2)
    _dev(topk_idx, "topk_idx", (torch.int32,), 2)
    _dev(out, "out", (torch.bfloat16,), 3)
    _dev(dout, "dout", (torch.bfloat16,), 3)
    _dev(softmax_max, "softmax_max", (torch.float32,), 2)
    _dev(softmax_sum, "softmax_sum", (torch.float32,), 2)
    n_q, h, d_qk = q.shape
    n_k = kv.shape[0]
    d_v = out.shape[2]
    topk = topk_idx.shape[1]
    if (kv.shape[1] != d_qk or topk_idx.shape[0] != n_q or out.shape[:2] != (n_q, h)
            or dout.shape != out.shape or softmax_max.shape != (n_q, h)
            or softmax_sum.shape != (n_q, h)):
        raise ValueError("backward tensor shapes do not match q [n_q,h,d_qk] / kv [n_k,d_qk]")
    dev = q.device
    if dq is None:
        dq = torch.empty(n_q, h, d_qk, dtype=torch.bfloat16, device=dev)
    if dkv is None:
        dkv = torch.zeros(n_k, d_qk, dtype=torch.float32, device=dev)
    _dev(dq, "dq", (torch.bfloat16,), 3)
    _dev(dkv, "dkv", (torch.float32,), 2)
    sh = _shape(n_q=n_q, n_k=n_k, h=h, d_qk=d_qk, d_v=d_v, topk=topk,
                softmax_scale=softmax_scale)
    if workspace is None:
        nb = dsa_sparse_attn_bwd_workspace_bytes(n_q, n_k, topk, h, d_qk, d_v)
        workspace = torch.empty(max(nb, 1), dtype=torch.uint8, device=dev)
    _check(load_library().dsa_sparse_attn_bwd(
        ctypes.byref(sh), _ptr(q), _ptr(kv), _ptr(topk_idx), _ptr(out), _ptr(dout),
        _ptr(softmax_max), _ptr(softmax_sum), _ptr(dq), _ptr(dkv), _ptr(workspace),
        ctypes.c_size_t(workspace.numel() * workspace.element_size()), _stream(dev, stream)))
    return dq, dkv


def dsa_indexer_kl_workspace_bytes(n_q: int, n_k: int, topk: int) -> int:
    sh = _shape(n_q=n_q, n_k=n_k, h_idx=64, d_idx=128, h=128, d_qk=576, d_v=512, topk=topk,
                softmax_scale=1.0)
    n = ctypes.c_size_t(0)
    _check(load_library().dsa_indexer_kl_workspace_bytes(ctypes.byref(sh), ctypes.byref(n)))
    return int(n.value)


def dsa_indexer_kl_loss_grad(q_idx, k_idx, w_idx, q, kv, topk_idx, softmax_max, softmax_sum,
                             softmax_scale: float, loss_grad: float = 1.0, dk_idx=None,
                             workspace=None, stream=None):
    """Indexer KL loss against the head-summed attention distribution, and its gradients.

    Returns (loss fp32 [1], loss_rows fp32 [n_q], dq_idx bf16 [n_q,64,128], dw_idx fp32
    [n_q,64], dk_idx fp32 [n_k,128]); a given ``dk_idx`` is accumulated into, a new one starts
    at zero."""
    _dev(q_idx, "q_idx", (torch.bfloat16,), 3)
    _dev(k_idx, "k_idx", (torch.bfloat16,), 2)
    _dev(w_idx, "w_idx", (torch.float32,), 2)
    _dev(q, "q", (torch.bfloat16,), 3)
    _dev(kv, "kv", (torch.bfloat16,), 2)
    _dev(topk_idx, "topk_idx", (torch.int32,), 2)
    _dev(softmax_max, "softmax_max", (torch.float32,), 2)
    _dev(softmax_sum, "softmax_sum", (torch.float32,), 2)
    n_q, h_idx, d_idx = q_idx.shape
    n_k = k_idx.shape[0]
    _, h, d_qk = q.shape
    topk = topk_idx.shape[1]
    if (k_idx.shape[1] != d_idx or w_idx.shape != (n_q, h_idx) or q.shape[0] != n_q
            or kv.shape != (n_k, d_qk) or topk_idx.shape[0] != n_q
            or softmax_max.shape != (n_q, h) or softmax_sum.shape != (n_q, h)):
        raise ValueError("indexer loss tensor shapes do not match q_idx [n_q,h_idx,d_idx] / "
                         "k_idx [n_k,d_idx] / q [n_q,h,d_qk] / kv [n_k,d_qk]")
    dev = q.device
    loss = torch.empty(1, dtype=torch.float32, device=dev)
    loss_rows = torch.empty(n_q, dtype=torch.float32, device=dev)
    dq_idx = torch.empty(n_q, h_idx, d_idx, dtype=torch.bfloat16, device=dev)
    dw_idx = torch.empty(n_q, h_idx, dtype=torch.float32, device=dev)
    if dk_idx is None:
        dk_idx = torch.zeros(n_k, d_idx, dtype=torch.float32, device=dev)
    _dev(dk_idx, "dk_idx", (torch.float32,), 2)
    sh = _shape(n_q=n_q, n_k=n_k, h_idx=h_idx, d_idx=d_idx, h=h, d_qk=d_qk, d_v=512, topk=topk,
                softmax_scale=softmax_scale)
    if workspace is None:
        nb = dsa_indexer_kl_workspace_bytes(n_q, n_k, topk)
        workspace = torch.empty(max(nb, 1), dtype=torch.uint8, device=dev)
    _check(load_library().dsa_indexer_kl_loss_grad(
        ctypes.byref(sh), _ptr(q_idx), _ptr(k_idx), _ptr(w_idx), _ptr(q), _ptr(kv),
        _ptr(topk_idx), _ptr(softmax_max), _ptr(softmax_sum), ctypes.c_float(loss_grad),
        _ptr(loss_rows), _ptr(loss), _ptr(dq_idx), _ptr(dw_idx), _ptr(dk_idx), _ptr(workspace),
        ctypes.c_size_t(workspace.numel() * workspace.element_size()), _stream(dev, stream)))
    return loss, loss_rows, dq_idx, dw_idx, dk_idx


def dsa_sparse_attn_bwd_indexer_kl_workspace_bytes(n_q: int, n_k: int, topk: int) -> int:
    sh = _shape(n_q=n_q, n_k=n_k, h_idx=64, d_idx=128, h=128, d_qk=576, d_v=512, topk=topk,
                softmax_scale=1.0)
    n = ctypes.c_size_t(0)
    _check(load_library().dsa_sparse_attn_bwd_indexer_kl_workspace_bytes(ctypes.byref(sh),
                                                                         ctypes.byref(n)))
    return int(n.value)


def dsa_sparse_attn_bwd_indexer_kl(q, kv, topk_idx, out, dout, softmax_max, softmax_sum,
                                   softmax_scale: float, q_idx, k_idx, w_idx,
                                   loss_grad: float = 1.0, dq=None, dkv=None, dk_idx=None,
                                   workspace=None, stream=None):
    """The attention backward and the indexer KL loss of one step in one call.

    Returns (dq, dkv, loss, loss_rows, dq_idx, dw_idx, dk_idx) as dsa_sparse_attn_bwd and
    dsa_indexer_kl_loss_grad; a given ``dkv`` / ``dk_idx`` is accumulated into, a new one
    starts at zero."""
    _dev(q, "q", (torch.bfloat16,), 3)
    _dev(kv, "kv", (torch.bfloat16,), 2)
    _dev(topk_idx, "topk_idx", (torch.int32,), 2)
    _dev(out, "out", (torch.bfloat16,), 3)
    _dev(dout, "dout", (torch.bfloat16,), 3)
    _dev(softmax_max, "softmax_max", (torch.float32,), 2)
    _dev(softmax_sum, "softmax_sum", (torch.float32,), 2)
    _dev(q_idx, "q_idx", (torch.bfloat16,), 3)
    _dev(k_idx, "k_idx", (torch.bfloat16,), 2)
    _dev(w_idx, "w_idx", (torch.float32,), 2)
    n_q, h, d_qk = q.shape
    n_k = kv.shape[0]
    d_v = out.shape[2]
    topk = topk_idx.shape[1]
    _, h_idx, d_idx = q_idx.shape
    if (kv.shape[1] != d_qk or topk_idx.shape[0] != n_q or out.shape[:2] != (n_q, h)
            or dout.shape != out.shape or softmax_max.shape != (n_q, h)
            or softmax_sum.shape != (n_q, h) or q_idx.shape[0] != n_q
            or k_idx.shape != (n_k, d_idx) or w_idx.shape != (n_q, h_idx)):
        raise ValueError("backward / indexer loss tensor shapes do not match q [n_q,h,d_qk], "
                         "kv [n_k,d_qk], q_idx [n_q,h_idx,d_idx], k_idx [n_k,d_idx]")
    dev = q.device
    if dq is None:
        dq = torch.empty(n_q, h, d_qk, dtype=torch.bfloat16, device=dev)
    if dkv is None:
        dkv = torch.zeros(n_k, d_qk, dtype=torch.float32, device=dev)
    if dk_idx is None:
        dk_idx = torch.zeros(n_k, d_idx, dtype=torch.float32, device=dev)
    _dev(dq, "dq", (torch.bfloat16,), 3)
    _dev(dkv, "dkv", (torch.float32,), 2)
    _dev(dk_idx, "dk_idx", (torch.float32,), 2)
    loss = torch.empty(1, dtype=torch.float32, device=dev)
    loss_rows = torch.empty(n_q, dtype=torch.float32, device=dev)
    dq_idx = torch.empty(n_q, h_idx, d_idx, dtype=torch.bfloat16, device=dev)
    dw_idx = torch.empty(n_q, h_idx, dtype=torch.float32, device=dev)
    sh = _shape(n_q=n_q, n_k=n_k, h_idx=h_idx, d_idx=d_idx, h=h, d_qk=d_qk, d_v=d_v, topk=topk,
                softmax_scale=softmax_scale)
    if workspace is None:
        nb = dsa_sparse_attn_bwd_indexer_kl_workspace_bytes(n_q, n_k, topk)
        workspace = torch.empty(max(nb, 1), dtype=torch.uint8, device=dev)
    _check(load_library().dsa_sparse_attn_bwd_indexer_kl(
        ctypes.byref(sh), _ptr(q), _ptr(kv), _ptr(topk_idx), _ptr(out), _ptr(dout),
        _ptr(softmax_max), _ptr(softmax_sum), _ptr(dq), _ptr(dkv), _ptr(q_idx), _ptr(k_idx),
        _ptr(w_idx), ctypes.c_float(loss_grad), _ptr(loss_rows), _ptr(loss), _ptr(dq_idx),
        _ptr(dw_idx), _ptr(dk_idx), _ptr(workspace),
        ctypes.c_size_t(workspace.numel() * workspace.element_size()), _stream(dev, stream)))
    return dq, dkv, loss, loss_rows, dq_idx, dw_idx, dk_idx


def dsa_forward(q_idx, k_idx, w_idx, q, kv, segments, topk: int, softmax_scale: float,
                d_v: int, q_scale=None, k_scale=None, out=None, return_idx=True, stats=True,
                workspace=None, stream=None):
    """Fused indexer -> top-k -> sparse attention on one CP rank's share.

    Returns (out, topk_idx or None, softmax_max or None, softmax_sum or None)."""
    fp8, n_q, h_idx, d_idx = _idx_inputs(q_idx, k_idx, w_idx, q_scale, k_scale)
    _dev(q, "q", (torch.bfloat16,), 3)
    _dev(kv, "kv", (torch.bfloat16,), 2)
    n_k = k_idx.shape[0]
    _, h, d_qk = q.shape
    if q.shape[0] != n_q or kv.shape != (n_k, d_qk):
        raise ValueError("q [n_q,h,d_qk] / kv [n_k,d_qk] do not match the index tensors")
    dev = q.device
    if out is None:
        out = torch.empty(n_q, h, d_v, dtype=torch.bfloat16, device=dev)
    _dev(out, "out", (torch.bfloat16,), 3)
    idx = torch.empty(n_q, topk, dtype=torch.int32, device=dev) if return_idx else None
    smax = torch.empty(n_q, h, dtype=torch.float32, device=dev) if stats else None
    ssum = torch.empty(n_q, h, dtype=torch.float32, device=dev) if stats else None
    sh = _shape(n_q=n_q, n_k=n_k, h_idx=h_idx, d_idx=d_idx, h=h, d_qk=d_qk, d_v=d_v, topk=topk,
                softmax_scale=softmax_scale,
                idx_dtype=DSA_IDX_FP8_E4M3 if fp8 else DSA_IDX_BF16, segments=segments)
    nbytes = ctypes.c_size_t(0)
    lib = load_library()
    _check(lib.dsa_workspace_bytes(ctypes.byref(sh), ctypes.byref(nbytes)))
    if workspace is None:
        workspace = torch.empty(max(1, nbytes.value), dtype=torch.uint8, device=dev)
    _dev(workspace, "workspace", (torch.uint8,))
    _check(lib.dsa_forward(ctypes.byref(sh), _ptr(q_idx), _ptr(q_scale), _ptr(k_idx),
                           _ptr(k_scale), _ptr(w_idx), _ptr(q), _ptr(kv), _ptr(out), _ptr(idx),
                           _ptr(smax), _ptr(ssum), _ptr(workspace),
                           ctypes.c_size_t(workspace.numel()), _stream(dev, stream)))
    return out, idx, smax, ssum


def dsa_forward_noalloc(q_idx, k_idx, w_idx, q, kv, segments, topk: int, softmax_scale: float,
                        d_v: int, out, topk_idx=None, softmax_max=None, softmax_sum=None,
                        q_scale=None, k_scale=None, stream=None):
    """dsa_forward with the library's fixed per-GPU scratch as its workspace: every output is
    given by the caller (topk_idx / softmax_max / softmax_sum may be None) and nothing is
    allocated.  Returns (out, topk_idx, softmax_max, softmax_sum)."""
    fp8, n_q, h_idx, d_idx = _idx_inputs(q_idx, k_idx, w_idx, q_scale, k_scale)
    _dev(q, "q", (torch.bfloat16,), 3)
    _dev(kv, "kv", (torch.bfloat16,), 2)
    _dev(out, "out", (torch.bfloat16,), 3)
    n_k = k_idx.shape[0]
    _, h, d_qk = q.shape
    if q.shape[0] != n_q or kv.shape != (n_k, d_qk) or tuple(out.shape) != (n_q, h, d_v):
        raise ValueError("q [n_q,h,d_qk] / kv [n_k,d_qk] / out [n_q,h,d_v] do not match")
    for t, name, shp in ((topk_idx, "topk_idx", (n_q, topk)), (softmax_max, "softmax_max", (n_q, h)),
                         (softmax_sum, "softmax_sum", (n_q, h))):
        if t is not None:
            _dev(t, name, (torch.int32,) if name == "topk_idx" else (torch.float32,), 2)
            if tuple(t.shape) != shp:
                raise ValueError(f"{name} must be {shp}")
    sh = _shape(n_q=n_q, n_k=n_k, h_idx=h_idx, d_idx=d_idx, h=h, d_qk=d_qk, d_v=d_v, topk=topk,
                softmax_scale=softmax_scale,
                idx_dtype=DSA_IDX_FP8_E4M3 if fp8 else DSA_IDX_BF16, segments=segments)
    _check(load_library().dsa_forward_noalloc(
        ctypes.byref(sh), _ptr(q_idx), _ptr(q_scale), _ptr(k_idx), _ptr(k_scale), _ptr(w_idx),
        _ptr(q), _ptr(kv), _ptr(out), _ptr(topk_idx), _ptr(softmax_max), _ptr(softmax_sum),
        _stream(q.device, stream)))
    return out, topk_idx, softmax_max, softmax_sum


def dsa_quantize_fp8_rows(x, out=None, scale=None, stream=None):
    """Per-row e4m3fn quantization of a bf16 tensor viewed as [rows, cols] (rows = dim 0).
    Returns (codes uint8 of x's shape, scale fp32 [rows])."""
    _dev(x, "x", (torch.bfloat16,))
    rows = x.shape[0]
    cols = x.numel() // max(1, rows)
    if out is None:
        out = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    if scale is None:
        scale = torch.empty(rows, dtype=torch.float32, device=x.device)
    _dev(out, "out", (torch.uint8,))
    _dev(scale, "scale", (torch.float32,), 1)
    _check(load_library().dsa_quantize_fp8_rows(_ptr(x), ctypes.c_int64(rows),
                                                ctypes.c_int32(cols), _ptr(out), _ptr(scale),
                                                _stream(x.device, stream)))
    return out, scale
