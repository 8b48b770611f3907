"""Seeded synthetic inputs for the DSA forward workloads.

This module only draws random tensors and builds segment tables; it holds none of the
method's arithmetic.  Both the HIP path's tests and the oracle's tests take their inputs from
here, so the two sides always see the same numbers.

The workloads stand in for DeepSeek-V3.2 32K continued pretraining (weights and corpus are not
available): Gaussian index queries/keys and latent rows, uniform per-token index weights, with
the model's shapes (64 index heads of width 128, 128 query heads over a 576-wide latent row
whose first 512 columns are the value).  Random data makes the selected keys close to uniform
over each window, the worst case for gather locality.

Every tensor is drawn on a CPU ``torch.Generator`` seeded with ``1000 + workload number``
(unless a seed is given) in the fixed order q_idx, k_idx, w_idx, q, kv, dout, in float32, and
rounded to bfloat16 with round-to-nearest-even.  Index weights are also rounded to bfloat16
values and then carried as float32, so an fp32 and a bf16 consumer see the same numbers.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    n_q: int                 # local query rows T
    n_k: int                 # gathered key rows S_k
    h_idx: int
    d_idx: int
    h: int
    d_qk: int
    d_v: int
    topk: int
    segments: tuple          # ((q_start, q_len, k_start, k_len, pos0), ...)
    w_scale: float           # w_idx ~ U(0,1) * w_scale
    kv_std: float = 1.0
    softmax_scale: float = 0.0
    fp8_indexer: bool = False
    with_dout: bool = False
    seed: int = 0
    doc: str = field(default="", compare=False)

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


def _largest_remainder(weights: np.ndarray, total: int) -> np.ndarray:
    raw = weights * total
    base = np.floor(raw).astype(np.int64)
    rem = total - int(base.sum())
    frac = raw - base
    order = np.lexsort((np.arange(len(weights)), -frac))   # largest fraction first, then index
    base[order[:rem]] += 1
    return base


def varlen_doc_lengths(seed: int, total: int = 32768, n_docs: int = 8, min_len: int = 512):
    """Document lengths for the packed (TND) workload: a seeded Dirichlet(1) split of the
    tokens above the per-document minimum, rounded by largest remainder so they sum to total."""
    rng = np.random.default_rng(seed)
    p = rng.dirichlet(np.ones(n_docs))
    return [int(min_len + x) for x in _largest_remainder(p, total - n_docs * min_len)]


def head_tail_segments(seq: int, cp: int, rank: int):
    """Head-tail load-balanced CP share: the sequence is cut into 2*cp chunks and rank r holds
    chunks r and 2*cp-1-r, both attending the full gathered keys [0, seq)."""
    c = seq // (2 * cp)
    return ((0, c, 0, seq, rank * c), (c, c, 0, seq, (2 * cp - 1 - rank) * c))


def _workloads():
    w = {}
    w[1] = Workload(
        name="tiny-S256", n_q=256, n_k=256, h_idx=4, d_idx=32, h=8, d_qk=80, d_v=64, topk=64,
        segments=((0, 256, 0, 256, 0),), w_scale=1.0 / math.sqrt(4),
        softmax_scale=1.0 / math.sqrt(80), seed=1001,
        doc="Tiny DSA forward, S=256 causal, 4x32 indexer, topk 64, 8 heads x 80-d latent")
    w[2] = Workload(
        name="v32-S4096", n_q=4096, n_k=4096, h_idx=64, d_idx=128, h=128, d_qk=576, d_v=512,
        topk=2048, segments=((0, 4096, 0, 4096, 0),), w_scale=1.0 / 8, kv_std=0.5,
        softmax_scale=1.0 / math.sqrt(576), seed=1002,
        doc="DeepSeek-V3.2-shaped single-rank forward, S=4096 causal")
    w[3] = Workload(
        name="cp2-rank1-32K", n_q=16384, n_k=32768, h_idx=64, d_idx=128, h=128, d_qk=576,
        d_v=512, topk=2048, segments=((0, 16384, 0, 32768, 16384),), w_scale=1.0 / 8,
        softmax_scale=1.0 / math.sqrt(576), seed=1003,
        doc="32K sequence, CP degree 2, second rank: 16384 local queries at positions "
            "16384..32767 against the full 32768-token keys")
    w[4] = Workload(
        name="cp8-headtail-rank0-32K", n_q=4096, n_k=32768, h_idx=64, d_idx=128, h=128,
        d_qk=576, d_v=512, topk=2048, segments=head_tail_segments(32768, 8, 0),
        w_scale=1.0 / 8, softmax_scale=1.0 / math.sqrt(576), seed=1004,
        doc="32K sequence, CP degree 8 head-tail, rank 0: positions 0..2047 and 30720..32767")
    lens = varlen_doc_lengths(1005)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(int)
    w[5] = Workload(
        name="varlen-T32768-8docs", n_q=32768, n_k=32768, h_idx=64, d_idx=128, h=128,
        d_qk=576, d_v=512, topk=2048,
        segments=tuple((int(cu[g]), lens[g], int(cu[g]), lens[g], 0) for g in range(8)),
        w_scale=1.0 / 8, softmax_scale=1.0 / math.sqrt(576), with_dout=True, seed=1005,
        doc="Packed varlen TND, 8 documents (Dirichlet(1) lengths, min 512), per-document "
            "causal, forward + sparse-attention backward")
    return w


WORKLOADS = _workloads()


def workload(n: int) -> Workload:
    return WORKLOADS[n]


def _bf16(x: torch.Tensor) -> torch.Tensor:
    return x.to(torch.bfloat16)


def generate(wl: Workload, seed: int | None = None, device="cpu", gen_device="cpu"):
    """Draw the inputs of ``wl``.  Returns a dict of tensors on ``device``:

    q_idx bf16 [n_q, h_idx, d_idx], k_idx bf16 [n_k, d_idx], w_idx fp32 [n_q, h_idx],
    q bf16 [n_q, h, d_qk], kv bf16 [n_k, d_qk] and, when the workload has a backward,
    dout bf16 [n_q, h, d_v].  With gen_device='cuda' the numbers come from the device
    generator instead (same distributions, different stream; used only for timing runs)."""
    g = torch.Generator(device=gen_device)
    g.manual_seed(wl.seed if seed is None else seed)
    kw = dict(generator=g, device=gen_device, dtype=torch.float32)
    out = {}
    out["q_idx"] = _bf16(torch.randn(wl.n_q, wl.h_idx, wl.d_idx, **kw))
    out["k_idx"] = _bf16(torch.randn(wl.n_k, wl.d_idx, **kw))
    out["w_idx"] = _bf16(torch.rand(wl.n_q, wl.h_idx, **kw) * wl.w_scale).float()
    # large tensors are drawn in chunks to bound the float32 staging memory
    q = torch.empty(wl.n_q, wl.h, wl.d_qk, dtype=torch.bfloat16, device=gen_device)
    step = max(1, (1 << 26) // (wl.h * wl.d_qk))
    for r in range(0, wl.n_q, step):
        n = min(step, wl.n_q - r)
        q[r:r + n] = _bf16(torch.randn(n, wl.h, wl.d_qk, **kw))
    out["q"] = q
    out["kv"] = _bf16(torch.randn(wl.n_k, wl.d_qk, **kw) * wl.kv_std)
    if wl.with_dout:
        d = torch.empty(wl.n_q, wl.h, wl.d_v, dtype=torch.bfloat16, device=gen_device)
        step = max(1, (1 << 26) // (wl.h * wl.d_v))
        for r in range(0, wl.n_q, step):
            n = min(step, wl.n_q - r)
            d[r:r + n] = _bf16(torch.randn(n, wl.h, wl.d_v, **kw))
        out["dout"] = d
    if str(device) != str(gen_device):
        out = {k: v.to(device) for k, v in out.items()}
    return out


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact float64 copy of a bf16 / fp32 tensor, for the oracle."""
    return t.detach().to("cpu").double().numpy()


# ---- dense causal attention of an Ulysses head shard ---------------------------------------
# DeepSeek-V3's attention (the dense model the CP pages run under Ulysses) in its training
# form: 128 heads, q/k heads 192 wide (128 + 64 rope), v heads 128 wide.  One rank of an
# 8-way Ulysses group holds all 32K positions of 16 heads.  Q, K and V are N(0, 1) in bf16,
# drawn in that order on a CPU generator seeded with 2000 + workload number.


@dataclass(frozen=True)
class DenseWorkload:
    name: str
    n: int                   # query rows = key rows (the packed sequence)
    h: int                   # heads of the shard
    segments: tuple
    d_qk: int = 192
    d_v: int = 128
    seed: int = 2000

    @property
    def softmax_scale(self) -> float:
        return 1.0 / math.sqrt(self.d_qk)


DENSE_WORKLOADS = {
    0: DenseWorkload("ulysses-tiny-S300-h3", 300, 3, ((0, 300, 0, 300, 0),), seed=2000),
    1: DenseWorkload("ulysses-cp8-rank-32K-h16", 32768, 16, ((0, 32768, 0, 32768, 0),),
                     seed=2001),
}


def dense_workload(n: int) -> DenseWorkload:
    return DENSE_WORKLOADS[n]


def generate_dense(wl: DenseWorkload, seed: int | None = None, device="cpu", gen_device="cpu"):
    """q [n, h, d_qk], k [n, h, d_qk], v [n, h, d_v], bf16 N(0, 1), on ``device``."""
    g = torch.Generator(device=gen_device)
    g.manual_seed(wl.seed if seed is None else seed)
    kw = dict(generator=g, device=gen_device, dtype=torch.float32)
    out = {}
    for name, width in (("q", wl.d_qk), ("k", wl.d_qk), ("v", wl.d_v)):
        t = torch.empty(wl.n, wl.h, width, dtype=torch.bfloat16, device=gen_device)
        step = max(1, (1 << 26) // (wl.h * width))
        for r in range(0, wl.n, step):
            m = min(step, wl.n - r)
            t[r:r + m] = _bf16(torch.randn(m, wl.h, width, **kw))
        out[name] = t
    if str(device) != str(gen_device):
        out = {k: v.to(device) for k, v in out.items()}
    return out
