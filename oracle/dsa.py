"""Plain float64 oracle for the DSA forward (with the sparse-attention backward and the indexer
KL loss) on one CP rank, and for the dense causal attention of an Ulysses head shard.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the bench's CPU-baseline
leg, never by the product path.  Nothing here is blocked, fused or reordered beyond what the
definitions state; a NumPy matmul or sort serves as a single step where the definition is a
matrix product or an ordering.

Sources (four web pages on DeepSeek Sparse Attention and its context parallelism):

* Page "CANNTorchTitan: DeepSeek-V3.2 32k长序列预训练昇腾优化实践", section
  "SparseLightningIndexerGradKLLoss": the Lightning Indexer top-k value formula (per-token
  weights times ReLU of the merged index-head query against the index keys) and the Sparse
  Flash Attention formula (softmax of q K_topk^T / sqrt(d)); section "SparseFlashAttentionGrad":
  the backward (Gather, recomputed P, dP = dY V^T, dS = P * (dP - FlashSoftmaxGrad(dY, out)),
  dQ = dS K_topk / sqrt(d), dK = ScatterAdd(dS^T Q / sqrt(d)), dV = P^T dY); section
  "自定义CP策略": a CP rank's local queries must see the full all-gathered keys and values;
  section "SparseLightningIndexerGradKLLoss" also gives the indexer loss (KL divergence of the
  indexer's softmax from the head-summed, L1-normalised attention probabilities) and its
  gradients with respect to the index weights, queries and keys.
* Page "CANN/torchtitan-npu融合算子适配", section "DSA": the indexer selects a small set of
  high-value token indices that the sparse multi-query attention then consumes.
* Page "context_parallel.md" (HyperParallel CP guide), section "DSA CP": the indexer boundary
  (query, key, weights), the sparse-attention boundary (query, key, value, topk_indices,
  query_rope, key_rope) with query-side tensors sharded along the sequence and key-side tensors
  replicated, the indexer-loss boundary that consumes softmax_max / softmax_sum, and the BSND /
  TND layouts; section "基础用法" / load_balance: with head-tail balance the mask is built from
  K's (global) length; section "适用边界": position ids and masks align with the global window;
  section "ContextParallel 模式": the Pure Ulysses / Hybrid placements of the dense attention.
* Page "自定义Context Parallel特性", section "SDPA Ulysses CP": the dense model's attention runs
  as an ordinary SDPA on a head shard that holds the whole sequence.

Readings where the pages are silent (each also listed in the design notes):

* causal window of a local row: inclusive diagonal, keys ``k_start .. k_start + pos0 + r``;
* rows whose window is shorter than top-k select the whole window and pad with -1;
* ties in the indexer score go to the lower key index; -0.0 equals +0.0;
* selected indices are emitted in ascending key order, absolute rows of the key tensor;
* the value is the first ``d_v`` columns of the shared latent row, the rope part the rest;
* ``softmax_max`` is the maximum scaled logit, ``softmax_sum`` the sum of exp(z - max);
* FlashSoftmaxGrad(dY, out) is the row sum of dY * out;
* fp8 indexer inputs: OCP e4m3fn with one fp32 scale per token row, scale = amax / 448;
* indexer loss: the sum over tokens of each token's KL term over its selected slots (a
  repeated key is one entry per slot), the target recomputed from the selected rows; ReLU
  passes no gradient at exactly 0; the incoming loss gradient scales dI.
"""

from __future__ import annotations

import numpy as np

# ----------------------------------------------------------------------------------------
# number formats
# ----------------------------------------------------------------------------------------


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Decode bfloat16 bit patterns (uint16 / int16) exactly into float64.

    A bfloat16 is the upper half of an IEEE binary32, so the decode is a 16-bit shift."""
    b = np.asarray(bits).astype(np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


E4M3_MAX = 448.0  # largest finite OCP e4m3fn value: exponent field 15, mantissa 6 -> 1.75 * 2^8


def e4m3fn_decode(codes) -> np.ndarray:
    """Decode OCP 8-bit float E4M3 ("fn": finite, no infinity) codes to float64.

    Layout: 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits.  Exponent field 0 holds
    subnormals m * 2^-9; code S.1111.111 is NaN; everything else is (1 + m/8) * 2^(e-7)."""
    c = np.asarray(codes).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & ((c & 7) == 7), np.nan, mag)
    return sign * mag


def e4m3fn_encode(x) -> np.ndarray:
    """Round values to OCP e4m3fn codes: round-to-nearest-even, saturating at +-448.

    Written from the format definition: find the binade of |x|, the spacing of representable
    values there (2^(E-3) for normal binades E >= -6, 2^-9 below), round |x| / spacing to the
    nearest integer with ties to even, then clamp to the largest finite value."""
    v = np.asarray(x, dtype=np.float64)
    a = np.abs(v)
    neg = np.signbit(v)
    out = np.zeros(a.shape, dtype=np.uint8)
    nan = np.isnan(a)
    fin = ~nan
    _, ex = np.frexp(np.where(fin & (a > 0), a, 1.0))  # a = f * 2^ex, f in [0.5, 1)
    binade = ex - 1                                      # floor(log2 a)
    spacing = np.exp2(np.where(binade < -6, -9, binade - 3).astype(np.float64))
    r = np.rint(np.where(fin, a, 0.0) / spacing) * spacing  # np.rint rounds half to even
    r = np.minimum(r, E4M3_MAX)
    # encode the rounded magnitude
    is_sub = r < 2.0 ** -6
    msub = np.rint(r * 2.0 ** 9).astype(np.int64)
    _, ex2 = np.frexp(np.where(is_sub, 1.0, r))
    E = ex2 - 1
    mnorm = np.rint((r / np.exp2(E.astype(np.float64)) - 1.0) * 8.0).astype(np.int64)
    code = np.where(is_sub, msub, ((E + 7) << 3) | mnorm)
    out = np.where(nan, 0x7F, code).astype(np.uint8)
    out = out | np.where(neg & ~nan, 0x80, 0).astype(np.uint8)
    return out


def quantize_fp8_rows(x) -> tuple[np.ndarray, np.ndarray]:
    """Per-row (per-token) e4m3fn quantization of a 2-D array of float32-exact values.

    scale = amax(|row|) / 448 (1.0 for an all-zero row), y = x / scale, code = e4m3fn(y).
    Both the scale and y are computed in IEEE float32 with correctly rounded division, the
    precision the kernel takes the decision in; the code is then the RNE e4m3fn of that y.
    Returns (codes uint8 [rows, cols], scales float32 [rows])."""
    x32 = np.asarray(x, dtype=np.float32)
    assert x32.ndim == 2
    amax = np.max(np.abs(x32), axis=1)
    scale = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    y = (x32 / scale[:, None]).astype(np.float32)
    return e4m3fn_encode(y), scale


# ----------------------------------------------------------------------------------------
# windows of a CP rank's local rows
# ----------------------------------------------------------------------------------------


def row_windows(segments, n_q: int, n_k: int):
    """Causal key window of every local query row.

    ``segments`` is a list of (q_start, q_len, k_start, k_len, pos0).  Local row
    i = q_start + r sits at global position p = pos0 + r of its sequence (the CP guide: local
    slices keep positions aligned with the global window; with head-tail balance the global
    length comes from K), and attends keys k_start .. k_start + p inclusive, so its window
    length is p + 1.  Returns (k_lo, L) int64 arrays of length n_q; rows covered by no segment
    get k_lo = L = -1."""
    k_lo = np.full(n_q, -1, dtype=np.int64)
    L = np.full(n_q, -1, dtype=np.int64)
    for (q_start, q_len, k_start, k_len, pos0) in segments:
        if q_len < 0 or k_len < 0 or pos0 < 0:
            raise ValueError("negative segment field")
        if q_start < 0 or q_start + q_len > n_q or k_start < 0 or k_start + k_len > n_k:
            raise ValueError("segment out of range")
        if q_len > 0 and pos0 + q_len > k_len:
            raise ValueError("query position beyond the segment's key length")
        rows = np.arange(q_start, q_start + q_len)
        if np.any(L[rows] >= 0):
            raise ValueError("segments overlap")
        k_lo[rows] = k_start
        L[rows] = pos0 + (rows - q_start) + 1
    return k_lo, L


# ----------------------------------------------------------------------------------------
# Lightning Indexer scores
# ----------------------------------------------------------------------------------------


def indexer_scores_row(q_i, k_win, w_i) -> np.ndarray:
    """Indexer score of one query token against the keys of its window.

    I[s] = sum_j w[j] * ReLU(q[j, :] . k[s, :]) -- the Lightning Indexer top-k value formula
    (page "CANNTorchTitan: ...", section "SparseLightningIndexerGradKLLoss"): the token's index
    heads are merged, each head's dot product with the shared index key goes through ReLU, and
    the per-token weights combine the heads.  No extra scale factor is applied inside.
    q_i [H_idx, d_idx], k_win [L, d_idx], w_i [H_idx] -> [L] float64."""
    q_i = np.asarray(q_i, dtype=np.float64)
    k_win = np.asarray(k_win, dtype=np.float64)
    w_i = np.asarray(w_i, dtype=np.float64)
    dots = k_win @ q_i.T                 # [L, H_idx]: every head against every key
    return np.maximum(dots, 0.0) @ w_i   # ReLU per (head, key), then weighted head sum


def indexer_scores(q_idx, k_idx, w_idx, segments, rows=None, q_scale=None, k_scale=None):
    """Dense indexer scores [len(rows), n_k] in float64, -inf outside each row's window.

    q_idx [n_q, H_idx, d_idx], k_idx [n_k, d_idx], w_idx [n_q, H_idx] are the real values the
    inputs represent (bf16 decoded, or fp8 codes decoded).  With fp8 inputs, ``q_scale`` [n_q]
    and ``k_scale`` [n_k] are the per-token dequantization scales: the represented query is
    q_scale[i] * q8[i] and the represented key k_scale[s] * k8[s]."""
    q_idx = np.asarray(q_idx, dtype=np.float64)
    k_idx = np.asarray(k_idx, dtype=np.float64)
    n_q, n_k = q_idx.shape[0], k_idx.shape[0]
    k_lo, L = row_windows(segments, n_q, n_k)
    rows = np.arange(n_q) if rows is None else np.asarray(rows)
    out = np.full((len(rows), n_k), -np.inf)
    for o, i in enumerate(rows):
        if L[i] < 0:
            continue
        qi = q_idx[i] if q_scale is None else q_idx[i] * float(q_scale[i])
        kw = k_idx[k_lo[i]:k_lo[i] + L[i]]
        if k_scale is not None:
            kw = kw * np.asarray(k_scale, dtype=np.float64)[k_lo[i]:k_lo[i] + L[i], None]
        out[o, k_lo[i]:k_lo[i] + L[i]] = indexer_scores_row(qi, kw, w_idx[i])
    return out


# ----------------------------------------------------------------------------------------
# top-k selection
# ----------------------------------------------------------------------------------------


def topk_row(scores_win, k_lo: int, topk: int) -> np.ndarray:
    """Top-k key indices of one row from the scores of its window.

    n = min(topk, L) keys with the largest score; equal scores go to the lower key index and
    -0.0 counts as +0.0.  The chosen indices are returned in ascending key order as absolute
    rows (k_lo + window offset), padded with -1 to length topk."""
    s = np.asarray(scores_win, dtype=np.float64)
    if not np.all(np.isfinite(s)):
        raise ValueError("non-finite score inside a window")
    L = s.shape[0]
    n = min(topk, L)
    pos = np.arange(L)
    order = np.lexsort((pos, -s))        # primary key: score descending; then index ascending
    chosen = np.sort(order[:n]) + k_lo
    out = np.full(topk, -1, dtype=np.int64)
    out[:n] = chosen
    return out


def topk_select(scores, segments, topk: int, n_q: int | None = None, rows=None) -> np.ndarray:
    """Per-row top-k over dense scores [n_rows, n_k] (windows from ``segments``).

    Without ``rows`` the score rows are all n_q local rows.  With ``rows`` (local row numbers,
    ``n_q`` then required) score row o belongs to local row rows[o]."""
    scores = np.asarray(scores)
    if rows is None:
        rows_arr = np.arange(scores.shape[0])
        n_q = scores.shape[0]
    else:
        rows_arr = np.asarray(rows)
        if n_q is None:
            raise ValueError("n_q is required with rows")
    k_lo, L = row_windows(segments, n_q, scores.shape[1])
    out = np.full((len(rows_arr), topk), -1, dtype=np.int64)
    for o, i in enumerate(rows_arr):
        if L[i] < 0:
            continue
        out[o] = topk_row(scores[o, k_lo[i]:k_lo[i] + L[i]], k_lo[i], topk)
    return out


# ----------------------------------------------------------------------------------------
# sparse multi-query attention over the shared latent rows
# ----------------------------------------------------------------------------------------


def attention_row(q_i, kv, idx_i, scale: float, d_v: int):
    """Sparse MQA of one query token over its selected latent rows.

    K_topk = kv[idx] (the Gather of the selected rows); per head h,
    z = scale * q[h] . K_topk^T, p = softmax(z), out[h] = p . V_topk with V the first d_v
    columns of the same latent rows (page "CANNTorchTitan: ...", Sparse Flash Attention
    formula; weight absorption makes key and value one shared latent row).  Also returns
    softmax_max = max z and softmax_sum = sum exp(z - max) per head, the statistics the
    indexer-loss boundary consumes.  Slots holding -1 are empty.  With no valid slot the
    output is 0, max -inf and sum 0."""
    q_i = np.asarray(q_i, dtype=np.float64)
    idx_i = np.asarray(idx_i)
    sel = idx_i[idx_i >= 0]
    H = q_i.shape[0]
    if sel.size == 0:
        return np.zeros((H, d_v)), np.full(H, -np.inf), np.zeros(H)
    K = np.asarray(kv, dtype=np.float64)[sel]          # [n, D]
    z = scale * (q_i @ K.T)                            # [H, n]
    m = z.max(axis=1)
    e = np.exp(z - m[:, None])
    l = e.sum(axis=1)
    out = (e @ K[:, :d_v]) / l[:, None]
    return out, m, l


def sparse_attn(q, kv, idx, scale: float, d_v: int, rows=None):
    """Row loop of ``attention_row`` over q [n_q, H, D] and idx [n_q, topk].

    With ``rows``, only those local rows are computed; idx still has one row per local row.
    Returns (out [n, H, d_v], softmax_max [n, H], softmax_sum [n, H]) for the computed rows."""
    q = np.asarray(q)
    rows_arr = np.arange(q.shape[0]) if rows is None else np.asarray(rows)
    H = q.shape[1]
    out = np.zeros((len(rows_arr), H, d_v))
    mx = np.zeros((len(rows_arr), H))
    sm = np.zeros((len(rows_arr), H))
    for o, i in enumerate(rows_arr):
        out[o], mx[o], sm[o] = attention_row(q[i], kv, idx[i], scale, d_v)
    return out, mx, sm


# ----------------------------------------------------------------------------------------
# the DSA forward on a CP rank's share: indexer -> top-k -> sparse attention
# ----------------------------------------------------------------------------------------


def dsa_forward(q_idx, k_idx, w_idx, q, kv, segments, topk: int, scale: float, d_v: int,
                rows=None, q_scale=None, k_scale=None):
    """The composed forward for the requested local rows.

    The local query rows (and their index queries and weights) are this rank's sequence shard;
    k_idx and kv are the full, already all-gathered sequence, as the CP strategy of page
    "CANNTorchTitan: ..." (section "自定义CP策略") and the DSA CP styles of the HyperParallel
    guide require.  Returns a dict with, per requested row: 'scores' (dense, -inf outside the
    window), 'idx' (top-k, ascending, -1 padded), 'out', 'softmax_max', 'softmax_sum'."""
    n_q = np.asarray(q_idx).shape[0]
    rows_arr = np.arange(n_q) if rows is None else np.asarray(rows)
    scores = indexer_scores(q_idx, k_idx, w_idx, segments, rows=rows_arr,
                            q_scale=q_scale, k_scale=k_scale)
    k_lo, L = row_windows(segments, n_q, np.asarray(k_idx).shape[0])
    idx = np.full((len(rows_arr), topk), -1, dtype=np.int64)
    for o, i in enumerate(rows_arr):
        if L[i] >= 0:
            idx[o] = topk_row(scores[o, k_lo[i]:k_lo[i] + L[i]], k_lo[i], topk)
    q = np.asarray(q)
    H = q.shape[1]
    out = np.zeros((len(rows_arr), H, d_v))
    mx = np.zeros((len(rows_arr), H))
    sm = np.zeros((len(rows_arr), H))
    for o, i in enumerate(rows_arr):
        out[o], mx[o], sm[o] = attention_row(q[i], kv, idx[o], scale, d_v)
    return {"scores": scores, "idx": idx, "out": out, "softmax_max": mx, "softmax_sum": sm,
            "rows": rows_arr}


# ----------------------------------------------------------------------------------------
# sparse attention backward
# ----------------------------------------------------------------------------------------


def attention_bwd_row(q_i, kv, idx_i, dout_i, scale: float, d_v: int):
    """Gradients of one query token's sparse attention (page "CANNTorchTitan: ...", section
    "SparseFlashAttentionGrad").

    K_topk = Gather(kv, idx); P = softmax(scale * q K_topk^T) recomputed; out = P V_topk;
    D = rowsum(dY * out) (FlashSoftmaxGrad of the output gradient and the forward output);
    dP = dY V_topk^T; dS = P * (dP - D); dQ = scale * dS K_topk;
    dK rows = scale * dS^T q (scatter-added into the selected rows);
    dV rows = P^T dY, added into the first d_v columns of the same latent rows.
    Returns (dq_i [H, D], sel [n], dkv_rows [n, D])."""
    q_i = np.asarray(q_i, dtype=np.float64)
    dout_i = np.asarray(dout_i, dtype=np.float64)
    idx_i = np.asarray(idx_i)
    sel = idx_i[idx_i >= 0]
    H, D = q_i.shape
    if sel.size == 0:
        return np.zeros((H, D)), sel, np.zeros((0, D))
    K = np.asarray(kv, dtype=np.float64)[sel]
    V = K[:, :d_v]
    z = scale * (q_i @ K.T)
    m = z.max(axis=1)
    e = np.exp(z - m[:, None])
    P = e / e.sum(axis=1)[:, None]
    out = P @ V
    Dsum = np.sum(dout_i * out, axis=1)
    dP = dout_i @ V.T
    dS = P * (dP - Dsum[:, None])
    dq = scale * (dS @ K)
    dkv_rows = scale * (dS.T @ q_i)
    dkv_rows[:, :d_v] += P.T @ dout_i
    return dq, sel, dkv_rows


def sparse_attn_bwd(q, kv, idx, dout, scale: float, d_v: int):
    """Full backward: dq [n_q, H, D] and dkv [n_k, D] (scatter-add over every row's selection)."""
    q = np.asarray(q)
    kv = np.asarray(kv, dtype=np.float64)
    dq = np.zeros(q.shape)
    dkv = np.zeros(kv.shape)
    for i in range(q.shape[0]):
        dq[i], sel, rows = attention_bwd_row(q[i], kv, idx[i], dout[i], scale, d_v)
        np.add.at(dkv, sel, rows)
    return dq, dkv


# ----------------------------------------------------------------------------------------
# indexer KL loss and its gradients
# ----------------------------------------------------------------------------------------


def indexer_kl_row(q_idx_i, k_idx, w_i, q_i, kv, idx_i, scale: float, loss_grad: float = 1.0):
    """KL loss of one query token's indexer distribution and its gradients (page
    "CANNTorchTitan: ...", section "SparseLightningIndexerGradKLLoss", the loss and gradient
    formulas after the two top-k value formulas).

    Over the token's selected keys (slots holding -1 are empty; a repeated key is one entry
    per slot):
      target   P[h, s] = softmax_s(scale * q[h] . kv[sel[s]]), the Sparse Flash Attention
               probabilities; p = sum_h P[h, :], then divided by its L1 norm over the slots;
      indexer  S = q_idx K_sel^T [h_idx, n] with K_sel = k_idx[sel] (S is the product of the
               index queries and keys); I = sum_j w[j] ReLU(S[j, :]);
      loss     = D_KL(p || softmax(I)) = sum_s p_s log(p_s / softmax(I)_s) (0 log 0 = 0);
      dI       = loss_grad * (softmax(I) - p);
      dW       = ReLU(S) dI  (for each index head j: sum_s dI_s ReLU(S[j, s]));
      dS       = w[j] dI_s where S[j, s] > 0, else 0 (ReLU passes no gradient at 0);
      dq_idx   = dS K_sel;   dK rows = dS^T q_idx (added into k_idx's selected rows).
    The target carries no gradient.  loss_grad is the gradient arriving at this token's loss
    term (1 for the plain sum over tokens).
    Returns (loss, dq_idx_i [h_idx, d_idx], dw_i [h_idx], sel [n], dk_rows [n, d_idx])."""
    q_idx_i = np.asarray(q_idx_i, dtype=np.float64)
    w_i = np.asarray(w_i, dtype=np.float64)
    idx_i = np.asarray(idx_i)
    sel = idx_i[idx_i >= 0]
    G, d = q_idx_i.shape
    if sel.size == 0:
        return 0.0, np.zeros((G, d)), np.zeros(G), sel, np.zeros((0, d))
    # target distribution from the attention probabilities
    K = np.asarray(kv, dtype=np.float64)[sel]
    z = scale * (np.asarray(q_i, dtype=np.float64) @ K.T)      # [H, n]
    e = np.exp(z - z.max(axis=1)[:, None])
    P = e / e.sum(axis=1)[:, None]
    p = P.sum(axis=0)
    p = p / np.abs(p).sum()
    # indexer distribution
    Ki = np.asarray(k_idx, dtype=np.float64)[sel]              # [n, d]
    S = q_idx_i @ Ki.T                                         # [G, n]
    R = np.maximum(S, 0.0)
    I = w_i @ R
    lse = I.max() + np.log(np.sum(np.exp(I - I.max())))
    logr = I - lse
    r = np.exp(logr)
    pos = p > 0
    loss = float(np.sum(p[pos] * (np.log(p[pos]) - logr[pos])))
    # gradients
    dI = loss_grad * (r - p)
    dw = R @ dI
    dS = np.where(S > 0, w_i[:, None] * dI[None, :], 0.0)
    dq = dS @ Ki
    dk_rows = dS.T @ q_idx_i
    return loss, dq, dw, sel, dk_rows


def indexer_kl_loss_grad(q_idx, k_idx, w_idx, q, kv, idx, scale: float, loss_grad: float = 1.0):
    """Row loop of ``indexer_kl_row``: per-token losses [n_q] (their sum is the loss of the
    page's formula), dq_idx [n_q, h_idx, d_idx], dw [n_q, h_idx] and dk_idx [n_k, d_idx] (the
    scatter-add of every row's key-row gradients)."""
    q_idx = np.asarray(q_idx)
    n_q, G, d = q_idx.shape
    dk = np.zeros((np.asarray(k_idx).shape[0], d))
    losses = np.zeros(n_q)
    dq = np.zeros((n_q, G, d))
    dw = np.zeros((n_q, G))
    k64 = np.asarray(k_idx, dtype=np.float64)
    kv64 = np.asarray(kv, dtype=np.float64)
    for i in range(n_q):
        losses[i], dq[i], dw[i], sel, rows = indexer_kl_row(q_idx[i], k64, w_idx[i], q[i], kv64,
                                                            idx[i], scale, loss_grad)
        np.add.at(dk, sel, rows)
    return losses, dq, dw, dk


# ----------------------------------------------------------------------------------------
# dense causal attention on an Ulysses head shard
# ----------------------------------------------------------------------------------------


def dense_attn_row(q_i, k_win, v_win, scale: float):
    """Causal softmax attention of one query token over the keys of its window, head by head.

    Page "自定义Context Parallel特性", section "SDPA Ulysses CP": an all-to-all turns the
    sequence-sharded Q/K/V into head-sharded ones, so one device holds the whole context of
    its heads and runs the ordinary SDPA on them; per head h,
    z = scale * q[h] . K[:, h]^T over the window, p = softmax(z), out[h] = p . V[:, h].  Also
    returns lse = log sum exp z (natural log, scaled logits), the statistic a backward uses.
    q_i [H, D], k_win [L, H, D], v_win [L, H, D_v]; L >= 1."""
    q_i = np.asarray(q_i, dtype=np.float64)
    k_win = np.asarray(k_win, dtype=np.float64)
    v_win = np.asarray(v_win, dtype=np.float64)
    z = scale * np.einsum("hd,lhd->hl", q_i, k_win)     # [H, L]
    m = z.max(axis=1)
    e = np.exp(z - m[:, None])
    l = e.sum(axis=1)
    out = np.einsum("hl,lhd->hd", e, v_win) / l[:, None]
    return out, m + np.log(l)


def dense_attn(q, k, v, segments, scale: float, rows=None):
    """``dense_attn_row`` over the local rows: q [n_q, H, D], k [n_k, H, D], v [n_k, H, D_v].

    Row i of a segment attends keys k_start .. k_start + pos0 + r of k and v (``row_windows``):
    one segment with pos0 = 0 is plain causal attention over a sequence (pure Ulysses: page
    "context_parallel.md", section "ContextParallel 模式", Q/K/V moved from a sequence shard to a
    head shard); a segment with pos0 > 0 is a sequence shard of the queries against the whole
    gathered K/V (the Hybrid mode, which also gathers K/V over the Colossal group); packed
    documents are one segment each.  Returns (out [n, H, D_v], lse [n, H]) for the computed
    rows; rows covered by no segment give out 0 and lse -inf."""
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    n_q, H = q.shape[0], q.shape[1]
    k_lo, L = row_windows(segments, n_q, k.shape[0])
    rows_arr = np.arange(n_q) if rows is None else np.asarray(rows)
    out = np.zeros((len(rows_arr), H, v.shape[2]))
    lse = np.full((len(rows_arr), H), -np.inf)
    for o, i in enumerate(rows_arr):
        if L[i] < 0:
            continue
        lo, hi = k_lo[i], k_lo[i] + L[i]
        out[o], lse[o] = dense_attn_row(q[i], k[lo:hi], v[lo:hi], scale)
    return out, lse
