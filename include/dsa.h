/*
 * dsa.h -- C ABI of libdsa: the DeepSeek Sparse Attention (DSA) forward on one
 * context-parallel (CP) rank's share, for AMD Instinct MI355X (gfx950).
 *
 * The share is a slice of local query rows scored by the Lightning Indexer, reduced to each
 * row's causal top-k keys, and attended with multi-query attention over the selected rows of
 * the FULL, already all-gathered key / latent-KV sequence.  Sources:
 *   - page "CANNTorchTitan: DeepSeek-V3.2 32k长序列预训练昇腾优化实践", section
 *     "SparseLightningIndexerGradKLLoss" (Lightning Indexer and Sparse Flash Attention
 *     formulas), section "SparseFlashAttentionGrad" (backward), section "自定义CP策略"
 *     (CP = local queries against all-gathered keys/values);
 *   - page "context_parallel.md" (HyperParallel CP guide), section "DSA CP" (the indexer,
 *     sparse-attention and indexer-loss boundaries and their query/key placements, BSND/TND
 *     layouts), and the load_balance note (head-tail shares, masks from K's global length);
 *   - page "CANN/torchtitan-npu融合算子适配", section "DSA" (indexer selects the indices the
 *     sparse multi-query attention consumes).
 *
 * Conventions for every entry point:
 *   - Tensor pointers are DEVICE memory owned by the caller; the library never allocates or
 *     frees device memory.  Scratch space for dsa_forward comes from the caller's workspace,
 *     sized by dsa_workspace_bytes.  The dsa_shape struct and its segment array are HOST
 *     memory, read before the call returns.
 *   - Tensors are dense row-major.  bf16 values are raw IEEE bfloat16 bit patterns.
 *   - Key indices are absolute rows of k_idx / kv; -1 marks an empty top-k slot.
 *   - Arguments are validated synchronously: DSA_ERR_INVALID_ARG / DSA_ERR_UNSUPPORTED /
 *     DSA_ERR_WORKSPACE return without launching anything.  Otherwise the work is enqueued on
 *     `stream` (a hipStream_t; NULL means the default stream) and DSA_OK is returned with no
 *     host synchronisation.  A failed launch returns DSA_ERR_HIP.  Device-side faults surface
 *     at the caller's next synchronisation.  dsa_last_error() describes the last non-OK status
 *     of the calling thread.  No C++ exception crosses this interface.
 *   - Alignment: the kernels read and write rows in 16-byte pieces, so q_idx, k_idx, q, kv,
 *     out, dout, dq, dkv and workspaces must be 16-byte aligned; index lists, scores, weights,
 *     scales and softmax statistics 4-byte aligned (bf16 quantizer input 2-byte).  A
 *     misaligned pointer is DSA_ERR_INVALID_ARG, naming the argument.
 *   - Supported dimensions (anything else is DSA_ERR_UNSUPPORTED):
 *       indexer (h_idx, d_idx) in {(4, 32), (64, 128)};
 *       attention (h, d_qk, d_v) in {(8, 80, 64), (128, 576, 512)};
 *       1 <= topk <= 4096; every window length <= 65536 keys; the latent KV (n_k * d_qk
 *       bf16 values) at most 4 GiB.
 */
#ifndef DSA_H
#define DSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DSA_ABI_VERSION 1

typedef enum {
  DSA_OK = 0,
  DSA_ERR_INVALID_ARG = 1, /* null pointer, negative size, bad segment table        */
  DSA_ERR_UNSUPPORTED = 2, /* dimensions or options this build has no kernel for    */
  DSA_ERR_WORKSPACE = 3,   /* workspace missing or smaller than dsa_workspace_bytes  */
  DSA_ERR_HIP = 4          /* a HIP runtime call or kernel launch failed             */
} dsa_status;

/* Element type of the index query / index key tensors. */
typedef enum {
  DSA_IDX_BF16 = 0,    /* q_idx, k_idx are bf16; q_scale, k_scale must be NULL          */
  DSA_IDX_FP8_E4M3 = 1 /* q_idx, k_idx are OCP e4m3fn codes (uint8) with one fp32 scale
                          per token row: represented value = code value * row scale    */
} dsa_idx_dtype;

/*
 * One run of local query rows sharing a key sequence (the CP guide's DSA CP placements:
 * query side sharded along the sequence, key side replicated).  Local rows
 * [q_start, q_start + q_len) sit at global positions pos0 .. pos0 + q_len - 1 of a sequence
 * whose keys are rows [k_start, k_start + k_len) of k_idx / kv.  Row q_start + r attends
 * keys k_start .. k_start + pos0 + r inclusive (causal, diagonal included), so its window
 * holds pos0 + r + 1 keys; pos0 + q_len <= k_len is required.
 *   - an unsharded causal sequence is one segment with pos0 = 0;
 *   - a CP rank's contiguous share of a gathered sequence sets pos0 to its offset;
 *   - a head-tail balanced share is two segments (two chunks, each with its own pos0);
 *   - BSND with B sequences / packed TND documents are one segment per sequence.
 * Segments must not overlap in query rows.  Rows covered by no segment are left untouched
 * by the indexer, top-k and fused forward.
 */
typedef struct {
  int32_t q_start, q_len, k_start, k_len, pos0;
} dsa_segment;

typedef struct {
  int32_t n_q, n_k;       /* local query rows, gathered key rows                          */
  int32_t h_idx, d_idx;   /* index heads, index head width                                */
  int32_t h, d_qk, d_v;   /* query heads, latent row width (value + rope), value width    */
  int32_t topk;           /* selected keys per row; a row keeps min(topk, window) of them */
  float softmax_scale;    /* multiplies q.k before the softmax (1/sqrt(d_qk) usually)     */
  int32_t idx_dtype;      /* dsa_idx_dtype                                                 */
  const dsa_segment *segs; /* host array of n_segs segments                                */
  int32_t n_segs;
} dsa_shape;

/* DSA_ABI_VERSION of the built library. */
int dsa_abi_version(void);

/* Message for the calling thread's last non-OK status ("" if none).  Valid until the next
 * call on the same thread. */
const char *dsa_last_error(void);

/*
 * Workspace bytes dsa_forward and dsa_indexer_topk use by default for `shape`: one candidate
 * count per row, the [n_q, topk] indices (used when the caller does not keep them), then
 * `cap` candidate slots per row, as fp32 scores and, in a second region, 16-bit window
 * offsets of their keys; each region starts on a 256-byte boundary:
 *     round256(4 n_q) + round256(4 n_q topk) + round256(4 n_q cap) + round256(2 n_q cap),
 *     cap = min(W, max(T + 192, round64(ceil(4.5 topk))))
 * with W the longest window and T topk, both rounded up to a multiple of 64.  A smaller
 * workspace is accepted down to cap = min(W, T + 192) (the calls use the most slots it holds);
 * rows whose candidates outgrow their slots are compacted in place, so fewer slots cost time,
 * not results.  Host-only.
 */
dsa_status dsa_workspace_bytes(const dsa_shape *shape, size_t *bytes);

/*
 * Lightning Indexer scores (page "CANNTorchTitan: ...", section
 * "SparseLightningIndexerGradKLLoss", indexer top-k value formula; the CP guide's indexer
 * boundary (query, key, weights)):
 *     scores[i, s] = sum_j w_idx[i, j] * ReLU( q_idx[i, j, :] . k_idx[s, :] )
 * for s in row i's window, -inf for every other column of a covered row.
 *   q_idx   [n_q, h_idx, d_idx]  bf16 (or e4m3fn codes with q_scale [n_q] fp32)
 *   k_idx   [n_k, d_idx]         bf16 (or e4m3fn codes with k_scale [n_k] fp32)
 *   w_idx   [n_q, h_idx]         fp32 per-token head weights (any sign)
 *   scores  [n_q, n_k]           fp32 output
 * bf16 products are accumulated in fp32 (MFMA); ReLU, weights and the head sum are fp32.
 */
dsa_status dsa_indexer_scores(const dsa_shape *shape, const void *q_idx, const float *q_scale,
                              const void *k_idx, const float *k_scale, const float *w_idx,
                              float *scores, void *stream);

/*
 * Per-row causal top-k over indexer scores laid out as dsa_indexer_scores writes them
 * ([n_q, n_k] fp32; only each row's window is read).  Row i keeps n_i = min(topk, window)
 * keys with the largest scores; equal scores go to the lower key index and -0.0 equals +0.0.
 * topk_idx [n_q, topk] int32 receives the kept absolute key rows in ascending order followed
 * by -1.  Scores inside a window must be finite (NaN ordering is unspecified).
 */
dsa_status dsa_topk_select(const dsa_shape *shape, const float *scores, int32_t *topk_idx,
                           void *stream);

/*
 * The indexer fused with the top-k (page "CANN/torchtitan-npu融合算子适配", section "DSA":
 * the indexer operator returns the selected indices, not the scores): the same indices as
 * dsa_indexer_scores followed by dsa_topk_select on the same inputs, bit for bit (the scores
 * come from the same kernels), without writing every score.  Per row the indexer keeps a
 * running lower bound of the row's k-th largest score and writes only the scores at or above
 * it, with their keys, to the row's candidate slots in `workspace`; when they would outgrow
 * the slots the row finds its k-th largest candidate and keeps only what can still be
 * selected.  The selection then runs over those candidates.
 * topk_idx [n_q, topk] int32 receives, for every covered row, its kept keys in ascending order
 * followed by -1.  workspace: dsa_workspace_bytes bytes or fewer, down to the minimum stated
 * there (DSA_ERR_WORKSPACE below it).  Arguments and index dtypes as for dsa_indexer_scores;
 * rows covered by no segment are left untouched.
 */
dsa_status dsa_indexer_topk(const dsa_shape *shape, const void *q_idx, const float *q_scale,
                            const void *k_idx, const float *k_scale, const float *w_idx,
                            int32_t *topk_idx, void *workspace, size_t workspace_bytes,
                            void *stream);

/*
 * Sparse multi-query attention over gathered latent rows (page "CANNTorchTitan: ...",
 * Sparse Flash Attention formula; the CP guide's sparse-attention boundary with key = value
 * = the shared latent row under weight absorption, rope = its last d_qk - d_v columns):
 *     z[h, t]       = softmax_scale * q[i, h, :] . kv[topk_idx[i, t], :]
 *     out[i, h, :]  = sum_t softmax_t(z[h, :]) * kv[topk_idx[i, t], :d_v]
 *     softmax_max[i, h] = max_t z[h, t];  softmax_sum[i, h] = sum_t exp(z[h, t] - max)
 *   q [n_q, h, d_qk] bf16, kv [n_k, d_qk] bf16, topk_idx [n_q, topk] int32,
 *   out [n_q, h, d_v] bf16; softmax_max / softmax_sum [n_q, h] fp32 (either may be NULL).
 * Every row 0..n_q-1 is computed (segments are not used).  Slots holding a negative index or
 * an index >= n_k are skipped; a row with no valid slot gets out = 0, max = -inf, sum = 0.
 * bf16 MFMA with fp32 accumulation and an fp32 online softmax.
 */
dsa_status dsa_sparse_attn(const dsa_shape *shape, const void *q, const void *kv,
                           const int32_t *topk_idx, void *out, float *softmax_max,
                           float *softmax_sum, void *stream);

/*
 * The fused DSA forward on one CP rank's share: the fused indexer + top-k
 * (dsa_indexer_topk) -> sparse attention, enqueued back to back on `stream` (the page
 * "CANNTorchTitan: ..." section "自定义CP策略": the CP forward is the plain forward over
 * all-gathered keys).  Arguments as above; only candidate scores are written, to
 * `workspace` (never the full [n_q, n_k]; sizes as for dsa_indexer_topk).  topk_idx may be
 * NULL (then the indices stay in the workspace), softmax_max / softmax_sum may be NULL.
 * Rows covered by no segment are left untouched.
 */
dsa_status dsa_forward(const dsa_shape *shape, const void *q_idx, const float *q_scale,
                       const void *k_idx, const float *k_scale, const float *w_idx,
                       const void *q, const void *kv, void *out, int32_t *topk_idx,
                       float *softmax_max, float *softmax_sum, void *workspace,
                       size_t workspace_bytes, void *stream);

/*
 * Dense causal attention of an Ulysses head shard (page "自定义Context Parallel特性", section
 * "SDPA Ulysses CP": an all-to-all moves Q/K/V from a sequence shard to a head shard, so one
 * device runs ordinary SDPA over the whole sequence of its heads; page "context_parallel.md",
 * section "ContextParallel 模式": Pure Ulysses and Hybrid placements).  Per local row i of a
 * segment (row r of it, window keys k_start .. k_start + pos0 + r, as for the DSA calls) and
 * head h:
 *   z_s = softmax_scale * q[i,h,:] . k[s,h,:];  out[i,h,:] = sum_s softmax(z)_s v[s,h,:];
 *   lse[i,h] = log(sum_s exp(z_s)) (natural log).
 * One segment (0, S, 0, S, 0) is plain causal attention over a sequence; a query shard of
 * the sequence against gathered K/V (Hybrid) sets pos0 to the shard's offset; packed
 * documents are one segment each.  Used fields of `shape`: n_q, n_k, h (the shard's heads,
 * >= 1), d_qk = 192, d_v = 128 (the only dims built: DSA_ERR_UNSUPPORTED otherwise),
 * softmax_scale (finite, > 0), segs / n_segs; the rest is ignored.
 *   q [n_q, h, 192], k [n_k, h, 192], v [n_k, h, 128], out [n_q, h, 128]: bf16 (BSHD with the
 *   batch folded into rows), 16-byte aligned; lse [n_q, h] fp32, may be NULL.
 * n_k * h * 192 * 2 bytes must stay below 4 GiB.  Rows covered by no segment are left
 * untouched.  bf16 MFMA with fp32 accumulation; the softmax max is rebased only when it grows
 * by more than 2^8, so probabilities stay below 2^8 before normalisation.  Device memory owned
 * by the caller; nothing is allocated.
 */
dsa_status dsa_dense_attn(const dsa_shape *shape, const void *q, const void *k, const void *v,
                          void *out, float *lse, void *stream);

/*
 * Sparse-attention backward (page "CANNTorchTitan: ...", section "SparseFlashAttentionGrad"):
 * for each row i, head h and selected slot s (valid index k = topk_idx[i][s]):
 *   z = softmax_scale * q[i,h,:] . kv[k,:];  P = exp(z - softmax_max[i,h]) / softmax_sum[i,h];
 *   D = sum_c dout[i,h,c] * out[i,h,c];  dP = dout[i,h,:] . kv[k,:d_v];  dS = P * (dP - D);
 *   dq[i,h,:]   = softmax_scale * sum_s dS * kv[k,:]
 *   dkv[k,:]   += softmax_scale * sum_h dS * q[i,h,:]
 *   dkv[k,:d_v] += sum_h P * dout[i,h,:]
 * q [n_q, h, d_qk], kv [n_k, d_qk], out / dout [n_q, h, d_v] bf16 (out and the statistics as
 * written by the forward); topk_idx [n_q, topk] as for dsa_sparse_attn (empty slots skipped);
 * dq [n_q, h, d_qk] bf16 (written); dkv [n_k, d_qk] fp32 (16-byte aligned) is ADDED to, so
 * the caller zeroes it (or accumulates into it); the order in which a key's contributions
 * are summed is not fixed.
 * Built for (h, d_qk, d_v) = (128, 576, 512) only (else DSA_ERR_UNSUPPORTED).  The workspace
 * (16-byte aligned) holds per-key counters and, for a chunk of rows, bf16 P and dS, the bf16
 * dKV contribution of every selected slot and the per-key entry lists; rows are processed in
 * chunks of as many rows as it fits (DSA_ERR_WORKSPACE if not even one).  dkv is updated
 * with plain read-modify-writes (each key's sum is formed by one wave), so calls that
 * update the same dkv must not overlap.
 */
dsa_status dsa_sparse_attn_bwd(const dsa_shape *shape, const void *q, const void *kv,
                               const int32_t *topk_idx, const void *out, const void *dout,
                               const float *softmax_max, const float *softmax_sum, void *dq,
                               float *dkv, void *workspace, size_t workspace_bytes,
                               void *stream);

/* Workspace size for dsa_sparse_attn_bwd that processes up to 2048 rows per pass:
 * (4 * topk_p * h + 2 * topk_p * d_qk + 4 * topk) bytes per row, topk_p = topk rounded up to a
 * multiple of 96, plus 4 * (3 * n_k + 1) bytes rounded up to 256 and 2 KiB of alignment
 * slack. */
dsa_status dsa_sparse_attn_bwd_workspace_bytes(const dsa_shape *shape, size_t *bytes);

/*
 * Indexer KL loss and its gradients (page "CANNTorchTitan: ...", section
 * "SparseLightningIndexerGradKLLoss": the loss and gradient formulas that follow the indexer
 * and Sparse Flash Attention top-k value formulas; the CP guide's indexer-loss boundary, which
 * consumes softmax_max / softmax_sum).  For each row i, over its valid slots s (index
 * k = topk_idx[i][s] in [0, n_k); a repeated key is one entry per slot):
 *   P[h, s] = exp(softmax_scale * q[i,h,:] . kv[k,:] - softmax_max[i,h]) / softmax_sum[i,h]
 *   p[s]    = sum_h P[h, s] / sum_{h,s'} P[h, s']           (target, L1-normalised)
 *   S[j, s] = q_idx[i,j,:] . k_idx[k,:];   I[s] = sum_j w_idx[i,j] * ReLU(S[j, s])
 *   loss_rows[i] = sum_s p[s] * (log p[s] - log softmax(I)[s])  (terms with p[s] = 0 are 0)
 *   dI[s]   = loss_grad * (softmax(I)[s] - p[s])
 *   dw_idx[i, j]  = sum_s dI[s] * ReLU(S[j, s])
 *   dS[j, s] = w_idx[i,j] * dI[s] if S[j, s] > 0 else 0
 *   dq_idx[i, j, :] = sum_s dS[j, s] * k_idx[k, :];   dk_idx[k, :] += sum_j dS[j, s] * q_idx[i, j, :]
 * The target carries no gradient; loss_grad is the gradient arriving at each row's term (1 for
 * the plain sum).  A row with no valid slot gets loss 0 and zero dq_idx / dw_idx.
 *   q_idx [n_q, 64, 128] bf16, k_idx [n_k, 128] bf16, w_idx [n_q, 64] fp32,
 *   q [n_q, 128, 576] bf16, kv [n_k, 576] bf16, topk_idx [n_q, topk] int32,
 *   softmax_max / softmax_sum [n_q, 128] fp32 as written by the forward for these indices;
 *   loss_rows [n_q] fp32 (written); loss [1] fp32 = sum of loss_rows in a fixed order (written;
 *   may be NULL); dq_idx [n_q, 64, 128] bf16 and dw_idx [n_q, 64] fp32 (written);
 *   dk_idx [n_k, 128] fp32 is ADDED to (the caller zeroes it), each key's sum in an order
 *   that is not fixed.  Every row 0..n_q-1 is computed (segments are not used).
 * Built for bf16 index tensors with (h_idx, d_idx, h, d_qk) = (64, 128, 128, 576) and
 * 1 <= topk <= 2048 (else DSA_ERR_UNSUPPORTED); d_v is not used.  q_idx, k_idx, w_idx, q, kv,
 * the statistics, dk_idx and the workspace must be 16-byte aligned, dq_idx 8-byte aligned
 * (DSA_ERR_INVALID_ARG).  The workspace holds per-key counters and, for a chunk of rows, the
 * bf16 key gradient and fp32 dI of every slot and the per-key entry lists; rows are processed in chunks
 * of as many rows as it fits (DSA_ERR_WORKSPACE if not even one).  Calls that update the same
 * dk_idx must not overlap.  Products in bf16 MFMA with fp32 accumulation; softmax, logarithms
 * and the loss in fp32.
 */
dsa_status dsa_indexer_kl_loss_grad(const dsa_shape *shape, const void *q_idx, const void *k_idx,
                                    const float *w_idx, const void *q, const void *kv,
                                    const int32_t *topk_idx, const float *softmax_max,
                                    const float *softmax_sum, float loss_grad, float *loss_rows,
                                    float *loss, void *dq_idx, float *dw_idx, float *dk_idx,
                                    void *workspace, size_t workspace_bytes, void *stream);

/* Workspace size for dsa_indexer_kl_loss_grad that processes up to 2048 rows per pass:
 * (260 * topk_p + 4 * topk) bytes per row, topk_p = topk rounded up to a multiple of 96, plus
 * 4 * (3 * n_k + 1) bytes rounded up to 256, 1 KiB, and 2 KiB of alignment slack. */
dsa_status dsa_indexer_kl_workspace_bytes(const dsa_shape *shape, size_t *bytes);

/*
 * The attention backward and the indexer KL loss of one training step in one call (page
 * "CANNTorchTitan: ...", sections "SparseFlashAttentionGrad" and
 * "SparseLightningIndexerGradKLLoss": both consume the same recomputed probabilities
 * P[h, s] and the same top-k indices).  Results as dsa_sparse_attn_bwd followed by
 * dsa_indexer_kl_loss_grad with the same arguments (dq bit for bit; dkv and dk_idx up to the
 * order of their per-key sums; the losses, dq_idx and dw_idx up to fp32 rounding of the target:
 * its per-slot head sums come from the backward's probabilities instead of a second
 * recomputation).  Over each chunk of rows the per-key entry lists are built once for both,
 * and the indexer loss neither gathers latent rows nor recomputes logits.
 *   Arguments: those of dsa_sparse_attn_bwd (q .. dkv), then those of dsa_indexer_kl_loss_grad
 *   that it does not share (q_idx .. dk_idx); the same layouts, alignment, accumulation
 *   (dkv and dk_idx are ADDED to) and supported dimensions as those two calls (the union of
 *   their DSA_ERR_UNSUPPORTED cases).  The workspace holds both calls' per-chunk arrays, the
 *   indexer loss's reusing the backward's once consumed, plus 4 * topk_p bytes per row of
 *   head sums; rows are processed in chunks of as many rows as it fits (DSA_ERR_WORKSPACE
 *   if not even one).  Calls that update the same dkv or dk_idx must not overlap.
 */
dsa_status dsa_sparse_attn_bwd_indexer_kl(
    const dsa_shape *shape, const void *q, const void *kv, const int32_t *topk_idx,
    const void *out, const void *dout, const float *softmax_max, const float *softmax_sum,
    void *dq, float *dkv, const void *q_idx, const void *k_idx, const float *w_idx,
    float loss_grad, float *loss_rows, float *loss, void *dq_idx, float *dw_idx, float *dk_idx,
    void *workspace, size_t workspace_bytes, void *stream);

/* Workspace size for dsa_sparse_attn_bwd_indexer_kl that processes up to 2048 rows per pass:
 * dsa_sparse_attn_bwd's bytes per row plus 4 * topk_p, plus its fixed part. */
dsa_status dsa_sparse_attn_bwd_indexer_kl_workspace_bytes(const dsa_shape *shape, size_t *bytes);

/* Bytes of the fixed device array dsa_forward_noalloc works in (one per GPU). */
#define DSA_NOALLOC_SCRATCH_BYTES (256u << 20)

/*
 * dsa_forward for callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  Arguments, results and errors are
 * those of dsa_forward without the workspace (the same kernels run, so the results are the
 * same bit for bit).  The workspace is a device array of DSA_NOALLOC_SCRATCH_BYTES bytes that
 * the library holds on every GPU it runs on until the process ends; the local rows go through
 * it in consecutive passes of as many rows as it holds with the default candidate slots
 * (DSA_ERR_UNSUPPORTED if not even one row's workspace fits).  Nothing in it needs to start
 * at zero.  The call allocates no device memory and does not synchronise; its first call on a
 * device looks up that device's array address (make it before any graph capture).  `stream`
 * must belong to the current device (DSA_ERR_INVALID_ARG otherwise).  Every call on a GPU
 * shares that GPU's array: calls that overlap on one GPU (other streams, other host threads)
 * race and must be serialised by the caller.
 */
dsa_status dsa_forward_noalloc(const dsa_shape *shape, const void *q_idx, const float *q_scale,
                               const void *k_idx, const float *k_scale, const float *w_idx,
                               const void *q, const void *kv, void *out, int32_t *topk_idx,
                               float *softmax_max, float *softmax_sum, void *stream);

/*
 * Per-row (per-token) fp8 quantization for the fp8 indexer: for each of `rows` rows of
 * `cols` bf16 values, scale = amax(|row|) / 448 (1.0 for an all-zero row) and
 * code = e4m3fn(round-to-nearest-even(x / scale)), saturating at +-448; scale and x / scale
 * are computed in fp32 with correctly rounded division.
 *   x_bf16 [rows, cols] bf16 -> x_fp8 [rows, cols] uint8 codes, scale [rows] fp32.
 * For the index query use rows = n_q, cols = h_idx * d_idx (one scale per token).
 */
dsa_status dsa_quantize_fp8_rows(const void *x_bf16, int64_t rows, int32_t cols, void *x_fp8,
                                 float *scale, void *stream);

#ifdef __cplusplus
} /* extern "C" */
#endif

#endif /* DSA_H */
