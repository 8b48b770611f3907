"""DSA forward benchmark on one MI355X: one CP rank's share of a 32K sequence.

A step is one fused forward (indexer fused with the top-k -> sparse attention) over the
whole local share, inputs resident in HBM.  Prints one JSON line: useful TFLOP/s of the step (indexer
2*H_idx*d_idx per window key + attention 2*H*(d_qk+d_v) per selected key), queries/s, a
roofline entry for the dominant kernel (sparse attention, MFMA-bound), per-stage timings, the
head-tail CP-degree-8 share with its indexer in bf16 and in fp8, the training-side kernels on
the packed varlen workload, and the CPU oracle's throughput on a bounded row sample.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 3] [--no-cpu-baseline]
"""

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from sparse_attention_11_amd import dsa, inputs as I  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0      # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")
_CSRC = os.path.join(ROOT, "sparse_attention_11_amd", "csrc")
# kernel families of the forward whose HBM bytes the counter record holds, the sources each is
# built from (the record is valid for those sources only) and the name prefix of its kernels
# in the profiler's dispatch table
TRAFFIC_KERNELS = {
    "attention": (("attention.hip", "attn_common.h", "dsa_device.h"),
                  ("k_sparse_attn_ring<128, 576, 512>",)),
    "indexer_candidates": (("indexer.hip", "dsa_device.h"), ("k_indexer_bf16<64, 128, true>",)),
    "topk_candidates": (("topk.hip", "dsa_device.h"),
                        ("k_topk<256, 8, true>", "k_topk<512, 16, true>", "k_topk<512, 32, true>",
                         "k_topk<1024, 32, true>")),
}


def source_hash(files):
    h = hashlib.sha256()
    for f in files:
        h.update(open(os.path.join(_CSRC, f), "rb").read())
    return h.hexdigest()


def work(wl):
    """Algorithmic work of the forward for the workload's segments."""
    L = []
    for (qs, ql, ks, kl, p0) in wl.segments:
        L.append(np.arange(p0 + 1, p0 + ql + 1, dtype=np.int64))
    L = np.concatenate(L) if L else np.zeros(0, np.int64)
    n = np.minimum(L, wl.topk)
    f_idx = float(2 * wl.h_idx * wl.d_idx * L.sum())
    f_attn = float(2 * wl.h * (wl.d_qk + wl.d_v) * n.sum())
    return dict(rows=int(L.size), window_keys=int(L.sum()), selected=int(n.sum()),
                f_idx=f_idx, f_attn=f_attn,
                gather_bytes=float(n.sum() * wl.d_qk * 2),
                topk_bytes=float(L.sum() * 4 + L.size * wl.topk * 4))


def time_launches(fn, reps, stream, trials=3):
    """Average duration of fn() over reps back-to-back launches, HIP events on the launch
    stream; the median of `trials` such averages (one slow stretch of the box does not set the
    figure; every launch of the median trial counts)."""
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    fn()
    torch.cuda.synchronize()
    avg = []
    for _ in range(trials):
        start.record(stream)
        for _ in range(reps):
            fn()
        end.record(stream)
        torch.cuda.synchronize()
        avg.append(start.elapsed_time(end) / reps)
    return float(np.median(avg))


def per_step_timing(step, stream, reps, cold_reps=5, scratch_bytes=512 << 20):
    """Each forward step timed on its own (HIP events on the launch stream): median and min
    with the caches warm (steps back to back), and with them cold (a 512 MB buffer, twice the
    256 MB MALL, is overwritten before each timed step; the fill is outside the timed span)."""
    def one(before=None):
        if before is not None:
            before()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        step()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)
    warm = [one() for _ in range(reps)]
    scratch = torch.empty(scratch_bytes, dtype=torch.uint8, device=torch.device("cuda:0"))
    cold = [one(lambda i=i: scratch.fill_(i & 0xFF)) for i in range(cold_reps)]
    del scratch
    return {"warm": {"median_ms": float(np.median(warm)), "min_ms": float(np.min(warm)),
                     "steps": reps},
            "cold": {"median_ms": float(np.median(cold)), "min_ms": float(np.min(cold)),
                     "steps": cold_reps,
                     "flush": "512 MB buffer overwritten before each timed step"}}


def cpu_baseline(wl, budget_s=15.0, max_rows=2048):
    """The float64 oracle on a seeded sample of the workload's rows, on the host cores."""
    import oracle
    from threadpoolctl import threadpool_info
    x = I.generate(wl)                     # CPU generator: the oracle's own inputs
    f64 = I.to_f64
    qi, ki, wi, q, kv = (f64(x[k]) for k in ("q_idx", "k_idx", "w_idx", "q", "kv"))
    rng = np.random.default_rng(0)
    order = rng.permutation(wl.n_q)
    segs = list(wl.segments)
    done, flops, t0 = [], 0.0, time.perf_counter()
    k_lo, L = oracle.row_windows(segs, wl.n_q, wl.n_k)
    for r in order[:max_rows]:
        if L[r] < 0:
            continue
        oracle.dsa_forward(qi, ki, wi, q, kv, segs, wl.topk, wl.softmax_scale, wl.d_v,
                           rows=np.array([r]))
        done.append(int(r))
        n = min(wl.topk, int(L[r]))
        flops += 2 * wl.h_idx * wl.d_idx * int(L[r]) + 2 * wl.h * (wl.d_qk + wl.d_v) * n
        if time.perf_counter() - t0 > budget_s and len(done) >= 4:
            break
    dt = time.perf_counter() - t0
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle", "queries_per_s": len(done) / dt, "cpu_model": host_cpu_model(),
            "sample": f"{len(done)} seeded random rows of {wl.name} (indexer over each row's "
                      f"window, top-k, attention), float64 NumPy, {dt:.1f} s"}


def backward_stage(args, n=5):
    """Training-side kernels on the packed varlen workload (8 documents, 32768 tokens): the
    GPU forward supplies indices, output and softmax statistics; the sparse-attention backward
    (P / dS, dQ, dKV kernels) and the indexer KL loss with its gradients are each timed on
    their own with HIP events, then both in the one combined call."""
    wl = I.workload(n)
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    g = I.generate(wl, device=dev, gen_device="cuda")
    out, idx, smax, ssum = dsa.dsa_forward(g["q_idx"], g["k_idx"], g["w_idx"], g["q"], g["kv"],
                                           wl.segments, wl.topk, wl.softmax_scale, wl.d_v)
    dq = torch.empty_like(g["q"])
    dkv = torch.zeros(wl.n_k, wl.d_qk, dtype=torch.float32, device=dev)
    nb = dsa.dsa_sparse_attn_bwd_workspace_bytes(wl.n_q, wl.n_k, wl.topk)
    ws = torch.empty(nb, dtype=torch.uint8, device=dev)

    def bwd():
        dsa.dsa_sparse_attn_bwd(g["q"], g["kv"], idx, out, g["dout"], smax, ssum,
                                wl.softmax_scale, dq=dq, dkv=dkv, workspace=ws)
    reps = max(3, min(args.steps, 10))
    ms = time_launches(bwd, reps, stream)
    n_sel = int((idx >= 0).sum())
    flop = 2.0 * wl.h * (3 * wl.d_qk + 2 * wl.d_v) * n_sel
    print(f"bench: backward {wl.name} {ms:.3f} ms", file=sys.stderr, flush=True)
    rec = {"workload": wl.name, "ms": ms, "selected_keys": n_sel, "flop": flop,
           "tflops": flop / (ms * 1e-3) / 1e12,
           "mfma_frac": flop / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}
    del dq, ws
    # indexer KL loss and its gradients on the same forward outputs: per selected slot the
    # recomputed attention logits (2 h d_qk) and the index scores, dq_idx and dk_idx products
    # (3 x 2 h_idx d_idx)
    dk = torch.zeros(wl.n_k, wl.d_idx, dtype=torch.float32, device=dev)
    kws = torch.empty(dsa.dsa_indexer_kl_workspace_bytes(wl.n_q, wl.n_k, wl.topk),
                      dtype=torch.uint8, device=dev)

    def kl():
        dsa.dsa_indexer_kl_loss_grad(g["q_idx"], g["k_idx"], g["w_idx"], g["q"], g["kv"], idx,
                                     smax, ssum, wl.softmax_scale, dk_idx=dk, workspace=kws)
    kms = time_launches(kl, reps, stream)
    kflop = 2.0 * n_sel * (wl.h * wl.d_qk + 3 * wl.h_idx * wl.d_idx)
    print(f"bench: indexer KL loss + gradients {wl.name} {kms:.3f} ms", file=sys.stderr,
          flush=True)
    rec["indexer_kl"] = {"ms": kms, "flop": kflop, "tflops": kflop / (kms * 1e-3) / 1e12,
                         "mfma_frac": kflop / (kms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}
    del kws
    # both in one call (dsa_sparse_attn_bwd_indexer_kl): the indexer loss takes its target
    # from the backward's probabilities and shares its key lists; the useful work is the
    # backward's plus the indexer part of the loss (3 x 2 h_idx d_idx per slot)
    dq = torch.empty_like(g["q"])
    cws = torch.empty(dsa.dsa_sparse_attn_bwd_indexer_kl_workspace_bytes(wl.n_q, wl.n_k, wl.topk),
                      dtype=torch.uint8, device=dev)

    def both():
        dsa.dsa_sparse_attn_bwd_indexer_kl(g["q"], g["kv"], idx, out, g["dout"], smax, ssum,
                                           wl.softmax_scale, g["q_idx"], g["k_idx"], g["w_idx"],
                                           dq=dq, dkv=dkv, dk_idx=dk, workspace=cws)
    cms = time_launches(both, reps, stream)
    cflop = flop + 2.0 * n_sel * 3 * wl.h_idx * wl.d_idx
    print(f"bench: backward + indexer loss in one call {wl.name} {cms:.3f} ms (separate "
          f"{ms + kms:.3f} ms)", file=sys.stderr, flush=True)
    rec["with_indexer_kl"] = {"ms": cms, "separate_ms": ms + kms, "flop": cflop,
                              "tflops": cflop / (cms * 1e-3) / 1e12,
                              "mfma_frac": cflop / (cms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}
    return rec


def dense_stage(args):
    """Dense causal attention of one 8-way Ulysses rank (32768 positions, 16 of DeepSeek-V3's
    128 heads, q/k 192 and v 128 wide): time per call and useful TFLOP/s (every causal
    (query, key) pair once, 2 (192 + 128) flop per pair and head)."""
    wl = I.dense_workload(1)
    stream = torch.cuda.current_stream()
    g = I.generate_dense(wl, device=torch.device("cuda:0"), gen_device="cuda")
    out = torch.empty(wl.n, wl.h, wl.d_v, dtype=torch.bfloat16, device="cuda:0")
    reps = max(3, min(args.steps, 10))
    ms = time_launches(lambda: dsa.dsa_dense_attn(g["q"], g["k"], g["v"], wl.segments,
                                                  wl.softmax_scale, out=out), reps, stream)
    pairs = sum(L * (L + 1) // 2 for (_, L, _, _, _) in wl.segments)
    flop = 2.0 * pairs * wl.h * (wl.d_qk + wl.d_v)
    tf = flop / (ms * 1e-3) / 1e12
    print(f"bench: dense attention {wl.name} {ms:.3f} ms {tf:.1f} TFLOP/s", file=sys.stderr,
          flush=True)
    return {"workload": wl.name, "ms": ms, "flop": flop, "tflops": tf,
            "mfma_frac": tf / PEAK_BF16_TFLOPS}


def head_tail_stage(args):
    """The CP-degree-8 head-tail share (two 2048-query chunks against 32768 keys): the fused
    indexer + top-k with bf16 index inputs and with e4m3 codes and per-token scales (quantized
    on the GPU, outside the timed span), and the whole bf16 forward, each timed on its own."""
    wl = I.workload(4).with_(with_dout=False)
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    g = I.generate(wl, device=dev, gen_device="cuda")
    W = work(wl)
    reps = max(3, min(args.steps, 10))
    qc, qs = dsa.dsa_quantize_fp8_rows(g["q_idx"])
    kc, ks = dsa.dsa_quantize_fp8_rows(g["k_idx"])
    tk = torch.empty(wl.n_q, wl.topk, dtype=torch.int32, device=dev)
    ws = torch.empty(dsa.dsa_workspace_bytes(wl.n_q, wl.n_k, wl.topk, wl.segments),
                     dtype=torch.uint8, device=dev)
    bf = time_launches(lambda: dsa.dsa_indexer_topk(g["q_idx"], g["k_idx"], g["w_idx"],
                                                    wl.segments, wl.topk, out=tk, workspace=ws),
                       reps, stream)
    f8 = time_launches(lambda: dsa.dsa_indexer_topk(qc, kc, g["w_idx"], wl.segments, wl.topk,
                                                    q_scale=qs, k_scale=ks, out=tk, workspace=ws),
                       reps, stream)
    out = torch.empty(wl.n_q, wl.h, wl.d_v, dtype=torch.bfloat16, device=dev)
    fw = time_launches(lambda: dsa.dsa_forward(g["q_idx"], g["k_idx"], g["w_idx"], g["q"],
                                               g["kv"], wl.segments, wl.topk, wl.softmax_scale,
                                               wl.d_v, out=out, workspace=ws), reps, stream)
    print(f"bench: head-tail {wl.name}: indexer+top-k bf16 {bf:.3f} ms, fp8 {f8:.3f} ms, "
          f"forward {fw:.3f} ms", file=sys.stderr, flush=True)
    fi = W["f_idx"]
    return {"workload": wl.name,
            "indexer_topk_bf16_ms": bf, "indexer_topk_bf16_tflops": fi / (bf * 1e-3) / 1e12,
            "indexer_topk_fp8_ms": f8, "indexer_topk_fp8_tflops": fi / (f8 * 1e-3) / 1e12,
            "indexer_topk_fp8_frac_of_fp8_peak": fi / (f8 * 1e-3) / 1e12 / PEAK_FP8_TFLOPS,
            "forward_bf16_ms": fw,
            "forward_tflops": (W["f_idx"] + W["f_attn"]) / (fw * 1e-3) / 1e12,
            "forward_queries_per_s": wl.n_q / (fw * 1e-3)}


def traffic_record():
    """Counter-based HBM bytes per forward of each kernel family (see TRAFFIC_KERNELS), for the
    families whose sources are unchanged since the counters were taken; {} without a record."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return {}
    out = {}
    for fam, (srcs, _) in TRAFFIC_KERNELS.items():
        e = t.get("kernels", {}).get(fam)
        if e and e.get("source_sha256") == source_hash(srcs):
            out[fam] = e
    return out


def _counter_rows(d, counter):
    import csv
    import glob
    rows = []
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] == counter:
                rows.append((int(r["Dispatch_Id"]), r["Kernel_Name"], float(r["Counter_Value"])))
    return sorted(rows)


def write_traffic_record(fetch_dir, write_dir, steps):
    """HBM bytes per forward of each kernel family: FETCH_SIZE and WRITE_SIZE (KiB-like units
    as read) scaled by what the same counters read for the 1 GiB device copy of the same run,
    summed over the family's dispatches and divided by the forwards run (warm-up + timed)."""
    scale, rows = {}, {}
    for name, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows[name] = _counter_rows(d, name)
        copies = [v for _, k, v in rows[name] if "copyBuffer" in k or "copy" in k.lower()]
        scale[name] = float(1 << 30) / max(copies)   # bytes per unit: the largest copy is 1 GiB
    rec = {"forwards": steps, "bytes_per_unit": scale, "kernels": {}}
    for fam, (srcs, prefixes) in TRAFFIC_KERNELS.items():
        e = {"source_sha256": source_hash(srcs), "kernels": list(prefixes)}
        for name in ("FETCH_SIZE", "WRITE_SIZE"):
            vals = [v for _, k, v in rows[name] if any(p in k for p in prefixes)]
            e[name] = {"dispatches": len(vals),
                       "bytes_per_forward": sum(vals) * scale[name] / steps}
        e["hbm_bytes_per_forward"] = e["FETCH_SIZE"]["bytes_per_forward"] + \
            e["WRITE_SIZE"]["bytes_per_forward"]
        rec["kernels"][fam] = e
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec, indent=1))


def kernel_times(fn, reps):
    """Average duration (ms) of every GPU kernel fn() launches, per call of fn, from the
    profiler's device activity trace (the HIP runtime's own dispatch timestamps); None when
    the trace is not available."""
    try:
        from torch.profiler import ProfilerActivity, profile
        fn()
        torch.cuda.synchronize()
        with profile(activities=[ProfilerActivity.CUDA]) as prof:
            for _ in range(reps):
                fn()
            torch.cuda.synchronize()
        out = {}
        for e in prof.key_averages():
            tot = getattr(e, "device_time_total", None)
            if tot is None:
                tot = getattr(e, "cuda_time_total", 0.0)
            if tot and e.key.startswith(("dsa::", "void dsa::")):
                out[e.key.replace("void ", "")] = tot / 1000.0 / reps
        return out or None
    except Exception as ex:  # noqa: BLE001
        print(f"bench: kernel trace unavailable ({type(ex).__name__}: {ex})", file=sys.stderr)
        return None


def _family_ms(ktimes, fam):
    if not ktimes:
        return None
    prefixes = TRAFFIC_KERNELS[fam][1]
    t = sum(v for k, v in ktimes.items() if any(p in k for p in prefixes))
    return t or None


def host_cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-stages", action="store_true")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the packed-varlen forward + backward timing")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write the HBM traffic record of the forward's kernels from two "
                         "rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of "
                         "'bench.py --calibrate-copy --no-stages --no-backward' with the same "
                         "--steps/--warmup, and exit")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run one 1 GiB device copy (reference for HBM byte counters)")
    args = ap.parse_args()
    if args.traffic_from:
        write_traffic_record(*args.traffic_from, steps=args.steps + args.warmup)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU's share only (got --gpus {args.gpus}); the CP "
              "all-gather and multi-GPU runs are not part of this build", file=sys.stderr)
        sys.exit(2)

    wl = I.workload(args.workload).with_(with_dout=False)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    print(f"bench: {wl.name} n_q={wl.n_q} n_k={wl.n_k} topk={wl.topk}", file=sys.stderr, flush=True)
    g = I.generate(wl, device=dev, gen_device="cuda")
    W = work(wl)
    if args.calibrate_copy:
        # a plain copy of known size: its FETCH_SIZE / WRITE_SIZE under rocprofv3 --pmc give
        # the scale from counter units to bytes for the kernels measured in the same run
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    out = torch.empty(wl.n_q, wl.h, wl.d_v, dtype=torch.bfloat16, device=dev)
    ws = torch.empty(dsa.dsa_workspace_bytes(wl.n_q, wl.n_k, wl.topk, wl.segments),
                     dtype=torch.uint8, device=dev)

    def step():
        return dsa.dsa_forward(g["q_idx"], g["k_idx"], g["w_idx"], g["q"], g["kv"],
                               wl.segments, wl.topk, wl.softmax_scale, wl.d_v, out=out,
                               return_idx=True, stats=True, workspace=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(args.steps):
        res = step()
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    print(f"bench: forward {ms:.3f} ms/step", file=sys.stderr, flush=True)
    idx = res[1]
    # (left out of the counter runs: cold steps would change the per-launch averages there;
    # an auxiliary figure, so a failure here is reported in the line instead of ending the run)
    timing = None
    if not args.calibrate_copy:
        try:
            timing = per_step_timing(step, stream, reps=max(3, min(args.steps, 10)))
        except Exception as e:  # noqa: BLE001
            timing = {"error": f"{type(e).__name__}: {e}"}

    stages = {}
    if not args.no_stages:
        reps = max(3, min(args.steps, 10))
        scores = torch.empty(wl.n_q, wl.n_k, dtype=torch.float32, device=dev)
        stages["indexer_ms"] = time_launches(
            lambda: dsa.dsa_indexer_scores(g["q_idx"], g["k_idx"], g["w_idx"], wl.segments,
                                           out=scores), reps, stream)
        tk = torch.empty(wl.n_q, wl.topk, dtype=torch.int32, device=dev)
        stages["topk_ms"] = time_launches(
            lambda: dsa.dsa_topk_select(scores, wl.segments, wl.topk, out=tk), reps, stream)
        del scores
        stages["indexer_topk_fused_ms"] = time_launches(
            lambda: dsa.dsa_indexer_topk(g["q_idx"], g["k_idx"], g["w_idx"], wl.segments,
                                         wl.topk, out=tk, workspace=ws), reps, stream)
        stages["attention_ms"] = time_launches(
            lambda: dsa.dsa_sparse_attn(g["q"], g["kv"], idx, wl.softmax_scale, wl.d_v, out=out),
            reps, stream)
        # per-kernel durations of one forward (the profiler's dispatch timestamps): the
        # candidate-mode indexer and the top-k tiers are two kernels inside one fused call
        stages["kernels_ms"] = kernel_times(step, reps)
    t_attn = stages.get("attention_ms")
    attn_tf = W["f_attn"] / (t_attn * 1e-3) / 1e12 if t_attn else None

    line = {
        "metric": "DSA fwd useful TFLOP/s + queries/s at 32K CP shard; % MFMA peak, HBM GB/s",
        "value": (W["f_idx"] + W["f_attn"]) / (ms * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded Gaussian index/query/latent rows, uniform index weights)",
        "config": {"workload": wl.name, "local_queries": wl.n_q, "keys": wl.n_k,
                   "segments": [list(s) for s in wl.segments], "topk": wl.topk,
                   "index_heads": wl.h_idx, "index_dim": wl.d_idx, "heads": wl.h,
                   "d_qk": wl.d_qk, "d_v": wl.d_v, "parallelism": "one CP rank's share"},
        "queries_per_s": wl.n_q / (ms * 1e-3),
        "useful_tflop": (W["f_idx"] + W["f_attn"]) / 1e12,
        "step_timing": timing,
        "workspace_bytes": int(ws.numel()),
    }
    if stages:
        ti, tt = stages["indexer_ms"], stages["topk_ms"]
        kt = stages["kernels_ms"]
        t_ic = _family_ms(kt, "indexer_candidates")
        t_tk = _family_ms(kt, "topk_candidates")
        t_ak = _family_ms(kt, "attention")
        tr = traffic_record()

        def gbs(fam, t_ms, minus=0.0, part="hbm_bytes_per_forward"):
            e = tr.get(fam)
            if not e or not t_ms:
                return None
            b = (e[part]["bytes_per_forward"] if part != "hbm_bytes_per_forward" else e[part])
            return (b - minus) / (t_ms * 1e-3) / 1e9
        q_bytes = wl.n_q * wl.h * wl.d_qk * 2.0
        idx_bytes = wl.n_q * wl.topk * 4.0
        line["stages"] = {
            "dense_indexer_ms_incl_minus_inf_fill": ti,
            "dense_indexer_tflops": W["f_idx"] / (ti * 1e-3) / 1e12,
            "dense_indexer_mfma_frac": W["f_idx"] / (ti * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
            "dense_topk_ms": tt,
            "dense_topk_logical_gbs": W["topk_bytes"] / (tt * 1e-3) / 1e9,
            "indexer_topk_fused_ms": stages["indexer_topk_fused_ms"],
            "indexer_candidates_kernel_ms": t_ic,
            "indexer_candidates_tflops": W["f_idx"] / (t_ic * 1e-3) / 1e12 if t_ic else None,
            "indexer_candidates_mfma_frac":
                W["f_idx"] / (t_ic * 1e-3) / 1e12 / PEAK_BF16_TFLOPS if t_ic else None,
            "topk_candidates_kernels_ms": t_tk,
            # HBM bytes from the rocprofv3 FETCH_SIZE / WRITE_SIZE record of these kernels
            # (null when their sources changed since it was taken) over their live duration
            "topk_candidates_hbm_gbs": gbs("topk_candidates", t_tk),
            "attention_ms": t_attn,
            "attention_kernel_ms": t_ak,
            "attention_tflops": attn_tf,
            "attention_mfma_frac": attn_tf / PEAK_BF16_TFLOPS,
            "attention_hbm_gbs": gbs("attention", t_ak),
            # the attention kernel's fetched bytes less its compulsory reads (q, indices):
            # the latent-row gather's traffic past L2 (HBM and the MALL behind it)
            "kv_gather_hbm_gbs": gbs("attention", t_ak, q_bytes + idx_bytes, "FETCH_SIZE"),
            "kv_gather_logical_gbs": W["gather_bytes"] / (t_attn * 1e-3) / 1e9,
            "kernels_ms": kt,
        }
        traffic = tr["attention"]["hbm_bytes_per_forward"] if "attention" in tr else None
        line["roofline"] = {"bound": "mfma", "kernel": "k_sparse_attn_ring (sparse MQA attention)",
                            "achieved": attn_tf, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                            "frac": attn_tf / PEAK_BF16_TFLOPS, "traffic": traffic,
                            "per_launch_flop": W["f_attn"]}
    if stages:
        line["head_tail"] = head_tail_stage(args)
        line["dense_attn"] = dense_stage(args)
    if not args.no_backward:
        line["backward"] = backward_stage(args)
    if not args.no_cpu_baseline:
        print("bench: timing the CPU oracle on a row sample", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
