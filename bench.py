"""Throughput of packed (THD) sink attention on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                [--no-cpu-baseline] [--no-configs]

One step = the whole hot path over one batch: the host tile schedule
(sink_attn_metadata, sink_attn_metadata_paged or sink_attn_metadata_padded)
and its copy to the device, the forward (sink_attn_fwd, sink_attn_fwd_paged
reading a paged K/V cache, or sink_attn_fwd_padded for a batch-padded
layout) and, for training workloads, the backward (sink_attn_bwd or
sink_attn_bwd_padded), all through the C ABI on torch's current stream. Inputs are resident in HBM
before timing starts. Prints one JSON line.

With the default workload (train_varlen, the configuration the headline
metric is quoted on) the line also carries "configs": the prefill, GQA
sliding-window training and decode configurations timed in the same run,
each in its own launch configuration.

FLOPs count only kept (query row, key, q-head) pairs: 4*D per pair forward,
10*D backward (the backward recomputes S). Bytes (decode) count K and V read
once plus q, out, lse.
"""
import argparse
import dataclasses
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0
METRIC = "sink-attention fwd+bwd TFLOP/s and % of bf16 MFMA peak, varlen THD causal"
TRAIN = {"train_varlen", "gqa_window", "gqa_window_bnsd", "train_varlen_d256"}


def kept_pairs(cu_q, cu_k, causal, wl, wr):
    """Kept (row, key) pairs per head, counted row by row from the
    bottom-right aligned mask bounds."""
    total = 0
    for b in range(len(cu_q) - 1):
        lq, lk = int(cu_q[b + 1] - cu_q[b]), int(cu_k[b + 1] - cu_k[b])
        if lq == 0 or lk == 0:
            continue
        pos = np.arange(lq, dtype=np.int64) + (lk - lq)
        lo = np.maximum(0, pos - wl) if wl >= 0 else np.zeros(lq, np.int64)
        if causal:
            hi = np.minimum(lk - 1, pos)
        elif wr >= 0:
            hi = np.minimum(lk - 1, pos + wr)
        else:
            hi = np.full(lq, lk - 1, np.int64)
        total += int(np.maximum(0, hi - lo + 1).sum())
    return total


def to_dev(p, name):
    import torch
    x = np.ascontiguousarray(getattr(p, name))
    if p.dtype == "bf16":
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(x).cuda()


def cpu_baseline(p, train, seconds):
    """The fp64 oracle on the host over a bounded sample of the workload:
    whole (sequence, q-head) slices, forward (+ backward for training),
    taken in a fixed order (median-length sequence first, heads in order)
    until about `seconds` of work has been done."""
    import oracle as O
    lens = np.diff(p.cu_q)
    order = list(np.argsort(lens, kind="stable"))
    order = order[len(order) // 2:] + order[:len(order) // 2][::-1]
    G = p.num_heads_q // p.num_heads_k
    pairs = 0
    done = []
    t0 = time.perf_counter()
    for b in order:
        sub = p.sub_batch([int(b)])
        sp = kept_pairs(sub.cu_q, sub.cu_k, p.causal, p.win_left, p.win_right)
        for h in range(p.num_heads_q):
            hk = h // G
            args = (sub.as_f32("q")[:, h:h + 1], sub.as_f32("k")[:, hk:hk + 1],
                    sub.as_f32("v")[:, hk:hk + 1], sub.cu_q, sub.cu_k,
                    sub.sinks[h:h + 1].astype(np.float64), float(p.scale), p.causal,
                    p.win_left, p.win_right)
            if train:
                O.sink_attention_backward(sub.as_f32("dout")[:, h:h + 1], *args)
            else:
                O.sink_attention_forward(*args)
            pairs += sp
            done.append((int(b), h))
            if time.perf_counter() - t0 >= seconds:
                break
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    flops = pairs * p.head_dim * (14 if train else 4)
    threads = blas_threads()
    seqs = sorted({b for b, _ in done})
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle", **host_cores(),
            "sample": f"{len(done)} (sequence, q-head) slices from sequences {seqs}: "
                      f"{'forward+backward' if train else 'forward'}, {pairs} kept pairs, "
                      f"{dt:.1f} s (FLOPs counted as in value)"}


def blas_threads():
    """Threads of the BLAS library NumPy calls (the oracle's matrix products
    run on these; its elementwise work runs on one core)."""
    from threadpoolctl import threadpool_info
    return max([i.get("num_threads", 1) for i in threadpool_info()
                if i.get("user_api") == "blas"] or [1])


def host_cores():
    """The host's logical CPUs, the CPUs this process may run on, and the
    BLAS thread count, reported beside the oracle's rate."""
    return {"cpu_count": os.cpu_count(), "affinity": len(os.sched_getaffinity(0)),
            "blas_threads": blas_threads()}


def other_configs():
    """The other reference configurations, each timed in a process of its
    own (as a standalone run of this script would time it) and in its own
    default launch configuration (forward-only workloads: 100 steps after
    20; the GQA window training step: 10 after 3): step time, throughput and
    the dominant kernel's share of its roofline."""
    import subprocess
    out = {}
    for name in ("prefill_varlen", "gqa_window", "decode_softmax_n"):
        print(f"# configuration {name}", file=sys.stderr, flush=True)
        r = subprocess.run([sys.executable, os.path.abspath(__file__), "--workload", name,
                            "--no-cpu-baseline"], capture_output=True, text=True, timeout=600)
        lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
        if r.returncode != 0 or not lines:
            raise RuntimeError(f"configuration {name} failed (exit {r.returncode}):\n"
                               f"{r.stderr[-2000:]}")
        d = json.loads(lines[-1])
        roof = d["roofline"]
        c = {"metric": d["metric"], "ms_per_step": d["ms_per_step"], "steps": d["steps"],
             "warmup": d["warmup"], "dtype": d["dtype"]}
        if "value_gbs" in d:
            c.update(value=d["value_gbs"], unit="GB/s",
                     frac_of_hbm_peak=d["value_gbs"] / PEAK_HBM_GBS, tflops=d["value"])
        else:
            c.update(value=d["value"], unit="TFLOP/s",
                     frac_of_bf16_peak=d["value"] / PEAK_BF16_TFLOPS)
        c["roofline"] = {k: roof[k] for k in ("bound", "kernel", "achieved", "peak", "unit",
                                              "frac", "traffic", "launch_ms")}
        c["config"] = d["config"]
        out[name] = c
    return out


def traffic_record(workload, kernel):
    """HBM bytes per launch of `kernel` from the committed counter summary,
    if it was taken on the current kernel source and compile flags; else
    None."""
    import hashlib
    from softmax_sink_amd.build import SOURCE_FLAGS
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get(workload)
    if not rec or rec.get("kernel") != kernel or "sources" not in rec:
        return None
    # the kernel's source file and every header it includes, in order
    h = hashlib.sha256()
    for name in rec["sources"]:
        h.update(open(os.path.join(ROOT, "softmax_sink_amd", "csrc", name), "rb").read())
    # extra compile flags of the kernel's source file, where it has any
    flags = SOURCE_FLAGS.get(rec["sources"][0], [])
    if flags:
        h.update(" ".join(flags).encode())
    if h.hexdigest() != rec["sources_sha256"]:
        return None
    return rec["hbm_bytes_per_launch"]


def bench_merge(args):
    """Context-parallel merge: 4 sink-free bf16 partials of the prefill
    workload's shape (16 sequences, 16640 tokens, 32 heads, D 128) merged into
    one bf16 output. HBM-bound: the bytes are the partials and their lse read
    once, the output and lse written once."""
    import torch
    from softmax_sink_amd import binding as B
    from softmax_sink_amd import workloads as W
    import oracle as O
    P, Hq, D = 4, 32, 128
    Tq = W.config("prefill_varlen").total_q
    outs, lses, sinks = W.merge_inputs(61, P, Tq, Hq, D)
    po = torch.from_numpy(outs.view(np.int16)).view(torch.bfloat16).cuda()
    pl = torch.from_numpy(lses).cuda()
    sk = torch.from_numpy(sinks).cuda()
    out = torch.empty(Tq, Hq, D, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(Hq, Tq, dtype=torch.float32, device="cuda")
    ev = []
    def step(timed):
        if timed:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            B.sink_attn_arm_timing(e0, e1)
            ev.append((e0, e1))
        B.sink_attn_merge(P, Tq, Hq, D, B.BF16, B.BF16, po, pl, sk, out, lse)
    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(args.steps):
        step(True)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    kms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    nbytes = float(P * Tq * Hq * D * 2 + P * Hq * Tq * 4 + Tq * Hq * D * 2 + Hq * Tq * 4 + Hq * 4)
    res = {"metric": "context-parallel merge GB/s (sink-free partials -> sink attention)",
           "value": nbytes / (ms * 1e-3) / 1e9, "unit": "GB/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic",
           "config": {"workload": "cp_merge", "parts": P, "total_q": Tq, "heads_q": Hq,
                      "head_dim": D, "seed": 61},
           "main_kernel_ms": {"merge": kms},
           "roofline": {"bound": "hbm", "kernel": "merge_kernel",
                        "achieved": nbytes / (kms * 1e-3) / 1e9, "peak": PEAK_HBM_GBS,
                        "unit": "GB/s", "frac": nbytes / (kms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                        "traffic": traffic_record("cp_merge", "merge_kernel"),
                        "launch_ms": kms, "bytes_per_launch": nbytes}}
    if not args.no_cpu_baseline:
        rows, t = 0, time.perf_counter()
        while time.perf_counter() - t < min(args.cpu_seconds, 5.0):
            a = rows % Tq
            b = min(Tq, a + 1024)
            O.merge_partials(W.bf16_bits_to_f32(outs[:, a:b]), lses[:, :, a:b], sinks)
            rows += b - a
        dt = time.perf_counter() - t
        res["cpu_baseline"] = {"value": nbytes * rows / Tq / dt / 1e9, "unit": "GB/s",
                               "cores": 1, "kind": "oracle", **host_cores(),
                               "sample": f"{rows} of {Tq} token rows (all heads), {dt:.1f} s"}
    print(json.dumps(res), flush=True)


def run_workload(name, steps, warmup, progress=True):
    """Times `steps` steps of workload `name` after `warmup` untimed ones.
    Returns (result dict, the workload's Problem, training?)."""
    import torch
    from softmax_sink_amd import binding as B
    from softmax_sink_amd import workloads as W

    p = W.config(name)
    train = name in TRAIN
    paged = "paged" in p.meta
    decode = name in ("decode_softmax_n", "decode_paged")
    padded = p.meta.get("layout")          # "BNSD": a batch-padded layout
    D, Hq, Hk = p.head_dim, p.num_heads_q, p.num_heads_k
    if padded:
        lens_q, lens_k = np.diff(p.cu_q), np.diff(p.cu_k)
        seq_q, seq_k = int(lens_q.max()), int(lens_k.max())
        assert (lens_q == seq_q).all() and (lens_k == seq_k).all()
        # device copies in the padded layout; p itself stays packed (the
        # oracle's sample reads it)
        src = dataclasses.replace(p, **{
            t: W.pad_rows(getattr(p, t), cu, seq, padded, 0)
            for t, cu, seq in (("q", p.cu_q, seq_q), ("k", p.cu_k, seq_k),
                                  ("v", p.cu_k, seq_k), ("dout", p.cu_q, seq_q))})
    else:
        src = p
    q = to_dev(src, "q")
    if paged:
        layout = p.meta["paged"]
        kv_desc = B.PagedKV(layout.block_size, layout.block_table.shape[1], layout.num_blocks)
        k = torch.from_numpy(W.scatter_to_pages(p.k, p.cu_k, layout).view(np.int16)).view(
            torch.bfloat16).cuda()
        v = torch.from_numpy(W.scatter_to_pages(p.v, p.cu_k, layout).view(np.int16)).view(
            torch.bfloat16).cuda()
        bt_host = np.ascontiguousarray(layout.block_table, dtype=np.int32)
        used_host = np.ascontiguousarray(layout.seqused, dtype=np.int32)
        bt_dev = torch.from_numpy(bt_host).cuda()
        used_dev = torch.from_numpy(used_host).cuda()
    else:
        k, v = to_dev(src, "k"), to_dev(src, "v")
    dout = to_dev(src, "dout") if train else None
    sinks = torch.from_numpy(p.sinks).cuda()
    scale = float(p.scale)
    dtype_code = B.BF16 if p.dtype == "bf16" else B.FP32
    problem = B.make_problem(p.cu_q, p.cu_k, Hq, Hk, D, p.causal, p.win_left, p.win_right,
                             dtype_code)
    cu_q_dev = torch.from_numpy(p.cu_q).cuda()
    cu_k_dev = torch.from_numpy(p.cu_k).cuda()
    if paged:
        problem = B.make_problem_paged(p.cu_q, used_host, Hq, Hk, D, p.causal, p.win_left,
                                       p.win_right, dtype_code)
        meta0, fws = B.sink_attn_metadata_paged(problem, kv_desc, p.cu_q, used_host, bt_host)
        bws = 0
    elif padded:
        problem = B.make_problem_padded(p.batch, seq_q, seq_k, None, None, Hq, Hk, D,
                                        p.causal, p.win_left, p.win_right, dtype_code,
                                        padded)
        meta0, fws, bws = B.sink_attn_metadata_padded(problem, None, None)
    else:
        meta0, fws, bws = B.sink_attn_metadata(problem, p.cu_q, p.cu_k)
    # two pinned host / device metadata buffers, alternated across steps
    meta_host = [torch.empty(len(meta0), dtype=torch.int32).pin_memory() for _ in range(2)]
    meta_dev = [torch.empty(len(meta0), dtype=torch.int32, device="cuda") for _ in range(2)]
    copied = [None, None]
    out = torch.empty_like(q)
    lse = (torch.empty(p.batch, Hq, seq_q, dtype=torch.float32, device="cuda") if padded
           else torch.empty(Hq, p.total_q, dtype=torch.float32, device="cuda"))
    fwd_ws = torch.empty(max(fws, 1), dtype=torch.uint8, device="cuda")
    if train:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        dsink = torch.empty(Hq, dtype=torch.float32, device="cuda")
        bwd_ws = torch.empty(max(bws, 1), dtype=torch.uint8, device="cuda")
    cq = np.ascontiguousarray(p.cu_q)
    ck = np.ascontiguousarray(p.cu_k)
    main_events = []

    def step(n, timed):
        slot = n & 1
        if copied[slot] is not None:
            copied[slot].synchronize()       # the host buffer is free again
        mh = meta_host[slot].numpy()          # the table is written straight here
        if paged:
            B.sink_attn_metadata_paged(problem, kv_desc, cq, used_host, bt_host, out=mh)
        elif padded:
            B.sink_attn_metadata_padded(problem, None, None, out=mh)
        else:
            B.sink_attn_metadata(problem, cq, ck, out=mh)
        # the table goes to the device with the library's upload kernel on
        # the stream (no DMA-engine copy, and no cross-engine wait, before
        # the attention kernels); a forward-only step copies just the prefix
        # the forward reads
        words = len(mh) if train else B.forward_table_words(mh)
        B.sink_attn_upload_table(meta_host[slot], meta_dev[slot], words)
        ev = torch.cuda.Event()
        ev.record()
        copied[slot] = ev
        if timed:
            s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            B.sink_attn_arm_timing(s0, s1)
        if paged:
            B.sink_attn_fwd_paged(problem, kv_desc, mh, meta_dev[slot], q, k, v, bt_dev,
                                  cu_q_dev, used_dev, sinks, scale, out, lse, fwd_ws, fws)
        elif padded:
            B.sink_attn_fwd_padded(problem, mh, meta_dev[slot], q, k, v, None, None, sinks,
                                   scale, out, lse, fwd_ws, fws)
        else:
            B.sink_attn_fwd(problem, mh, meta_dev[slot], q, k, v, cu_q_dev, cu_k_dev, sinks,
                            scale, out, lse, fwd_ws, fws)
        if timed and not train:
            main_events.append(("fwd", s0, s1))
        if train:
            if timed:
                b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                B.sink_attn_arm_timing(b0, b1)
                main_events.append(("fwd", s0, s1))
            if padded:
                B.sink_attn_bwd_padded(problem, mh, meta_dev[slot], dout, q, k, v, out, lse,
                                       None, None, sinks, scale, dq, dk, dv, dsink, bwd_ws,
                                       bws)
            else:
                B.sink_attn_bwd(problem, mh, meta_dev[slot], dout, q, k, v, out, lse,
                                cu_q_dev, cu_k_dev, sinks, scale, dq, dk, dv, dsink, bwd_ws,
                                bws)
            if timed:
                main_events.append(("bwd", b0, b1))

    for i in range(warmup):
        step(i, False)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(steps):
        step(warmup + i, True)
        if progress:
            print(f"# step {i + 1}/{steps} enqueued", file=sys.stderr, flush=True)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps

    pairs = kept_pairs(p.cu_q, p.cu_k, p.causal, p.win_left, p.win_right) * Hq
    fwd_flops = 4.0 * D * pairs
    bwd_flops = 10.0 * D * pairs
    step_flops = fwd_flops + (bwd_flops if train else 0.0)
    value = step_flops / (ms * 1e-3) / 1e12
    kms = {}
    for ev, a, b in main_events:
        kms.setdefault(ev, []).append(a.elapsed_time(b))
    kavg = {n: float(np.mean(x)) for n, x in kms.items()}
    esize = 2 if p.dtype == "bf16" else 4
    if decode:
        kv_bytes = 2.0 * p.total_k * Hk * D * esize
        qo_bytes = 2.0 * p.total_q * Hq * D * esize + 4.0 * p.total_q * Hq
        alg_bytes = kv_bytes + qo_bytes
        if paged:   # the block-table entries of the pages in use
            alg_bytes += 4.0 * int(((used_host + layout.block_size - 1) // layout.block_size).sum())
        achieved = alg_bytes / (kavg["fwd"] * 1e-3) / 1e9
        roof = {"bound": "hbm", "kernel": "fwd_split_kernel", "achieved": achieved,
                "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS,
                "traffic": traffic_record(name, "fwd_split_kernel"),
                "launch_ms": kavg["fwd"], "bytes_per_launch": alg_bytes}
    else:
        # dominant kernel: the dK/dV loop (S, dP, dV, dK: 8*D per kept pair)
        # for training, the prefill tile loop (QK^T, PV: 4*D) otherwise
        phase = "bwd" if train else "fwd"
        flops = (8.0 * D * pairs) if train else fwd_flops
        kname = "bwd_dkdv_kernel" if train else "fwd_prefill_kernel"
        peak = PEAK_BF16_TFLOPS if p.dtype == "bf16" else PEAK_FP32_TFLOPS
        achieved = flops / (kavg[phase] * 1e-3) / 1e12
        roof = {"bound": "mfma", "kernel": kname, "achieved": achieved, "peak": peak,
                "unit": "TFLOP/s", "frac": achieved / peak,
                "traffic": traffic_record(name, kname),
                "launch_ms": kavg[phase], "flop_per_launch": flops}
    res = {
        "metric": METRIC if train else
        ("sink-attention decode forward TFLOP/s (split-KV" + (", paged K/V)" if paged else ")")
         if decode else "sink-attention forward TFLOP/s" + (" (paged K/V)" if paged else "")),
        "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": steps,
        "warmup": warmup, "ms_per_step": ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": p.dtype, "data": "synthetic",
        "config": {"workload": name, "batch": p.batch, "total_q": p.total_q,
                   "total_k": p.total_k, "heads_q": Hq, "heads_kv": Hk, "head_dim": D,
                   "causal": p.causal, "window": [p.win_left, p.win_right],
                   "seed": p.seed, "kept_pairs": pairs,
                   **({"layout": padded} if padded else {}),
                   "passes": "metadata+fwd+bwd" if train else "metadata+fwd",
                   **({"kv_pages": {"block_size": layout.block_size,
                                    "num_blocks": layout.num_blocks}} if paged else {})},
        "frac_of_bf16_peak": value / PEAK_BF16_TFLOPS,
        "main_kernel_ms": kavg,
        "roofline": roof,
    }
    if decode:
        res["value_gbs"] = alg_bytes / (ms * 1e-3) / 1e9
    return res, p, train


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default: 10 for training workloads, 100 otherwise)")
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed steps first (default: 3 for training workloads, 20 otherwise)")
    ap.add_argument("--workload", default="train_varlen")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="with the default workload, skip timing the other reference "
                         "configurations (prefill_varlen, gqa_window, decode_softmax_n)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="first run a plain device-to-device copy of BYTES bytes "
                         "three times (reference for HBM traffic counters)")
    args = ap.parse_args()
    # A forward-only step takes well under a millisecond: ten of them time a
    # few milliseconds of work, which reads 5-15% slower than a longer run.
    if args.steps is None:
        args.steps = 10 if args.workload in TRAIN else 100
    if args.warmup is None:
        args.warmup = 3 if args.workload in TRAIN else 20
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus})", file=sys.stderr)
        sys.exit(2)

    import torch
    from softmax_sink_amd import binding as B
    from softmax_sink_amd import workloads as W

    torch.cuda.set_device(0)
    if args.calibrate_copy:
        src = torch.empty(args.calibrate_copy, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.workload == "cp_merge":
        bench_merge(args)
        return
    res, p, train = run_workload(args.workload, args.steps, args.warmup)
    if args.workload == "train_varlen" and not args.no_configs:
        res["configs"] = other_configs()
    if not args.no_cpu_baseline:
        print("# timing the oracle on the host", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(p, train, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
