#!/usr/bin/env python
"""Benchmark of the Parallax attention hot path on one MI355X.

Default (--workload metric): the headline is large-batch decode, bf16,
B=2048, Hq=16, Hkv=8, D=128, 2048 cached keys per sequence (17.2 GB of K/V),
q/r/K/V ~ N(0,1)/sqrt(128), seeded: the largest single-GPU decode
configuration of the metric. A step is one parallax_decode call over the
batch. Inputs are resident in HBM before timing; a cache smaller than four
times the 256 MB Infinity Cache is replicated into enough copies that
consecutive steps never find their keys there, and steps rotate through the
copies. The warmup steps and the timed steps are captured into HIP graphs and
replayed; the timed steps run as ten equal replays, each between HIP events
on the replay stream, bracketed by device synchronisation: value is the mean
over all timed steps, us_per_step the q05 / q50 / q95 over the replays.

Also measured in the same run, for each workload:
  * the dominant streaming kernel against the HBM roofline (8 TB/s), from
    algorithmic bytes K + V + q + r (+ o when the kernel writes o itself);
  * softmax_decode on the same inputs (the cost of the correction branch);
  * the CPU oracle on the same inputs (cpu_baseline: bounded sample, every core).
The default line carries sub-records for the tiny fp32 decode and the
long-context decode (each with the oracle's full step on one thread and on
every core), the varlen decode batch and the causal prefill (TFLOP/s against
the bf16 dense MFMA peak), these two with the oracle on a bounded sample.

Other workloads (--workload tiny | long | varlen | large | prefill | backward |
grid | prefill-varlen) print their own line; prefill-varlen times the packed
forward and backward of 16 sequences of U{256..4096} tokens; backward times parallax_prefill_backward (row pass + key
pass) on the causal-prefill shapes; grid runs the pages' own decode shapes
(multi-head H = 8, B in {1, 32}, L in {512 .. 16384}) and reports a table, each
row also timed with the Infinity Cache defeated.
Prints one JSON line on stdout.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "Parallax decode µs/step + achieved HBM TB/s vs roofline; prefill TFLOP/s"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
MALL_BYTES = 256 << 20


def parse():
    ap = argparse.ArgumentParser(description=__doc__,
                                 formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="metric",
                    choices=["metric", "tiny", "long", "varlen", "large", "prefill", "backward",
                             "grid", "prefill-varlen"])
    ap.add_argument("--num-splits", type=int, default=0, help="0: library plan")
    ap.add_argument("--window", type=int, default=0,
                    help="sliding window (keys a query sees); 0: none")
    ap.add_argument("--block-density", type=float, default=0.0,
                    help="> 0: a seeded block-sparse mask (128-position blocks, one per "
                         "sequence and KV head) with this fraction of blocks visible (decode, "
                         "prefill and backward workloads; no window)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target wall time of the CPU oracle sample")
    ap.add_argument("--cpu-seconds-one", type=float, default=3.0,
                    help="target wall time of each oracle figure of the sub-records in the "
                         "default run (one-thread and all-core full steps of the small decodes, "
                         "bounded samples of the varlen decode and the prefill)")
    ap.add_argument("--eager", action="store_true",
                    help="launch steps one by one instead of replaying a HIP graph (for profilers)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain copy kernel of known size (HBM counter calibration)")
    return ap.parse_args()


def upload_cache(torch, spec, synth, tid, tokens, chunk=1 << 16):
    row = spec.Hkv * spec.D
    out = torch.empty((tokens, spec.Hkv, spec.D), dtype=torch.bfloat16, device="cuda")
    host = torch.empty((chunk, spec.Hkv, spec.D), dtype=torch.bfloat16, pin_memory=True)
    hv = host.view(torch.int16).numpy().view(np.uint16)
    t0 = 0
    while t0 < tokens:
        n = min(chunk, tokens - t0)
        synth.normal(spec.seed, tid, (n, spec.Hkv, spec.D), spec.scale, spec.dtype,
                     first=t0 * row, out=hv[:n])
        out[t0:t0 + n].copy_(host[:n])
        t0 += n
    torch.cuda.synchronize()
    return out


EAGER = False


def visible_pairs(L, W):
    """(query, key) pairs a causal prefill of length L sees with window W (0: none)."""
    if W <= 0 or W >= L:
        return L * (L + 1) // 2
    return W * (W + 1) // 2 + (L - W) * W


MASK_SEED = 4242
MASK_BLOCK = 128


def prefill_mask(synth, B, Hkv, L, density):
    """The seeded prefill block mask [B, Hkv, nb, nb], or None."""
    if density <= 0:
        return None
    nb = -(-L // MASK_BLOCK)
    return synth.block_mask(MASK_SEED, (B, Hkv, nb, nb), density)


def masked_pairs(m, L):
    """Visible (query, key) pairs of one query head per (sequence, KV head), summed:
    causal pairs inside each diagonal block, whole 128 x 128 blocks below it where
    the mask shows them."""
    nb = m.shape[-1]
    total = 0
    for qb in range(nb):
        rows = min(L, (qb + 1) * MASK_BLOCK) - qb * MASK_BLOCK
        diag = rows * (rows + 1) // 2
        below = int(m[:, :, qb, :qb].sum()) * rows * MASK_BLOCK
        total += diag * m.shape[0] * m.shape[1] + below
    return total


def timed_steps(torch, fn, steps, warmup, trials=10):
    """Exactly `steps` timed calls of fn(i), after `warmup` untimed ones.

    Graph mode (default): the warmup calls are captured into one graph and the
    timed calls into graphs of n = steps // trials calls (plus one graph of the
    remainder). After the warmup replay, each timed replay runs between HIP
    events recorded on the replay stream; the timed region is bracketed by
    device synchronisation. Returns seconds per step: the mean over all timed
    steps, and q05 / q50 / q95 over the equal-size replays (the pages' replay
    sweep reports q50 with q05 / q95). With --eager every call is launched and
    timed on its own."""
    stream = torch.cuda.Stream()
    trials = max(1, min(trials, steps))
    if EAGER:
        with torch.cuda.stream(stream):
            for i in range(warmup):
                fn(i)
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
        with torch.cuda.stream(stream):
            for i, (e0, e1) in enumerate(ev):
                e0.record(stream)
                fn(warmup + i)
                e1.record(stream)
        torch.cuda.synchronize()
        per = np.array([e0.elapsed_time(e1) * 1e-3 for e0, e1 in ev])
        q = np.quantile(per, [0.05, 0.5, 0.95])
        return {"mean": float(per.mean()), "q05": q[0], "q50": q[1], "q95": q[2]}
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        for i in range(2):  # eager warm calls before capture
            fn(i)
    torch.cuda.synchronize()
    n = steps // trials
    rem = steps - n * trials
    gw = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gw, stream=stream):
        for i in range(max(warmup, 1)):
            fn(i)
    gs = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gs, stream=stream):
        for i in range(n):
            fn(i)
    gr = None
    if rem:
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr, stream=stream):
            for i in range(rem):
                fn(n + i)
    torch.cuda.synchronize()
    if warmup > 0:
        gw.replay()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(trials + (1 if rem else 0))]
    with torch.cuda.stream(stream):
        for t in range(trials):
            ev[t][0].record(stream)
            gs.replay()
            ev[t][1].record(stream)
        if rem:
            ev[-1][0].record(stream)
            gr.replay()
            ev[-1][1].record(stream)
    torch.cuda.synchronize()
    per = np.array([ev[t][0].elapsed_time(ev[t][1]) * 1e-3 / n for t in range(trials)])
    total = per.sum() * n + (ev[-1][0].elapsed_time(ev[-1][1]) * 1e-3 if rem else 0.0)
    q = np.quantile(per, [0.05, 0.5, 0.95])
    return {"mean": float(total / steps), "q05": q[0], "q50": q[1], "q95": q[2]}


def graph_time(torch, fn, steps, warmup):
    """Mean seconds per step of timed_steps."""
    return timed_steps(torch, fn, steps, warmup)["mean"]


def us_quantiles(t):
    return {"q05": round(t["q05"] * 1e6, 3), "q50": round(t["q50"] * 1e6, 3),
            "q95": round(t["q95"] * 1e6, 3)}


def measured_traffic(workload):
    """HBM bytes per launch of the roofline kernel from the committed counter
    summaries (profiles/*_hbm_traffic.json), or None when none covers this
    workload (for decode: the workload name and its split plan), or when the
    kernel sources changed since the counters were taken."""
    import glob
    import hashlib
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*_hbm_traffic.json"))):
        with open(path) as f:
            rec = json.load(f)
        if rec["workload"] != workload:
            continue
        h = hashlib.sha256()
        for src in rec["sources"]:
            with open(os.path.join(ROOT, src), "rb") as f:
                h.update(f.read())
        return rec["traffic_bytes_per_launch"] if h.hexdigest() == rec["source_sha256"] else None
    return None


# Elements whose reference magnitude is below this fraction of the row's largest are left
# out of the per-element relative error (an elementwise ratio is unbounded where the
# reference crosses zero).
REL_FLOOR = 1e-2


def elementwise_rel_err(o, ref):
    """Worst per-element relative error |o - ref| / |ref| over the elements with
    |ref| >= REL_FLOOR x the largest |ref| of their row (last axis): the pages'
    accuracy figure, beside the max-norm error used for the parity bar."""
    o, ref = np.asarray(o, dtype=np.float64), np.asarray(ref, dtype=np.float64)
    big = np.abs(ref) >= REL_FLOOR * np.abs(ref).max(axis=-1, keepdims=True)
    return float((np.abs(o - ref)[big] / np.abs(ref)[big]).max())


def omp_threads():
    env = os.environ.get("OMP_NUM_THREADS")
    n = len(os.sched_getaffinity(0))
    if env and env.isdigit():
        return min(int(env), n)
    return n


def upload_any(torch, spec, synth, tid, tokens):
    if spec.dtype == synth.BF16:
        return upload_cache(torch, spec, synth, tid, tokens)
    a = synth.normal(spec.seed, tid, (tokens, spec.Hkv, spec.D), spec.scale, spec.dtype)
    return torch.from_numpy(a).cuda()


def to_device(torch, a, synth, dtype):
    t = torch.from_numpy(np.ascontiguousarray(a))
    return (t.view(torch.bfloat16) if dtype == synth.BF16 else t).cuda()


def decode_record(args, torch, plx, synth, oracle, idx, steps, warmup, cpu="cores", cpu_seconds=None):
    """One decode workload (idx 1..4: tiny fp32, long-context, varlen batch,
    large batch), timed as a step of parallax_decode over the batch. cpu:
    "cores" (the oracle on a bounded sample with every core, for cpu_seconds,
    default --cpu-seconds), "one" (the oracle's full step on one thread), "none"."""
    if cpu_seconds is None:
        cpu_seconds = args.cpu_seconds
    spec = synth.decode_spec(idx)
    lens = spec.seq_lengths()
    T = int(lens.sum())
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    q_np, r_np = synth.decode_qr(spec)
    q = to_device(torch, q_np, synth, spec.dtype)
    r = to_device(torch, r_np, synth, spec.dtype)
    k0 = upload_any(torch, spec, synth, synth.TID_K, T)
    v0 = upload_any(torch, spec, synth, synth.TID_V, T)
    esize = k0.element_size()
    kv_bytes = 2 * k0.numel() * esize
    copies = max(1, min(4, math.ceil(3 * MALL_BYTES / kv_bytes) + 1)) if kv_bytes < 4 * MALL_BYTES \
        else 1
    ks = [k0] + [k0.clone() for _ in range(copies - 1)]
    vs = [v0] + [v0.clone() for _ in range(copies - 1)]
    varlen = spec.varlen is not None
    cu_t = torch.from_numpy(cu.astype(np.int32)).cuda() if varlen else None
    if not varlen:
        ks = [k.view(spec.B, spec.L, spec.Hkv, spec.D) for k in ks]
        vs = [v.view(spec.B, spec.L, spec.Hkv, spec.D) for v in vs]
    code = plx.PLX_BF16 if spec.dtype == synth.BF16 else plx.PLX_F32
    ns = args.num_splits
    W = args.window
    splits = plx.decode_num_splits(spec.B, spec.Hq, spec.Hkv, spec.D, spec.L, code, ns, W)
    ws_bytes = plx.decode_workspace_bytes(spec.B, spec.Hq, spec.Hkv, spec.D, spec.L, code, ns, W)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
    out = torch.empty((spec.B, spec.Hq, spec.D), dtype=q.dtype, device="cuda")
    out_s = torch.empty_like(out)
    recs = torch.empty((spec.B, spec.Hq, splits, 2 * spec.D + 4), dtype=torch.float32,
                       device="cuda")
    mask = None
    if args.block_density > 0:
        assert W == 0, "block masks are benchmarked without a window"
        mask = synth.block_mask(MASK_SEED, (spec.B, spec.Hkv, -(-spec.L // MASK_BLOCK)),
                                args.block_density)
    kw = dict(cu_seqlens_k=cu_t, kv_len=spec.L, num_splits=ns, window=W,
              block_mask=None if mask is None else torch.from_numpy(mask).cuda())

    def step(i):
        c = i % copies
        plx.decode(q, r, ks[c], vs[c], out=out, workspace=ws, **kw)

    def step_softmax(i):
        c = i % copies
        plx.softmax_decode(q, ks[c], vs[c], out=out_s, workspace=ws, **kw)

    def step_stream_only(i):
        c = i % copies
        plx.decode_partial(q, r, ks[c], vs[c], records=recs, **kw)

    tt = timed_steps(torch, step, steps, warmup)
    t_step = tt["mean"]
    t_soft = timed_steps(torch, step_softmax, steps, warmup)
    # The roofline kernel: with one split per sequence the step is a single fused
    # streaming kernel; a packed cache with the automatic plan runs the stream-K
    # kernel, which has no streaming-only entry point (its roofline is taken over
    # the whole step); otherwise the streaming kernel is timed alone through
    # parallax_decode_partial (the same kernel and plan, records instead of o).
    mfma = code == plx.PLX_BF16 and spec.D == 128
    stream_k = varlen and ns == 0 and W == 0 and mfma and spec.Hq // spec.Hkv <= 8
    fused = splits == 1 and not stream_k
    if stream_k or fused:
        t_kern = t_step
    else:
        t_kern = timed_steps(torch, step_stream_only, steps, warmup)["mean"]
    kname = ("decode_mfma_streamk + decode_reduce (whole step)" if stream_k else
             ("decode_mfma_bf16_d128" if mfma else "decode_generic")
             + (" (fused: one split, o written directly)" if fused else
                " (streaming, split records)"))

    # algorithmic bytes: K + V over the visible keys, plus q, r and o
    T_vis = int(np.minimum(lens, W).sum()) if W > 0 else T
    kv_vis = kv_bytes * T_vis // T
    if mask is not None:
        # per (sequence, KV head): the visible blocks' keys (the last key's block always)
        head_keys = 0
        for b in range(spec.B):
            n = int(lens[b])
            if n == 0:
                continue
            nb_b = -(-n // MASK_BLOCK)
            last = n - (nb_b - 1) * MASK_BLOCK
            head_keys += spec.Hkv * last + int(mask[b, :, :nb_b - 1].sum()) * MASK_BLOCK
        T_vis = head_keys / spec.Hkv  # key rows of all heads, in units of tokens
        kv_vis = int(head_keys * 2 * spec.D * esize)
    qr_bytes = 2 * q.numel() * esize
    o_bytes = out.numel() * esize
    step_bytes = kv_vis + qr_bytes + o_bytes
    kern_bytes = kv_vis + qr_bytes + (o_bytes if (stream_k or fused) else 0)
    flops = 8 * spec.D * spec.Hq * T_vis
    res = {
        "metric": METRIC,
        "value": round(t_step * 1e6, 3),
        "unit": "us/step",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(t_step * 1e3, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if spec.dtype == synth.BF16 else "f32",
        "data": "synthetic",
        "config": {"workload": spec.name + (f" window{W}" if W > 0 else "")
                   + (f" block-density{args.block_density}" if mask is not None else ""),
                   "B": spec.B, "Hq": spec.Hq, "Hkv": spec.Hkv, "head_dim": spec.D,
                   "kv_len": spec.L, "total_kv_tokens": T, "visible_kv_tokens": T_vis,
                   "window": W, "block_density": args.block_density,
                   "kv_cache_copies": copies, "splits": splits},
        "us_per_step": us_quantiles(tt),
        "hbm_tb_s": round(step_bytes / t_step / 1e12, 4),
        "hbm_frac_of_8tbs": round(step_bytes / t_step / 1e9 / HBM_PEAK_GBS, 4),
        "tflops": round(flops / t_step / 1e12, 3),
        "softmax_decode_us": round(t_soft["mean"] * 1e6, 3),
        "softmax_decode_us_q50": round(t_soft["q50"] * 1e6, 3),
        "parallax_over_softmax": round(t_step / t_soft["mean"], 4),
        "roofline": {"bound": "hbm", "kernel": kname,
                     "achieved": round(kern_bytes / t_kern / 1e9, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(kern_bytes / t_kern / 1e9 / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(f"{spec.name}, {splits} splits")
                     if W == 0 and mask is None else None,
                     "avg_us": round(t_kern * 1e6, 3),
                     "bytes_per_launch": kern_bytes},
    }
    if idx == 1:  # 256 keys: latency-bound, no roofline claim
        res["roofline"]["bound"] = "latency"
    if cpu == "cores" and mask is None:
        oracle.set_num_threads(omp_threads())
        if varlen or spec.B > 64:
            # bounded sample: the first sequences, regenerated from the same streams
            nb = 4 if spec.B > 64 else 8
            sub = slice(0, nb)
            toks = int(cu[nb])
            k_h = synth.decode_kv_rows(spec, synth.TID_K, 0, toks)
            v_h = synth.decode_kv_rows(spec, synth.TID_V, 0, toks)
            qs, rs = np.ascontiguousarray(q_np[sub]), np.ascontiguousarray(r_np[sub])
            t = time.perf_counter()
            reps = 0
            while True:
                oracle.decode(qs, rs, k_h, v_h, seq_start=cu[:nb], seq_len=lens[:nb], window=W)
                reps += 1
                if time.perf_counter() - t > cpu_seconds:
                    break
            per_seq = (time.perf_counter() - t) / reps / nb
            # scale by tokens: the oracle's cost is linear in the visible keys
            toks_vis = int(np.minimum(lens[:nb], W).sum()) if W > 0 else toks
            us = per_seq * nb / toks_vis * T_vis * 1e6
            sample = f"{nb} of {spec.B} sequences ({toks_vis} of {T_vis} visible keys), " \
                     f"{reps} repeats, scaled to the full step by key count"
            threads = min(omp_threads(), nb * spec.Hq)
        else:
            k_h, v_h = dense_kv_host(synth, spec, T)
            us, reps = time_oracle_decode(oracle, q_np, r_np, k_h, v_h, cpu_seconds, W)
            sample = f"the full step (all {spec.Hq} heads x {T_vis} keys), {reps} repeats"
            threads = min(omp_threads(), spec.B * spec.Hq)
        res["cpu_baseline"] = {"value": round(us, 1), "unit": "us/step", "cores": threads,
                               "kind": "oracle", "sample": sample}
    elif cpu == "one" and mask is None and not varlen:
        # the full step on one core (per-core figure), and on every core
        k_h, v_h = dense_kv_host(synth, spec, T)
        oracle.set_num_threads(1)
        us1, reps1 = time_oracle_decode(oracle, q_np, r_np, k_h, v_h, args.cpu_seconds_one, W)
        oracle.set_num_threads(omp_threads())
        usn, repsn = time_oracle_decode(oracle, q_np, r_np, k_h, v_h, args.cpu_seconds_one, W)
        res["cpu_oracle_1thread"] = {"value": round(us1, 2), "unit": "us/step", "cores": 1,
                                     "kind": "oracle", "sample": f"the full step, {reps1} repeats"}
        res["cpu_oracle_all_cores"] = {"value": round(usn, 2), "unit": "us/step",
                                       "cores": min(omp_threads(), spec.B * spec.Hq),
                                       "kind": "oracle", "sample": f"the full step, {repsn} repeats"}
    # parity of the timed configuration on a few rows (the full check lives in the tests)
    o_full = out.float().cpu().numpy().astype(np.float64)
    rows = [(0, 0), (spec.B - 1, spec.Hq - 1), (spec.B // 2, min(3, spec.Hq - 1))]
    errs, rel = [], []
    for b, h in rows:
        toks = int(lens[b])
        k_h = synth.decode_kv_rows(spec, synth.TID_K, int(cu[b]), toks)[None]
        v_h = synth.decode_kv_rows(spec, synth.TID_V, int(cu[b]), toks)[None]
        ref = oracle.decode(np.ascontiguousarray(q_np[b:b + 1]), np.ascontiguousarray(r_np[b:b + 1]),
                            k_h, v_h, window=W,
                            block_mask=None if mask is None else mask[b:b + 1, :,
                                                                      :-(-toks // MASK_BLOCK)])[0, h]
        errs.append(float(np.abs(o_full[b, h] - ref).max() / np.abs(ref).max()))
        rel.append(elementwise_rel_err(o_full[b, h], ref))
    res["sampled_parity_max_norm_err"] = max(errs)
    res["sampled_elementwise_rel_err"] = max(rel)
    del ks, vs, k0, v0
    torch.cuda.empty_cache()
    return res


def dense_kv_host(synth, spec, T):
    k_h = synth.decode_kv_rows(spec, synth.TID_K, 0, T).reshape(spec.B, spec.L, spec.Hkv, spec.D)
    v_h = synth.decode_kv_rows(spec, synth.TID_V, 0, T).reshape(spec.B, spec.L, spec.Hkv, spec.D)
    return k_h, v_h


def time_oracle_decode(oracle, q, r, k, v, seconds, window=0):
    """The oracle's full decode step, repeated to fill about `seconds` of wall
    time. Returns (us_per_step, repeats)."""
    t = time.perf_counter()
    oracle.decode(q, r, k, v, window=window)
    one = time.perf_counter() - t
    reps = max(1, int(seconds / max(one, 1e-6)))
    t = time.perf_counter()
    for _ in range(reps):
        oracle.decode(q, r, k, v, window=window)
    return (time.perf_counter() - t) / reps * 1e6, reps + 1


def run_decode_workload(args, torch, plx, synth, oracle):
    idx = {"tiny": 1, "long": 2, "varlen": 3, "large": 4}[args.workload]
    return decode_record(args, torch, plx, synth, oracle, idx, args.steps, args.warmup,
                         "none" if args.no_cpu_baseline else "cores")


SUB_KEYS = ("value", "unit", "steps", "warmup", "ms_per_step", "dtype", "config", "us_per_step",
            "hbm_tb_s", "hbm_frac_of_8tbs", "tflops", "tflops_q50", "softmax_decode_us",
            "softmax_decode_us_q50", "parallax_over_softmax", "roofline", "cpu_baseline",
            "cpu_oracle_1thread", "cpu_oracle_all_cores", "sampled_parity_max_norm_err",
            "sampled_elementwise_rel_err")


def run_metric_workload(args, torch, plx, synth, oracle):
    """The default line. The metric's decode half is headlined on the largest
    single-GPU decode configuration (large-batch decode, B = 2048, 2048 keys
    each: 17.2 GB of K/V per step), with its roofline and the oracle's CPU
    baseline; the other configurations ride along as sub-records, each with
    its own timing (q05 / q50 / q95 over graph replays) and roofline fraction:
    tiny fp32 decode and long-context decode (with one-thread and all-core
    oracle figures of the full step), the varlen batch and the causal prefill
    (the metric's TFLOP/s half, against the bf16 dense MFMA peak), these two
    with the oracle timed on a bounded sample."""
    cpu = "none" if args.no_cpu_baseline else "cores"
    one = "none" if args.no_cpu_baseline else "one"
    head = decode_record(args, torch, plx, synth, oracle, 4, args.steps, args.warmup, cpu)
    subs = []
    for idx, mode in ((1, one), (2, one), (3, cpu)):
        rec = decode_record(args, torch, plx, synth, oracle, idx, 200, 20, mode,
                            cpu_seconds=args.cpu_seconds_one)
        subs.append({k: rec[k] for k in SUB_KEYS if k in rec})
    rec = prefill_record(args, torch, plx, synth, oracle, 100, COMPUTE_WARMUP, cpu == "cores",
                         cpu_seconds=args.cpu_seconds_one)
    subs.append({k: rec[k] for k in SUB_KEYS if k in rec})
    head["configs"] = subs
    return head


# The compute-bound kernels (prefill, backward) run about 20% slower for the first
# ~30 ms of sustained load on this part (measured: prefill replays ramp from 910 to a
# steady ~1140 TFLOP/s over the first 25 launches; the memory-bound decode steps
# do not ramp). Their lines therefore warm up for at least 100 steps, as the pages'
# replay protocol does, before the timed steps.
COMPUTE_WARMUP = 100


def run_prefill_workload(args, torch, plx, synth, oracle):
    return prefill_record(args, torch, plx, synth, oracle, max(1, min(args.steps, 100)),
                          max(args.warmup, COMPUTE_WARMUP), not args.no_cpu_baseline)


def prefill_record(args, torch, plx, synth, oracle, steps, warm, cpu, cpu_seconds=None):
    if cpu_seconds is None:
        cpu_seconds = args.cpu_seconds
    spec = synth.prefill_spec(5)
    B, Hq, Hkv, L, D = spec.B, spec.Hq, spec.Hkv, spec.L, spec.D
    arrs = {}
    for name, tid, H in (("q", synth.TID_Q, Hq), ("r", synth.TID_R, Hq), ("k", synth.TID_K, Hkv),
                         ("v", synth.TID_V, Hkv)):
        a = synth.normal(spec.seed, tid, (B, H, L, D), spec.scale, spec.dtype)
        arrs[name] = a
    t = {n: torch.from_numpy(a).view(torch.bfloat16).cuda() for n, a in arrs.items()}
    out = torch.empty_like(t["q"])

    W = args.window
    mask = prefill_mask(synth, B, Hkv, L, args.block_density)
    assert mask is None or W == 0, "block masks are benchmarked without a window"
    mask_t = None if mask is None else torch.from_numpy(mask).cuda()

    def step(i):
        plx.prefill(t["q"], t["r"], t["k"], t["v"], out=out, window=W, block_mask=mask_t)

    tt = timed_steps(torch, step, steps, warm)
    ts = tt["mean"]
    pairs = B * visible_pairs(L, W) if mask is None else masked_pairs(mask, L)
    flops = 8 * D * Hq * pairs if mask is None else 8 * D * (Hq // Hkv) * pairs
    res = {
        "metric": METRIC, "value": round(flops / ts / 1e12, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": steps, "warmup": warm, "ms_per_step": round(ts * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": spec.name + (f" window{W}" if W > 0 else "")
                   + (f" block-density{args.block_density}" if mask is not None else ""),
                   "B": B, "Hq": Hq, "Hkv": Hkv, "L": L, "head_dim": D, "window": W,
                   "block_density": args.block_density},
        "roofline": {"bound": "mfma", "kernel": "prefill", "achieved": round(flops / ts / 1e12, 2),
                     "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(flops / ts / 1e12 / BF16_PEAK_TFLOPS, 4),
                     "traffic": measured_traffic(spec.name) if W == 0 and mask is None else None,
                     "avg_us": round(ts * 1e6, 1), "flops_per_launch": flops},
        "us_per_step": us_quantiles(tt),
        "tflops_q50": round(flops / tt["q50"] / 1e12, 2),
    }
    rows = np.array([[0, 0, 0], [B - 1, Hq - 1, L - 1], [3, 5, 1000], [7, 8, 2047]])
    o = out.float().cpu().numpy()
    ref = oracle.prefill(arrs["q"], arrs["r"], arrs["k"], arrs["v"], rows=rows, window=W,
                         block_mask=mask)
    got = o[rows[:, 0], rows[:, 1], rows[:, 2]]
    res["sampled_parity_max_norm_err"] = float(
        (np.abs(got - ref).max(axis=1) / np.abs(ref).max(axis=1)).max())  # worst row
    res["sampled_elementwise_rel_err"] = elementwise_rel_err(got, ref)
    if cpu and mask is None:
        # bounded sample: rows spread over the causal range, scaled by visible keys
        oracle.set_num_threads(omp_threads())
        g = np.random.default_rng(0)
        n = 512
        sample_rows = np.stack([g.integers(0, B, n), g.integers(0, Hq, n),
                                g.integers(0, L, n)], axis=1)
        tt = time.perf_counter()
        reps = 0
        while True:
            oracle.prefill(arrs["q"], arrs["r"], arrs["k"], arrs["v"], rows=sample_rows, window=W)
            reps += 1
            if time.perf_counter() - tt > cpu_seconds:
                break
        per = (time.perf_counter() - tt) / reps
        vis = sample_rows[:, 2] + 1
        keys_sample = float((np.minimum(vis, W) if W > 0 else vis).sum())
        keys_full = B * Hq * visible_pairs(L, W)
        sec_full = per * keys_full / keys_sample
        res["cpu_baseline"] = {"value": round(flops / sec_full / 1e12, 6), "unit": "TFLOP/s",
                               "cores": min(omp_threads(), n), "kind": "oracle",
                               "sample": f"{n} random query rows, {reps} repeats, scaled to the "
                                         f"full step by visible keys ({sec_full:.0f} s/step)"}
    return res


def run_backward_workload(args, torch, plx, synth, oracle):
    spec = synth.prefill_spec(5)
    B, Hq, Hkv, L, D = spec.B, spec.Hq, spec.Hkv, spec.L, spec.D
    arrs = {}
    for name, tid, H, sc in (("q", synth.TID_Q, Hq, spec.scale), ("r", synth.TID_R, Hq, spec.scale),
                             ("k", synth.TID_K, Hkv, spec.scale), ("v", synth.TID_V, Hkv, spec.scale),
                             ("do", synth.TID_DO, Hq, 1.0)):
        arrs[name] = synth.normal(spec.seed, tid, (B, H, L, D), sc, spec.dtype)
    t = {n: torch.from_numpy(a).view(torch.bfloat16).cuda() for n, a in arrs.items()}
    W = args.window
    mask = prefill_mask(synth, B, Hkv, L, args.block_density)
    assert mask is None or W == 0, "block masks are benchmarked without a window"
    mask_t = None if mask is None else torch.from_numpy(mask).cuda()
    # the forward stores the softmax readout, as the autograd entry point does
    vbar = torch.empty_like(t["q"])
    o, lse, sbar = plx.prefill(t["q"], t["r"], t["k"], t["v"], return_stats=True, window=W,
                               vbar_out=vbar, block_mask=mask_t)
    grads = (torch.empty_like(t["q"]), torch.empty_like(t["r"]), torch.empty_like(t["k"]),
             torch.empty_like(t["v"]))
    ws = torch.empty(int(plx.lib().parallax_prefill_backward_workspace_bytes(B, Hq, L)),
                     dtype=torch.uint8, device="cuda")

    def step(i):
        plx.prefill_backward(t["q"], t["r"], t["k"], t["v"], o, t["do"], lse, sbar,
                             workspace=ws, out=grads, window=W, vbar=vbar, block_mask=mask_t)

    steps = max(1, min(args.steps, 40))
    warm = max(args.warmup, COMPUTE_WARMUP // 3)  # a backward step is three forward steps long
    tt = timed_steps(torch, step, steps, warm)
    ts = tt["mean"]
    # algorithmic: 8 contractions of 2D flops per visible (query, key) pair and query head --
    # recompute Z, S, U; dV; dQ, dR; dK from dZ and dS
    pairs = B * visible_pairs(L, W) if mask is None else masked_pairs(mask, L)
    flops = 16 * D * Hq * pairs if mask is None else 16 * D * (Hq // Hkv) * pairs
    res = {
        "metric": METRIC, "value": round(flops / ts / 1e12, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": steps, "warmup": warm, "ms_per_step": round(ts * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "causal-prefill-backward-bf16 B8 L4096 Hq16 Hkv8 D128"
                               + (f" window{W}" if W > 0 else "")
                               + (f" block-density{args.block_density}" if mask is not None
                                  else ""), "B": B, "Hq": Hq, "Hkv": Hkv,
                   "L": L, "head_dim": D, "window": W, "block_density": args.block_density},
        "roofline": {"bound": "mfma", "kernel": "prefill_backward (row pass + key pass)",
                     "achieved": round(flops / ts / 1e12, 2), "peak": BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(flops / ts / 1e12 / BF16_PEAK_TFLOPS, 4),
                     "traffic": None, "avg_us": round(ts * 1e6, 1), "flops_per_launch": flops,
                     "executed_flops_per_launch": flops * 11 // 8},
        "us_per_step": us_quantiles(tt),
    }
    # parity and CPU baseline: the oracle's complete gradients of one (sequence, KV head) unit
    units = np.array([[0, 0]])
    G = Hq // Hkv
    tt = time.perf_counter()
    reps = 0
    while True:
        ref = oracle.prefill_backward(arrs["q"], arrs["r"], arrs["k"], arrs["v"], arrs["do"],
                                      units=units, window=W, block_mask=mask)
        reps += 1
        if args.no_cpu_baseline or time.perf_counter() - tt > args.cpu_seconds:
            break
    per = (time.perf_counter() - tt) / reps
    got = [grads[0][0, :G], grads[1][0, :G], grads[2][0, 0], grads[3][0, 0]]
    errs = {}
    for name, a, b in zip(("dq", "dr", "dk", "dv"), got, ref):
        a = a.float().cpu().numpy()
        errs[name] = float(np.abs(a - b[0]).max() / np.abs(b[0]).max())
    res["sampled_parity_max_norm_err"] = errs
    if not args.no_cpu_baseline and mask is None:
        sec_full = per * B * Hkv
        res["cpu_baseline"] = {"value": round(flops / sec_full / 1e12, 6), "unit": "TFLOP/s",
                               "cores": omp_threads(), "kind": "oracle",
                               "sample": f"complete gradients of 1 of {B * Hkv} (sequence, KV "
                                         f"head) units, {reps} repeats, scaled by {B * Hkv} "
                                         f"({sec_full:.0f} s/step)"}
    return res


def run_prefill_varlen_workload(args, torch, plx, synth, oracle):
    spec = synth.prefill_varlen_spec()
    lens = spec.lengths
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    T, Hq, Hkv, D, W = int(cu[-1]), spec.Hq, spec.Hkv, spec.D, args.window
    arrs = {}
    for name, tid, H, sc in (("q", synth.TID_Q, Hq, spec.scale), ("r", synth.TID_R, Hq, spec.scale),
                             ("k", synth.TID_K, Hkv, spec.scale), ("v", synth.TID_V, Hkv, spec.scale),
                             ("do", synth.TID_DO, Hq, 1.0)):
        arrs[name] = synth.normal(spec.seed, tid, (T, H, D), sc, spec.dtype)
    t = {n: torch.from_numpy(a).view(torch.bfloat16).cuda() for n, a in arrs.items()}
    cu_t = torch.from_numpy(cu.astype(np.int32)).cuda()
    max_len = int(lens.max())
    out = torch.empty_like(t["q"])
    lse = torch.empty((T, Hq), dtype=torch.float32, device="cuda")
    sbar = torch.empty_like(lse)
    grads = (torch.empty_like(t["q"]), torch.empty_like(t["r"]), torch.empty_like(t["k"]),
             torch.empty_like(t["v"]))
    ws = torch.empty(int(plx.lib().parallax_prefill_varlen_workspace_bytes(Hq, T, 1)),
                     dtype=torch.uint8, device="cuda")
    ws_f = torch.empty(int(plx.lib().parallax_prefill_varlen_workspace_bytes(Hq, T, 0)),
                       dtype=torch.uint8, device="cuda")

    def fwd(i):
        plx.prefill_varlen(t["q"], t["r"], t["k"], t["v"], cu_t, max_len, out=out, window=W,
                           workspace=ws_f)

    vbar = torch.empty_like(t["q"])
    o, lse, sbar = plx.prefill_varlen(t["q"], t["r"], t["k"], t["v"], cu_t, max_len,
                                      return_stats=True, window=W, vbar_out=vbar)

    def bwd(i):
        plx.prefill_varlen_backward(t["q"], t["r"], t["k"], t["v"], o, t["do"], lse, sbar, cu_t,
                                    max_len, window=W, workspace=ws, out=grads, vbar=vbar)

    steps = max(1, min(args.steps, 40))
    warm = max(args.warmup, COMPUTE_WARMUP)
    tf = graph_time(torch, fwd, steps, warm)
    tb = graph_time(torch, bwd, steps, warm // 3)
    pairs = sum(visible_pairs(int(n), W) for n in lens)
    flops = 8 * D * Hq * pairs
    res = {
        "metric": METRIC, "value": round(flops / tf / 1e12, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": steps, "warmup": warm, "ms_per_step": round(tf * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": spec.name + (f" window{W}" if W > 0 else ""), "sequences": len(lens),
                   "total_tokens": T, "max_len": max_len, "Hq": Hq, "Hkv": Hkv, "head_dim": D,
                   "window": W},
        "roofline": {"bound": "mfma", "kernel": "prefill (packed)",
                     "achieved": round(flops / tf / 1e12, 2), "peak": BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(flops / tf / 1e12 / BF16_PEAK_TFLOPS, 4),
                     "traffic": None, "avg_us": round(tf * 1e6, 1), "flops_per_launch": flops},
        "backward_ms": round(tb * 1e3, 4),
        "backward_tflops": round(2 * flops / tb / 1e12, 3),
    }
    # parity: the full output and gradients of three sequences
    errs = []
    for b in (0, len(lens) // 2, len(lens) - 1):
        s0, s1 = int(cu[b]), int(cu[b + 1])
        sub = {n: np.ascontiguousarray(a[s0:s1]) for n, a in arrs.items()}
        scu = np.array([0, s1 - s0])
        ref = oracle.prefill_varlen(sub["q"], sub["r"], sub["k"], sub["v"], scu, window=W)
        got = out[s0:s1].float().cpu().numpy()
        errs.append(float(np.abs(got - ref).max() / np.abs(ref).max()))
        gref = oracle.prefill_varlen_backward(sub["q"], sub["r"], sub["k"], sub["v"], sub["do"],
                                              scu, window=W)
        for g, gr in zip(grads, gref):
            a = g[s0:s1].float().cpu().numpy()
            errs.append(float(np.abs(a - gr).max() / np.abs(gr).max()))
    res["sampled_parity_max_norm_err"] = max(errs)
    return res


# The pages' H200 Parallax decode latencies for the same shapes (PyPI README of
# parallax-kernel, small- and large-batch decode tables; q50, CUDA-graph replay).
# Context only: another machine's numbers, not a target.
PAGES_H200_PARALLAX_US = {(1, 512): 5.79, (1, 1024): 6.48, (1, 4096): 8.61, (1, 16384): 21.53,
                          (32, 512): 24.02, (32, 1024): 39.55, (32, 4096): 279.96,
                          (32, 16384): 1094.37}


ROTATE_BYTES = 1 << 30  # K/V bytes a cache-defeating rotation cycles through


def graph_trials(torch, fn, iters, trials, warmup):
    """Per-step seconds of `trials` replays of one graph of `iters` calls (after
    `warmup` eager calls): the pages' q05 / q50 / q95 replay sweep."""
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        for i in range(warmup):
            fn(i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for i in range(iters):
            fn(i)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    out = []
    with torch.cuda.stream(stream):
        for _ in range(trials):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            g.replay()
            e1.record(stream)
            e1.synchronize()
            out.append(e0.elapsed_time(e1) * 1e-3 / iters)
    return np.quantile(np.array(out), [0.05, 0.5, 0.95])


def run_grid_workload(args, torch, plx, synth, oracle):
    rows = []
    for spec in synth.pages_decode_grid():
        shp = (spec.B, spec.L, spec.Hkv, spec.D)
        q_np, r_np = synth.decode_qr(spec)
        k_np = synth.normal(spec.seed, synth.TID_K, shp, spec.scale, spec.dtype)
        v_np = synth.normal(spec.seed, synth.TID_V, shp, spec.scale, spec.dtype)
        q, r, k, v = (torch.from_numpy(a).view(torch.bfloat16).cuda()
                      for a in (q_np, r_np, k_np, v_np))
        ws = torch.empty(max(1, plx.decode_workspace_bytes(spec.B, spec.Hq, spec.Hkv, spec.D,
                                                           spec.L, plx.PLX_BF16)),
                         dtype=torch.uint8, device="cuda")
        out = torch.empty((spec.B, spec.Hq, spec.D), dtype=torch.bfloat16, device="cuda")
        out_s = torch.empty_like(out)
        trials = max(3, min(args.steps, 20))
        tq = graph_trials(torch, lambda i: plx.decode(q, r, k, v, out=out, workspace=ws), 50,
                          trials, max(1, min(args.warmup, 100)))
        ts = graph_trials(torch, lambda i: plx.softmax_decode(q, k, v, out=out_s, workspace=ws),
                          50, trials, max(1, min(args.warmup, 100)))
        kv_bytes = 2 * k.numel() * 2
        # the same step with the Infinity Cache defeated: a graph of n steps over n
        # copies of K and V, n * kv_bytes >= 1 GiB (four times the cache), so no
        # replay finds its keys there
        n_rot = 1 if kv_bytes >= ROTATE_BYTES else min(512, -(-ROTATE_BYTES // kv_bytes))
        if n_rot > 1:
            ks, vs = [k] + [k.clone() for _ in range(n_rot - 1)], [v] + [v.clone() for _ in range(n_rot - 1)]
            tr = graph_trials(torch, lambda i: plx.decode(q, r, ks[i % n_rot], vs[i % n_rot], out=out,
                                                          workspace=ws),
                              n_rot, trials, max(1, min(args.warmup, 100)))
            del ks, vs
        else:
            tr = tq
        plx.decode(q, r, k, v, out=out, workspace=ws)
        ref = oracle.decode(q_np, r_np, k_np, v_np)
        got = out.float().cpu().numpy().astype(np.float64)
        rows.append({"B": spec.B, "L": spec.L, "us_q05": round(tq[0] * 1e6, 2),
                     "us_q50": round(tq[1] * 1e6, 2), "us_q95": round(tq[2] * 1e6, 2),
                     "kv_gb_s": round(kv_bytes / tq[1] / 1e9, 1),
                     "us_q50_cache_defeated": round(tr[1] * 1e6, 2),
                     "kv_copies_cache_defeated": n_rot,
                     "softmax_decode_us_q50": round(ts[1] * 1e6, 2),
                     "max_norm_err": float(np.abs(got - ref).max() / np.abs(ref).max()),
                     "elementwise_rel_err": elementwise_rel_err(got, ref),
                     "splits": plx.decode_num_splits(spec.B, spec.Hq, spec.Hkv, spec.D, spec.L,
                                                     plx.PLX_BF16),
                     "pages_h200_parallax_us": PAGES_H200_PARALLAX_US[(spec.B, spec.L)]})
    big = rows[-1]
    return {
        "metric": METRIC, "value": big["us_q50"], "unit": "us/step", "n_gpus": 1,
        "steps": 50, "warmup": max(1, min(args.warmup, 100)), "ms_per_step": big["us_q50"] / 1e3,
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "pages-grid-decode-bf16 H8 D128 B{1,32} L{512..16384}",
                   "value_row": "B32 L16384", "timing": "q50 of graph replays of 50 steps, "
                   "inputs not rotated (the pages' replay sweep); us_q50_cache_defeated: "
                   "q50 of replays of one step per K/V copy over >= 1 GiB of copies"},
        "table": rows,
    }


def calibrate_copy(torch):
    """A plain copy kernel of known size, for scaling HBM byte counters."""
    n = 64 << 20  # floats: 256 MiB read + 256 MiB written
    x = torch.ones(n, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    torch.mul(x, 2.0, out=y)  # one elementwise kernel: reads 4n bytes, writes 4n bytes
    torch.cuda.synchronize()
    return 4 * n


def main():
    args = parse()
    global EAGER
    EAGER = args.eager
    if args.gpus != 1:
        print(f"bench.py runs on one GPU; --gpus {args.gpus} is not supported "
              "(the decode and prefill paths are single-GPU kernels).", file=sys.stderr)
        sys.exit(2)
    import torch

    import oracle
    import parameterized_local_linear_amd as plx
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    plx.lib()
    if args.calibrate_copy:
        calibrate_copy(torch)
    if args.workload == "metric":
        res = run_metric_workload(args, torch, plx, synth, oracle)
    elif args.workload == "prefill":
        res = run_prefill_workload(args, torch, plx, synth, oracle)
    elif args.workload == "backward":
        res = run_backward_workload(args, torch, plx, synth, oracle)
    elif args.workload == "grid":
        res = run_grid_workload(args, torch, plx, synth, oracle)
    elif args.workload == "prefill-varlen":
        res = run_prefill_varlen_workload(args, torch, plx, synth, oracle)
    else:
        res = run_decode_workload(args, torch, plx, synth, oracle)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
