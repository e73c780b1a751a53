#!/usr/bin/env python3
"""Decode throughput of the HIP KV-cached decode path on one MI355X.

A step is one decode forward of the whole batch (all layers, logits and greedy
argmax, tokens fed on the device), replayed as one hipGraph. Inputs are the seeded
synthetic workloads of synth/ (random-init weights of the named shape, random
prompt ids); prefill is untimed (reported as time to first token).

Every workload of the five configurations is measured (C1 tiny, C2 GPT-2 124M batch
1, C3 stress init to n_ctx, C4 batch 32 fp32 and bf16, C5 Llama-style paged batch 8):
  window       K steps from the end of the prompts, timed 5 times (median reported)
  full         every decode step of the generation, timed 5 times (median)
  step         algorithmic bytes per step over the step time, against 8 TB/s and a
               measured device-to-device copy; a synchronous variant (tokens read back
               and the stream synchronized every step)
  roofline     the dominant kernel (largest share of the step's kernel time):
               algorithmic bytes per launch / mean launch time, from HIP event pairs
               around every launch of a profiled pass whose steps are each enqueued
               whole behind a short hold, so host enqueue gaps fall outside the pairs
  gemm_mfma    per linear role of the batched workloads: 2 M N K / mean launch time
               against the fp32 matrix peak, the bf16 peak and the attainable roofline
  tokens       checksum of every generated token, GPU against the oracle
  cpu_baseline the CPU oracle timed on a bounded sample of the workload (worker
               processes started before the GPU work, one thread each)

Prints ONE JSON line on stdout (everything else goes to stderr); the top level is the
C2 workload (GPT-2 124M shape, batch 1, fp32), the others are under "workloads".
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
MFMA_FP32_TFLOPS = 157.3    # dense fp32 matrix peak
MFMA_BF16_TFLOPS = 2500.0   # dense bf16 matrix peak
METRIC = "decode tok/s at GPT-2-124M shape, batch 1 and 32; achieved HBM GB/s"


T0 = time.perf_counter()


def log(*a):
    print(f"{time.perf_counter() - T0:8.2f}s", *a, file=sys.stderr, flush=True)


def setup(wname: str):
    import torch
    import synth
    import transformer_gpt_decode_amd as gd
    w = synth.WORKLOADS[wname]
    W = synth.make_weights(w.shape, w.init, w.seed)
    prompts = synth.make_prompts(w)
    kw = dict(max_seqs=w.batch, max_batch=w.batch, kv_dtype=gd.KV_BF16 if w.init.kv_bf16 else gd.KV_F32)
    tables = None
    if w.kv_block:
        tables, pool = synth.make_block_tables(w, prompts)
        kw.update(kv_block_size=w.kv_block, kv_num_blocks=pool)
    wdt = gd.WEIGHT_BF16 if w.init.bf16 else (gd.WEIGHT_Q8 if w.init.q8 else gd.WEIGHT_F32)
    m = gd.Model.from_shape(w.shape, wdt, **kw)
    m.load_weights(W)
    if tables is not None:
        for b in range(w.batch):
            m.set_block_table(b, tables[b][tables[b] >= 0])
    dev = torch.device("cuda", 0)
    tok = torch.zeros(w.batch, dtype=torch.int32, device=dev)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for b, p in enumerate(prompts):
        m.prefill(b, p, tok[b:b + 1])
    torch.cuda.synchronize()
    ttft = time.perf_counter() - t0
    first = tok.clone()
    plen = [len(p) for p in prompts]
    return w, W, prompts, m, tok, first, plen, ttft


def rewind(m, tok, first, plen):
    for b, n in enumerate(plen):
        m.truncate_seq(b, n)
    tok.copy_(first)


def timed_steps(m, tok, first, plen, K, seq_ids, runs):
    """ms per step of K decode steps from the end of the prompts, timed `runs` times
    (GPU events around the K graph launches, and the host clock; the larger counts)."""
    import torch
    out = []
    for _ in range(runs):
        rewind(m, tok, first, plen)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        wall0 = time.perf_counter()
        e0.record()
        for _ in range(K):
            m.decode_step(seq_ids, tok, tok)
        e1.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - wall0
        out.append(max(e0.elapsed_time(e1), wall * 1e3) / K)
    return out


def measure(wname: str, steps, warmup: int, runs: int, full: bool):
    import torch
    import transformer_gpt_decode_amd as gd
    w, W, prompts, m, tok, first, plen, ttft = setup(wname)
    log(f"[bench] {wname}: prompts prefilled ({ttft:.3f} s)")
    if PROFILE_MODE[0] == 1:
        # counter runs: every step launched eagerly (under counter collection each
        # dispatch costs ~170 us, and graph-replayed passes ran for minutes without output)
        m.set_option(gd.OPT_USE_GRAPH, 0)
    n_decode = w.n_generate - 1
    K = min(steps, n_decode) if steps else n_decode
    seq_ids = list(range(w.batch))
    # warm-up: W steps from the end of the prompts (rewound after each whole generation)
    left = max(1, warmup)
    while left > 0:
        rewind(m, tok, first, plen)
        for _ in range(min(left, n_decode)):
            m.decode_step(seq_ids, tok, tok)
        left -= min(left, n_decode)
    torch.cuda.synchronize()
    log(f"[bench] {wname}: warm-up done")
    win = timed_steps(m, tok, first, plen, K, seq_ids, runs)
    assert m.device_errors() == 0
    log(f"[bench] {wname}: {runs} timed runs of {K} steps: " + " ".join(f"{x:.4f}" for x in win) + " ms/step")
    fullg = timed_steps(m, tok, first, plen, n_decode, seq_ids, runs) if (full and n_decode != K) else win
    if full and n_decode != K:
        log(f"[bench] {wname}: {runs} timed runs of the whole generation ({n_decode} steps): "
            + " ".join(f"{x:.4f}" for x in fullg) + " ms/step")
    if PROFILE_MODE[0] == 1:
        # counter runs collect per dispatch, serialized: only the passes they profile
        ms_sync, gpu_tokens = float("nan"), first.cpu().numpy()[:, None]
    else:
        # synchronous variant: the new tokens read back and the stream synchronized every step
        rewind(m, tok, first, plen)
        host = torch.empty(tok.shape, dtype=tok.dtype, pin_memory=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(K):
            m.decode_step(seq_ids, tok, tok)
            host.copy_(tok, non_blocking=True)
            torch.cuda.current_stream().synchronize()
        ms_sync = (time.perf_counter() - t0) * 1e3 / K
        log(f"[bench] {wname}: synchronous run done")
        # every generated token (the first from the prompt) for the checksum against the oracle
        rewind(m, tok, first, plen)
        hist = [first.cpu().numpy().copy()]
        for _ in range(n_decode):
            m.decode_step(seq_ids, tok, tok)
            hist.append(tok.clone())
        gpu_tokens = np.stack([h if isinstance(h, np.ndarray) else h.cpu().numpy() for h in hist], 1)
    assert m.device_errors() == 0
    # profiled eager pass over the window: per-kernel time and bytes
    rewind(m, tok, first, plen)
    m.set_option(gd.OPT_PROFILE, PROFILE_MODE[0])
    m.profile_read(reset=True)
    for _ in range(K):
        m.decode_step(seq_ids, tok, tok)
    stats = m.profile_read(reset=True)
    log(f"[bench] {wname}: profiled pass done ({K} steps)")
    m.set_option(gd.OPT_PROFILE, 0)
    m.close()
    torch.cuda.synchronize()
    return dict(w=w, prompts=prompts, plen=plen, K=K, win=win, full=fullg, n_decode=n_decode, ttft=ttft,
                stats=stats, P=K, gpu_tokens=gpu_tokens, ms_sync=ms_sync)


def kernel_table(stats, P):
    by_kernel = {}
    for s in stats:
        k = by_kernel.setdefault(s["kernel"], dict(kernel=s["kernel"], roles=[], launches=0, total_us=0.0, bytes=0.0))
        k["roles"].append(s["role"])
        k["launches"] += s["launches"]
        k["total_us"] += s["total_us"]
        k["bytes"] += s["bytes"]
    rows = []
    for k in by_kernel.values():
        avg_us = k["total_us"] / k["launches"]
        bpl = k["bytes"] / k["launches"]
        rows.append(dict(kernel=k["kernel"], roles=sorted(set(k["roles"])), launches_per_step=k["launches"] / P,
                         avg_us=round(avg_us, 3), bytes_per_launch=bpl, gbps=round(bpl / avg_us / 1e3, 1),
                         share=0.0, _total=k["total_us"]))
    tot = sum(r["_total"] for r in rows)
    for r in rows:
        r["share"] = round(r.pop("_total") / tot, 4)
    rows.sort(key=lambda r: -r["share"])
    step_bytes = sum(s["bytes"] for s in stats) / P
    return rows, step_bytes, tot / P


def gemm_table(stats, P, w):
    """Per linear role: 2 M N K flops per launch over the mean launch time, as a fraction of
    the fp32 matrix peak (the MFMA these kernels issue: bf16 weights are widened to fp32),
    of the bf16 peak, and of the attainable min(fp32 peak, intensity x 8 TB/s)."""
    s = w.shape
    qdim, kdim = s.n_head * s.head_dim, s.n_kv_head * s.head_dim
    fc_n = s.d_ff if s.arch == 0 else 2 * s.d_ff
    nk = {"linear.qkv": (qdim + 2 * kdim, s.d_model), "linear.o": (s.d_model, qdim), "linear.fc": (fc_n, s.d_model),
          "linear.down": (s.d_model, s.d_ff), "linear.head": (s.vocab, s.d_model)}
    elt = 2 if w.init.bf16 else 4
    out = []
    for st in stats:
        if st["role"] not in nk or st["launches"] == 0:
            continue
        n, k = nk[st["role"]]
        avg_us = st["total_us"] / st["launches"]
        flops = 2.0 * w.batch * n * k
        tf = flops / (avg_us * 1e-6) / 1e12
        # attainable: min(fp32 matrix peak, arithmetic intensity x 8 TB/s), with the weights
        # and the activation rows in and out as the bytes
        ai = flops / (n * k * elt + 4.0 * w.batch * (n + k))
        attain = min(MFMA_FP32_TFLOPS, ai * HBM_PEAK_GBPS / 1e3)
        out.append(dict(role=st["role"], kernel=st["kernel"], launches_per_step=round(st["launches"] / P, 2),
                        avg_us=round(avg_us, 3), tflops=round(tf, 2),
                        frac_fp32_peak=round(tf / MFMA_FP32_TFLOPS, 4), frac_bf16_peak=round(tf / MFMA_BF16_TFLOPS, 5),
                        attainable_tflops=round(attain, 1), frac_attainable=round(tf / attain, 4)))
    return out


def gemm_step(gemms, w):
    """All linear layers of one step: their summed kernel time and the step's GEMM flops
    (2 B x linear and head parameters) over it, against the fp32 and bf16 matrix peaks
    and against the attainable time (each GEMM at its own attainable rate)."""
    us = sum(g["launches_per_step"] * g["avg_us"] for g in gemms)
    flops = sum(g["launches_per_step"] * g["tflops"] * 1e12 * g["avg_us"] * 1e-6 for g in gemms)
    at_us = sum(g["launches_per_step"] * g["tflops"] * g["avg_us"] / g["attainable_tflops"] for g in gemms)
    tf = flops / (us * 1e-6) / 1e12 if us else 0.0
    return dict(us_per_step=round(us, 1), gflop_per_step=round(flops / 1e9, 3), tflops=round(tf, 2),
                frac_fp32_peak=round(tf / MFMA_FP32_TFLOPS, 4), frac_bf16_peak=round(tf / MFMA_BF16_TFLOPS, 5),
                attainable_us_per_step=round(at_us, 1), frac_attainable=round(at_us / us, 4) if us else 0.0)


def kernel_sources_sha256() -> str:
    """SHA-256 over the HIP sources of the library (names and contents, sorted)."""
    import hashlib
    d = os.path.join(ROOT, "transformer_gpt_decode_amd", "csrc")
    h = hashlib.sha256()
    for name in sorted(os.listdir(d)):
        if name.endswith((".h", ".hip")):
            h.update(name.encode())
            with open(os.path.join(d, name), "rb") as f:
                h.update(f.read())
    return h.hexdigest()


def load_traffic_record():
    """profiles/hbm_traffic.json, or None when absent or taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except OSError:
        return None
    return rec if rec.get("sources_sha256") == kernel_sources_sha256() else None


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, calibrated) of a kernel in a
    workload, recorded in profiles/hbm_traffic.json, or None when not recorded or when
    the kernel sources have changed since."""
    rec = load_traffic_record()
    if rec is None:
        return None
    ks = rec.get("workloads", {}).get(workload, {}).get("kernels", {})
    k = next((v for name, v in ks.items() if name.startswith(kernel.rstrip(">"))), None)
    return None if k is None else k["fetch_bytes"] + k["write_bytes"]


def dominant(rows):
    """The kernel with the largest share of the step's kernel time. Shares within 2 % of
    the largest are measurement noise between kernels of the same length (the batch-1
    step runs four kernels of ~4.2 us per layer, whose order changes from run to run), so
    among those the one that moves the most bytes per step is taken: the choice then
    follows the workload, not the run."""
    top = rows[0]["share"]
    near = [r for r in rows if r["share"] >= 0.98 * top]
    return max(near, key=lambda r: (r["bytes_per_launch"] * r["launches_per_step"], r["share"]))


def roofline(rows, workload: str):
    top = dominant(rows)
    ach = top["bytes_per_launch"] / (top["avg_us"] * 1e-6) / 1e9
    tr = measured_traffic(top["kernel"], workload)
    return {"bound": "hbm", "kernel": top["kernel"], "achieved": round(ach, 1), "peak": HBM_PEAK_GBPS,
            "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBPS, 4), "traffic": round(tr) if tr else None,
            "bytes_per_launch": round(top["bytes_per_launch"]), "avg_launch_us": top["avg_us"]}


# Oracle samples (workload: timed decode forwards). The sequence is the one with the
# shortest prompt (the oracle's untimed prefill grows with it); C1 and C2 time their
# whole generation, which also gives every token of it for the checksum.
CPU_SAMPLE_FORWARDS = {"tiny": None, "gpt2_b1": None, "gpt2_stress": 16, "gpt2_b32": 16, "gpt2_b32_bf16": 16,
                       "llama_b8": 8, "gpt2_b32_kv16": 16, "gpt2_b1_q8": None}
# no oracle sample: its untimed prefill of a 2976-id prompt alone takes the oracle ~20 min
NO_CPU_SAMPLE = {"llama_long": "the oracle's untimed prefill of the shortest (2976-id) prompt takes ~20 minutes"}


def _shortest(w, prompts):
    return min(range(len(prompts)), key=lambda b: (len(prompts[b]), b))


def oracle_sample(wname: str):
    """Runs in a worker process: the single-threaded oracle prefills one sequence
    (untimed), then runs its timed decode forwards (see CPU_SAMPLE_FORWARDS)."""
    import oracle
    import synth
    w = synth.WORKLOADS[wname]
    W = synth.make_weights(w.shape, w.init, w.seed)
    prompts = synth.make_prompts(w)
    b = _shortest(w, prompts)
    n = CPU_SAMPLE_FORWARDS[wname] or (w.n_generate - 1)
    om = oracle.for_workload(w, W)
    s = om.new_seq(len(prompts[b]) + w.n_generate)
    t0 = time.perf_counter()
    tok = -1
    for t in prompts[b]:
        tok = s.forward(int(t))
    prefill_s = time.perf_counter() - t0
    toks = [tok]
    t0 = time.perf_counter()
    for _ in range(n):
        toks.append(s.forward(toks[-1]))
    dt = time.perf_counter() - t0
    return dict(workload=wname, seq=b, prompt=len(prompts[b]), forwards=n, seconds=dt, prefill_s=prefill_s,
                tokens=toks)


def start_cpu_samples(wnames):
    """Worker processes for the oracle samples, started before anything touches the GPU
    (forked from a fresh server process; one thread each)."""
    import multiprocessing as mp
    ctx = mp.get_context("forkserver")
    todo = [wn for wn in wnames if wn not in NO_CPU_SAMPLE]
    pool = ctx.Pool(max(1, min(len(todo), 8)))
    return pool, {wn: pool.apply_async(oracle_sample, (wn,)) for wn in todo}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(sample, res, n_workers):
    w = res["w"]
    k = len(sample["tokens"])
    g = res["gpu_tokens"][sample["seq"], :k]
    unit = "tok/s"
    return {"value": round(sample["forwards"] / sample["seconds"], 3), "unit": unit, "cores": 1, "kind": "oracle",
            "sample": f"{w.name}: sequence {sample['seq']} ({sample['prompt']}-id prompt, the shortest) prefilled "
                      f"untimed ({sample['prefill_s']:.1f} s), then {sample['forwards']} single-token decode forwards "
                      f"({sample['seconds']:.2f} s, 1 thread; {n_workers} such samples ran at once, one per "
                      f"workload, each on its own core)",
            "host_cpus": os.cpu_count(), "cpu_model": cpu_model(),
            "tokens_match_gpu": bool(np.array_equal(g, np.array(sample["tokens"]))), "tokens_compared": int(k)}


def golden_tokens(wname: str):
    """The oracle's greedy tokens [B][n_generate] of a full-size workload, as written by
    tests/golden/make_golden.py (None when there is no golden or it came from another
    oracle source)."""
    import hashlib
    path = os.path.join(ROOT, "tests", "golden", f"{wname}.npz")
    if not os.path.exists(path):
        return None
    h = hashlib.sha256()
    for f in ("oracle.c", "oracle.h"):
        with open(os.path.join(ROOT, "oracle", f), "rb") as fh:
            h.update(fh.read())
    with np.load(path, allow_pickle=False) as z:
        if str(z["oracle_hash"]) != h.hexdigest()[:16]:
            return None
        return z["tokens"].copy(), z["margin"].copy()


def token_checksum(tokens) -> str:
    import hashlib
    return hashlib.sha256(np.ascontiguousarray(tokens, dtype=np.int32).tobytes()).hexdigest()[:16]


def token_record(res, sample):
    """Checksum of every generated token of every sequence, GPU and oracle; the oracle's
    tokens come from the golden file (full-size workloads) or from the oracle sample
    when it covers the whole generation (C1, C2, one sequence)."""
    gpu = res["gpu_tokens"]
    rec = {"gpu_checksum": token_checksum(gpu), "tokens": int(gpu.size)}
    g = golden_tokens(res["w"].name)
    ref = None
    if g is not None:
        ref, margin = g
        rec["oracle_source"] = "tests/golden (oracle)"
    elif sample is not None and res["w"].batch == 1 and len(sample["tokens"]) == gpu.shape[1]:
        ref, margin = np.array([sample["tokens"]], np.int32), None
        rec["oracle_source"] = "oracle sample (this run)"
    if ref is None:
        rec["oracle_checksum"] = None
        return rec
    rec["oracle_checksum"] = token_checksum(ref)
    rec["identical"] = bool(np.array_equal(gpu, ref))
    flips = []
    for b in range(gpu.shape[0]):
        d = np.nonzero(gpu[b] != ref[b])[0]
        if len(d):
            i = int(d[0])
            flips.append({"seq": b, "step": i, "oracle_margin": None if margin is None else float(margin[b, i])})
    rec["first_divergence"] = flips
    return rec


def summary(res):
    import statistics
    rows, step_bytes, kern_us = kernel_table(res["stats"], res["P"])
    w = res["w"]
    ms = statistics.median(res["win"])
    ms_full = statistics.median(res["full"])
    step_gbps = step_bytes / (ms * 1e-3) / 1e9
    p0, p1 = min(res["plen"]), max(res["plen"])
    return rows, dict(value=round(w.batch / (ms * 1e-3), 1), ms_per_step=round(ms, 4), steps=res["K"],
                      runs=len(res["win"]), ms_per_step_runs=[round(x, 4) for x in res["win"]],
                      window=f"decode steps 1..{res['K']} after the prompts (positions {p0}..{p0 + res['K'] - 1}"
                             + (f" to {p1}..{p1 + res['K'] - 1}" if p1 != p0 else "") + ")",
                      algo_bytes_per_step=round(step_bytes), step_gbps=round(step_gbps, 1),
                      step_hbm_frac=round(step_gbps / HBM_PEAK_GBPS, 4),
                      copy_gbps=round(COPY_GBPS[0], 1) if COPY_GBPS[0] else None,
                      step_copy_frac=round(step_gbps / COPY_GBPS[0], 4) if COPY_GBPS[0] else None,
                      kernel_us_per_step=round(kern_us, 2), ttft_s=round(res["ttft"], 4),
                      sync_ms_per_step=round(res["ms_sync"], 4), sync_value=round(w.batch / (res["ms_sync"] * 1e-3), 1),
                      full_generation=dict(steps=res["n_decode"], ms_per_step=round(ms_full, 4),
                                           value=round(w.batch / (ms_full * 1e-3), 1),
                                           ms_per_step_runs=[round(x, 4) for x in res["full"]]))


def _short_name(n: str) -> str:
    n = n.replace("void ", "")
    return n[:n.index("(")] if "(" in n else n


def profiled_regions(rows, steps_per_pass=None):
    """Row ranges [lo, hi) of the profiled passes in a rocprofv3 CSV of a bench.py run,
    rows in dispatch order. Every profiled step is held by one k_gate and ends with one
    k_argmax_finalize; the gates of a pass need not sit beside their steps (the helper
    stream that holds them runs ahead of the host's enqueues), so a pass is taken as its
    K gates in order and spans from its first gate to the K-th finalize after it.
    steps_per_pass gives K for each pass; without it all gates form one pass."""
    gates = [i for i, r in enumerate(rows) if _short_name(r["Kernel_Name"]) == "k_gate"]
    fins = [i for i, r in enumerate(rows) if _short_name(r["Kernel_Name"]) == "k_argmax_finalize"]
    if not gates:
        # ungated profiling (--profile-mode 1): one workload, whose profiled pass is the
        # last thing the run does, its K steps end with the last K finalizes
        k = steps_per_pass[0] if steps_per_pass else 0
        if k <= 0 or len(fins) <= k:
            return []
        return [(fins[-k - 1] + 1, fins[-1] + 1, k)]
    counts = list(steps_per_pass) if steps_per_pass else [len(gates)]
    regions, gi = [], 0
    for k in counts:
        if k <= 0 or gi + k > len(gates):
            break
        lo = gates[gi]
        after = [i for i in fins if i > lo]
        if len(after) < k:
            break
        regions.append((lo, after[k - 1] + 1, k))
        gi += k
    return regions


def counter_means(csv_path: str, calib_mib: int, steps=None):
    """The profiled pass (of `steps` steps; required when the run was not gated) of a
    rocprofv3 --pmc CSV of a bench.py run with one workload: {kernel: mean bytes per
    dispatch}, the counter scaled by the calibration copy (see trace_summary)."""
    import csv
    import statistics

    rows = sorted(csv.DictReader(open(csv_path)), key=lambda r: int(r["Dispatch_Id"]))
    cp = next(r for r in rows if "copyBuffer" in r["Kernel_Name"])
    factor = calib_mib * 1024.0 / float(cp["Counter_Value"])
    out = []
    for lo, hi, _ in profiled_regions(rows, [steps] if steps else None):
        d = {}
        for r in rows[lo:hi]:
            k = _short_name(r["Kernel_Name"])
            if k == "k_gate" or "at::native" in k or "rocclr" in k:
                continue
            d.setdefault(k, []).append(float(r["Counter_Value"]) * factor * 1024.0)
        out.append({k: statistics.mean(v) for k, v in d.items()})
    return out, factor


def traffic_json(fetch_csv: str, write_csv: str, calib_mib: int, commands, workload: str, steps=None):
    """Records in profiles/hbm_traffic.json, under the workload's name, the HBM bytes
    per dispatch of each kernel of the first profiled pass of the FETCH_SIZE and
    WRITE_SIZE runs (the bench's main workload), with the hash of the kernel sources they
    were measured on; records of other workloads on the same sources are kept."""
    f, ff = counter_means(fetch_csv, calib_mib, steps)
    w, wf = counter_means(write_csv, calib_mib, steps)
    rec = load_traffic_record() or {"sources_sha256": kernel_sources_sha256(), "workloads": {}}
    rec.setdefault("workloads", {})[workload] = {
        "pass": "the profiled pass of bench.py (see commands)",
        "commands": list(commands),
        "calibration": {"copy_mib_each_way": calib_mib, "fetch_kib_factor": round(ff, 4),
                        "write_kib_factor": round(wf, 4)},
        "kernels": {k: {"fetch_bytes": round(f[0][k]), "write_bytes": round(w[0].get(k, 0.0))} for k in sorted(f[0])}}
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    with open(path, "w") as fh:
        json.dump(rec, fh, indent=1)
    print(f"wrote {path}: {workload}, {len(rec['workloads'][workload]['kernels'])} kernels")


def trace_summary(csv_path: str, bench_json: str | None, calib_mib: int = 0, run_json: str | None = None):
    """Markdown summary of a rocprofv3 CSV of a bench.py run (--kernel-trace, or --pmc with
    one counter): per kernel, over the dispatches of each profiled pass (the steps that
    follow a k_gate hold; these are the launches bench.py times), the mean execution time
    or the mean counter value. A counter in KiB is scaled to bytes by the first
    __amd_rocclr_copyBuffer dispatch, the copy of calib_mib MiB each way that
    `bench.py --copy-mib` runs first. With the bench's JSON line, its mean time and
    algorithmic bytes per launch are shown beside. run_json, the JSON line of the traced
    run itself when it measured a subset of bench_json's workloads, gives the order and
    step counts of its profiled passes (workloads are matched by name)."""
    import csv
    import statistics

    # dispatch order (under counter collection the start times of a held kernel and
    # of the launches queued behind it do not follow it)
    rows = sorted(csv.DictReader(open(csv_path)), key=lambda r: int(r["Dispatch_Id"]))
    counter = rows[0].get("Counter_Name") if rows else None
    factor = None
    if counter and calib_mib:
        cp = next(r for r in rows if "copyBuffer" in r["Kernel_Name"])
        factor = calib_mib * 1024.0 / float(cp["Counter_Value"])
        print(f"{counter}: the calibration copy ({calib_mib} MiB read, {calib_mib} MiB written) counts "
              f"{float(cp['Counter_Value']):.1f} KiB, so bytes = {counter} x {factor:.3f} KiB")
    bench_sets, steps, names = [], None, []
    if bench_json:
        def last_json(path):
            with open(path) as f:
                return json.loads(f.read().strip().splitlines()[-1])
        bench = last_json(bench_json)
        run = last_json(run_json) if run_json else bench
        entries = run.get("workloads_order") or [run["config"]["workload"]]
        steps = []
        for name in entries:
            e = bench["workloads"][name] if "workloads" in bench else bench
            bench_sets.append({k["kernel"]: k for k in e.get("kernels", [])})
            steps.append((run["workloads"][name] if "workloads" in run else run)["steps"])
            names.append(name)
    for pi, (lo, hi, nsteps) in enumerate(profiled_regions(rows, steps)):
        d = {}
        for r in rows[lo:hi]:
            k = _short_name(r["Kernel_Name"])
            if k == "k_gate" or "at::native" in k or "rocclr" in k:
                continue
            v = float(r["Counter_Value"]) if counter else (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0
            d.setdefault(k, []).append(v)
        bs = bench_sets[pi] if pi < len(bench_sets) else {}
        label = f" ({names[pi]})" if pi < len(names) else ""
        print(f"\nProfiled pass {pi + 1}{label}: {nsteps} steps, dispatches {lo}..{hi}\n")
        if counter:
            print(f"| kernel | dispatches | mean {counter} KiB | MB per dispatch | bench.py algorithmic MB | ratio |")
            print("|---|---|---|---|---|---|")
        else:
            print("| kernel | dispatches | rocprofv3 mean us | bench.py mean us |")
            print("|---|---|---|---|")
        for k, v in sorted(d.items(), key=lambda kv: -sum(kv[1])):
            b = next((x for name, x in bs.items() if k.startswith(name.rstrip(">"))), None)
            mean = statistics.mean(v)
            if counter:
                mb = mean * factor * 1024 / 1e6 if factor else None
                alg = b["bytes_per_launch"] / 1e6 if b else None
                ratio = f"{mb / alg:.3f}" if (mb and alg) else "-"
                print(f"| `{k}` | {len(v)} | {mean:.1f} | {f'{mb:.3f}' if mb else '-'} | "
                      f"{f'{alg:.3f}' if alg else '-'} | {ratio} |")
            else:
                print(f"| `{k}` | {len(v)} | {mean:.2f} | {b['avg_us'] if b else '-'} |")


def counter_table(csv_paths, clock_ghz: float = 2.4, top: int = 16):
    """Markdown table of rocprofv3 --pmc CSVs of the same command (one per counter pass):
    per kernel and grid size, the number of dispatches, the mean of every counter per
    dispatch, the dispatch's mean duration in that run, and what follows from them where
    the counters are present: MFMA busy cycles per SIMD (1024 SIMDs) and as a share of
    the duration at clock_ghz, L2 hit rate, mean L2 read latency (cycles per request),
    and the shares of wave time spent waiting and issuing VALU and LDS instructions. The
    `top` kernels by total duration are listed."""
    import csv
    import statistics

    agg = {}
    for path in csv_paths:
        per = {}
        for r in csv.DictReader(open(path)):
            k = _short_name(r["Kernel_Name"])
            if "at::native" in k or "rocclr" in k or k == "k_gate":
                continue
            grid = int(r["Grid_Size"]) if "Grid_Size" in r else (
                int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"]))
            key = (k, grid)
            d = per.setdefault(key, {}).setdefault(int(r["Dispatch_Id"]), {})
            if "Counter_Name" in r:
                d[r["Counter_Name"]] = float(r["Counter_Value"])
            d["_us"] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0
        for key, ds in per.items():
            a = agg.setdefault(key, {"n": len(ds)})
            for c in {c for d in ds.values() for c in d}:
                a[c] = statistics.mean(d[c] for d in ds.values() if c in d)
    counters = sorted({c for a in agg.values() for c in a if c not in ("n", "_us")})
    cols = ["kernel", "grid", "dispatches", "mean us"] + [c.replace("_sum", "") for c in counters]
    derived = []
    if "SQ_VALU_MFMA_BUSY_CYCLES" in counters:
        derived += ["MFMA busy cycles / SIMD", "MFMA busy % of duration"]
    if "TCC_HIT_sum" in counters:
        derived += ["L2 hit %"]
    if "TCP_TCC_READ_REQ_LATENCY_sum" in counters:
        derived += ["L2 read latency (cycles / request)"]
    if "SQ_WAVE_CYCLES" in counters:
        derived += ["wait % of wave time", "VALU % of wave time", "LDS % of wave time"]
    print("| " + " | ".join(cols + derived) + " |")
    print("|" + "---|" * (len(cols) + len(derived)))
    for key in sorted(agg, key=lambda k: -agg[k]["n"] * agg[k].get("_us", 0.0))[:top]:
        a = agg[key]
        row = [f"`{key[0]}`", str(key[1]), str(a["n"]), f"{a.get('_us', 0.0):.2f}"]
        row += [f"{a[c]:.4g}" if c in a else "-" for c in counters]
        if "SQ_VALU_MFMA_BUSY_CYCLES" in counters:
            b = a.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / 1024
            row += [f"{b:.0f}", f"{100 * b / (a['_us'] * clock_ghz * 1e3):.1f}" if a.get("_us") else "-"]
        if "TCC_HIT_sum" in counters:
            h, m = a.get("TCC_HIT_sum", 0.0), a.get("TCC_MISS_sum", 0.0)
            row += [f"{100 * h / (h + m):.1f}" if h + m else "-"]
        if "TCP_TCC_READ_REQ_LATENCY_sum" in counters:
            q = a.get("TCP_TCC_READ_REQ_sum", 0.0)
            row += [f"{a.get('TCP_TCC_READ_REQ_LATENCY_sum', 0.0) / q:.0f}" if q else "-"]
        if "SQ_WAVE_CYCLES" in counters:
            w = a.get("SQ_WAVE_CYCLES", 0.0)
            row += [f"{100 * a.get(c, 0.0) / w:.1f}" if w else "-"
                    for c in ("SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS")]
        print("| " + " | ".join(row) + " |")


COPY_GBPS = [None]   # measured device-to-device copy rate (read + write bytes / time)
PROFILE_MODE = [2]   # GD_OPT_PROFILE of the per-kernel pass (--profile-mode)


def copy_rate():
    """Read + write bytes per second of a 1 GiB device-to-device copy (best of 6)."""
    import torch
    n = (1 << 30) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    best = 1e9
    for _ in range(6):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1))
    del src, dst
    return 2.0 * (1 << 30) / (best * 1e-3) / 1e9


WORKLOADS = ["gpt2_b1", "tiny", "gpt2_stress", "gpt2_b32", "gpt2_b32_bf16", "llama_b8", "gpt2_b32_kv16",
             "llama_long", "gpt2_b1_q8"]
SHAPES = {"tiny": "tiny GPT-2 (2x64, 4 heads, ff 256, vocab 512)",
          "gpt2_b1": "GPT-2 124M (12x768, 12 heads, ff 3072, vocab 50257)",
          "gpt2_stress": "GPT-2 124M, W_fc ~ N(0, 0.5)",
          "gpt2_b32": "GPT-2 124M (12x768, 12 heads, ff 3072, vocab 50257)",
          "gpt2_b32_bf16": "GPT-2 124M, bf16 weights",
          "llama_b8": "Llama-style (32x960, 15/5 heads, SwiGLU 2560, vocab 49152), paged KV",
          "gpt2_b32_kv16": "GPT-2 124M, bf16 KV cache",
          "llama_long": "Llama-style, n_ctx 4096, bf16 weights, bf16 paged KV",
          "gpt2_b1_q8": "GPT-2 124M, 8-bit block weights"}


def entry(res):
    rows, summ = summary(res)
    w = res["w"]
    e = dict(workload=w.name, shape=SHAPES[w.name], batch=w.batch, weights=w.weight_dtype,
             prompt_len=list(w.prompt_len), n_generate=w.n_generate, **summ)
    if w.name == "tiny":
        # 548 KB of weights stay in cache: the step is launch-bound, a roofline
        # fraction says nothing about it
        e["roofline"] = None
    else:
        e["roofline"] = roofline(rows, w.name)
    if w.batch > 1:
        gemms = gemm_table(res["stats"], res["P"], w)
        e["gemm_mfma"] = gemms
        e["gemm_step"] = gemm_step(gemms, w)
    e["kernels"] = rows
    return e


# Prompt workloads: (workload whose weights and prompts are used, sequence)
PREFILL = [("gpt2_stress", 0), ("llama_b8", 4)]


def measure_prefill(wname: str, seq: int, runs: int, untiled: bool = True):
    """Prompt throughput of one sequence's prompt: the tiled prompt pass (median of
    `runs`), the same prompt through the decode kernels (32 rows per pass; skipped with
    untiled=False), and a profiled pass giving each GEMM's 2 M N K over its mean time."""
    import statistics
    import torch
    import synth
    import transformer_gpt_decode_amd as gd
    w = synth.WORKLOADS[wname]
    W = synth.make_weights(w.shape, w.init, w.seed)
    prompts = synth.make_prompts(w)
    P = prompts[seq]
    kw = dict(max_seqs=w.batch, max_batch=w.batch, kv_dtype=gd.KV_BF16 if w.init.kv_bf16 else gd.KV_F32)
    if w.kv_block:
        tables, pool = synth.make_block_tables(w, prompts)
        kw.update(kv_block_size=w.kv_block, kv_num_blocks=pool)
    wdt = gd.WEIGHT_BF16 if w.init.bf16 else (gd.WEIGHT_Q8 if w.init.q8 else gd.WEIGHT_F32)
    m = gd.Model.from_shape(w.shape, wdt, **kw)
    m.load_weights(W)
    if w.kv_block:
        m.set_block_table(seq, tables[seq][tables[seq] >= 0])
    tok = torch.zeros(1, dtype=torch.int32, device="cuda")

    def run(tiled, n):
        m.set_option(gd.OPT_TILED_PREFILL, 1 if tiled else 0)
        out = []
        for _ in range(n + 1):   # the first run is a warm-up
            m.reset_seq(seq)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            m.prefill(seq, P, tok)
            e1.record()
            torch.cuda.synchronize()
            out.append(e0.elapsed_time(e1))
        return out[1:], int(tok.item())

    tiled, t1 = run(True, runs)
    untiled, t2 = run(False, runs) if untiled else ([float("nan")], t1)
    m.set_option(gd.OPT_TILED_PREFILL, 1)
    m.reset_seq(seq)
    m.set_option(gd.OPT_PROFILE, 1)
    m.profile_read(reset=True)
    m.prefill(seq, P, tok)
    stats = m.profile_read(reset=True)
    m.set_option(gd.OPT_PROFILE, 0)
    m.close()
    n = len(P)
    s = w.shape
    qdim, kdim = s.n_head * s.head_dim, s.n_kv_head * s.head_dim
    fc_n = s.d_ff if s.arch == 0 else 2 * s.d_ff
    nk = {"pf.qkv": (qdim + 2 * kdim, s.d_model), "pf.o": (s.d_model, qdim), "pf.fc": (fc_n, s.d_model),
          "pf.down": (s.d_model, s.d_ff)}
    gemms, g_us, g_fl = [], 0.0, 0.0
    chunks = -(-n // 512)   # launches per role = layers x 512-row chunks; the chunks cover the n rows once
    for st in stats:
        if st["role"] not in nk:
            continue
        N, K = nk[st["role"]]
        flops = 2.0 * n * N * K * st["launches"] / chunks
        tf = flops / (st["total_us"] * 1e-6) / 1e12
        g_us += st["total_us"]
        g_fl += flops
        # k_gemm_pf<w, epi, true, nrm>: the products in bf16 parts on the bf16 matrix cores (3 bf16
        # MFMA products per product with bf16 weights, 6 with fp32 weights)
        parts = ", true" in st["kernel"]
        issued = (3 if w.init.bf16 else 6) if parts else 1
        gemms.append(dict(role=st["role"], kernel=st["kernel"], launches=st["launches"],
                          avg_us=round(st["total_us"] / st["launches"], 2), tflops=round(tf, 2),
                          frac_fp32_peak=round(tf / MFMA_FP32_TFLOPS, 4),
                          mfma="bf16 parts" if parts else "fp32", issued_tflops=round(tf * issued, 2),
                          frac_issued_peak=round(tf * issued / (MFMA_BF16_TFLOPS if parts else MFMA_FP32_TFLOPS), 4)))
    other = {st["role"]: round(st["total_us"], 1) for st in stats if st["role"] not in nk}
    med = statistics.median(tiled)
    tf = g_fl / (g_us * 1e-6) / 1e12 if g_us else 0.0
    return dict(workload=wname, sequence=seq, prompt_len=n, weights=w.weight_dtype,
                ms=round(med, 3), ms_runs=[round(x, 3) for x in tiled], tok_s=round(n / (med * 1e-3), 1),
                untiled_ms=round(statistics.median(untiled), 3),
                untiled_tok_s=round(n / (statistics.median(untiled) * 1e-3), 1),
                same_first_token=t1 == t2, gemm=gemms,
                gemm_total=dict(us=round(g_us, 1), gflop=round(g_fl / 1e9, 2), tflops=round(tf, 2),
                                frac_fp32_peak=round(tf / MFMA_FP32_TFLOPS, 4)),
                other_us=other)


def log_entry(e):
    log(f"[bench] {e['workload']}: {e['value']} tok/s, {e['ms_per_step']} ms/step (median of {e['runs']}), "
        f"whole generation {e['full_generation']['ms_per_step']} ms/step")
    for r in e["kernels"]:
        log(f"  {r['kernel']:<34} {str(r['roles']):<28} {r['launches_per_step']:6.1f}/step {r['avg_us']:9.2f} us "
            f"{r['gbps']:8.1f} GB/s  {100 * r['share']:5.1f}%")
    for g in e.get("gemm_mfma", []):
        log(f"  {g['role']:<12} {g['avg_us']:8.2f} us {g['tflops']:7.2f} TFLOP/s  "
            f"{100 * g['frac_fp32_peak']:5.1f}% of fp32 MFMA peak, {100 * g['frac_attainable']:5.1f}% of attainable")


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20, help="timed decode steps per run (capped at a workload's "
                    "generation; 0: the whole generation)")
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--runs", type=int, default=5, help="timed runs per workload (the median is reported)")
    ap.add_argument("--workloads", default=",".join(WORKLOADS), help="comma-separated; the first is the headline")
    ap.add_argument("--no-full", action="store_true", help="skip the timed runs of the whole generation")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle samples (CPU baseline)")
    ap.add_argument("--no-prefill", action="store_true", help="skip the prompt-throughput measurements")
    ap.add_argument("--no-decode", action="store_true", help="measure the prompt pass only (no decode workload)")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="first run one device-to-device copy of this many MiB (a kernel of known traffic that "
                         "scales the HBM byte counters of a rocprofv3 --pmc run)")
    ap.add_argument("--trace-summary", metavar="CSV", help="print a markdown summary of a rocprofv3 kernel trace "
                    "of a bench.py run (no GPU needed) and exit")
    ap.add_argument("--bench-json", metavar="FILE", help="with --trace-summary: the bench's JSON line to compare")
    ap.add_argument("--run-json", metavar="FILE", help="with --trace-summary: the traced run's own JSON line (its "
                    "workloads and step counts, when it measured a subset of --bench-json's)")
    ap.add_argument("--calib-mib", type=int, default=0, help="with --trace-summary of a --pmc CSV: the size of the "
                    "--copy-mib calibration copy")
    ap.add_argument("--traffic-json", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/hbm_traffic.json from the two --pmc CSVs (with --calib-mib) and exit")
    ap.add_argument("--traffic-cmd", action="append", default=[], help="with --traffic-json: a command to record")
    ap.add_argument("--counter-table", nargs="+", metavar="CSV", help="print a markdown table of rocprofv3 --pmc "
                    "CSVs of one command (one per counter pass): counters and derived figures per kernel")
    ap.add_argument("--counter-top", type=int, default=16, help="with --counter-table: kernels listed (by total time)")
    ap.add_argument("--traffic-workload", default="gpt2_b1", help="with --traffic-json: the profiled workload")
    ap.add_argument("--profile-mode", type=int, choices=(1, 2), default=2,
                    help="per-kernel timing pass: 2 holds each step behind a gate kernel on a helper stream so "
                         "that its launches run back to back (timing); 1 launches as enqueued, with no "
                         "cross-stream wait and no graphs in any pass (for counter collection, which "
                         "serializes dispatches; its step times are not representative)")
    args = ap.parse_args()
    if args.traffic_json:
        steps = None
        if args.bench_json:
            with open(args.bench_json) as f:
                b = json.loads(f.read().strip().splitlines()[-1])
                steps = b["workloads"][args.traffic_workload]["steps"] if "workloads" in b else b["steps"]
        traffic_json(args.traffic_json[0], args.traffic_json[1], args.calib_mib, args.traffic_cmd,
                     args.traffic_workload, steps)
        return
    if args.counter_table:
        counter_table(args.counter_table, top=args.counter_top)
        return
    if args.trace_summary:
        trace_summary(args.trace_summary, args.bench_json, args.calib_mib, args.run_json)
        return
    if args.gpus != 1:
        print("bench.py runs on one GPU only: the decode path has no multi-GPU code (decode would shard "
              "by sequence, one weight copy per GPU); use --gpus 1", file=sys.stderr)
        sys.exit(2)
    wnames = [x for x in args.workloads.split(",") if x]
    for wn in wnames:
        if wn not in SHAPES:
            sys.exit(f"unknown workload {wn}; choose from {','.join(WORKLOADS)}")
    # the oracle samples start first, in processes that never touch the GPU
    pool, jobs = (None, {}) if (args.no_cpu or args.no_decode) else start_cpu_samples(wnames)
    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.copy_mib > 0:
        n = args.copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] calibration copy: {args.copy_mib} MiB read + {args.copy_mib} MiB written")
        del src, dst

    PROFILE_MODE[0] = args.profile_mode
    COPY_GBPS[0] = copy_rate()
    log(f"[bench] device-to-device copy: {COPY_GBPS[0]:.0f} GB/s (read + write)")
    results, entries = {}, {}
    if args.no_decode:
        prefill = [measure_prefill(pw, ps, args.runs, untiled=PROFILE_MODE[0] != 1) for pw, ps in PREFILL]
        for r in prefill:
            log(f"[bench] prefill {r['workload']} seq {r['sequence']} ({r['prompt_len']} ids): {r['ms']} ms = "
                f"{r['tok_s']} tok/s; GEMMs {r['gemm_total']}")
        print(json.dumps({"prefill": prefill}), flush=True)
        return
    for wn in wnames:
        log(f"[bench] workload {wn}: warmup {args.warmup}, {args.runs} runs of {args.steps or 'all'} steps")
        results[wn] = measure(wn, args.steps, args.warmup, args.runs, not args.no_full)
        entries[wn] = entry(results[wn])
        log_entry(entries[wn])
    prefill = []
    if not args.no_prefill:
        for pw, ps in PREFILL:
            r = measure_prefill(pw, ps, args.runs)
            prefill.append(r)
            log(f"[bench] prefill {pw} seq {ps} ({r['prompt_len']} ids): {r['ms']} ms = {r['tok_s']} tok/s "
                f"(decode kernels: {r['untiled_ms']} ms); GEMMs {r['gemm_total']}")
    if pool is not None:
        log("[bench] waiting for the oracle samples ...")
        for wn in wnames:
            if wn not in jobs:
                entries[wn]["cpu_baseline"] = {"value": None, "note": NO_CPU_SAMPLE[wn]}
                entries[wn]["tokens"] = token_record(results[wn], None)
                continue
            smp = jobs[wn].get(900)
            entries[wn]["cpu_baseline"] = cpu_baseline(smp, results[wn], len(jobs))
            entries[wn]["tokens"] = token_record(results[wn], smp)
            log(f"[bench] {wn}: oracle {entries[wn]['cpu_baseline']['value']} tok/s on 1 core; tokens "
                f"{entries[wn]['tokens']}")
        pool.terminate()
        pool.join()
    else:
        for wn in wnames:
            entries[wn]["tokens"] = token_record(results[wn], None)
    head = entries[wnames[0]]
    hw = results[wnames[0]]["w"]
    out = {"metric": METRIC, "value": head["value"], "unit": "tok/s",
           "n_gpus": 1, "steps": head["steps"], "warmup": args.warmup, "ms_per_step": head["ms_per_step"],
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "f32" if hw.weight_dtype == "f32" else "bf16-weights/f32", "data": "synthetic",
           "config": {"workload": hw.name, "batch": hw.batch, "prompt_len": hw.prompt_len[0],
                      "n_generate": hw.n_generate, "timed": head["window"], "runs": head["runs"],
                      "shape": head["shape"], "weights": hw.weight_dtype},
           "roofline": head["roofline"], "cpu_baseline": head.get("cpu_baseline"), "tokens": head["tokens"],
           "step": {k: head[k] for k in ("value", "ms_per_step", "ms_per_step_runs", "algo_bytes_per_step",
                                         "step_gbps", "step_hbm_frac", "copy_gbps", "step_copy_frac",
                                         "kernel_us_per_step", "ttft_s", "sync_ms_per_step", "sync_value",
                                         "full_generation")},
           "workloads_order": wnames, "workloads": entries, "prefill": prefill}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
