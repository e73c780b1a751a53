#!/usr/bin/env python3
"""Decode throughput of the HIP KV-cached decode path on one MI355X.

A step is one decode forward of the whole batch (all layers, logits and greedy
argmax, tokens fed on the device), replayed as one hipGraph. Inputs are the seeded
synthetic workloads of synth/ (random-init weights of the named shape, random
prompt ids); prefill is untimed.

Prints ONE JSON line on stdout (everything else goes to stderr):
  value        decode tokens/s of the headline workload (GPT-2 124M shape, batch 1)
  roofline     the dominant kernel (largest share of the step's kernel time):
               algorithmic bytes per launch / mean launch time, from HIP event pairs
               around every launch of a profiled pass whose steps are each enqueued
               whole behind a short hold, so host enqueue gaps fall outside the pairs
  step         achieved algorithmic GB/s of the whole step against 8 TB/s and against a
               measured device-to-device copy; a synchronous variant (token read back
               and stream synchronized every step)
  cpu_baseline the CPU oracle timed on a bounded sample of the same workload
  batch32      the same measurements for 32 sequences (GPT-2 124M shape, fp32)
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


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def setup(wname: str):
    import torch
    import synth
    import transformer_gpt_decode_amd as gd
    w = synth.WORKLOADS[wname]
    W = synth.make_weights(w.shape, w.init, w.seed)
    prompts = synth.make_prompts(w)
    kw = dict(max_seqs=w.batch, max_batch=w.batch)
    tables = None
    if w.kv_block:
        tables, pool = synth.make_block_tables(w, prompts)
        kw.update(kv_block_size=w.kv_block, kv_num_blocks=pool)
    m = gd.Model.from_shape(w.shape, gd.WEIGHT_BF16 if w.init.bf16 else gd.WEIGHT_F32, **kw)
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


def run_steps(m, tok, first, plen, n_steps, n_decode, seq_ids):
    """n_steps decode steps; after each full generation (n_decode steps) rewind to the prompt end."""
    done = 0
    while done < n_steps:
        k = min(n_steps - done, n_decode)
        for _ in range(k):
            m.decode_step(seq_ids, tok, tok)
        done += k
        if done < n_steps:
            rewind(m, tok, first, plen)


def measure(wname: str, steps, warmup: int):
    import torch
    import transformer_gpt_decode_amd as gd
    w, W, prompts, m, tok, first, plen, ttft = setup(wname)
    log(f"[bench] {wname}: prompts prefilled")
    if PROFILE_MODE[0] == 1:
        # counter runs: every step launched eagerly (under counter collection, runs stalled
        # inside back-to-back graph replays)
        m.set_option(gd.OPT_USE_GRAPH, 0)
    n_decode = w.n_generate - 1
    K = steps if steps else n_decode
    seq_ids = list(range(w.batch))
    # warmup (captures the graph), then rewind to the end of the prompts
    run_steps(m, tok, first, plen, max(1, warmup), n_decode, seq_ids)
    rewind(m, tok, first, plen)
    torch.cuda.synchronize()
    log(f"[bench] {wname}: warm-up done")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    e0.record()
    run_steps(m, tok, first, plen, K, n_decode, seq_ids)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    gpu_ms = e0.elapsed_time(e1)
    ms_step = max(gpu_ms, wall * 1e3) / K
    assert m.device_errors() == 0
    log(f"[bench] {wname}: timed run done ({K} steps)")
    # synchronous variant: the new tokens read back and the stream synchronized every step
    rewind(m, tok, first, plen)
    S = min(K, n_decode)
    host = torch.empty(tok.shape, dtype=tok.dtype, pin_memory=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(S):
        m.decode_step(seq_ids, tok, tok)
        host.copy_(tok, non_blocking=True)
        torch.cuda.current_stream().synchronize()
    ms_sync = (time.perf_counter() - t0) * 1e3 / S
    log(f"[bench] {wname}: synchronous run done")
    # greedy tokens of the first steps after the prompt (for the oracle cross-check)
    rewind(m, tok, first, plen)
    hist = [first.cpu().numpy().copy()]
    for _ in range(min(n_decode, 24)):
        m.decode_step(seq_ids, tok, tok)
        hist.append(tok.cpu().numpy().copy())
    gpu_tokens = np.stack(hist, 1)
    # profiled eager pass over one generation window: per-kernel time and bytes
    rewind(m, tok, first, plen)
    m.set_option(gd.OPT_PROFILE, PROFILE_MODE[0])
    m.profile_read(reset=True)
    P = min(K, n_decode)
    for _ in range(P):
        m.decode_step(seq_ids, tok, tok)
    stats = m.profile_read(reset=True)
    log(f"[bench] {wname}: profiled pass done ({P} steps)")
    m.set_option(gd.OPT_PROFILE, 0)
    m.close()
    torch.cuda.synchronize()
    return dict(w=w, W=W, prompts=prompts, ms_step=ms_step, K=K, ttft=ttft, stats=stats, P=P,
                gpu_tokens=gpu_tokens, gpu_ms=gpu_ms, wall_s=wall, ms_sync=ms_sync, S=S)


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
    (2 B x linear and head parameters) over it."""
    us = sum(g["launches_per_step"] * g["avg_us"] for g in gemms)
    flops = sum(g["launches_per_step"] * g["tflops"] * 1e12 * g["avg_us"] * 1e-6 for g in gemms)
    tf = flops / (us * 1e-6) / 1e12 if us else 0.0
    return dict(us_per_step=round(us, 1), gflop_per_step=round(flops / 1e9, 3), tflops=round(tf, 2),
                frac_fp32_peak=round(tf / MFMA_FP32_TFLOPS, 4))


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


def roofline(rows, workload: str):
    top = rows[0]
    ach = top["bytes_per_launch"] / (top["avg_us"] * 1e-6) / 1e9
    tr = measured_traffic(top["kernel"], workload)
    return {"bound": "hbm", "kernel": top["kernel"], "achieved": round(ach, 1), "peak": HBM_PEAK_GBPS,
            "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBPS, 4), "traffic": round(tr) if tr else None,
            "bytes_per_launch": round(top["bytes_per_launch"]), "avg_launch_us": top["avg_us"]}


def cpu_baseline(res, budget_s: float):
    """The oracle (single-threaded C) on a bounded sample: prompt prefilled untimed, then
    single-token decode forwards of sequence 0 until the budget is spent."""
    import oracle
    w, W, prompts = res["w"], res["W"], res["prompts"]
    om = oracle.Model(w.shape, W)
    p = prompts[0]
    s = om.new_seq(len(p) + w.n_generate)
    tok = -1
    for t in p:
        tok = s.forward(int(t))
    toks = [tok]
    t0 = time.perf_counter()
    n = 0
    while n < w.n_generate - 1 and (time.perf_counter() - t0) < budget_s:
        tok = s.forward(toks[-1])
        toks.append(tok)
        n += 1
    dt = time.perf_counter() - t0
    g = res["gpu_tokens"][0]
    k = min(len(g), len(toks))
    return {"value": round(n / dt, 3), "unit": "tok/s", "cores": 1, "kind": "oracle",
            "sample": f"{w.name}: sequence 0, {len(p)}-id prompt prefilled untimed, then {n} single-token decode "
                      f"forwards ({dt:.1f} s, 1 thread)",
            "host_cpus": os.cpu_count(), "tokens_match_gpu": bool(np.array_equal(g[:k], np.array(toks[:k]))),
            "tokens_compared": int(k)}


def summary(res):
    rows, step_bytes, kern_us = kernel_table(res["stats"], res["P"])
    w = res["w"]
    tps = w.batch / (res["ms_step"] * 1e-3)
    step_gbps = step_bytes / (res["ms_step"] * 1e-3) / 1e9
    return rows, dict(value=round(tps, 1), ms_per_step=round(res["ms_step"], 4), steps=res["K"],
                      algo_bytes_per_step=round(step_bytes), step_gbps=round(step_gbps, 1),
                      step_hbm_frac=round(step_gbps / HBM_PEAK_GBPS, 4),
                      copy_gbps=round(COPY_GBPS[0], 1) if COPY_GBPS[0] else None,
                      step_copy_frac=round(step_gbps / COPY_GBPS[0], 4) if COPY_GBPS[0] else None,
                      kernel_us_per_step=round(kern_us, 2), ttft_s=round(res["ttft"], 4),
                      sync_ms_per_step=round(res["ms_sync"], 4), sync_value=round(w.batch / (res["ms_sync"] * 1e-3), 1))


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


def trace_summary(csv_path: str, bench_json: str | None, calib_mib: int = 0):
    """Markdown summary of a rocprofv3 CSV of a bench.py run (--kernel-trace, or --pmc with
    one counter): per kernel, over the dispatches of each profiled pass (the steps that
    follow a k_gate hold; these are the launches bench.py times), the mean execution time
    or the mean counter value. A counter in KiB is scaled to bytes by the first
    __amd_rocclr_copyBuffer dispatch, the copy of calib_mib MiB each way that
    `bench.py --copy-mib` runs first. With the bench's JSON line, its mean time and
    algorithmic bytes per launch are shown beside."""
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
    bench_sets, steps = [], None
    if bench_json:
        with open(bench_json) as f:
            bench = json.loads(f.read().strip().splitlines()[-1])
        bench_sets.append({k["kernel"]: k for k in bench.get("kernels", [])})
        steps = [bench["steps"]]
        if "batch32" in bench:
            bench_sets.append({k["kernel"]: k for k in bench["batch32"].get("kernels", [])})
            steps.append(bench["batch32"]["steps"])
    for pi, (lo, hi, nsteps) in enumerate(profiled_regions(rows, steps)):
        d = {}
        for r in rows[lo:hi]:
            k = _short_name(r["Kernel_Name"])
            if k == "k_gate" or "at::native" in k or "rocclr" in k:
                continue
            v = float(r["Counter_Value"]) if counter else (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0
            d.setdefault(k, []).append(v)
        bs = bench_sets[pi] if pi < len(bench_sets) else {}
        print(f"\nProfiled pass {pi + 1}: {nsteps} steps, dispatches {lo}..{hi}\n")
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


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=0, help="timed decode steps (default: one full generation)")
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="gpt2_b1")
    ap.add_argument("--batch32", default="gpt2_b32", help="second workload reported beside ('' to skip)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="oracle sample budget (0 to skip)")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="first run one device-to-device copy of this many MiB (a kernel of known traffic that "
                         "scales the HBM byte counters of a rocprofv3 --pmc run)")
    ap.add_argument("--trace-summary", metavar="CSV", help="print a markdown summary of a rocprofv3 kernel trace "
                    "of a bench.py run (no GPU needed) and exit")
    ap.add_argument("--bench-json", metavar="FILE", help="with --trace-summary: the bench's JSON line to compare")
    ap.add_argument("--calib-mib", type=int, default=0, help="with --trace-summary of a --pmc CSV: the size of the "
                    "--copy-mib calibration copy")
    ap.add_argument("--traffic-json", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/hbm_traffic.json from the two --pmc CSVs (with --calib-mib) and exit")
    ap.add_argument("--traffic-cmd", action="append", default=[], help="with --traffic-json: a command to record")
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
                steps = json.loads(f.read().strip().splitlines()[-1])["steps"]
        traffic_json(args.traffic_json[0], args.traffic_json[1], args.calib_mib, args.traffic_cmd,
                     args.traffic_workload, steps)
        return
    if args.trace_summary:
        trace_summary(args.trace_summary, args.bench_json, args.calib_mib)
        return
    if args.gpus != 1:
        print("bench.py runs on one GPU only: the decode path has no multi-GPU code (decode would shard "
              "by sequence, one weight copy per GPU); use --gpus 1", file=sys.stderr)
        sys.exit(2)
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
    log(f"[bench] workload {args.workload}: warmup {args.warmup}, steps {args.steps or 'one generation'}")
    res = measure(args.workload, args.steps, args.warmup)
    rows, summ = summary(res)
    log(f"[bench] {args.workload}: {summ['value']} tok/s, {summ['ms_per_step']} ms/step")
    for r in rows:
        log(f"  {r['kernel']:<28} {str(r['roles']):<40} {r['launches_per_step']:6.1f}/step {r['avg_us']:9.2f} us "
            f"{r['gbps']:8.1f} GB/s  {100 * r['share']:5.1f}%")
    out = {"metric": METRIC, "value": summ["value"], "unit": "tok/s",
           "n_gpus": 1, "steps": res["K"], "warmup": args.warmup, "ms_per_step": summ["ms_per_step"],
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
           "config": {"workload": res["w"].name, "batch": res["w"].batch, "prompt_len": res["w"].prompt_len[0],
                      "n_generate": res["w"].n_generate, "shape": "GPT-2 124M (12x768, 12 heads, ff 3072, "
                      "vocab 50257)", "weights": "f32"},
           "roofline": roofline(rows, res["w"].name), "step": summ, "kernels": rows}
    if args.cpu_seconds > 0:
        log("[bench] oracle CPU baseline ...")
        out["cpu_baseline"] = cpu_baseline(res, args.cpu_seconds)
    if args.batch32:
        log(f"[bench] workload {args.batch32} ...")
        r32 = measure(args.batch32, 0, args.warmup)
        rows32, summ32 = summary(r32)
        log(f"[bench] {args.batch32}: {summ32['value']} tok/s, {summ32['ms_per_step']} ms/step")
        for r in rows32:
            log(f"  {r['kernel']:<28} {str(r['roles']):<40} {r['launches_per_step']:6.1f}/step "
                f"{r['avg_us']:9.2f} us {r['gbps']:8.1f} GB/s  {100 * r['share']:5.1f}%")
        gemms = gemm_table(r32["stats"], r32["P"], r32["w"])
        for g in gemms:
            log(f"  {g['role']:<12} {g['avg_us']:8.2f} us {g['tflops']:7.2f} TFLOP/s  "
                f"{100 * g['frac_fp32_peak']:5.1f}% of fp32 MFMA peak, {100 * g['frac_attainable']:5.1f}% of attainable")
        out["batch32"] = dict(workload=r32["w"].name, dtype=r32["w"].weight_dtype, **summ32,
                              roofline=roofline(rows32, r32["w"].name), gemm_mfma=gemms, gemm_step=gemm_step(gemms, r32["w"]),
                              kernels=rows32)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
