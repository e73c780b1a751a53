#!/usr/bin/env python3
"""Writes the oracle's greedy generations for the full-size workloads to tests/golden/.

Only the CPU oracle (oracle/) and the seeded input generator (synth/) are used: no
value here comes from the GPU library. For every sequence of a workload the file
holds

  tokens     [B][n_generate]   greedy tokens (first from the prompt, then fed back)
  top_idx    [B][n_generate][TOPK]  indices of the TOPK largest logits, descending
  top_val    [B][n_generate][TOPK]  their logits
  margin     [B][n_generate]   logit gap between the two largest entries
  probe_idx  [NPROBE]          fixed vocabulary entries (seeded), same for every step
  probe_val  [B][n_generate][NPROBE]  their logits
  full_steps [S]               steps whose whole logit row is kept, for sequence 0
  full_val   [S][V]            those rows

Usage: python tests/golden/make_golden.py [workload ...]  (default: all full-size ones)
Runs one worker process per sequence (up to the host's CPU count, at most 8).
"""
import argparse
import hashlib
import multiprocessing as mp
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth  # noqa: E402

TOPK = 8
NPROBE = 24
FULL_SEQ_STEPS = 3
WORKLOADS = ["gpt2_stress", "gpt2_b32", "gpt2_b32_bf16", "llama_b8", "gpt2_b32_kv16", "llama_long"]

_W = None


def _init(wname):
    global _W
    w = synth.WORKLOADS[wname]
    _W = (w, synth.make_weights(w.shape, w.init, w.seed))


def _one(args):
    b, prompt, probe, full_steps = args
    w, W = _W
    t0 = time.time()
    m = oracle.for_workload(w, W)
    toks, lg = oracle.generate(m, prompt, w.n_generate, want_logits=True)
    order = np.argsort(-lg.astype(np.float64), axis=1, kind="stable")[:, :TOPK]
    top_val = np.take_along_axis(lg, order, axis=1)
    srt = np.sort(lg.astype(np.float64), axis=1)
    margin = (srt[:, -1] - srt[:, -2]).astype(np.float32)
    full = lg[full_steps] if b == 0 else None
    return b, toks, order.astype(np.int32), top_val, margin, lg[:, probe], full, time.time() - t0


def oracle_hash():
    h = hashlib.sha256()
    for f in ("oracle.c", "oracle.h"):
        h.update(open(os.path.join(ROOT, "oracle", f), "rb").read())
    return h.hexdigest()[:16]


def make(wname, procs):
    w = synth.WORKLOADS[wname]
    prompts = synth.make_prompts(w)
    probe = np.sort(np.random.default_rng(1000 + w.seed).choice(w.shape.vocab, NPROBE, replace=False)).astype(np.int32)
    n = w.n_generate
    full_steps = np.array(sorted({0, n // 2, n - 1}), np.int32)
    B = w.batch
    out = dict(tokens=np.zeros((B, n), np.int32), top_idx=np.zeros((B, n, TOPK), np.int32),
               top_val=np.zeros((B, n, TOPK), np.float32), margin=np.zeros((B, n), np.float32),
               probe_idx=probe, probe_val=np.zeros((B, n, NPROBE), np.float32), full_steps=full_steps)
    jobs = [(b, prompts[b], probe, full_steps) for b in range(B)]
    t0 = time.time()
    with mp.get_context("fork").Pool(min(procs, B), initializer=_init, initargs=(wname,)) as pool:
        for b, toks, ti, tv, mg, pv, full, dt in pool.imap_unordered(_one, jobs):
            out["tokens"][b], out["top_idx"][b], out["top_val"][b] = toks, ti, tv
            out["margin"][b], out["probe_val"][b] = mg, pv
            if full is not None:
                out["full_val"] = full
            print(f"[golden] {wname} seq {b}: {len(prompts[b])} prompt ids, {dt:.0f} s "
                  f"(elapsed {time.time() - t0:.0f} s)", flush=True)
    out["oracle_hash"] = np.array(oracle_hash())
    path = os.path.join(HERE, f"{wname}.npz")
    np.savez_compressed(path, **out)
    print(f"[golden] wrote {path} ({os.path.getsize(path) / 1e6:.2f} MB)", flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("workloads", nargs="*", default=WORKLOADS)
    ap.add_argument("--procs", type=int, default=min(8, os.cpu_count() or 1))
    a = ap.parse_args()
    for wname in a.workloads:
        make(wname, a.procs)


if __name__ == "__main__":
    main()
