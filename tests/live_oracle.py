"""Oracle generations for the full-size parity tests, computed in the background.

The full-size workloads take the oracle minutes per sequence, so whole logit rows
(every vocabulary entry at every generated step) are computed while the other GPU
tests run: a pool of worker processes is started when the session begins (before
any test touches the GPU; the workers are forked from a fresh server process and
never load the HIP library) and each full-size test collects the sequences it
compares whole.

Only the CPU oracle (oracle/) and the seeded input generator (synth/) run here.
"""
from __future__ import annotations

import multiprocessing as mp
import os
from typing import Dict, List, Optional, Tuple

import numpy as np

# Sequences whose every logit is compared at every step, per workload: the ones with
# the shortest prompts (the oracle's time per sequence grows with the prompt).
# llama_long (prompts of 1536-3840 ids) would take the oracle over ten minutes per
# sequence: it is compared on the goldens' sampled entries only.
FULL_ROW_SEQS = {"gpt2_stress": 1, "gpt2_b32": 6, "gpt2_b32_bf16": 6, "llama_b8": 2, "gpt2_b32_kv16": 6,
                 "llama_long": 0}

_pool = None
_jobs: Dict[Tuple[str, int], "mp.pool.AsyncResult"] = {}
_W = {}


def full_row_seqs(wname: str) -> List[int]:
    import synth
    w = synth.WORKLOADS[wname]
    lens = [len(p) for p in synth.make_prompts(w)]
    order = sorted(range(w.batch), key=lambda b: (lens[b], b))
    return sorted(order[:FULL_ROW_SEQS[wname]])


def _generate(wname: str, b: int):
    import oracle
    import synth
    w = synth.WORKLOADS[wname]
    if wname not in _W:
        _W.clear()   # one workload's weights per worker at a time
        _W[wname] = oracle.for_workload(w, synth.make_weights(w.shape, w.init, w.seed))
    prompt = synth.make_prompts(w)[b]
    return oracle.generate(_W[wname], prompt, w.n_generate, want_logits=True)


def start(wnames: List[str], procs: Optional[int] = None) -> None:
    """Submits every full-row sequence of the given workloads (longest jobs first)."""
    global _pool
    if _pool is not None or not wnames:
        return
    import synth
    n = procs or max(1, min(12, (os.cpu_count() or 2) - 2))
    ctx = mp.get_context("forkserver")
    _pool = ctx.Pool(n)
    jobs = []
    for wname in wnames:
        w = synth.WORKLOADS[wname]
        lens = [len(p) for p in synth.make_prompts(w)]
        cost = 3.0 if w.shape.arch == synth.ARCH_LLAMA else 1.0
        for b in full_row_seqs(wname):
            jobs.append((cost * (lens[b] + w.n_generate), wname, b))
    for _, wname, b in sorted(jobs, reverse=True):
        _jobs[(wname, b)] = _pool.apply_async(_generate, (wname, b))


def result(wname: str, b: int, timeout: float = 900.0):
    """(tokens [n_generate], logits [n_generate][V]) of one sequence; computed here if
    the pool was not started (e.g. a single test run by name)."""
    job = _jobs.get((wname, b))
    if job is None:
        return _generate(wname, b)
    return job.get(timeout)


def stop() -> None:
    global _pool
    if _pool is not None:
        _pool.terminate()
        _pool.join()
        _pool = None
        _jobs.clear()

