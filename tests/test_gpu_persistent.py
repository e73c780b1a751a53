"""Parity of the single-launch decode step (one sequence, GPT-2 layout) against the oracle.

With GD_OPT_PERSISTENT on (off by default), a batch-1 decode step of the GPT-2 layout
runs as one launch with one workgroup per CU whose phases hand over through tagged
words in device memory. These tests switch it on and cover what
the kernel-chain tests do not: several attention chunks per head (contexts past 256
positions), paged caches with shuffled block tables, sequence slots other than 0
interleaved step by step, bf16 weights, and a step abandoned at its wait bound
(forced from the host with a zero bound: every kernel still exits normally).

Bar: identical greedy tokens and every logit within 1e-3 (fp32 weights) or 2e-2 (bf16).
"""
import dataclasses

import numpy as np
import pytest

import synth
from tests.gpu_util import (compare_generation, device, gd_model, gpu_generate, oracle_generate,
                             perturb_norms_and_biases)

pytestmark = pytest.mark.gpu

DERR_SYNC = 8


def _check(w, W, prompts, tol, tables=None, pool=None):
    ref_tok, ref_lg = oracle_generate(w, W, prompts)
    m = gd_model(w, W, pool_blocks=pool, persistent=True)
    tok, lg = gpu_generate(m, prompts, w.n_generate, tables=tables)
    assert m.device_errors() == 0
    rep = compare_generation(tok, lg, ref_tok, ref_lg, tol)
    assert not rep["near_ties"], rep
    m.close()
    return rep


def test_tiny():
    w = synth.WORKLOADS["tiny"]
    W = synth.make_weights(w.shape, w.init, w.seed)
    print("tiny", _check(w, W, synth.make_prompts(w), 1e-3))


def test_tiny_random_norms_and_biases():
    """Norm gains and shifts and every bias drawn at random (the workloads hold them at
    1 and 0)."""
    w = synth.WORKLOADS["tiny"]
    W = perturb_norms_and_biases(w.shape, synth.make_weights(w.shape, w.init, w.seed), 103)
    print("tiny random norms", _check(w, W, synth.make_prompts(w), 1e-3))


def test_tiny_long_context_chunks():
    """Contexts from 701 to 720 positions: three attention chunks of 256 per head."""
    shape = dataclasses.replace(synth.WORKLOADS["tiny"].shape, n_ctx=1024)
    w = synth.Workload("tiny_1k", shape, synth.Init(), 21, 1, (700, 700), 20)
    W = synth.make_weights(w.shape, w.init, w.seed)
    print("tiny_1k", _check(w, W, synth.make_prompts(w), 1e-3))


def test_tiny_bf16_paged_shuffled():
    w = synth.Workload("tiny_paged", synth.WORKLOADS["tiny"].shape, synth.Init(bf16=True), 22, 1, (30, 30), 24,
                       kv_block=16)
    W = synth.make_weights(w.shape, w.init, w.seed)
    prompts = synth.make_prompts(w)
    tab, pool = synth.make_block_tables(w, prompts)
    print("tiny_paged", _check(w, W, prompts, 2e-2, tables=tab, pool=pool))


def test_interleaved_sequence_slots():
    """Three sequences decoded one step at a time in turn (batch 1 each step), in slots
    0..2 of a paged cache with shuffled block tables."""
    import torch
    w = synth.Workload("tiny_slots", synth.WORKLOADS["tiny"].shape, synth.Init(), 23, 3, (5, 20), 12, kv_block=16)
    W = synth.make_weights(w.shape, w.init, w.seed)
    prompts = synth.make_prompts(w)
    tab, pool = synth.make_block_tables(w, prompts)
    ref_tok, ref_lg = oracle_generate(w, W, prompts)
    dev = device()
    m = gd_model(w, W, pool_blocks=pool, max_batch=1, persistent=True)
    for b in range(w.batch):
        m.set_block_table(b, tab[b][tab[b] >= 0])
    V = w.shape.vocab
    tok = torch.zeros(w.batch, dtype=torch.int32, device=dev)
    lg = torch.empty((w.batch, w.n_generate, V), dtype=torch.float32, device=dev)
    out = torch.zeros((w.batch, w.n_generate), dtype=torch.int32, device=dev)
    for b, p in enumerate(prompts):
        m.prefill(b, p, tok[b:b + 1], lg[b, 0])
        out[b, 0] = tok[b]
    for i in range(1, w.n_generate):
        for b in range(w.batch):
            m.decode_step([b], tok[b:b + 1], tok[b:b + 1], lg[b, i])
            out[b, i] = tok[b]
    torch.cuda.synchronize()
    assert m.device_errors() == 0
    rep = compare_generation(out.cpu().numpy(), lg.cpu().numpy(), ref_tok, ref_lg, 1e-3)
    assert not rep["near_ties"], rep
    m.close()


def test_gpt2_124m_bf16_paged():
    """GPT-2 124M shape, bf16 weights, paged cache (block 16, shuffled), one sequence."""
    base = synth.WORKLOADS["gpt2_b32_bf16"]
    w = dataclasses.replace(base, name="gpt2_bf16_paged", batch=1, prompt_len=(20, 20), n_generate=12, kv_block=16)
    W = synth.make_weights(w.shape, w.init, w.seed)
    prompts = synth.make_prompts(w)
    tab, pool = synth.make_block_tables(w, prompts)
    print("gpt2_bf16_paged", _check(w, W, prompts, 2e-2, tables=tab, pool=pool))


def test_abandoned_step_is_flagged_and_recoverable():
    """With a zero wait bound the step is abandoned (device error bit 3), every kernel
    exits; after restoring the bound and rewinding, the generation matches the oracle."""
    import torch
    import transformer_gpt_decode_amd as gd
    w = synth.WORKLOADS["tiny"]
    W = synth.make_weights(w.shape, w.init, w.seed)
    prompts = synth.make_prompts(w)
    ref_tok, ref_lg = oracle_generate(w, W, prompts)
    dev = device()
    m = gd_model(w, W, persistent=True)
    tok = torch.zeros(1, dtype=torch.int32, device=dev)
    m.prefill(0, prompts[0], tok)
    m.set_option(gd.OPT_PERSISTENT_SPIN_US, 0)
    for _ in range(3):
        m.decode_step([0], tok, tok)
    torch.cuda.synchronize()
    assert m.device_errors() & DERR_SYNC
    m.set_option(gd.OPT_PERSISTENT_SPIN_US, 20000)
    tok2, lg2 = gpu_generate(m, prompts, w.n_generate)   # resets the slot and prefills again
    assert m.device_errors() == 0
    rep = compare_generation(tok2, lg2, ref_tok, ref_lg, 1e-3)
    assert not rep["near_ties"], rep
    m.close()
