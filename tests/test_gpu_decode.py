"""End-to-end parity of the decode path (C ABI, hipGraph steps) against the oracle.

Bar: identical greedy tokens and every logit within 1e-3 (fp32 weights) or 2e-2 (bf16
weights) at every generated step of every sequence; a flip is accepted only as a
near tie (see gpu_util.compare_generation), after which the rest of that sequence is
compared teacher-forced.
"""
import dataclasses

import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import (compare_generation, device, gd_model, gpu_generate, near_tie_margin, oracle_generate,
                             perturb_norms_and_biases)

pytestmark = pytest.mark.gpu

TINY_LLAMA = synth.Shape(synth.ARCH_LLAMA, 2, 96, 6, 2, 16, 128, 300, 64, 1e-5, 1e4)
# head_dim 64 with 3 query heads per KV head (the C5 attention shape) in a small model
LLAMA_HD64 = synth.Shape(synth.ARCH_LLAMA, 2, 192, 3, 1, 64, 256, 300, 320, 1e-5, 1e5)


def _run_and_compare(w, W, prompts, tol, variant=0, graph=True, tables=None, pool=None, max_seqs=None,
                     fold=True, chunks=0, config=None, logits_slices=False):
    ref_tok, ref_lg = oracle_generate(w, W, prompts)
    m = gd_model(w, W, max_seqs=max_seqs, pool_blocks=pool, variant=variant, graph=graph, fold=fold, chunks=chunks)
    tok, lg = gpu_generate(m, prompts, w.n_generate, tables=tables, logits_slices=logits_slices)
    assert m.device_errors() == 0
    rep = compare_generation(tok, lg, ref_tok, ref_lg, tol, config or w.name, sampling=w.sampling,
                             plens=[len(p) for p in prompts], tie=near_tie_margin(w))
    if rep["flips"]:
        # continue teacher-forced with the oracle's tokens; logits must still meet the bar
        tok2, lg2 = gpu_generate(m, prompts, w.n_generate, tables=tables, forced=ref_tok)
        d = float(np.max(np.abs(lg2 - ref_lg)))
        rep["forced_max_dlogit"] = d
        assert d <= tol, d
    m.close()
    return rep, tok, lg


@pytest.mark.parametrize("graph", [True, False], ids=["graph", "eager"])
@pytest.mark.parametrize("variant", [0, 1, 2], ids=["auto", "gemv", "mfma"])
def test_tiny_gpt2(variant, graph):
    w = synth.WORKLOADS["tiny"]
    W = synth.make_weights(w.shape, w.init, w.seed)
    prompts = synth.make_prompts(w)
    rep, _, _ = _run_and_compare(w, W, prompts, 1e-3, variant, graph, config=f"tiny (C1, variant {variant})")
    assert not rep["flips"]


@pytest.mark.parametrize("variant", [0, 1, 2], ids=["auto", "gemv", "mfma"])
def test_tiny_gpt2_batched(variant):
    """Six ragged sequences. With the GEMV forced (variant 1) the six rows also take the
    short-context attention fused with the output projection (k_attn_o) in one launch."""
    w = dataclasses.replace(synth.WORKLOADS["tiny"], batch=6, prompt_len=(1, 30), n_generate=20)
    W = synth.make_weights(w.shape, w.init, w.seed)
    prompts = synth.make_prompts(w)
    _run_and_compare(w, W, prompts, 1e-3, variant)


@pytest.mark.parametrize("shuffled", [True, False], ids=["shuffled", "identity"])
def test_tiny_llama_paged(shuffled):
    w = synth.Workload("tiny_llama", TINY_LLAMA, synth.Init(bf16=True), 7, 3, (5, 40), 12, kv_block=8)
    W = synth.make_weights(w.shape, w.init, w.seed)
    prompts = synth.make_prompts(w)
    tab, pool = (synth.make_block_tables if shuffled else synth.identity_block_tables)(w, prompts)
    _run_and_compare(w, W, prompts, 2e-2, tables=tab, pool=pool)


@pytest.mark.parametrize("mode", ["fused_attn_o", "gemv_split_context", "mfma_split_context"])
def test_llama_hd64_gqa_paged(mode):
    """head_dim 64, 3 query heads per KV head, paged, bf16 weights. Rows at contexts of at
    most 256 positions whose projections run on the GEMV take attention fused with the
    output projection; with the GEMV forced, 8 rows at 250-310 positions run
    split-context attention whose partials the GEMV projection (two launches of 4 rows)
    merges in its prologue; with the MFMA forced, the MFMA projection merges the
    split-context partials of its 6 rows while staging them."""
    batch, plen, variant = {"fused_attn_o": (2, (5, 60), 0), "gemv_split_context": (8, (250, 300), 1),
                            "mfma_split_context": (6, (5, 60), 2)}[mode]
    w = synth.Workload("llama_hd64", LLAMA_HD64, synth.Init(bf16=True), 11, batch, plen, 10, kv_block=16)
    W = synth.make_weights(w.shape, w.init, w.seed)
    prompts = synth.make_prompts(w)
    tab, pool = synth.make_block_tables(w, prompts)
    _run_and_compare(w, W, prompts, 2e-2, variant=variant, tables=tab, pool=pool, config=f"llama_hd64 ({mode})")


def test_llama_hd64_gqa_paged_one_chunk():
    """The one-chunk split-context attention (one workgroup per row and KV head writes the
    normalized output) on a shuffled paged cache with 3 query heads per KV head, followed
    by the matrix-core output projection."""
    w = synth.Workload("llama_hd64", LLAMA_HD64, synth.Init(bf16=True), 12, 6, (5, 200), 10, kv_block=16)
    W = synth.make_weights(w.shape, w.init, w.seed)
    prompts = synth.make_prompts(w)
    tab, pool = synth.make_block_tables(w, prompts)
    _run_and_compare(w, W, prompts, 2e-2, variant=2, tables=tab, pool=pool, chunks=1)


@pytest.mark.parametrize("mode", ["fused_attn_o", "one_chunk", "eight_chunks", "eight_chunks_20_rows"])
def test_llama_hd64_gqa_contiguous(mode):
    """3 query heads per KV head on a contiguous cache (no block table): 2 rows at short
    contexts take the fused attention + output projection; 6 rows run split-context
    attention with one or eight chunks per row and the matrix-core output projection
    (which merges the eight chunks while staging its rows); 20 rows with eight chunks
    take the merge launch and then the 32-row matrix-core projection."""
    fused = mode == "fused_attn_o"
    w = synth.Workload("llama_hd64", LLAMA_HD64, synth.Init(bf16=True), 14,
                       2 if fused else 20 if mode == "eight_chunks_20_rows" else 6, (5, 120 if fused else 200), 10)
    W = synth.make_weights(w.shape, w.init, w.seed)
    prompts = synth.make_prompts(w)
    _run_and_compare(w, W, prompts, 2e-2, variant=0 if fused else 2, chunks=8 if mode.startswith("eight_chunks") else
                     (1 if mode == "one_chunk" else 0))


def test_context_crosses_fused_limit():
    """A batch-1 generation whose context grows past 256 positions: the decode graph
    switches from the fused attention + output projection to split-context attention."""
    shape = dataclasses.replace(synth.WORKLOADS["tiny"].shape, n_ctx=400)
    w = synth.Workload("tiny_long", shape, synth.Init(), 5, 1, (248, 248), 20)
    W = synth.make_weights(w.shape, w.init, w.seed)
    prompts = synth.make_prompts(w)
    _run_and_compare(w, W, prompts, 1e-3)


# head_dim 64 (64 positions per load round of the attention scan) at contexts of up to
# 1024 positions, small enough for the oracle
GPT2_HD64_LONG = synth.Shape(synth.ARCH_GPT2, 2, 128, 2, 2, 64, 256, 300, 1024)


@pytest.mark.parametrize("chunks", [0, 1, 8], ids=["auto", "one_chunk", "eight_chunks"])
@pytest.mark.parametrize("variant", [1, 2], ids=["gemv", "mfma"])
def test_long_contexts_attention_chunks(variant, chunks):
    """Ragged contexts of 1..~900 positions: the scan runs 1..15 load rounds of 64
    positions, odd and even counts. With the matrix-core output projection and one
    chunk per row the attention writes its normalized output itself; with eight chunks
    the partials are merged while the projection stages its rows (the gemv projection
    always merges eight)."""
    w = synth.Workload("gpt2_hd64_long", GPT2_HD64_LONG, synth.Init(), 13, 5, (1, 880), 6)
    W = synth.make_weights(w.shape, w.init, w.seed)
    prompts = synth.make_prompts(w)
    _run_and_compare(w, W, prompts, 1e-3, variant, chunks=chunks)


@pytest.mark.parametrize("mode", ["folded_norm", "norm_applied"])
def test_gpt2_124m_batch1(mode):
    """GPT-2 124M shape, batch 1, 8 prompt ids, 128 generated tokens (fp32): every logit of
    every step against the oracle, with the pre-norms folded into the weights (default)
    or applied to the rows."""
    w = synth.WORKLOADS["gpt2_b1"]
    W = synth.make_weights(w.shape, w.init, w.seed)
    prompts = synth.make_prompts(w)
    rep, _, _ = _run_and_compare(w, W, prompts, 1e-3, fold=mode == "folded_norm", config=f"gpt2_b1 ({mode})")
    assert not rep["flips"], rep["flips"]


def test_graph_cache_eviction_with_per_step_logits():
    """Every step writes its logits to a new slice, so each step captures a new graph and
    the bounded graph cache evicts (16 kept); results stay exact."""
    w = dataclasses.replace(synth.WORKLOADS["tiny"], n_generate=40)
    W = synth.make_weights(w.shape, w.init, w.seed)
    prompts = synth.make_prompts(w)
    rep, _, _ = _run_and_compare(w, W, prompts, 1e-3, logits_slices=True, config="tiny (graph per step)")
    assert not rep["flips"]


def test_tiny_gpt2_batches_interleaved():
    """Random norm parameters and biases; three sequences decoded in batches of 1, 3 and
    then 2 (slots interleaved), so steps of different row counts and slot sets follow
    each other on the same model."""
    import torch
    w = dataclasses.replace(synth.WORKLOADS["tiny"], batch=3, prompt_len=(3, 20), n_generate=12)
    W = perturb_norms_and_biases(w.shape, synth.make_weights(w.shape, w.init, w.seed), 104)
    prompts = synth.make_prompts(w)
    ref_tok, ref_lg = oracle_generate(w, W, prompts)
    m = gd_model(w, W)
    dev = device()
    V = w.shape.vocab
    tok = torch.zeros(w.batch, dtype=torch.int32, device=dev)
    out = torch.zeros((w.batch, w.n_generate), dtype=torch.int32, device=dev)
    lg = torch.empty((w.batch, w.n_generate, V), dtype=torch.float32, device=dev)
    for b, p in enumerate(prompts):
        m.reset_seq(b)
        m.prefill(b, p, tok[b:b + 1], lg[b, 0])
        out[b, 0] = tok[b]
    step_lg = torch.empty((w.batch, V), dtype=torch.float32, device=dev)
    for i in range(1, w.n_generate):
        groups = [[0], [1], [2]] if i % 3 == 0 else ([[0, 1, 2]] if i % 3 == 1 else [[2, 0], [1]])
        for g in groups:
            t_in = torch.stack([tok[b] for b in g])
            t_out = torch.zeros(len(g), dtype=torch.int32, device=dev)
            m.decode_step(g, t_in, t_out, step_lg[:len(g)])
            for k, b in enumerate(g):
                tok[b] = t_out[k]
                out[b, i] = t_out[k]
                lg[b, i] = step_lg[k]
    torch.cuda.synchronize()
    assert m.device_errors() == 0
    rep = compare_generation(out.cpu().numpy(), lg.cpu().numpy(), ref_tok, ref_lg, 1e-3, "tiny (interleaved batches)")
    assert not rep["flips"], rep
    m.close()


def test_set_up_in_qkv_and_set_up_launch_alternate():
    """Steps of up to 4 rows run the step's set-up (embedding, row metadata) inside the
    first QKV launch and advance the sequence lengths in the argmax finalize; steps of 6
    rows stage their rows through the set-up launch, which advances them itself. Six
    sequences decoded alternately as one batch of 6 and as batches of 4 and 2 (slots
    reordered) must match the oracle at every step."""
    import torch
    w = dataclasses.replace(synth.WORKLOADS["tiny"], batch=6, prompt_len=(2, 24), n_generate=14)
    W = perturb_norms_and_biases(w.shape, synth.make_weights(w.shape, w.init, w.seed), 105)
    prompts = synth.make_prompts(w)
    ref_tok, ref_lg = oracle_generate(w, W, prompts)
    m = gd_model(w, W)
    dev = device()
    V = w.shape.vocab
    tok = torch.zeros(w.batch, dtype=torch.int32, device=dev)
    out = torch.zeros((w.batch, w.n_generate), dtype=torch.int32, device=dev)
    lg = torch.empty((w.batch, w.n_generate, V), dtype=torch.float32, device=dev)
    for b, p in enumerate(prompts):
        m.reset_seq(b)
        m.prefill(b, p, tok[b:b + 1], lg[b, 0])
        out[b, 0] = tok[b]
    step_lg = torch.empty((w.batch, V), dtype=torch.float32, device=dev)
    for i in range(1, w.n_generate):
        groups = [[0, 1, 2, 3, 4, 5]] if i % 2 else [[5, 3, 1, 0], [2, 4]]
        for g in groups:
            t_in = torch.stack([tok[b] for b in g])
            t_out = torch.zeros(len(g), dtype=torch.int32, device=dev)
            m.decode_step(g, t_in, t_out, step_lg[:len(g)])
            for k, b in enumerate(g):
                tok[b] = t_out[k]
                out[b, i] = t_out[k]
                lg[b, i] = step_lg[k]
    torch.cuda.synchronize()
    assert m.device_errors() == 0
    rep = compare_generation(out.cpu().numpy(), lg.cpu().numpy(), ref_tok, ref_lg, 1e-3,
                             "tiny (set-up in QKV / set-up launch alternating)")
    assert not rep["flips"], rep
    # (a device length out of step with the host's would have moved the attended
    # positions and the logits above)
    for b, p in enumerate(prompts):
        assert m.seq_len(b) == len(p) + w.n_generate - 1
    m.close()


@pytest.mark.parametrize("fold", [True, False], ids=["folded", "applied"])
@pytest.mark.parametrize("variant", [0, 2], ids=["auto", "mfma"])
def test_tiny_gpt2_random_norms_and_biases(variant, fold):
    """Norm gains and shifts and every bias drawn at random (the workloads hold them at
    1 and 0): the pre-norm folded into the weights (gain) and the bias (shift), or
    applied to the row, must match the oracle, on the GEMV and the MFMA paths."""
    w = dataclasses.replace(synth.WORKLOADS["tiny"], batch=3, prompt_len=(1, 30), n_generate=16)
    W = perturb_norms_and_biases(w.shape, synth.make_weights(w.shape, w.init, w.seed), 101)
    prompts = synth.make_prompts(w)
    rep, _, _ = _run_and_compare(w, W, prompts, 1e-3, variant, fold=fold)
    assert not rep["flips"]


def test_gpt2_124m_random_norms_and_biases():
    """GPT-2 124M shape, batch 1, random norm parameters and biases, folded pre-norms
    (the head's folded bias carries the final norm's shift through the tied embedding)."""
    w = dataclasses.replace(synth.WORKLOADS["gpt2_b1"], n_generate=24)
    W = perturb_norms_and_biases(w.shape, synth.make_weights(w.shape, w.init, w.seed), 102)
    prompts = synth.make_prompts(w)
    rep, _, _ = _run_and_compare(w, W, prompts, 1e-3, config="gpt2_b1 (random norms and biases)")
    assert not rep["flips"], rep["flips"]


@pytest.mark.parametrize("fold", [True, False], ids=["folded_norm", "norm_applied"])
def test_gpt2_124m_batched_random_norms_head_parts(fold):
    """GPT-2 124M shape, 6 sequences (matrix-core GEMMs), random norm parameters and
    biases: the head's 3142 column tiles stream through 256 workgroups, which multiply in
    exact bf16 parts, with the final norm folded into the tied embedding or applied to
    the rows."""
    w = dataclasses.replace(synth.WORKLOADS["gpt2_b32"], batch=6, prompt_len=(2, 30), n_generate=6)
    W = perturb_norms_and_biases(w.shape, synth.make_weights(w.shape, w.init, w.seed), 105)
    prompts = synth.make_prompts(w)
    rep, _, _ = _run_and_compare(w, W, prompts, 1e-3, fold=fold,
                                 config=f"gpt2 124M batch 6, random norms ({'folded' if fold else 'applied'})")
    assert not rep["flips"], rep["flips"]


# Llama layout, small but with a SwiGLU up-projection and a head wide enough (320 and 512
# column tiles) for their workgroups to stream several tiles (bf16 parts)
LLAMA_WIDE_FF = synth.Shape(synth.ARCH_LLAMA, 2, 192, 3, 1, 64, 2560, 8192, 256, 1e-5, 1e5)


def test_llama_wide_mlp_and_head_parts():
    """bf16 weights, 6 rows, paged: the SwiGLU up-projection (5120 rows) and the head
    (8192 rows) run in bf16 parts on the matrix cores, with random norm gains."""
    w = synth.Workload("llama_wide_ff", LLAMA_WIDE_FF, synth.Init(bf16=True), 19, 6, (5, 120), 8, kv_block=16)
    W = perturb_norms_and_biases(w.shape, synth.make_weights(w.shape, w.init, w.seed), 106)
    prompts = synth.make_prompts(w)
    tab, pool = synth.make_block_tables(w, prompts)
    rep, _, _ = _run_and_compare(w, W, prompts, 2e-2, tables=tab, pool=pool, config="llama wide MLP and head (bf16 parts)")
    assert not rep["flips"], rep["flips"]


@pytest.mark.parametrize("wdt", ["f32", "bf16"])
def test_gpt2_124m_batched_short(wdt):
    """GPT-2 124M shape, 5 sequences with ragged prompts, MFMA path for the linears."""
    w = dataclasses.replace(synth.WORKLOADS["gpt2_b32" if wdt == "f32" else "gpt2_b32_bf16"], batch=5,
                            prompt_len=(2, 40), n_generate=6)
    W = synth.make_weights(w.shape, w.init, w.seed)
    prompts = synth.make_prompts(w)
    _run_and_compare(w, W, prompts, 1e-3 if wdt == "f32" else 2e-2)


def test_out_of_range_tokens_on_both_set_up_paths():
    """A token id outside the vocabulary fed on the device is flagged and replaced by 0,
    both where the step's set-up runs inside the QKV launch (2 rows) and where it runs
    as a launch of its own (6 rows); the other rows of the step are unaffected and the
    next steps run normally."""
    import torch
    dev = device()
    w = dataclasses.replace(synth.WORKLOADS["tiny"], batch=6, prompt_len=(3, 12), n_generate=4)
    W = synth.make_weights(w.shape, w.init, w.seed)
    prompts = synth.make_prompts(w)
    V = w.shape.vocab
    om = oracle.Model(w.shape, W)
    m = gd_model(w, W)
    tok = torch.zeros(w.batch, dtype=torch.int32, device=dev)
    ref_next = []
    for b, p in enumerate(prompts):
        m.reset_seq(b)
        m.prefill(b, p, tok[b:b + 1])
        s = om.new_seq(len(p) + 4)
        ref = np.empty(V, np.float32)
        for t in p:
            s.forward(int(t), ref)
        ref_next.append((s, ref))
    torch.cuda.synchronize()
    assert m.device_errors() == 0
    for rows, bad in (([1, 4], 1), ([0, 1, 2, 3, 4, 5], 3)):
        feed = torch.tensor([int(tok[b]) for b in rows], dtype=torch.int32, device=dev)
        feed[bad] = V + 5 if len(rows) == 2 else -3
        out = torch.zeros(len(rows), dtype=torch.int32, device=dev)
        lg = torch.empty((len(rows), V), dtype=torch.float32, device=dev)
        m.decode_step(rows, feed, out, lg)
        torch.cuda.synchronize()
        assert m.device_errors() & 1, rows
        assert m.device_errors() == 0
        for k, b in enumerate(rows):
            s, ref = ref_next[b]
            fed = 0 if k == bad else int(feed[k])      # the replaced id
            nxt = s.forward(fed, ref)
            assert np.max(np.abs(lg[k].cpu().numpy() - ref)) <= 1e-3, (rows, b)
            assert int(out[k]) == nxt
            tok[b] = out[k]
    m.close()


def test_context_edges_and_errors():
    """Position n_ctx-1 runs; one more is refused on the host; bad ids are rejected."""
    import torch
    import transformer_gpt_decode_amd as gd
    dev = device()
    w = synth.WORKLOADS["tiny"]
    W = synth.make_weights(w.shape, w.init, w.seed)
    n_ctx = w.shape.n_ctx
    rng = np.random.default_rng(9)
    prompt = rng.integers(0, w.shape.vocab, size=n_ctx - 1).astype(np.int32)
    m = gd_model(w, W)
    tok = torch.zeros(1, dtype=torch.int32, device=dev)
    logits = torch.empty((2, w.shape.vocab), dtype=torch.float32, device=dev)
    m.prefill(0, prompt, tok, logits[0])
    torch.cuda.synchronize()
    tok0 = int(tok.item())                            # the prefill's greedy token
    m.decode_step([0], tok, tok, logits[1])          # position n_ctx - 1
    torch.cuda.synchronize()
    om = oracle.Model(w.shape, W)
    s = om.new_seq(n_ctx)
    ref = np.empty(w.shape.vocab, np.float32)
    for t in prompt:
        first = s.forward(int(t), ref)
    assert tok0 == int(first)
    r0 = ref.copy()
    second = s.forward(first, ref)
    assert np.max(np.abs(logits[0].cpu().numpy() - r0)) <= 1e-3
    assert np.max(np.abs(logits[1].cpu().numpy() - ref)) <= 1e-3
    assert int(tok.item()) == second
    assert m.seq_len(0) == n_ctx
    with pytest.raises(gd.GdError) as e:
        m.decode_step([0], tok, tok)
    assert e.value.status == gd.GD_ERR_CTX_FULL
    with pytest.raises(gd.GdError) as e:
        m.prefill(0, [1], tok)
    assert e.value.status == gd.GD_ERR_CTX_FULL
    m.reset_seq(0)
    with pytest.raises(gd.GdError) as e:
        m.prefill(0, [w.shape.vocab], tok)
    assert e.value.status == gd.GD_ERR_INVALID
    with pytest.raises(gd.GdError) as e:
        m.prefill(0, [], tok)
    assert e.value.status == gd.GD_ERR_INVALID
    # an out-of-range id fed on the device is flagged and replaced by 0 (no fault)
    m.prefill(0, [3], tok)
    bad = torch.tensor([w.shape.vocab + 5], dtype=torch.int32, device=dev)
    m.decode_step([0], bad, tok)
    assert m.device_errors() & 1
    assert m.device_errors() == 0
    # option values outside the documented sets are refused on the host
    for opt, bad in ((gd.OPT_ATTN_CHUNKS, 2), (gd.OPT_ATTN_CHUNKS, -1), (gd.OPT_ATTN_CHUNKS, 16),
                     (gd.OPT_LINEAR_VARIANT, 3), (gd.OPT_PROFILE, 5), (gd.OPT_PREFILL_BF16_PARTS, 3), (99, 0)):
        with pytest.raises(gd.GdError) as e:
            m.set_option(opt, bad)
        assert e.value.status == gd.GD_ERR_INVALID
    m.close()


@pytest.mark.parametrize("outlier,mean", [(20.0, 5.0), (0.0, 50.0), (200.0, 0.0), (200.0, 50.0)],
                         ids=["outlier20_mean5", "mean50", "outlier200", "outlier200_mean50"])
@pytest.mark.parametrize("fold", [True, False], ids=["folded", "applied"])
def test_gpt2_124m_prenorm_outlier_rows(outlier, mean, fold):
    """Rows where the folded pre-norm's shift (the row's first element) is far from the
    row mean: the learned position table gets `mean` added to every entry and `outlier`
    more on column 0, so every residual row has x0 - mean(x) of about -outlier (up to
    ~7000 times the spread of the other entries) and a large common offset. The folded
    form r((x - x0) . g W - a s) cancels terms of size |a| |s|; both forms must stay
    within 1e-3 of the oracle's double-accumulated LayerNorm."""
    w = dataclasses.replace(synth.WORKLOADS["gpt2_b1"], n_generate=6)
    W = synth.make_weights(w.shape, w.init, w.seed)
    off, shp = synth.offsets(w.shape)["wpe"]
    wpe = W[off:off + int(np.prod(shp))].reshape(shp)
    wpe += np.float32(mean)
    wpe[:, 0] += np.float32(outlier)
    prompts = synth.make_prompts(w)
    rep, _, _ = _run_and_compare(w, W, prompts, 1e-3, fold=fold,
                                 config=f"gpt2_b1 pre-norm rows (outlier {outlier:g}, mean {mean:g}, "
                                        f"{'folded' if fold else 'applied'})")
    assert not rep["flips"], rep["flips"]


# ------------------------------------------------------------- bfloat16 KV cache

@pytest.mark.parametrize("variant", [0, 2], ids=["auto", "mfma"])
def test_tiny_gpt2_kv_bf16(variant):
    """K and V rounded to bf16 as they enter the cache (the oracle rounds the same
    values): contiguous cache, GEMV and MFMA QKV epilogues, fused and split attention."""
    w = synth.Workload("tiny_kv16", synth.TINY, synth.Init(kv_bf16=True), 1, 4, (1, 40), 16)
    W = synth.make_weights(w.shape, w.init, w.seed)
    prompts = synth.make_prompts(w)
    rep, _, _ = _run_and_compare(w, W, prompts, 2e-2, variant, config=f"tiny kv bf16 (variant {variant})")
    assert not rep["flips"]


@pytest.mark.parametrize("mode", ["fused_attn_o", "one_chunk", "eight_chunks"])
def test_llama_hd64_kv_bf16_paged(mode):
    """bf16 KV on a shuffled paged cache with 3 query heads per KV head: the fused
    short-context attention, and split-context attention with one or eight chunks."""
    batch, plen, variant, chunks = {"fused_attn_o": (2, (5, 60), 0, 0), "one_chunk": (6, (5, 200), 2, 1),
                                    "eight_chunks": (6, (5, 200), 2, 8)}[mode]
    w = synth.Workload("llama_hd64_kv16", LLAMA_HD64, synth.Init(bf16=True, kv_bf16=True), 15, batch, plen, 10,
                       kv_block=16)
    W = synth.make_weights(w.shape, w.init, w.seed)
    prompts = synth.make_prompts(w)
    tab, pool = synth.make_block_tables(w, prompts)
    _run_and_compare(w, W, prompts, 2e-2, variant=variant, tables=tab, pool=pool, chunks=chunks,
                     config=f"llama_hd64 kv bf16 ({mode})")


@pytest.mark.parametrize("chunks", [1, 8], ids=["one_chunk", "eight_chunks"])
def test_long_contexts_kv_bf16(chunks):
    """bf16 KV at ragged contexts up to ~900 positions on the contiguous cache, the
    one-chunk attention fused with the output projection and the eight-chunk scan."""
    w = synth.Workload("gpt2_hd64_long_kv16", GPT2_HD64_LONG, synth.Init(kv_bf16=True), 16, 5, (1, 880), 6)
    W = synth.make_weights(w.shape, w.init, w.seed)
    prompts = synth.make_prompts(w)
    _run_and_compare(w, W, prompts, 2e-2, variant=2, chunks=chunks, config=f"gpt2_hd64_long kv bf16 ({chunks} chunks)")


# A small Llama-style model with contexts far past 1280 positions
LLAMA_LONG_SMALL = synth.Shape(synth.ARCH_LLAMA, 2, 192, 3, 1, 64, 256, 300, 4096, 1e-5, 1e5)


@pytest.mark.parametrize("kv", ["f32", "bf16", "q8_weights"])
def test_llama_contexts_past_1280(kv):
    """Split-context paged attention at 1300-3800 positions (n_ctx 4096), float or bf16
    KV, or 8-bit weights; shuffled block tables; the rows at different lengths share
    each step (32 chunks per row, merged by a launch of their own)."""
    q8 = kv == "q8_weights"
    init = synth.Init(q8=True) if q8 else synth.Init(bf16=True, kv_bf16=kv == "bf16")
    w = synth.Workload("llama_long_small", LLAMA_LONG_SMALL, init, 17, 2, (1300, 3800), 6, kv_block=16)
    W = synth.make_weights(w.shape, w.init, w.seed)
    prompts = synth.make_prompts(w)
    tab, pool = synth.make_block_tables(w, prompts)
    _run_and_compare(w, W, prompts, 1e-3 if q8 else 2e-2, tables=tab, pool=pool, config=f"llama long contexts ({kv})")


# ----------------------------------------------------------------- 8-bit weights

@pytest.mark.parametrize("batch", [1, 3, 6])
def test_tiny_gpt2_q8(batch):
    """8-bit block weights (quantized at load by the library; the oracle quantizes the
    same float weights itself): every matrix including the tied embedding and the
    position table, one launch of up to 4 rows or two."""
    w = synth.Workload("tiny_q8", synth.TINY, synth.Init(q8=True), 1, batch, (1, 30), 16)
    W = synth.make_weights(w.shape, w.init, w.seed)
    prompts = synth.make_prompts(w)
    rep, _, _ = _run_and_compare(w, W, prompts, 1e-3, config=f"tiny q8 (batch {batch})")
    assert not rep["flips"]


@pytest.mark.parametrize("kv", ["f32", "bf16"])
def test_llama_hd64_q8_paged(kv):
    """8-bit weights in the Llama layout (RoPE row pairs and gate/up rows interleaved at
    load, untied head), 3 query heads per KV head, shuffled paged cache."""
    w = synth.Workload("llama_hd64_q8", LLAMA_HD64, synth.Init(q8=True, kv_bf16=kv == "bf16"), 18, 3, (5, 300), 8,
                       kv_block=16)
    W = synth.make_weights(w.shape, w.init, w.seed)
    prompts = synth.make_prompts(w)
    tab, pool = synth.make_block_tables(w, prompts)
    _run_and_compare(w, W, prompts, 1e-3 if kv == "f32" else 2e-2, tables=tab, pool=pool,
                     config=f"llama_hd64 q8 ({kv} KV)")


def test_gpt2_124m_q8_batch1():
    """GPT-2 124M shape with 8-bit weights, batch 1, 8 prompt ids, 128 tokens: every
    logit of every step against the oracle."""
    w = synth.WORKLOADS["gpt2_b1_q8"]
    W = synth.make_weights(w.shape, w.init, w.seed)
    prompts = synth.make_prompts(w)
    rep, _, _ = _run_and_compare(w, W, prompts, 1e-3, config="gpt2_b1_q8")
    assert not rep["flips"], rep["flips"]


# ---------------------------------------------------------------------- sampling

@pytest.mark.parametrize("temp,top_k", [(0.8, 20), (1.5, 256), (0.3, 2)])
def test_tiny_gpt2_sampling(temp, top_k):
    """Temperature / top-k draws on the GPU (Philox4x64-10 uniforms keyed by seed,
    sequence slot and position) against the oracle's, token by token; three sequences
    decoded together, the first token drawn from the prefill's last row."""
    w = synth.Workload("tiny_sample", synth.TINY, synth.Init(), 1, 3, (1, 30), 24, sampling=(temp, top_k, 99))
    W = synth.make_weights(w.shape, w.init, w.seed)
    prompts = synth.make_prompts(w)
    rep, tok, _ = _run_and_compare(w, W, prompts, 1e-3, config=f"tiny sampled (T {temp}, top-{top_k})")
    assert len(set(tok.ravel().tolist())) > 3   # the draws spread over several tokens


def test_sampling_greedy_special_cases_and_nan():
    """top_k == 1 or temperature 0 is the greedy argmax; a NaN logit wins (first NaN)."""
    import torch
    import transformer_gpt_decode_amd as gd
    w = synth.WORKLOADS["tiny"]
    W = synth.make_weights(w.shape, w.init, w.seed)
    prompts = synth.make_prompts(w)
    ref_tok, _ = oracle_generate(w, W, prompts)
    for temp, k in ((0.7, 1), (0.0, 40)):
        m = gd_model(w, W)
        m.set_sampling(temp, k, 5)
        tok, _ = gpu_generate(m, prompts, w.n_generate)
        assert np.array_equal(tok, ref_tok)
        m.close()
    m = gd_model(w, W)
    for bad in ((0.7, 0), (0.7, 257), (float("nan"), 5)):
        with pytest.raises(gd.GdError) as e:
            m.set_sampling(*bad, 1)
        assert e.value.status == gd.GD_ERR_INVALID
    # NaN among the logits: an embedding row of NaNs through a 1-layer model is not
    # needed; the sampler's NaN rule is reached with NaN weights in the head instead
    Wn = W.copy()
    o, shp = synth.offsets(w.shape)["wte"]
    Wn[o + 77 * shp[1]:o + 78 * shp[1]] = np.nan   # row 77 of the tied embedding: logit 77 is NaN
    m2 = gd_model(w, Wn)
    m2.set_sampling(0.9, 30, 1)
    dev = device()
    t = torch.zeros(1, dtype=torch.int32, device=dev)
    m2.prefill(0, [1, 2, 3], t)
    torch.cuda.synchronize()
    assert int(t.item()) == 77
    m.close()
    m2.close()


def test_gpt2_124m_sampled_batch1():
    """GPT-2 124M shape, batch 1, temperature 0.7, top-k 40 (the batch_forge demo's
    temperature): 128 sampled tokens against the oracle's draws."""
    w = synth.WORKLOADS["gpt2_b1_sample"]
    W = synth.make_weights(w.shape, w.init, w.seed)
    prompts = synth.make_prompts(w)
    _run_and_compare(w, W, prompts, 1e-3, config="gpt2_b1 sampled (T 0.7, top-40)")


def test_llama_hd64_sampled_paged():
    """Sampling on the Llama layout (untied head, paged cache, 5 sequences)."""
    w = synth.Workload("llama_hd64_sample", LLAMA_HD64, synth.Init(bf16=True), 19, 5, (5, 100), 12, kv_block=16,
                       sampling=(1.0, 50, 7))
    W = synth.make_weights(w.shape, w.init, w.seed)
    prompts = synth.make_prompts(w)
    tab, pool = synth.make_block_tables(w, prompts)
    _run_and_compare(w, W, prompts, 2e-2, tables=tab, pool=pool, config="llama_hd64 sampled (T 1, top-50)")


# ------------------------------------------------------------- tiled prompt pass

@pytest.mark.parametrize("kv", ["f32", "bf16"])
@pytest.mark.parametrize("wdt", ["f32", "bf16"])
def test_tiled_prefill_gpt2(wdt, kv):
    """Prompts of 64-1000 ids take the tiled prompt pass (64 x 64 matrix-core GEMM tiles,
    tiled causal attention; two 512-row chunks past 512 ids, ragged last tiles), then
    decode; the first token and its logits come from the pass's last row."""
    w = synth.Workload("gpt2_hd64_prefill", GPT2_HD64_LONG, synth.Init(bf16=wdt == "bf16", kv_bf16=kv == "bf16"), 20,
                       4, (64, 1000), 6)
    W = synth.make_weights(w.shape, w.init, w.seed)
    prompts = synth.make_prompts(w)
    _run_and_compare(w, W, prompts, 1e-3 if (wdt, kv) == ("f32", "f32") else 2e-2,
                     config=f"tiled prefill gpt2 ({wdt} weights, {kv} KV)")


@pytest.mark.parametrize("parts", [2, 0], ids=["bf16_parts", "fp32_mfma"])
@pytest.mark.parametrize("wdt", ["f32", "bf16"])
def test_tiled_prefill_split_edges(wdt, parts):
    """Prompt lengths at the key-tile edges of the tiled pass: 64 ids (one key tile, the
    attention written unsplit), 65 and 128 (two tiles: one query tile's second split
    empty), 191 (three tiles, ragged last query tile); the GEMM products in bf16 parts
    (the default) and on the fp32 matrix cores."""
    import transformer_gpt_decode_amd as gd
    w = synth.Workload("gpt2_hd64_prefill_edges", GPT2_HD64_LONG, synth.Init(bf16=wdt == "bf16"), 23, 4, (191, 191), 6)
    W = synth.make_weights(w.shape, w.init, w.seed)
    full = synth.make_prompts(w)
    prompts = [full[0][:64], full[1][:65], full[2][:128], full[3][:191]]
    ref_tok, ref_lg = oracle_generate(w, W, prompts)
    m = gd_model(w, W)
    m.set_option(gd.OPT_PREFILL_BF16_PARTS, parts)
    tok, lg = gpu_generate(m, prompts, w.n_generate)
    assert m.device_errors() == 0
    rep = compare_generation(tok, lg, ref_tok, ref_lg, 1e-3 if wdt == "f32" else 2e-2,
                             f"tiled prefill gpt2 ({wdt} weights, {'bf16 parts' if parts else 'fp32 MFMA'}; 64, 65, 128, 191 ids)",
                             plens=[len(p) for p in prompts], tie=near_tie_margin(w))
    assert not rep["flips"]
    m.close()


def test_tiled_prefill_llama_long_paged():
    """Llama layout (RoPE in the QKV GEMM epilogue, 3 query heads per KV head, SwiGLU),
    shuffled paged bf16 cache, prompts of 600-2000 ids: up to four 512-row chunks, each
    attending to the positions the earlier chunks cached."""
    w = synth.Workload("llama_long_prefill", LLAMA_LONG_SMALL, synth.Init(bf16=True, kv_bf16=True), 21, 2,
                       (600, 2000), 6, kv_block=16)
    W = synth.make_weights(w.shape, w.init, w.seed)
    prompts = synth.make_prompts(w)
    tab, pool = synth.make_block_tables(w, prompts)
    _run_and_compare(w, W, prompts, 2e-2, tables=tab, pool=pool, config="tiled prefill llama (paged, bf16 KV)")


def test_prefill_in_two_calls():
    """A prompt prefilled in two calls (100 ids, then 260 more at positions 100..359:
    the second call's tiled pass attends to the first call's cache) equals the oracle
    run over the whole prompt; short prompts (< 64 ids) keep the decode kernels."""
    import torch
    w = synth.Workload("gpt2_hd64_prefill2", GPT2_HD64_LONG, synth.Init(), 22, 1, (360, 360), 8)
    W = synth.make_weights(w.shape, w.init, w.seed)
    prompt = synth.make_prompts(w)[0]
    ref_tok, ref_lg = oracle_generate(w, W, [prompt])
    m = gd_model(w, W)
    dev = device()
    tok = torch.zeros(1, dtype=torch.int32, device=dev)
    lg = torch.empty((w.n_generate, w.shape.vocab), dtype=torch.float32, device=dev)
    m.reset_seq(0)
    m.prefill(0, prompt[:100], tok)
    m.prefill(0, prompt[100:], tok, lg[0])
    out = [tok.clone()]
    step = torch.empty((1, w.shape.vocab), dtype=torch.float32, device=dev)
    for i in range(1, w.n_generate):
        m.decode_step([0], tok, tok, step)
        lg[i].copy_(step[0])
        out.append(tok.clone())
    torch.cuda.synchronize()
    got = torch.cat(out).cpu().numpy()[None]
    rep = compare_generation(got, lg.cpu().numpy()[None], ref_tok, ref_lg, 1e-3, "prefill in two calls")
    assert not rep["flips"]
    m.close()


# ------------------------------------------------------- replays and the NaN rule

def _replay_logits(m, plens, toks, n, dev):
    """Logits of the same decode step (every sequence rewound to its prompt end and fed
    the same token) replayed n times, as one [n][B][V] array."""
    import torch
    B = len(plens)
    out = []
    tok = torch.tensor(toks, dtype=torch.int32, device=dev)
    nxt = torch.empty(B, dtype=torch.int32, device=dev)
    lg = torch.empty((B, m.cfg.vocab), dtype=torch.float32, device=dev)
    for _ in range(n):
        for b, p in enumerate(plens):
            m.truncate_seq(b, p)
        m.decode_step(list(range(B)), tok, nxt, lg)
        out.append(lg.cpu().numpy().copy())
    return np.stack(out)


@pytest.mark.parametrize("fuse", [0, 1], ids=["unfused", "fused"])
def test_replay_determinism_batch1(fuse):
    """GPT-2 124M shape, batch 1: one decode step replayed 100 times (one hipGraph). With
    attention and the output projection in separate launches no float atomic is left and
    the logits must be bitwise identical; the fused attention adds the heads' shares of
    the projection with atomics in any order, so replays may differ in the last bits
    (bounded here by 1e-5)."""
    import transformer_gpt_decode_amd as gd
    w = synth.WORKLOADS["gpt2_b1"]
    W = synth.make_weights(w.shape, w.init, w.seed)
    prompts = synth.make_prompts(w)
    m = gd_model(w, W)
    m.set_option(gd.OPT_FUSE_ATTN_O, fuse)
    dev = device()
    import torch
    t = torch.zeros(1, dtype=torch.int32, device=dev)
    m.prefill(0, prompts[0], t)
    lg = _replay_logits(m, [len(prompts[0])], [int(t.item())], 100, dev)
    assert m.device_errors() == 0 and np.all(np.isfinite(lg))
    d = float(np.max(np.abs(lg - lg[0])))
    print(f"batch-1 replays (fuse {fuse}): max |dlogit| across 100 replays {d:.3e}", flush=True)
    if fuse == 0:
        assert d == 0.0, d
    else:
        assert d <= 1e-5, d
    m.close()


def test_replay_spread_batch32():
    """GPT-2 124M shape, 32 sequences: one decode step replayed 20 times. The split-K
    matrix-core GEMMs and the fused attention + projection add with float atomics, so
    replays may differ in the last bits; the spread is bounded (1e-5) and the greedy
    tokens equal in every replay."""
    w = synth.WORKLOADS["gpt2_b32"]
    W = synth.make_weights(w.shape, w.init, w.seed)
    prompts = synth.make_prompts(w)
    m = gd_model(w, W)
    dev = device()
    import torch
    t = torch.zeros(w.batch, dtype=torch.int32, device=dev)
    for b, p in enumerate(prompts):
        m.prefill(b, p, t[b:b + 1])
    lg = _replay_logits(m, [len(p) for p in prompts], t.cpu().tolist(), 20, dev)
    assert m.device_errors() == 0 and np.all(np.isfinite(lg))
    d = float(np.max(np.abs(lg - lg[0])))
    print(f"batch-32 replays: max |dlogit| across 20 replays {d:.3e}", flush=True)
    assert d <= 1e-5, d
    am = np.argmax(lg, axis=2)
    assert np.all(am == am[0])
    m.close()


def test_greedy_head_nan_rule():
    """Row 77 of the tied embedding set to NaN makes logit 77 NaN in every row: the greedy
    argmax of the fused head returns 77 for one row (GEMV head, decode-kernel prefill),
    for six rows fed finite tokens (matrix-core head) and after a 70-id prompt (tiled
    prompt pass); a row whose logits are all NaN (token 77 fed back) returns index 0, the
    first NaN."""
    import torch
    w = synth.Workload("gpt2_hd64_nan", GPT2_HD64_LONG, synth.Init(), 24, 6, (70, 70), 2)
    W = synth.make_weights(w.shape, w.init, w.seed)
    o, shp = synth.offsets(w.shape)["wte"]
    W[o + 77 * shp[1]:o + 78 * shp[1]] = np.nan
    prompts = [[78 if x == 77 else int(x) for x in p] for p in synth.make_prompts(w)]   # finite embeddings
    m = gd_model(w, W)
    dev = device()
    t = torch.zeros(w.batch, dtype=torch.int32, device=dev)
    m.prefill(0, prompts[0][:5], t[0:1])          # decode kernels, one row
    m.prefill(1, prompts[1], t[1:2])              # tiled prompt pass (70 ids)
    for b in range(2, w.batch):
        m.prefill(b, prompts[b][:3 + b], t[b:b + 1])
    torch.cuda.synchronize()
    assert t.cpu().tolist() == [77] * w.batch
    # six rows fed finite tokens: the matrix-core head
    feed = torch.tensor([1, 2, 3, 4, 5, 6], dtype=torch.int32, device=dev)
    nxt = torch.empty(w.batch, dtype=torch.int32, device=dev)
    m.decode_step(list(range(w.batch)), feed, nxt)
    torch.cuda.synchronize()
    assert nxt.cpu().tolist() == [77] * w.batch
    # token 77 fed back: its NaN embedding makes every logit NaN -> the first NaN, 0
    m.decode_step([0], nxt[0:1], nxt[0:1])
    torch.cuda.synchronize()
    assert int(nxt[0].item()) == 0
    assert m.device_errors() == 0
    m.close()


@pytest.mark.parametrize("fold", [True, False], ids=["in_gemm", "rownorm"])
@pytest.mark.parametrize("arch", ["gpt2", "llama"])
def test_tiled_prefill_prenorm(arch, fold):
    """The tiled prompt pass with its pre-norms inside the GEMMs (LayerNorm through the
    folded fp32 weights, RMSNorm with the gains applied as the tiles are staged) and
    applied to the rows first (k_rownorm): random norm gains, shifts and biases, and
    residual rows with a far-off first element and a large common offset (the folded
    LayerNorm shifts by the first element); 96- and 200-id prompts."""
    if arch == "gpt2":
        w = synth.Workload("gpt2_hd64_prefill_norm", GPT2_HD64_LONG, synth.Init(), 25, 2, (96, 200), 4)
    else:
        w = synth.Workload("llama_prefill_norm", LLAMA_HD64, synth.Init(), 25, 2, (96, 200), 4)
    W = perturb_norms_and_biases(w.shape, synth.make_weights(w.shape, w.init, w.seed), 26)
    name = "wpe" if arch == "gpt2" else "wte"
    off, shp = synth.offsets(w.shape)[name]
    tab = W[off:off + int(np.prod(shp))].reshape(shp)
    tab += np.float32(5.0)
    tab[:, 0] += np.float32(20.0)
    prompts = synth.make_prompts(w)
    rep, _, _ = _run_and_compare(w, W, prompts, 1e-3, fold=fold,
                                 config=f"tiled prefill {arch} pre-norm ({'in the GEMMs' if fold else 'rownorm'}, "
                                        f"random norms, offset rows)")
    assert not rep["flips"], rep["flips"]
