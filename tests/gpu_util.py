"""Helpers for the GPU tests: device, workloads through the HIP library, parity checks."""
from __future__ import annotations

import numpy as np

import oracle
import synth


def device():
    import torch
    assert torch.cuda.is_available(), "GPU tests need an MI355X (gfx950) device; select them with -m gpu"
    import transformer_gpt_decode_amd as gd
    gd.lib()   # fails loudly if the HIP library is missing
    return torch.device("cuda", 0)


def gd_model(workload, W, max_seqs=None, max_batch=None, pool_blocks=None, variant=0, graph=True, persistent=False,
             fold=True, mlp=False, chunks=0):
    import transformer_gpt_decode_amd as gd
    s = workload.shape
    kw = dict(max_seqs=max_seqs or workload.batch, max_batch=max_batch or workload.batch)
    if workload.kv_block:
        kw.update(kv_block_size=workload.kv_block, kv_num_blocks=pool_blocks)
    m = gd.Model.from_shape(s, gd.WEIGHT_BF16 if workload.init.bf16 else gd.WEIGHT_F32, **kw)
    m.load_weights(W)
    m.set_option(gd.OPT_LINEAR_VARIANT, variant)
    m.set_option(gd.OPT_USE_GRAPH, 1 if graph else 0)
    m.set_option(gd.OPT_PERSISTENT, 1 if persistent else 0)
    m.set_option(gd.OPT_FOLD_NORM, 1 if fold else 0)
    m.set_option(gd.OPT_FUSE_MLP, 1 if mlp else 0)
    m.set_option(gd.OPT_ATTN_CHUNKS, chunks)
    return m


def perturb_norms_and_biases(shape, W, seed):
    """A copy of W whose norm gains are 1 + 0.2 N(0, 1) and whose norm shifts and
    biases are 0.1 N(0, 1) (synth draws them constant: 1 and 0)."""
    import synth
    rng = np.random.default_rng(seed)
    W = W.copy()
    off = 0
    for name, shp, kind in synth.tensor_list(shape):
        n = int(np.prod(shp))
        if kind == "g":
            W[off:off + n] = 1.0 + 0.2 * rng.standard_normal(n, dtype=np.float32)
        elif kind == "b":
            W[off:off + n] = 0.1 * rng.standard_normal(n, dtype=np.float32)
        off += n
    return W


def gpu_generate(m, prompts, n_generate, tables=None, want_logits=True, forced=None):
    """Prefill each sequence, then n_generate-1 batched greedy decode steps fed on the device.

    Returns tokens [B][n_generate] and (optionally) logits [B][n_generate][V] as numpy.
    With ``forced`` ([B][n_generate]) the fed tokens are forced[b][i-1] (teacher forcing).
    """
    import torch
    dev = device()
    B = len(prompts)
    V = m.cfg.vocab
    if tables is not None:
        for b in range(B):
            m.set_block_table(b, tables[b][tables[b] >= 0])
    tok = torch.zeros(B, dtype=torch.int32, device=dev)
    logits = torch.empty((n_generate, B, V), dtype=torch.float32, device=dev) if want_logits else None
    for b, p in enumerate(prompts):
        m.reset_seq(b)
        m.prefill(b, p, tok[b:b + 1], logits[0, b] if want_logits else None)
    toks = [tok.clone()]
    forced_dev = None
    if forced is not None:
        forced_dev = torch.as_tensor(np.ascontiguousarray(np.asarray(forced, np.int32).T), device=dev)
    feed = torch.zeros(B, dtype=torch.int32, device=dev)
    for i in range(1, n_generate):
        if forced_dev is not None:
            feed.copy_(forced_dev[i - 1])
            m.decode_step(list(range(B)), feed, tok, logits[i] if want_logits else None)
        else:
            m.decode_step(list(range(B)), tok, tok, logits[i] if want_logits else None)
        toks.append(tok.clone())
    torch.cuda.synchronize()
    t = torch.stack(toks, 1).cpu().numpy()
    lg = logits.permute(1, 0, 2).cpu().numpy() if want_logits else None
    return t, lg


def oracle_generate(workload, W, prompts, n_generate=None, forced=None):
    om = oracle.Model(workload.shape, W)
    n = n_generate or workload.n_generate
    toks, lgs = [], []
    for b, p in enumerate(prompts):
        t, lg = oracle.generate(om, p, n, want_logits=True, forced=None if forced is None else forced[b])
        toks.append(t)
        lgs.append(lg)
    return np.stack(toks), np.stack(lgs)


def top2_margin(logits: np.ndarray) -> float:
    s = np.sort(logits.astype(np.float64))
    return float(s[-1] - s[-2])


def compare_generation(gpu_tok, gpu_lg, ref_tok, ref_lg, tol):
    """Parity bar: identical greedy tokens and |dlogit| <= tol at every step of every
    sequence. A token flip is tolerated only as a near tie: the oracle's top-2 margin at
    that step is at most twice the max |dlogit| seen up to it. Returns a report dict."""
    B, n = ref_tok.shape
    rep = {"max_dlogit": 0.0, "near_ties": [], "first_divergence": None}
    for b in range(B):
        seen = 0.0
        for i in range(n):
            d = float(np.max(np.abs(gpu_lg[b, i] - ref_lg[b, i])))
            seen = max(seen, d)
            rep["max_dlogit"] = max(rep["max_dlogit"], d)
            assert np.all(np.isfinite(gpu_lg[b, i])), f"non-finite logits seq {b} step {i}"
            assert d <= tol, f"seq {b} step {i}: max |dlogit| {d:.3e} > {tol}"
            if gpu_tok[b, i] != ref_tok[b, i]:
                m = top2_margin(ref_lg[b, i])
                assert m <= 2 * seen, f"seq {b} step {i}: token {gpu_tok[b, i]} != {ref_tok[b, i]}, margin {m:.3e}"
                rep["near_ties"].append((b, i, m))
                if rep["first_divergence"] is None:
                    rep["first_divergence"] = (b, i)
                break   # later steps of this sequence are compared teacher-forced by the caller
    return rep
