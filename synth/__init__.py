"""Seeded synthetic inputs shared by the oracle and the HIP path.

This module holds the workload shapes, the weight draws, the prompts and the
paged block tables. It contains none of the forward pass's arithmetic: both the
CPU oracle and the GPU library consume the exact bytes produced here.

Workloads (sizes as named by the model shapes they stand in for):

* ``tiny``         2-layer GPT-2-style decoder, d 64, 4 heads x 16, ff 256, vocab 512,
                   n_ctx 64; batch 1, 8 prompt ids, 16 generated tokens.
* ``gpt2_b1``      GPT-2 124M shape (12 x 768, 12 heads, ff 3072, vocab 50257, n_ctx
                   1024); batch 1, 8 prompt ids, 128 generated tokens.
* ``gpt2_stress``  the same shape with MLP c_fc weights ~N(0, 0.5) (drives GELU
                   pre-activations far beyond the tanh overflow point); batch 1,
                   512 prompt ids, 512 generated tokens (sequence reaches n_ctx).
* ``gpt2_b32`` / ``gpt2_b32_bf16``  batch 32, prompt lengths uniform in [16, 512],
                   256 generated tokens each; fp32 or bf16 weight storage.
* ``llama_b8``     Llama-style decoder: 32 layers, d 960, 15 query / 5 KV heads x 64,
                   SiLU-gated MLP 2560, RMSNorm, RoPE theta 1e5, vocab 49152, untied
                   head, bf16 weights; paged KV (block 16, shuffled tables); batch 8,
                   prompt lengths uniform in [32, 1024], 256 generated tokens.
* ``gpt2_b32_kv16`` the batch-32 GPT-2 workload with a bfloat16 KV cache.
* ``llama_long``   the Llama-style shape at n_ctx 4096 with a bfloat16 paged KV cache:
                   batch 4, prompt lengths uniform in [1536, 3840], 128 generated.
* ``gpt2_b1_q8``   the batch-1 GPT-2 workload with 8-bit block-quantized weights.
* ``gpt2_b1_sample`` the batch-1 GPT-2 workload sampled at temperature 0.7, top-k 40.

Draw rules: ``numpy.random.default_rng(seed)`` (PCG64) for weights, drawn in the
canonical tensor order below with ``standard_normal(dtype=float32) * sigma``;
tensors that are constant (biases 0, norm gains 1, norm shifts 0) consume no draws.
Prompts use ``default_rng(seed + 1)``: first the batch's prompt lengths (when they
are ranged), then each sequence's ids in turn. Paged block assignments use
``default_rng(seed + 2)``. Closed ranges ``[a, b]`` include ``b``.

Canonical weight order (float32, row-major, ``[out][in]`` for every matrix):

GPT-2 style: ``wte [V][d]``, ``wpe [n_ctx][d]``, then per layer ``ln1_g [d]``,
``ln1_b [d]``, ``w_qkv [3d][d]``, ``b_qkv [3d]``, ``w_o [d][d]``, ``b_o [d]``,
``ln2_g [d]``, ``ln2_b [d]``, ``w_fc [ff][d]``, ``b_fc [ff]``, ``w_proj [d][ff]``,
``b_proj [d]``; then ``lnf_g [d]``, ``lnf_b [d]``.

Llama style: ``wte [V][d]``, then per layer ``rms1 [d]``, ``w_q [Hq*hd][d]``,
``w_k [Hkv*hd][d]``, ``w_v [Hkv*hd][d]``, ``w_o [d][Hq*hd]``, ``rms2 [d]``,
``w_gate [ff][d]``, ``w_up [ff][d]``, ``w_down [d][ff]``; then ``rmsf [d]``,
``w_head [V][d]``.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Tuple

import numpy as np

ARCH_GPT2 = 0
ARCH_LLAMA = 1


@dataclasses.dataclass(frozen=True)
class Shape:
    arch: int
    n_layer: int
    d_model: int
    n_head: int
    n_kv_head: int
    head_dim: int
    d_ff: int
    vocab: int
    n_ctx: int
    norm_eps: float = 1e-5
    rope_theta: float = 0.0


@dataclasses.dataclass(frozen=True)
class Init:
    sigma: float = 0.02
    resid_sigma: Optional[float] = None   # sigma of w_o / w_proj (GPT-2 residual scaling)
    fc_sigma: Optional[float] = None      # sigma of w_fc (activation-stress init)
    bf16: bool = False                    # weight matrices rounded to bf16 (RNE)
    q8: bool = False                      # weight matrices in 8-bit blocks of 32 (quantized by each side)
    kv_bf16: bool = False                 # K and V rounded to bf16 as they enter the cache


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    shape: Shape
    init: Init
    seed: int
    batch: int
    prompt_len: Tuple[int, int]           # closed range [lo, hi]; lo == hi means fixed
    n_generate: int                       # generated tokens per sequence (argmax count)
    kv_block: int = 0                     # 0: contiguous per-sequence cache; else paged
    sampling: Optional[Tuple[float, int, int]] = None   # (temperature, top_k, seed); None: greedy

    @property
    def weight_dtype(self) -> str:
        return "bf16" if self.init.bf16 else ("q8" if self.init.q8 else "f32")


GPT2_124M = Shape(ARCH_GPT2, 12, 768, 12, 12, 64, 3072, 50257, 1024)
TINY = Shape(ARCH_GPT2, 2, 64, 4, 4, 16, 256, 512, 64)
# n_ctx of the Llama-style shape: longest prompt (1024) plus 256 generated tokens.
LLAMA_360M = Shape(ARCH_LLAMA, 32, 960, 15, 5, 64, 2560, 49152, 1280, 1e-5, 1e5)
LLAMA_360M_4K = Shape(ARCH_LLAMA, 32, 960, 15, 5, 64, 2560, 49152, 4096, 1e-5, 1e5)

_RESID = 0.02 / math.sqrt(24.0)

WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload("tiny", TINY, Init(), 1, 1, (8, 8), 16),
    "gpt2_b1": Workload("gpt2_b1", GPT2_124M, Init(resid_sigma=_RESID), 2, 1, (8, 8), 128),
    "gpt2_stress": Workload("gpt2_stress", GPT2_124M, Init(resid_sigma=_RESID, fc_sigma=0.5), 3, 1,
                            (512, 512), 512),
    "gpt2_b32": Workload("gpt2_b32", GPT2_124M, Init(resid_sigma=_RESID), 4, 32, (16, 512), 256),
    "gpt2_b32_bf16": Workload("gpt2_b32_bf16", GPT2_124M, Init(resid_sigma=_RESID, bf16=True), 4, 32,
                              (16, 512), 256),
    "llama_b8": Workload("llama_b8", LLAMA_360M, Init(bf16=True), 5, 8, (32, 1024), 256, kv_block=16),
    "gpt2_b32_kv16": Workload("gpt2_b32_kv16", GPT2_124M, Init(resid_sigma=_RESID, kv_bf16=True), 4, 32,
                              (16, 512), 256),
    "llama_long": Workload("llama_long", LLAMA_360M_4K, Init(bf16=True, kv_bf16=True), 6, 4, (1536, 3840), 128,
                           kv_block=16),
    "gpt2_b1_q8": Workload("gpt2_b1_q8", GPT2_124M, Init(resid_sigma=_RESID, q8=True), 2, 1, (8, 8), 128),
    "gpt2_b1_sample": Workload("gpt2_b1_sample", GPT2_124M, Init(resid_sigma=_RESID), 2, 1, (8, 8), 128,
                               sampling=(0.7, 40, 2024)),
}


def tensor_list(s: Shape) -> List[Tuple[str, Tuple[int, ...], str]]:
    """Canonical (name, shape, kind) list; kind is 'w' (drawn matrix), 'b' (zeros) or 'g' (ones)."""
    d, ff, V = s.d_model, s.d_ff, s.vocab
    out: List[Tuple[str, Tuple[int, ...], str]] = []
    if s.arch == ARCH_GPT2:
        out.append(("wte", (V, d), "w"))
        out.append(("wpe", (s.n_ctx, d), "w"))
        for l in range(s.n_layer):
            p = f"h{l}."
            out += [(p + "ln1_g", (d,), "g"), (p + "ln1_b", (d,), "b"),
                    (p + "w_qkv", (3 * d, d), "w"), (p + "b_qkv", (3 * d,), "b"),
                    (p + "w_o", (d, d), "w"), (p + "b_o", (d,), "b"),
                    (p + "ln2_g", (d,), "g"), (p + "ln2_b", (d,), "b"),
                    (p + "w_fc", (ff, d), "w"), (p + "b_fc", (ff,), "b"),
                    (p + "w_proj", (d, ff), "w"), (p + "b_proj", (d,), "b")]
        out += [("lnf_g", (d,), "g"), ("lnf_b", (d,), "b")]
    else:
        hq, hk, hd = s.n_head, s.n_kv_head, s.head_dim
        out.append(("wte", (V, d), "w"))
        for l in range(s.n_layer):
            p = f"h{l}."
            out += [(p + "rms1", (d,), "g"),
                    (p + "w_q", (hq * hd, d), "w"), (p + "w_k", (hk * hd, d), "w"),
                    (p + "w_v", (hk * hd, d), "w"), (p + "w_o", (d, hq * hd), "w"),
                    (p + "rms2", (d,), "g"),
                    (p + "w_gate", (ff, d), "w"), (p + "w_up", (ff, d), "w"),
                    (p + "w_down", (d, ff), "w")]
        out += [("rmsf", (d,), "g"), ("w_head", (V, d), "w")]
    return out


def weight_count(s: Shape) -> int:
    return sum(int(np.prod(shp)) for _, shp, _ in tensor_list(s))


def offsets(s: Shape) -> Dict[str, Tuple[int, Tuple[int, ...]]]:
    """Float offset and shape of every tensor inside the packed canonical buffer."""
    res, off = {}, 0
    for name, shp, _ in tensor_list(s):
        res[name] = (off, shp)
        off += int(np.prod(shp))
    return res


def round_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even), returned as float32."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def _sigma_for(name: str, init: Init) -> float:
    base = name.split(".")[-1]
    if base in ("w_o", "w_proj") and init.resid_sigma is not None:
        return init.resid_sigma
    if base == "w_fc" and init.fc_sigma is not None:
        return init.fc_sigma
    return init.sigma


def make_weights(s: Shape, init: Init, seed: int) -> np.ndarray:
    """Packed canonical float32 weights drawn from ``default_rng(seed)``.

    For bf16 variants every drawn matrix is rounded to bf16 (RNE); the returned
    float32 values are then exactly representable in bf16, and both sides use them.
    """
    rng = np.random.default_rng(seed)
    buf = np.empty(weight_count(s), dtype=np.float32)
    off = 0
    for name, shp, kind in tensor_list(s):
        n = int(np.prod(shp))
        view = buf[off:off + n]
        if kind == "w":
            view[:] = rng.standard_normal(n, dtype=np.float32)
            view *= np.float32(_sigma_for(name, init))
            if init.bf16:
                view[:] = round_bf16(view)
        elif kind == "g":
            view[:] = 1.0
        else:
            view[:] = 0.0
        off += n
    return buf


def make_prompts(w: Workload) -> List[np.ndarray]:
    """Per-sequence int32 prompt ids from ``default_rng(seed + 1)``."""
    rng = np.random.default_rng(w.seed + 1)
    lo, hi = w.prompt_len
    if lo == hi:
        lens = [lo] * w.batch
    else:
        lens = [int(x) for x in rng.integers(lo, hi + 1, size=w.batch)]
    return [rng.integers(0, w.shape.vocab, size=n).astype(np.int32) for n in lens]


def seq_capacity(w: Workload, prompt_len: int) -> int:
    """Positions a sequence needs: prompt plus generated tokens (last one never fed back)."""
    return prompt_len + w.n_generate - 1


def make_block_tables(w: Workload, prompts: List[np.ndarray]) -> Tuple[np.ndarray, int]:
    """Shuffled paged-KV block tables [batch][max_blocks] (-1 = unused) and the pool size.

    Each sequence gets ceil(capacity / block) blocks, drawn without replacement
    from a permutation of the pool made with ``default_rng(seed + 2)``.
    """
    assert w.kv_block > 0
    B = w.kv_block
    need = [-(-seq_capacity(w, len(p)) // B) for p in prompts]
    pool = int(sum(need))
    perm = np.random.default_rng(w.seed + 2).permutation(pool).astype(np.int32)
    max_blocks = -(-w.shape.n_ctx // B)
    tab = np.full((len(prompts), max_blocks), -1, dtype=np.int32)
    o = 0
    for i, n in enumerate(need):
        tab[i, :n] = perm[o:o + n]
        o += n
    return tab, pool


def identity_block_tables(w: Workload, prompts: List[np.ndarray]) -> Tuple[np.ndarray, int]:
    """Unshuffled tables over the same pool size (sequence i owns a contiguous run)."""
    B = w.kv_block
    need = [-(-seq_capacity(w, len(p)) // B) for p in prompts]
    max_blocks = -(-w.shape.n_ctx // B)
    tab = np.full((len(prompts), max_blocks), -1, dtype=np.int32)
    o = 0
    for i, n in enumerate(need):
        tab[i, :n] = np.arange(o, o + n, dtype=np.int32)
        o += n
    return tab, int(sum(need))
