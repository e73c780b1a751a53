"""ctypes wrapper of the CPU oracle (oracle/liboracle.so).

TEST INFRASTRUCTURE ONLY: imported by tests/, the smoke check and the benchmark's
CPU-baseline leg; never by the product package. See oracle.h for what it computes.
"""
from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_f32p = ctypes.POINTER(ctypes.c_float)
_i32p = ctypes.POINTER(ctypes.c_int)


class OrcConfig(ctypes.Structure):
    _fields_ = [("arch", ctypes.c_int), ("n_layer", ctypes.c_int), ("d_model", ctypes.c_int),
                ("n_head", ctypes.c_int), ("n_kv_head", ctypes.c_int), ("head_dim", ctypes.c_int),
                ("d_ff", ctypes.c_int), ("vocab", ctypes.c_int), ("n_ctx", ctypes.c_int),
                ("norm_eps", ctypes.c_double), ("rope_theta", ctypes.c_double), ("kv_bf16", ctypes.c_int),
                ("weight_q8", ctypes.c_int)]


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b
            _b.build()
        L = ctypes.CDLL(_LIB_PATH)
        L.orc_weight_count.restype = ctypes.c_size_t
        L.orc_weight_count.argtypes = [ctypes.POINTER(OrcConfig)]
        L.orc_model_create.restype = ctypes.c_void_p
        L.orc_model_create.argtypes = [ctypes.POINTER(OrcConfig), _f32p, ctypes.c_size_t]
        L.orc_model_free.argtypes = [ctypes.c_void_p]
        L.orc_seq_create.restype = ctypes.c_void_p
        L.orc_seq_create.argtypes = [ctypes.c_void_p, ctypes.c_int]
        L.orc_seq_free.argtypes = [ctypes.c_void_p]
        L.orc_seq_len.restype = ctypes.c_int
        L.orc_seq_len.argtypes = [ctypes.c_void_p]
        L.orc_forward.restype = ctypes.c_int
        L.orc_forward.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, _f32p]
        L.orc_forward_stateless.restype = ctypes.c_int
        L.orc_forward_stateless.argtypes = [ctypes.c_void_p, _i32p, ctypes.c_int, _f32p]
        L.orc_argmax.restype = ctypes.c_int
        L.orc_argmax.argtypes = [_f32p, ctypes.c_int]
        L.orc_layernorm.argtypes = [_f32p, _f32p, _f32p, ctypes.c_int, ctypes.c_double, _f32p]
        L.orc_rmsnorm.argtypes = [_f32p, _f32p, ctypes.c_int, ctypes.c_double, _f32p]
        L.orc_gelu.restype = ctypes.c_float
        L.orc_gelu.argtypes = [ctypes.c_float]
        L.orc_silu.restype = ctypes.c_float
        L.orc_silu.argtypes = [ctypes.c_float]
        L.orc_softmax.argtypes = [_f32p, ctypes.c_int, _f32p]
        L.orc_linear.argtypes = [_f32p, _f32p, _f32p, ctypes.c_int, ctypes.c_int, _f32p]
        L.orc_attend.argtypes = [_f32p, _f32p, _f32p, ctypes.c_int, ctypes.c_int, ctypes.c_int, _f32p]
        L.orc_rope.argtypes = [_f32p, ctypes.c_int, ctypes.c_int, ctypes.c_double]
        L.orc_set_mutation.argtypes = [ctypes.c_int]
        L.orc_round_bf16.restype = ctypes.c_float
        L.orc_round_bf16.argtypes = [ctypes.c_float]
        L.orc_quantize_q8.argtypes = [_f32p, ctypes.c_int, ctypes.POINTER(ctypes.c_int8), _f32p]
        _u64p = ctypes.POINTER(ctypes.c_uint64)
        L.orc_philox4x64.argtypes = [_u64p, _u64p, _u64p]
        L.orc_uniform.restype = ctypes.c_double
        L.orc_uniform.argtypes = [ctypes.c_uint64, ctypes.c_int, ctypes.c_int]
        L.orc_sample.restype = ctypes.c_int
        L.orc_sample.argtypes = [_f32p, ctypes.c_int, ctypes.c_double, ctypes.c_int, ctypes.c_double]
        _lib = L
    return _lib


def _fp(a: np.ndarray):
    assert a.dtype == np.float32 and a.flags.c_contiguous
    return a.ctypes.data_as(_f32p)


def _ip(a: np.ndarray):
    assert a.dtype == np.int32 and a.flags.c_contiguous
    return a.ctypes.data_as(_i32p)


def config_from_shape(s, kv_bf16: bool = False, weight_q8: bool = False) -> OrcConfig:
    return OrcConfig(s.arch, s.n_layer, s.d_model, s.n_head, s.n_kv_head, s.head_dim, s.d_ff, s.vocab,
                     s.n_ctx, s.norm_eps, s.rope_theta, int(kv_bf16), int(weight_q8))


def set_mutation(m: int) -> None:
    lib().orc_set_mutation(int(m))


# ----------------------------------------------------------------- components

def layernorm(x, g, b, eps=1e-5):
    x, g, b = (np.ascontiguousarray(a, np.float32) for a in (x, g, b))
    y = np.empty_like(x)
    lib().orc_layernorm(_fp(x), _fp(g), _fp(b), x.size, eps, _fp(y))
    return y


def rmsnorm(x, w, eps=1e-5):
    x, w = (np.ascontiguousarray(a, np.float32) for a in (x, w))
    y = np.empty_like(x)
    lib().orc_rmsnorm(_fp(x), _fp(w), x.size, eps, _fp(y))
    return y


def gelu(u) -> np.ndarray:
    u = np.asarray(u, np.float32)
    f = lib().orc_gelu
    return np.array([f(float(v)) for v in u.ravel()], dtype=np.float32).reshape(u.shape)


def silu(z) -> np.ndarray:
    z = np.asarray(z, np.float32)
    f = lib().orc_silu
    return np.array([f(float(v)) for v in z.ravel()], dtype=np.float32).reshape(z.shape)


def softmax(s):
    s = np.ascontiguousarray(s, np.float32)
    p = np.empty_like(s)
    lib().orc_softmax(_fp(s), s.size, _fp(p))
    return p


def linear(x, W, b=None):
    x = np.ascontiguousarray(x, np.float32)
    W = np.ascontiguousarray(W, np.float32)
    n_out, n_in = W.shape
    y = np.empty(n_out, np.float32)
    bp = _fp(np.ascontiguousarray(b, np.float32)) if b is not None else None
    if b is not None:
        bb = np.ascontiguousarray(b, np.float32)
        lib().orc_linear(_fp(x), _fp(W), _fp(bb), n_out, n_in, _fp(y))
    else:
        lib().orc_linear(_fp(x), _fp(W), None, n_out, n_in, _fp(y))
    del bp
    return y


def attend(q, K, V):
    q = np.ascontiguousarray(q, np.float32)
    K = np.ascontiguousarray(K, np.float32)
    V = np.ascontiguousarray(V, np.float32)
    T, hd = K.shape
    o = np.empty(hd, np.float32)
    lib().orc_attend(_fp(q), _fp(K), _fp(V), T, hd, hd, _fp(o))
    return o


def rope(v, pos, theta):
    v = np.array(v, np.float32, copy=True)
    lib().orc_rope(_fp(v), v.size, int(pos), float(theta))
    return v


def argmax(v) -> int:
    v = np.ascontiguousarray(v, np.float32)
    return int(lib().orc_argmax(_fp(v), v.size))


def round_bf16(x) -> np.ndarray:
    x = np.asarray(x, np.float32)
    f = lib().orc_round_bf16
    return np.array([f(float(v)) for v in x.ravel()], dtype=np.float32).reshape(x.shape)


def quantize_q8(x):
    """(q int8 [n], d float32 [n / 32]) of n values (n a multiple of 32)."""
    x = np.ascontiguousarray(x, np.float32).ravel()
    q = np.empty(x.size, np.int8)
    d = np.empty(x.size // 32, np.float32)
    lib().orc_quantize_q8(_fp(x), x.size, q.ctypes.data_as(ctypes.POINTER(ctypes.c_int8)), _fp(d))
    return q, d


def philox4x64(ctr, key):
    c = (ctypes.c_uint64 * 4)(*[int(v) for v in ctr])
    k = (ctypes.c_uint64 * 2)(*[int(v) for v in key])
    o = (ctypes.c_uint64 * 4)()
    lib().orc_philox4x64(c, k, o)
    return [int(v) for v in o]


def uniform(seed: int, seq: int, pos: int) -> float:
    return float(lib().orc_uniform(int(seed), int(seq), int(pos)))


def sample(logits, temperature: float, top_k: int, u: float) -> int:
    v = np.ascontiguousarray(logits, np.float32)
    return int(lib().orc_sample(_fp(v), v.size, float(temperature), int(top_k), float(u)))


# --------------------------------------------------------------------- model

class Model:
    """The oracle model over a packed canonical float32 weight buffer (kept alive here)."""

    def __init__(self, shape, weights: np.ndarray, kv_bf16: bool = False, weight_q8: bool = False):
        self.shape = shape
        self.cfg = config_from_shape(shape, kv_bf16, weight_q8)
        self.weights = np.ascontiguousarray(weights, np.float32)
        n = lib().orc_weight_count(ctypes.byref(self.cfg))
        if n != self.weights.size:
            raise ValueError(f"weight count {self.weights.size} != {n}")
        self._h = lib().orc_model_create(ctypes.byref(self.cfg), _fp(self.weights), n)
        if not self._h:
            raise ValueError("orc_model_create failed")

    def __del__(self):
        if getattr(self, "_h", None):
            lib().orc_model_free(self._h)
            self._h = None

    def new_seq(self, capacity: int) -> "Seq":
        return Seq(self, capacity)

    def stateless(self, tokens: Sequence[int]) -> np.ndarray:
        t = np.ascontiguousarray(np.asarray(tokens, np.int32))
        out = np.empty((t.size, self.shape.vocab), np.float32)
        rc = lib().orc_forward_stateless(self._h, _ip(t), t.size, _fp(out))
        if rc != 0:
            raise ValueError(f"orc_forward_stateless rc={rc}")
        return out


class Seq:
    def __init__(self, model: Model, capacity: int):
        self.model = model
        self._h = lib().orc_seq_create(model._h, int(capacity))
        if not self._h:
            raise MemoryError("orc_seq_create failed")

    def __del__(self):
        if getattr(self, "_h", None):
            lib().orc_seq_free(self._h)
            self._h = None

    def __len__(self) -> int:
        return lib().orc_seq_len(self._h)

    def forward(self, token: int, logits: Optional[np.ndarray] = None) -> int:
        if logits is not None:
            assert logits.dtype == np.float32 and logits.size == self.model.shape.vocab
            return int(lib().orc_forward(self.model._h, self._h, int(token), _fp(logits)))
        return int(lib().orc_forward(self.model._h, self._h, int(token), None))


def for_workload(w, weights: np.ndarray) -> Model:
    """The oracle model of a synth workload (its KV and weight precision choices)."""
    return Model(w.shape, weights, kv_bf16=w.init.kv_bf16, weight_q8=w.init.q8)


def generate(model: Model, prompt: Sequence[int], n_generate: int, capacity: Optional[int] = None,
             want_logits: bool = False, forced: Optional[Sequence[int]] = None, sampling=None):
    """Greedy (or sampled) generation: prefill the prompt, then feed each token back.

    Returns (tokens[n_generate], logits[n_generate][V] or None). The first generated
    token comes from the prompt's last position, so there are n_generate - 1 decode
    forwards after the prompt. With ``forced``, the fed tokens are ``forced`` instead
    of the generated ones (teacher forcing); the returned tokens are still the
    generated ones. ``sampling`` = (temperature, top_k, seed, slot) samples each token
    with orc_sample and the uniform of (seed, slot, position of the logits' row)
    instead of taking the argmax.
    """
    V = model.shape.vocab
    cap = capacity or (len(prompt) + n_generate)
    s = model.new_seq(cap)
    logits = np.empty((n_generate, V), np.float32) if want_logits else None
    buf = np.empty(V, np.float32)
    def pick(tok, pos):
        if sampling is None:
            return tok
        temp, top_k, seed, slot = sampling
        return sample(buf, temp, top_k, uniform(seed, slot, pos))

    tok = -1
    keep = want_logits or sampling is not None
    for i, t in enumerate(prompt):
        last = i == len(prompt) - 1
        tok = s.forward(int(t), buf if (last and keep) else None)
    out: List[int] = [pick(tok, len(prompt) - 1)]
    if want_logits:
        logits[0] = buf
    for i in range(1, n_generate):
        feed = out[-1] if forced is None else int(forced[i - 1])
        tok = s.forward(feed, buf if keep else None)
        if tok < 0:
            raise RuntimeError(f"oracle forward failed rc={tok}")
        out.append(pick(tok, len(prompt) + i - 1))
        if want_logits:
            logits[i] = buf
    return np.array(out, np.int32), logits
