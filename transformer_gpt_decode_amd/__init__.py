"""Python binding of libgptdecode.so, the MI355X (gfx950) KV-cached decode library.

Argument marshalling only: every step of the forward pass runs in the library's
HIP kernels (see include/gd.h). PyTorch supplies device memory and the stream.
The library must be built (``python -m transformer_gpt_decode_amd.build`` or
``__graft_entry__.build()``); importing the binding without it raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgptdecode.so")

GD_OK, GD_ERR_INVALID, GD_ERR_NO_DEVICE, GD_ERR_HIP, GD_ERR_OOM, GD_ERR_CTX_FULL, GD_ERR_STATE = 0, -1, -2, -3, -4, -5, -6
ARCH_GPT2, ARCH_LLAMA = 0, 1
WEIGHT_F32, WEIGHT_BF16, WEIGHT_Q8 = 0, 1, 2
KV_F32, KV_BF16 = 0, 1
OPT_LINEAR_VARIANT, OPT_USE_GRAPH, OPT_PROFILE, OPT_FUSE_ATTN_O = 1, 2, 3, 4
OPT_FOLD_NORM, OPT_ATTN_CHUNKS, OPT_TILED_PREFILL, OPT_PREFILL_BF16_PARTS = 7, 9, 10, 11
NORM_NONE, NORM_LAYER, NORM_RMS = 0, 1, 2
ACT_NONE, ACT_GELU = 0, 1

# Symbols declared in include/gd.h.
EXPORTS = ["gd_create", "gd_memory_requirements", "gd_bind_memory", "gd_load_weights", "gd_set_block_table",
           "gd_reset_seq", "gd_truncate_seq", "gd_seq_len", "gd_prefill", "gd_decode_step", "gd_device_errors",
           "gd_set_option", "gd_profile_read", "gd_destroy", "gd_last_error", "gd_linear_workspace", "gd_linear",
           "gd_argmax_workspace", "gd_argmax", "gd_argmax_static", "gd_set_sampling"]


class GdError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"gd status {status}: {msg}")
        self.status = status


class GdConfig(ctypes.Structure):
    _fields_ = [("arch", ctypes.c_int32), ("n_layer", ctypes.c_int32), ("d_model", ctypes.c_int32),
                ("n_head", ctypes.c_int32), ("n_kv_head", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("d_ff", ctypes.c_int32), ("vocab", ctypes.c_int32), ("n_ctx", ctypes.c_int32),
                ("norm_eps", ctypes.c_float), ("rope_theta", ctypes.c_float), ("weight_dtype", ctypes.c_int32),
                ("max_seqs", ctypes.c_int32), ("max_batch", ctypes.c_int32), ("kv_block_size", ctypes.c_int32),
                ("kv_num_blocks", ctypes.c_int32), ("kv_dtype", ctypes.c_int32)]


class KernelStat(ctypes.Structure):
    _fields_ = [("role", ctypes.c_char * 32), ("kernel", ctypes.c_char * 64), ("launches", ctypes.c_int64),
                ("total_us", ctypes.c_double), ("bytes", ctypes.c_double)]


_lib = None
_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_i32p = ctypes.POINTER(ctypes.c_int32)
_szp = ctypes.POINTER(ctypes.c_size_t)


def lib() -> ctypes.CDLL:
    """Load the HIP library; raises if it has not been built (no fallback exists)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with transformer_gpt_decode_amd/build.py")
        L = ctypes.CDLL(LIB_PATH)
        sigs = {
            "gd_create": [ctypes.POINTER(GdConfig), _vp, ctypes.POINTER(_vp)],
            "gd_memory_requirements": [_vp, _szp, _szp, _szp],
            "gd_bind_memory": [_vp, _vp, _vp, _vp],
            "gd_load_weights": [_vp, _vp, ctypes.c_size_t],
            "gd_set_block_table": [_vp, _i32, _i32p, _i32],
            "gd_reset_seq": [_vp, _i32],
            "gd_truncate_seq": [_vp, _i32, _i32],
            "gd_profile_read": [_vp, ctypes.POINTER(KernelStat), _i32, _i32p, _i32],
            "gd_seq_len": [_vp, _i32, _i32p],
            "gd_prefill": [_vp, _i32, _i32p, _i32, _vp, _vp],
            "gd_decode_step": [_vp, _i32, _i32p, _vp, _vp, _vp],
            "gd_device_errors": [_vp, _i32p],
            "gd_set_option": [_vp, _i32, _i32],
            "gd_linear_workspace": [_i32, _i32, _i32, _i32, _szp],
            "gd_linear": [_vp, _i32, _vp, _i32, _vp, _i32, _vp, _vp, ctypes.c_float, _i32, _vp, _i32, _vp, _i32,
                          _i32, _i32, _i32, _i32, _vp, ctypes.c_size_t, _vp],
            "gd_argmax_workspace": [_i32, _i32, _szp],
            "gd_argmax": [_vp, _i32, _i32, _vp, _vp, ctypes.c_size_t, _vp],
            "gd_argmax_static": [_vp, _i32, _i32, _vp, _vp],
            "gd_set_sampling": [_vp, ctypes.c_float, _i32, ctypes.c_uint64],
        }
        for name, args in sigs.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = ctypes.c_int
        L.gd_destroy.argtypes = [_vp]
        L.gd_destroy.restype = None
        L.gd_last_error.argtypes = []
        L.gd_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _check(status: int) -> None:
    if status != GD_OK:
        raise GdError(status, lib().gd_last_error().decode(errors="replace"))


def _stream_ptr(stream=None) -> Optional[int]:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream or None


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


class Model:
    """A decode model bound to torch-allocated device memory on the current device."""

    def __init__(self, arch: int, n_layer: int, d_model: int, n_head: int, n_kv_head: int, head_dim: int,
                 d_ff: int, vocab: int, n_ctx: int, norm_eps: float = 1e-5, rope_theta: float = 0.0,
                 weight_dtype: int = WEIGHT_F32, max_seqs: int = 1, max_batch: int = 1, kv_block_size: int = 0,
                 kv_num_blocks: int = 0, kv_dtype: int = KV_F32, stream=None):
        import torch
        self.cfg = GdConfig(arch, n_layer, d_model, n_head, n_kv_head, head_dim, d_ff, vocab, n_ctx, norm_eps,
                            rope_theta, weight_dtype, max_seqs, max_batch, kv_block_size, kv_num_blocks, kv_dtype)
        self.stream = stream if stream is not None else torch.cuda.current_stream()
        h = _vp()
        _check(lib().gd_create(ctypes.byref(self.cfg), _stream_ptr(self.stream), ctypes.byref(h)))
        self._h = h
        wb, kb, sb = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
        _check(lib().gd_memory_requirements(self._h, ctypes.byref(wb), ctypes.byref(kb), ctypes.byref(sb)))
        dev = torch.device("cuda", torch.cuda.current_device())
        self.weights_dev = torch.empty(wb.value, dtype=torch.uint8, device=dev)
        self.kv_dev = torch.empty(kb.value, dtype=torch.uint8, device=dev)
        self.scratch_dev = torch.empty(sb.value, dtype=torch.uint8, device=dev)
        self.sizes = (wb.value, kb.value, sb.value)
        _check(lib().gd_bind_memory(self._h, self.weights_dev.data_ptr(), self.kv_dev.data_ptr(),
                                    self.scratch_dev.data_ptr()))

    @classmethod
    def from_shape(cls, shape, weight_dtype: int = WEIGHT_F32, **kw) -> "Model":
        """Build from any object with the shape fields (arch, n_layer, d_model, ...)."""
        return cls(shape.arch, shape.n_layer, shape.d_model, shape.n_head, shape.n_kv_head, shape.head_dim,
                   shape.d_ff, shape.vocab, shape.n_ctx, shape.norm_eps, shape.rope_theta, weight_dtype, **kw)

    def close(self) -> None:
        if getattr(self, "_h", None):
            lib().gd_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def load_weights(self, w: np.ndarray) -> None:
        w = np.ascontiguousarray(w, dtype=np.float32)
        _check(lib().gd_load_weights(self._h, w.ctypes.data, w.size))

    def set_block_table(self, seq: int, blocks: Sequence[int]) -> None:
        b = np.ascontiguousarray(np.asarray(blocks, np.int32))
        _check(lib().gd_set_block_table(self._h, seq, b.ctypes.data_as(_i32p), b.size))

    def reset_seq(self, seq: int) -> None:
        _check(lib().gd_reset_seq(self._h, seq))

    def truncate_seq(self, seq: int, length: int) -> None:
        _check(lib().gd_truncate_seq(self._h, seq, length))

    def profile_read(self, reset: bool = True):
        """Per-kernel profile gathered with OPT_PROFILE on: list of dicts."""
        arr = (KernelStat * 64)()
        n = ctypes.c_int32()
        _check(lib().gd_profile_read(self._h, arr, 64, ctypes.byref(n), 1 if reset else 0))
        return [dict(role=a.role.decode(), kernel=a.kernel.decode(), launches=a.launches, total_us=a.total_us,
                     bytes=a.bytes) for a in arr[:min(n.value, 64)]]

    def seq_len(self, seq: int) -> int:
        v = ctypes.c_int32()
        _check(lib().gd_seq_len(self._h, seq, ctypes.byref(v)))
        return v.value

    def prefill(self, seq: int, tokens: Sequence[int], next_dev, logits_dev=None) -> None:
        t = np.ascontiguousarray(np.asarray(tokens, np.int32))
        _check(lib().gd_prefill(self._h, seq, t.ctypes.data_as(_i32p), t.size, next_dev.data_ptr(),
                                _ptr(logits_dev)))

    def decode_step(self, seq_ids: Sequence[int], tokens_dev, next_dev, logits_dev=None) -> None:
        s = np.ascontiguousarray(np.asarray(seq_ids, np.int32))
        _check(lib().gd_decode_step(self._h, s.size, s.ctypes.data_as(_i32p), tokens_dev.data_ptr(),
                                    next_dev.data_ptr(), _ptr(logits_dev)))

    def device_errors(self) -> int:
        v = ctypes.c_int32()
        _check(lib().gd_device_errors(self._h, ctypes.byref(v)))
        return v.value

    def set_option(self, opt: int, value: int) -> None:
        _check(lib().gd_set_option(self._h, opt, value))

    def set_sampling(self, temperature: float, top_k: int, seed: int) -> None:
        """Temperature / top-k sampling for later steps (temperature <= 0 or top_k == 1: greedy)."""
        _check(lib().gd_set_sampling(self._h, float(temperature), int(top_k), int(seed)))


def linear(x, W, weight_dtype: int = WEIGHT_F32, bias=None, norm: int = NORM_NONE, norm_g=None, norm_b=None,
           eps: float = 1e-5, act: int = ACT_NONE, resid=None, out=None, variant: int = 0, stream=None):
    """y = act(norm(x) . W^T + bias) (+ resid) on device tensors; W is float32 or bf16 bits (int16/uint16)."""
    import torch
    M, K = x.shape
    N = W.shape[0]
    y = out if out is not None else torch.empty((M, N), dtype=torch.float32, device=x.device)
    nb = ctypes.c_size_t()
    _check(lib().gd_linear_workspace(M, N, K, variant, ctypes.byref(nb)))
    ws = torch.zeros(max(nb.value, 256), dtype=torch.uint8, device=x.device)
    _check(lib().gd_linear(x.data_ptr(), x.stride(0), W.data_ptr(), weight_dtype, _ptr(bias), norm, _ptr(norm_g),
                           _ptr(norm_b), eps, act, _ptr(resid), resid.stride(0) if resid is not None else 0,
                           y.data_ptr(), y.stride(0), M, N, K, variant, ws.data_ptr(), ws.numel(),
                           _stream_ptr(stream)))
    return y


def argmax(logits, stream=None):
    """Greedy argmax of each row (NaN first, ties to the lowest index) -> int32 device tensor."""
    import torch
    rows, vocab = logits.shape
    nb = ctypes.c_size_t()
    _check(lib().gd_argmax_workspace(rows, vocab, ctypes.byref(nb)))
    ws = torch.zeros(nb.value, dtype=torch.uint8, device=logits.device)
    out = torch.empty(rows, dtype=torch.int32, device=logits.device)
    _check(lib().gd_argmax(logits.data_ptr(), rows, vocab, out.data_ptr(), ws.data_ptr(), ws.numel(),
                           _stream_ptr(stream)))
    return out


def argmax_static(logits, out=None, stream=None):
    """argmax() without a workspace: the library's static scratch holds the partials
    (calls on one GPU must not overlap). Writes into ``out`` if given."""
    import torch
    rows, vocab = logits.shape
    if out is None:
        out = torch.empty(rows, dtype=torch.int32, device=logits.device)
    _check(lib().gd_argmax_static(logits.data_ptr(), rows, vocab, out.data_ptr(), _stream_ptr(stream)))
    return out
