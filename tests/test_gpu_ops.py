"""Kernel-level parity through the C ABI: gd_linear and gd_argmax against the oracle.

Every kernel variant is forced on every shape (VALU GEMV and MFMA), with awkward
column counts (7, 33, 130, 50257 = the GPT-2 vocabulary) and both weight dtypes.
Tolerance for one output of a length-K fp32 dot product: 4 * sqrt(K) * 2^-24 *
sum_i |x_i w_i| (a few times the typical rounding of a blocked fp32 sum), plus the
rounding of the float32 output itself.
"""
import math

import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import device

pytestmark = pytest.mark.gpu

SHAPES = [(7, 64), (33, 768), (130, 256), (2304, 768), (768, 3072), (50257, 768)]
ROWS = [1, 3, 4, 5, 17, 32]


def _bf16_bits(a):
    r = synth.round_bf16(a)
    return r, (r.view(np.uint32) >> 16).astype(np.uint16)


def _ref(x, W, b, norm, g, nb, act):
    ys = []
    for r in x:
        if norm == 1:
            r = oracle.layernorm(r, g, nb, 1e-5)
        elif norm == 2:
            r = oracle.rmsnorm(r, g, 1e-5)
        y = oracle.linear(r, W, b)
        if act == 1:
            y = oracle.gelu(y)
        ys.append((y, np.abs(W.astype(np.float64)) @ np.abs(r.astype(np.float64))))
    return np.stack([a for a, _ in ys]), np.stack([s for _, s in ys])


@pytest.mark.parametrize("variant", [1, 2], ids=["gemv", "mfma"])
@pytest.mark.parametrize("wdt", ["f32", "bf16"])
@pytest.mark.parametrize("N,K", SHAPES, ids=[f"{n}x{k}" for n, k in SHAPES])
def test_linear_parity(N, K, wdt, variant):
    import torch
    import transformer_gpt_decode_amd as gd
    dev = device()
    rng = np.random.default_rng(N * 7 + K)
    rows = [1, 5] if N * K > 10_000_000 else ROWS
    W = (rng.standard_normal((N, K)) * 0.05).astype(np.float32)
    if wdt == "bf16":
        W, bits = _bf16_bits(W)
        Wd = torch.as_tensor(bits.view(np.int16), device=dev)
    else:
        Wd = torch.as_tensor(W, device=dev)
    b = rng.standard_normal(N).astype(np.float32)
    for M in rows:
        x = (rng.standard_normal((M, K)) * 2.0).astype(np.float32)
        xd = torch.as_tensor(x, device=dev)
        y = gd.linear(xd, Wd, gd.WEIGHT_BF16 if wdt == "bf16" else gd.WEIGHT_F32, bias=torch.as_tensor(b, device=dev),
                      variant=variant)
        ref, scale = _ref(x, W, b, 0, None, None, 0)
        tol = 4 * math.sqrt(K) * 2.0 ** -24 * scale + 2.0 ** -24 * np.abs(ref) + 1e-30
        got = y.cpu().numpy()
        bad = np.abs(got - ref) > tol
        assert not bad.any(), f"M={M}: {bad.sum()} outside tol, worst {np.max(np.abs(got - ref)):.3e}"


@pytest.mark.parametrize("variant", [1, 2], ids=["gemv", "mfma"])
@pytest.mark.parametrize("norm", [1, 2], ids=["layernorm", "rmsnorm"])
def test_linear_norm_gelu_resid(norm, variant):
    """Pre-norm prologue, GELU epilogue at stress magnitudes, and the residual add."""
    import torch
    import transformer_gpt_decode_amd as gd
    dev = device()
    rng = np.random.default_rng(5 + norm)
    K, N = 768, 3072
    W = (rng.standard_normal((N, K)) * 0.5).astype(np.float32)     # GELU pre-activations ~ N(0, 14^2)
    b = rng.standard_normal(N).astype(np.float32)
    g = (1 + 0.1 * rng.standard_normal(K)).astype(np.float32)
    nb = (0.1 * rng.standard_normal(K)).astype(np.float32)
    for M in (1, 7, 32):
        x = (rng.standard_normal((M, K)) * 30 + 3).astype(np.float32)
        res = rng.standard_normal((M, N)).astype(np.float32)
        t = lambda a: torch.as_tensor(a, device=dev)
        y = gd.linear(t(x), t(W), gd.WEIGHT_F32, bias=t(b), norm=norm, norm_g=t(g),
                      norm_b=t(nb) if norm == 1 else None, act=gd.ACT_GELU, resid=t(res), variant=variant)
        ref, scale = _ref(x, W, b, norm, g, nb if norm == 1 else None, 1)
        ref = ref.astype(np.float64) + res
        got = y.cpu().numpy()
        assert np.all(np.isfinite(got))
        # GELU has slope <= 1.13, so the pre-activation bound carries over; the normalized
        # input adds ~1e-6 relative; residual add rounds once.
        tol = 1.13 * (4 * math.sqrt(K) * 2.0 ** -24 + 2e-6) * scale + 2.0 ** -23 * np.abs(ref) + 1e-6
        bad = np.abs(got - ref) > tol
        assert not bad.any(), f"M={M}: worst {np.max(np.abs(got - ref)):.3e}"


def test_argmax_rules():
    import torch
    import transformer_gpt_decode_amd as gd
    dev = device()
    rng = np.random.default_rng(3)
    V = 50257
    L = rng.standard_normal((32, V)).astype(np.float32)
    L[1, :] = 0.5                       # all tied -> 0
    L[2, 100] = L[2, 40000] = 99.0      # tie -> 100
    L[3, 7] = np.nan
    L[3, 50000] = np.nan                # first NaN -> 7
    L[4, 50256] = 1e30                  # last element
    L[5, 4096] = 1e30                   # chunk boundary
    L[6, :] = -np.inf
    L[6, 33000] = -1e30
    got = gd.argmax(torch.as_tensor(L, device=dev)).cpu().numpy()
    ref = np.array([oracle.argmax(r) for r in L])
    assert np.array_equal(got, ref)
    assert list(got[1:7]) == [0, 100, 7, 50256, 4096, 33000]
