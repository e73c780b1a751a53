"""Pins of the CPU oracle against facts fixed by the pages and by mathematics.

Each ``check_*`` function asserts one family of facts. The tests in
test_oracle_pins.py run them as they stand (they must pass) and under planted
mistakes in the oracle (each mistake must make at least one of them fail).
"""
from __future__ import annotations

import math

import numpy as np
from scipy.special import erf, lambertw

import oracle
import synth

RNG = np.random.default_rng(1234)


def check_softmax():
    for n in (1, 2, 7, 64, 1000):
        s = (RNG.standard_normal(n) * 5).astype(np.float32)
        p = oracle.softmax(s)
        assert abs(float(np.sum(p, dtype=np.float64)) - 1.0) < 1e-6
        assert np.all(p >= 0)
    assert oracle.softmax(np.array([3.5], np.float32))[0] == 1.0
    u = oracle.softmax(np.full(10, 2.25, np.float32))
    assert np.all(u == np.float32(0.1))
    m = np.array([1.0, -np.inf, 2.0, -np.inf], np.float32)
    pm = oracle.softmax(m)
    assert pm[1] == 0.0 and pm[3] == 0.0
    e = math.exp(1.0)
    assert abs(pm[2] - e / (1 + e)) < 1e-7


def check_layernorm():
    d = 768
    for sigma, mu in ((0.02, 0.0), (1.0, 3.0), (50.0, -7.0)):
        x = (RNG.standard_normal(d) * sigma + mu).astype(np.float32)
        y = oracle.layernorm(x, np.ones(d, np.float32), np.zeros(d, np.float32), 1e-5)
        xd = x.astype(np.float64)
        var = xd.var()
        assert abs(y.astype(np.float64).mean()) <= 1e-6 * max(1.0, np.abs(y).max())
        # variance of the normalized row is var / (var + eps) (not 1 for small inputs)
        assert abs(y.astype(np.float64).var() - var / (var + 1e-5)) < 1e-5
    c = oracle.layernorm(np.full(16, 4.0, np.float32), np.full(16, 2.0, np.float32),
                         np.arange(16, dtype=np.float32), 1e-5)
    assert np.all(c == np.arange(16, dtype=np.float32))
    # gain and shift act elementwise on the normalized row
    x = RNG.standard_normal(32).astype(np.float32)
    g = RNG.standard_normal(32).astype(np.float32)
    b = RNG.standard_normal(32).astype(np.float32)
    y0 = oracle.layernorm(x, np.ones(32, np.float32), np.zeros(32, np.float32), 1e-5)
    y1 = oracle.layernorm(x, g, b, 1e-5)
    assert np.allclose(y1, y0.astype(np.float64) * g + b, atol=1e-6)


def check_rmsnorm():
    d = 960
    for sigma in (0.02, 1.0, 30.0):
        x = (RNG.standard_normal(d) * sigma + 0.5 * sigma).astype(np.float32)
        y = oracle.rmsnorm(x, np.ones(d, np.float32), 1e-5)
        ms = float(np.mean(x.astype(np.float64) ** 2))
        assert abs(float(np.mean(y.astype(np.float64) ** 2)) - ms / (ms + 1e-5)) < 1e-5
        # direction is preserved: y is a positive multiple of x
        r = y.astype(np.float64) / x
        assert np.allclose(r, r[0], rtol=1e-6)


def check_gelu():
    big = np.array([15.0, 15.5, 20.0, 70.0, 1e4, 3.0e38], np.float32)
    assert np.all(oracle.gelu(big) == big)                 # saturated: gelu(u) == u
    neg = -big
    gn = oracle.gelu(neg)
    assert np.all(np.abs(gn.astype(np.float64)) <= 1e-11 * np.abs(neg.astype(np.float64)))
    assert oracle.gelu(np.array([0.0], np.float32))[0] == 0.0
    # odd identity of the formula: gelu(u) - gelu(-u) = u
    u = (RNG.standard_normal(2000) * 4).astype(np.float32)
    d = oracle.gelu(u).astype(np.float64) - oracle.gelu(-u).astype(np.float64)
    assert np.allclose(d, u, rtol=2e-6, atol=1e-7)
    # the tanh form approximates u * Phi(u) to within 4.8e-4 everywhere
    v = np.linspace(-8, 8, 3201).astype(np.float32)
    exact = 0.5 * v.astype(np.float64) * (1.0 + erf(v.astype(np.float64) / math.sqrt(2.0)))
    assert np.max(np.abs(oracle.gelu(v) - exact)) < 4.8e-4
    # finite for stress-scale pre-activations (C3: sigma ~ 14, tails far past |70|)
    s = (RNG.standard_normal(20000) * 14.0).astype(np.float32)
    s[:4] = [80.0, -80.0, 1e30, -1e30]
    assert np.all(np.isfinite(oracle.gelu(s)))


def check_silu():
    z = (RNG.standard_normal(1000) * 6).astype(np.float32)
    d = oracle.silu(z).astype(np.float64) - oracle.silu(-z).astype(np.float64)
    assert np.allclose(d, z, rtol=2e-6, atol=1e-7)          # silu(z) - silu(-z) = z
    assert oracle.silu(np.array([0.0], np.float32))[0] == 0.0
    w = float(np.real(lambertw(math.exp(-1.0))))             # minimum at z = -1 - W(1/e)
    zmin = np.float32(-1.0 - w)
    assert abs(float(oracle.silu(np.array([zmin]))[0]) + w) < 1e-7
    assert oracle.silu(np.array([100.0], np.float32))[0] == 100.0


def check_linear():
    for n_out, n_in in ((7, 33), (130, 64), (33, 768)):
        W = RNG.standard_normal((n_out, n_in)).astype(np.float32)
        x = RNG.standard_normal(n_in).astype(np.float32)
        b = RNG.standard_normal(n_out).astype(np.float32)
        y = oracle.linear(x, W, b)
        ref = W.astype(np.float64) @ x.astype(np.float64) + b
        scale = np.abs(W.astype(np.float64)) @ np.abs(x.astype(np.float64)) + np.abs(b)
        assert np.all(np.abs(y - ref) <= 1e-6 * scale + 1e-30)
    x = RNG.standard_normal(16).astype(np.float32)
    b = RNG.standard_normal(16).astype(np.float32)
    assert np.all(oracle.linear(x, np.eye(16, dtype=np.float32), b) == (x + b))
    # orientation: y = x . W^T with W [out][in]
    W = np.zeros((3, 5), np.float32)
    W[2, 4] = 1.0
    x = np.arange(5, dtype=np.float32)
    assert list(oracle.linear(x, W)) == [0.0, 0.0, 4.0]


def _brute_attend(q, K, V):
    q, K, V = (a.astype(np.float64) for a in (q, K, V))
    s = K @ q / math.sqrt(q.size)
    p = np.exp(s - s.max())
    p /= p.sum()
    return p @ V


def check_attention():
    hd = 16
    for T in (1, 2, 5, 8):
        q = RNG.standard_normal(hd).astype(np.float32)
        K = RNG.standard_normal((T, hd)).astype(np.float32)
        V = RNG.standard_normal((T, hd)).astype(np.float32)
        o = oracle.attend(q, K, V)
        assert np.allclose(o, _brute_attend(q, K, V), atol=1e-6)
    V = RNG.standard_normal((1, hd)).astype(np.float32)
    assert np.all(oracle.attend(RNG.standard_normal(hd).astype(np.float32),
                                RNG.standard_normal((1, hd)).astype(np.float32), V) == V[0])
    V = RNG.standard_normal((6, hd)).astype(np.float32)
    Keq = np.tile(RNG.standard_normal(hd).astype(np.float32), (6, 1))
    mean = V.astype(np.float64).mean(axis=0)
    assert np.allclose(oracle.attend(RNG.standard_normal(hd).astype(np.float32), Keq, V), mean, atol=1e-6)
    assert np.allclose(oracle.attend(np.zeros(hd, np.float32), RNG.standard_normal((6, hd)).astype(np.float32), V),
                       mean, atol=1e-6)
    # a key far more aligned with q than the rest takes all the weight
    q = np.zeros(hd, np.float32)
    q[0] = 40.0
    K = np.zeros((4, hd), np.float32)
    K[2, 0] = 40.0
    o = oracle.attend(q, K, V[:4])
    assert np.allclose(o, V[2], atol=1e-6)


def check_rope():
    hd, theta = 64, 1e5
    v = RNG.standard_normal(hd).astype(np.float32)
    assert np.all(oracle.rope(v, 0, theta) == v)
    for p in (1, 7, 300, 1279):
        r = oracle.rope(v, p, theta)
        assert abs(np.linalg.norm(r.astype(np.float64)) - np.linalg.norm(v.astype(np.float64))) < 1e-5
    # the first pair rotates by exactly p radians: e0 -> cos(p) e0 + sin(p) e32
    e0 = np.zeros(hd, np.float32)
    e0[0] = 1.0
    for p in (1, 2, 5):
        r = oracle.rope(e0, p, theta)
        assert abs(r[0] - math.cos(p)) < 1e-7 and abs(r[32] - math.sin(p)) < 1e-7
        assert np.count_nonzero(r) == 2
    # the last pair turns by p * theta^(-62/64)
    e31 = np.zeros(hd, np.float32)
    e31[31] = 1.0
    r = oracle.rope(e31, 1000, theta)
    a = 1000 * theta ** (-62 / 64)
    assert abs(r[31] - math.cos(a)) < 1e-7 and abs(r[63] - math.sin(a)) < 1e-7
    # q(p) . k(j) depends only on p - j
    q = RNG.standard_normal(hd).astype(np.float32)
    k = RNG.standard_normal(hd).astype(np.float32)
    dots = [float(np.dot(oracle.rope(q, p + 5, theta).astype(np.float64),
                         oracle.rope(k, p, theta).astype(np.float64))) for p in (0, 10, 200, 900)]
    assert max(dots) - min(dots) < 1e-4


def check_argmax():
    assert oracle.argmax(np.array([1, 3, 3, 2], np.float32)) == 1
    assert oracle.argmax(np.array([5, 5, 5], np.float32)) == 0
    assert oracle.argmax(np.array([1, np.nan, 9, np.nan], np.float32)) == 1
    assert oracle.argmax(np.array([-np.inf, -1.0, np.inf, np.inf], np.float32)) == 2
    v = RNG.standard_normal(50257).astype(np.float32)
    assert oracle.argmax(v) == int(np.argmax(v))


# ------------------------------------------------------------ model-level pins

def _tiny_gpt2(n_layer=2, d=64, H=4, ff=256, V=512, n_ctx=64):
    return synth.Shape(synth.ARCH_GPT2, n_layer, d, H, H, d // H, ff, V, n_ctx)


def _tiny_llama(n_layer=2, d=48, H=6, Hk=2, hd=8, ff=96, V=300, n_ctx=40):
    return synth.Shape(synth.ARCH_LLAMA, n_layer, d, H, Hk, hd, ff, V, n_ctx, 1e-5, 1e4)


def _np_layernorm(x):
    x = x.astype(np.float64)
    return (x - x.mean()) / np.sqrt(x.var() + 1e-5)


def _np_rms(x):
    x = x.astype(np.float64)
    return x / np.sqrt(np.mean(x * x) + 1e-5)


def check_cached_equals_stateless():
    for shape, seed in ((_tiny_gpt2(), 11), (_tiny_llama(), 12)):
        W = synth.make_weights(shape, synth.Init(), seed)
        m = oracle.Model(shape, W)
        toks = np.random.default_rng(seed).integers(0, shape.vocab, size=20).astype(np.int32)
        st = m.stateless(toks)
        s = m.new_seq(32)
        buf = np.empty(shape.vocab, np.float32)
        for i, t in enumerate(toks):
            s.forward(int(t), buf)
            assert np.max(np.abs(buf - st[i])) < 1e-5, (shape.arch, i)


def check_zero_layers_closed_form():
    sh = _tiny_gpt2()
    W = synth.make_weights(sh, synth.Init(), 21)
    off = synth.offsets(sh)
    for name, (o, shp) in off.items():
        if name.startswith("h") and ("w_" in name or "b_" in name):
            W[o:o + int(np.prod(shp))] = 0.0
    m = oracle.Model(sh, W)
    wte = W[off["wte"][0]:off["wte"][0] + sh.vocab * sh.d_model].reshape(sh.vocab, sh.d_model)
    wpe = W[off["wpe"][0]:off["wpe"][0] + sh.n_ctx * sh.d_model].reshape(sh.n_ctx, sh.d_model)
    toks = [5, 77, 250, 2]
    st = m.stateless(toks)
    for p, t in enumerate(toks):
        x = wte[t].astype(np.float32) + wpe[p]
        ref = wte.astype(np.float64) @ _np_layernorm(x)
        assert np.max(np.abs(st[p] - ref)) < 1e-5
    sh = _tiny_llama()
    W = synth.make_weights(sh, synth.Init(), 22)
    off = synth.offsets(sh)
    for name, (o, shp) in off.items():
        if name.startswith("h") and "w_" in name:
            W[o:o + int(np.prod(shp))] = 0.0
    m = oracle.Model(sh, W)
    wte = W[off["wte"][0]:off["wte"][0] + sh.vocab * sh.d_model].reshape(sh.vocab, sh.d_model)
    head = W[off["w_head"][0]:off["w_head"][0] + sh.vocab * sh.d_model].reshape(sh.vocab, sh.d_model)
    st = m.stateless(toks)
    for p, t in enumerate(toks):
        ref = head.astype(np.float64) @ _np_rms(wte[t])
        assert np.max(np.abs(st[p] - ref)) < 1e-5


def _set(W, off, name, value):
    o, shp = off[name]
    W[o:o + int(np.prod(shp))] = np.asarray(value, np.float32).reshape(-1)


def check_gpt2_block_closed_forms():
    """Structured weights that reduce each block to a closed form built from pinned parts."""
    sh = _tiny_gpt2(n_layer=3)
    d, ff = sh.d_model, sh.d_ff
    rng = np.random.default_rng(31)
    W = synth.make_weights(sh, synth.Init(), 31)
    off = synth.offsets(sh)
    perm = rng.permutation(d)
    P = np.zeros((d, d), np.float32)
    P[np.arange(d), perm] = 1.0                       # (o . P^T)_i = o[perm[i]]
    cv = rng.standard_normal(d).astype(np.float32)
    bo = rng.standard_normal(d).astype(np.float32)
    bfc = rng.standard_normal(ff).astype(np.float32)
    bp = rng.standard_normal(d).astype(np.float32)
    Wfc = np.zeros((ff, d), np.float32)
    Wfc[:d] = np.eye(d, dtype=np.float32)[perm]       # u_j = a[perm[j]] for j < d
    Wp = np.zeros((d, ff), np.float32)
    Wp[:, ff - d:] = np.eye(d, dtype=np.float32)      # y_i = g[ff - d + i]
    Wfc[ff - d:] += np.eye(d, dtype=np.float32)
    for l in range(sh.n_layer):
        p = f"h{l}."
        _set(W, off, p + "w_qkv", 0.0)
        bqkv = np.zeros(3 * d, np.float32)
        bqkv[2 * d:] = cv                             # v = cv for every position
        bqkv[:d] = rng.standard_normal(d)             # q, k values are irrelevant here
        _set(W, off, p + "b_qkv", bqkv)
        _set(W, off, p + "w_o", P)
        _set(W, off, p + "b_o", bo)
        _set(W, off, p + "w_fc", Wfc)
        _set(W, off, p + "b_fc", bfc)
        _set(W, off, p + "w_proj", Wp)
        _set(W, off, p + "b_proj", bp)
    m = oracle.Model(sh, W)
    wte = W[off["wte"][0]:off["wte"][0] + sh.vocab * d].reshape(sh.vocab, d)
    wpe = W[off["wpe"][0]:off["wpe"][0] + sh.n_ctx * d].reshape(sh.n_ctx, d)
    toks = [9, 100, 4]
    st = m.stateless(toks)
    for pos, t in enumerate(toks):
        x = (wte[t] + wpe[pos]).astype(np.float32)
        for _ in range(sh.n_layer):
            x = (x + (cv[perm] + bo)).astype(np.float32)
            a = _np_layernorm(x)
            u = np.zeros(ff)
            u[:d] = a[perm]
            u[ff - d:] += a
            u += bfc
            g = oracle.gelu(u.astype(np.float32)).astype(np.float64)
            x = (x + (g[ff - d:] + bp)).astype(np.float32)
        ref = wte.astype(np.float64) @ _np_layernorm(x)
        assert np.max(np.abs(st[pos] - ref)) < 2e-5, pos


def check_llama_block_closed_forms():
    """GQA head mapping, W_o orientation and SwiGLU wiring at position 0 (attention = v)."""
    sh = _tiny_llama(n_layer=1, d=48, H=6, Hk=2, hd=8, ff=96)
    d, hd, H, Hk, ff = sh.d_model, sh.head_dim, sh.n_head, sh.n_kv_head, sh.d_ff
    rng = np.random.default_rng(41)
    W = synth.make_weights(sh, synth.Init(), 41)
    off = synth.offsets(sh)
    wv = rng.standard_normal((Hk, d)).astype(np.float32)
    Wv = np.repeat(wv, hd, axis=0)                    # every dim of kv head g equals a . wv[g]
    perm = rng.permutation(d)
    Wo = np.eye(d, dtype=np.float32)[perm]            # (o . Wo^T)_i = o[perm[i]]
    Wg = np.zeros((ff, d), np.float32)
    Wg[:d] = np.eye(d, dtype=np.float32)
    Wu = np.zeros((ff, d), np.float32)
    Wu[d:2 * d] = np.eye(d, dtype=np.float32)
    Wu[:d] = 2.0 * np.eye(d, dtype=np.float32)
    Wd = np.zeros((d, ff), np.float32)
    Wd[:, :d] = np.eye(d, dtype=np.float32)
    _set(W, off, "h0.w_v", Wv)
    _set(W, off, "h0.w_o", Wo)
    _set(W, off, "h0.w_gate", Wg)
    _set(W, off, "h0.w_up", Wu)
    _set(W, off, "h0.w_down", Wd)
    m = oracle.Model(sh, W)
    wte = W[off["wte"][0]:off["wte"][0] + sh.vocab * d].reshape(sh.vocab, d)
    head = W[off["w_head"][0]:off["w_head"][0] + sh.vocab * d].reshape(sh.vocab, d)
    for t in (3, 250):
        s = m.new_seq(4)
        buf = np.empty(sh.vocab, np.float32)
        s.forward(t, buf)
        x = wte[t].astype(np.float64)
        a = _np_rms(wte[t]).astype(np.float32).astype(np.float64)
        vg = wv.astype(np.float64) @ a                # value of kv head g
        o = np.concatenate([np.full(hd, vg[h // (H // Hk)]) for h in range(H)])
        x = (x + o[perm]).astype(np.float32)
        b = _np_rms(x).astype(np.float32)
        h = oracle.silu(b).astype(np.float64) * (2.0 * b.astype(np.float64))
        x = (x + h).astype(np.float32)
        ref = head.astype(np.float64) @ _np_rms(x)
        assert np.max(np.abs(buf - ref)) < 2e-5, t


def check_round_bf16():
    """bfloat16 rounding (nearest, ties to even) against torch's float32 -> bfloat16
    conversion, a library routine the oracle does not use."""
    import torch
    vals = [0.0, -0.0, 1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -7, -1.0 - 2.0 ** -8, 3.39e38, 3.4e38,
            1e-40, -1e-40, 6e-39, 65504.0, 1.0 / 3.0]
    x = np.concatenate([np.array(vals, np.float32)] +
                       [(RNG.standard_normal(4000) * s).astype(np.float32) for s in (1e-3, 1.0, 1e3, 1e30)])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    got = oracle.round_bf16(x)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    assert np.isnan(oracle.round_bf16(np.array([np.nan], np.float32))[0])


def check_kv_bf16_model():
    """With the bfloat16 KV cache: the cached path equals the stateless matrix form (both
    read rounded K and V), K/V that are exactly zero make it equal the float cache, and
    random K/V make it differ (the rounding is applied)."""
    for shape, seed in ((_tiny_gpt2(), 31), (_tiny_llama(), 32)):
        W = synth.make_weights(shape, synth.Init(), seed)
        m = oracle.Model(shape, W, kv_bf16=True)
        m32 = oracle.Model(shape, W)
        toks = np.random.default_rng(seed).integers(0, shape.vocab, size=16).astype(np.int32)
        st = m.stateless(toks)
        s = m.new_seq(32)
        buf = np.empty(shape.vocab, np.float32)
        for i, t in enumerate(toks):
            s.forward(int(t), buf)
            assert np.max(np.abs(buf - st[i])) < 1e-5, (shape.arch, i)
        assert np.max(np.abs(m32.stateless(toks) - st)) > 1e-6
    sh = _tiny_gpt2()
    W = synth.make_weights(sh, synth.Init(), 33)
    off = synth.offsets(sh)
    d = sh.d_model
    for l in range(sh.n_layer):
        o, _ = off[f"h{l}.w_qkv"]
        W[o + d * d:o + 3 * d * d] = 0.0   # k and v rows (their biases are zero)
    toks = [3, 9, 27, 81]
    assert np.array_equal(oracle.Model(sh, W, kv_bf16=True).stateless(toks), oracle.Model(sh, W).stateless(toks))


def check_quantize_q8():
    """8-bit blocks of 32: codes in [-127, 127], the largest magnitude of a block at 127,
    reconstruction within half a step, exact for values that are codes times a power of
    two, sign symmetry, all-zero blocks."""
    for sc in (1e-3, 0.02, 1.0, 50.0):
        x = (RNG.standard_normal(32 * 64) * sc).astype(np.float32)
        q, d = oracle.quantize_q8(x)
        assert q.min() >= -127 and q.max() <= 127
        qb = q.reshape(-1, 32).astype(np.int32)
        assert np.all(np.abs(qb).max(axis=1) == 127)
        err = np.abs(x.reshape(-1, 32).astype(np.float64) - qb * d[:, None].astype(np.float64))
        assert np.all(err <= 0.5 * d[:, None] * (1 + 1e-5) + 1e-12)
        q2, d2 = oracle.quantize_q8(-x)
        assert np.array_equal(q2, -q) and np.array_equal(d2, d)
    codes = RNG.integers(-127, 128, size=(8, 32)).astype(np.int32)
    codes[:, 5] = 127
    scale = 2.0 ** RNG.integers(-12, 4, size=8).astype(np.float64)
    x = (codes * scale[:, None]).astype(np.float32)
    q, d = oracle.quantize_q8(x)
    assert np.array_equal(q.reshape(8, 32), codes) and np.array_equal(d, scale.astype(np.float32))
    q, d = oracle.quantize_q8(np.zeros(64, np.float32))
    assert not q.any() and not d.any()


def check_q8_model():
    """The 8-bit model equals the float model run on weights whose every matrix (and
    only the matrices) is replaced row by row, block by block, by its dequantization."""
    for shape, seed in ((_tiny_gpt2(), 41), (_tiny_llama(d=64, H=8, Hk=2, hd=8, ff=96), 42)):
        W = synth.make_weights(shape, synth.Init(), seed)
        Wd = W.copy()
        off = 0
        for name, shp, kind in synth.tensor_list(shape):
            n = int(np.prod(shp))
            if kind == "w":
                rows = W[off:off + n].reshape(shp)
                q, d = oracle.quantize_q8(rows)
                Wd[off:off + n] = (q.astype(np.float32).reshape(-1, 32) * d[:, None]).reshape(-1)
            off += n
        toks = [1, 17, 200, 42, 7]
        a = oracle.Model(shape, W, weight_q8=True).stateless(toks)
        b = oracle.Model(shape, Wd).stateless(toks)
        assert np.array_equal(a, b)
        assert np.max(np.abs(a - oracle.Model(shape, W).stateless(toks))) > 1e-6


def check_sampling():
    """Philox4x64-10 against numpy's implementation (which advances the counter before a
    block); the sampling rule against scipy's softmax of the top-k logits over a fine
    grid of uniforms; its greedy special cases."""
    from scipy.special import softmax
    for key, ctr in (((0, 0), (0, 0, 0, 0)), ((7, 0), (1022, 31, 0, 0)), ((2 ** 63 + 5, 3), (2 ** 40, 9, 8, 7))):
        bg = np.random.Philox(key=np.array(key, dtype=np.uint64),
                              counter=np.array([ctr[0] - 1 if ctr[0] else 2 ** 64 - 1, ctr[1], ctr[2], ctr[3]]
                                               if ctr[0] else [2 ** 64 - 1, (ctr[1] - 1) % 2 ** 64, ctr[2], ctr[3]],
                                               dtype=np.uint64))
        want = [int(v) for v in bg.random_raw(4)]
        if ctr[0] == 0 and ctr[1] == 0:
            # the block before (0, 0, 0, 0) wraps words 0 and 1 and borrows from word 2
            bg = np.random.Philox(key=np.array(key, dtype=np.uint64),
                                  counter=np.array([2 ** 64 - 1, 2 ** 64 - 1, 2 ** 64 - 1, 2 ** 64 - 1], dtype=np.uint64))
            want = [int(v) for v in bg.random_raw(4)]
        assert oracle.philox4x64(ctr, key) == want, (ctr, key)
    for seed, seq, pos in ((0, 0, 0), (12345, 3, 511), (2 ** 40 + 1, 31, 1023)):
        bg = np.random.Philox(key=np.array([seed, 0], dtype=np.uint64),
                              counter=np.array([pos - 1 if pos else 2 ** 64 - 1, seq if pos else seq - 1, 0, 0]
                                               if (pos or seq) else [2 ** 64 - 1] * 4, dtype=np.uint64))
        w0 = int(bg.random_raw(1)[0])
        assert oracle.uniform(seed, seq, pos) == (w0 >> 40) / 2.0 ** 24
    logits = (RNG.standard_normal(12) * 2).astype(np.float32)
    order = sorted(range(12), key=lambda i: (-float(logits[i]), i))
    assert oracle.sample(logits, 0.7, 1, 0.9) == order[0]
    assert oracle.sample(logits, 0.0, 5, 0.9) == order[0]
    assert oracle.sample(logits, 0.7, 5, 0.0) == order[0]
    for T, k in ((0.7, 4), (1.3, 0), (0.25, 12), (2.0, 7)):
        kk = 12 if k == 0 else k
        p = softmax(logits[order[:kk]].astype(np.float64) / T)
        n = 20000
        picks = np.array([oracle.sample(logits, T, k, (i + 0.5) / n) for i in range(n)])
        assert set(picks.tolist()) <= set(order[:kk])
        freq = np.array([np.mean(picks == order[r]) for r in range(kk)])
        assert np.max(np.abs(freq - p)) <= 1.5 / n + 1e-9, (T, k)
    tie = np.array([1.0, 1.0], np.float32)
    assert oracle.sample(tie, 1.0, 0, 0.49) == 0 and oracle.sample(tie, 1.0, 0, 0.51) == 1
    nan = np.array([0.0, np.nan, 5.0, np.nan], np.float32)
    assert oracle.sample(nan, 1.0, 0, 0.3) == 1


COMPONENT_CHECKS = [check_softmax, check_layernorm, check_rmsnorm, check_gelu, check_silu, check_linear,
                    check_attention, check_rope, check_argmax, check_round_bf16, check_quantize_q8, check_sampling]
MODEL_CHECKS = [check_cached_equals_stateless, check_zero_layers_closed_form, check_gpt2_block_closed_forms,
                check_llama_block_closed_forms, check_kv_bf16_model, check_q8_model]
ALL_CHECKS = COMPONENT_CHECKS + MODEL_CHECKS
