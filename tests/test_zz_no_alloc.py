"""gd_argmax_static (no workspace: partials in the library's static device scratch)
against gd_argmax (caller workspace) through the C ABI, on two calls in a row, the
second smaller, and its size limits. Integer results: bit-exact."""
import numpy as np
import pytest

import oracle
from tests.gpu_util import device

pytestmark = pytest.mark.gpu


def _logits(rng, rows, vocab):
    L = rng.standard_normal((rows, vocab)).astype(np.float32)
    L[0, :] = 0.25                         # all tied: index 0
    if rows > 2:
        L[1, 3] = L[1, vocab - 2] = 50.0   # tie: the lower index
        L[2, 5] = np.nan
        L[2, vocab - 1] = np.nan           # first NaN wins
    if rows > 4 and vocab > 4096:
        L[3, 4096] = 1e30                  # chunk boundary
        L[4, :] = -np.inf
        L[4, vocab - 1] = -1e30
    return L


def test_argmax_static_matches_workspace_argmax():
    import torch
    import transformer_gpt_decode_amd as gd
    dev = device()
    rng = np.random.default_rng(21)
    for rows, vocab in ((32, 50257), (5, 3000)):
        L = torch.as_tensor(_logits(rng, rows, vocab), device=dev)
        ref = gd.argmax(L).cpu().numpy()
        out = torch.full((rows,), -1, dtype=torch.int32, device=dev)
        gd.argmax_static(L, out)
        got = out.cpu().numpy()
        assert np.array_equal(got, ref), (rows, vocab, got, ref)
        assert np.array_equal(got, [oracle.argmax(r) for r in L.cpu().numpy()])


def test_argmax_static_refuses_sizes_beyond_its_scratch():
    import torch
    import transformer_gpt_decode_amd as gd
    dev = device()
    big = torch.zeros((1, (1 << 20) + 1), dtype=torch.float32, device=dev)
    with pytest.raises(gd.GdError) as e:
        gd.argmax_static(big)
    assert e.value.status == gd.GD_ERR_INVALID
    with pytest.raises(gd.GdError) as e:
        gd.argmax_static(torch.zeros((33, 10), dtype=torch.float32, device=dev))
    assert e.value.status == gd.GD_ERR_INVALID
