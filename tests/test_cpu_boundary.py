"""Host-side checks of the C ABI that need no GPU: the library loads, exports every
symbol include/gd.h declares, and rejects bad configs before touching a device."""
import ctypes
import os
import re
import subprocess

import pytest

import transformer_gpt_decode_amd as gd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "gd.h")).read()
    return sorted(set(re.findall(r"\b(gd_[a-z_]+)\s*\(", src)))


def test_header_matches_binding_list():
    assert sorted(gd.EXPORTS) == _declared()


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", gd.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    syms = set(l.split()[-1] for l in out.splitlines() if l.strip())
    missing = [s for s in _declared() if s not in syms]
    assert not missing, missing
    L = gd.lib()
    for s in _declared():
        assert hasattr(L, s)


def test_library_carries_gfx950_code_object(tmp_path):
    """The device code embedded in the library (its .hip_fatbin section) targets gfx950."""
    sec = tmp_path / "fatbin"
    subprocess.run(["objcopy", "-O", "binary", "--only-section=.hip_fatbin", gd.LIB_PATH, str(sec)], check=True)
    data = sec.read_bytes()
    assert b"amdgcn-amd-amdhsa--gfx950" in data


def _cfg(**kw):
    base = dict(arch=0, n_layer=2, d_model=64, n_head=4, n_kv_head=4, head_dim=16, d_ff=256, vocab=512, n_ctx=64,
                norm_eps=1e-5, rope_theta=0.0, weight_dtype=0, max_seqs=1, max_batch=1, kv_block_size=0,
                kv_num_blocks=0, kv_dtype=0)
    base.update(kw)
    return gd.GdConfig(**base)


@pytest.mark.parametrize("bad", [dict(arch=7), dict(head_dim=32, d_model=128), dict(max_batch=33),
                                 dict(n_kv_head=2), dict(weight_dtype=3), dict(norm_eps=0.0),
                                 dict(d_model=60, head_dim=15), dict(kv_dtype=2)])
def test_create_rejects_bad_config(bad):
    h = ctypes.c_void_p()
    st = gd.lib().gd_create(ctypes.byref(_cfg(**bad)), None, ctypes.byref(h))
    assert st == gd.GD_ERR_INVALID
    assert gd.lib().gd_last_error()


def test_workspace_queries():
    n = ctypes.c_size_t()
    assert gd.lib().gd_linear_workspace(1, 50257, 768, 0, ctypes.byref(n)) == gd.GD_OK
    assert gd.lib().gd_linear_workspace(0, 10, 64, 0, ctypes.byref(n)) == gd.GD_ERR_INVALID
    assert gd.lib().gd_linear_workspace(4, 10, 60, 0, ctypes.byref(n)) == gd.GD_ERR_INVALID
    assert gd.lib().gd_argmax_workspace(32, 50257, ctypes.byref(n)) == gd.GD_OK
    assert n.value > 0


def test_binding_refuses_missing_library(tmp_path, monkeypatch):
    monkeypatch.setattr(gd, "LIB_PATH", str(tmp_path / "nope.so"))
    monkeypatch.setattr(gd, "_lib", None)
    with pytest.raises(ImportError):
        gd.lib()
