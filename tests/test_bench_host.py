"""Host logic of bench.py that needs no GPU: how a profiled pass is found in a rocprofv3
CSV (gated and ungated runs), and the rule that recorded HBM traffic is only reported for
the kernel sources it was measured on."""
import json

import bench


def _row(i, name):
    return {"Dispatch_Id": str(i), "Kernel_Name": name}


STEP = ["k_setup_decode(RowParams)", "void k_gemv<0, 3, 1, 4, 0, 2>(LinParams)",
        "void k_attn_o<64, 1, 4, false, 0>(AttnParams, AttnOParams)",
        "void k_gemv<0, 3, 4, 3, 0, 2>(LinParams)", "k_argmax_finalize(float const*, int const*, int, int, int*)"]


def _rows(names):
    return [_row(i + 1, n) for i, n in enumerate(names)]


def test_gated_pass_with_gates_dispatched_ahead():
    """Gates of a pass may be dispatched before their steps (here: all three first); the
    pass still spans its first gate to its third finalize, and a second workload's pass
    follows after unrelated dispatches."""
    names = ["void k_mm<0, 1, 0, 0, false>(LinParams)"] * 5          # prefill
    names += ["k_gate(long long)"] * 3 + STEP * 3                    # pass 1: 3 steps
    names += ["__amd_rocclr_copyBuffer"] * 4 + STEP * 2              # other work
    names += ["k_gate(long long)", *STEP, "k_gate(long long)", *STEP]   # pass 2: 2 steps
    rows = _rows(names)
    regions = bench.profiled_regions(rows, [3, 2])
    assert len(regions) == 2
    (lo1, hi1, k1), (lo2, hi2, k2) = regions
    assert (k1, k2) == (3, 2)
    assert rows[lo1]["Kernel_Name"].startswith("k_gate") and lo1 == 5
    assert hi1 == 5 + 3 + 3 * len(STEP)
    fin = [r for r in rows[lo1:hi1] if r["Kernel_Name"].startswith("k_argmax_finalize")]
    assert len(fin) == 3
    assert rows[lo2]["Kernel_Name"].startswith("k_gate") and hi2 == len(rows)


def test_ungated_pass_is_the_last_k_steps():
    names = ["void k_mm<0, 1, 0, 0, false>(LinParams)"] * 4 + STEP * 5   # 5 steps, 2 profiled
    rows = _rows(names)
    (lo, hi, k), = bench.profiled_regions(rows, [2])
    assert k == 2 and hi == len(rows) and hi - lo == 2 * len(STEP)
    assert rows[lo]["Kernel_Name"].startswith("k_setup_decode")
    assert bench.profiled_regions(rows, None) == []          # ungated needs the step count
    assert bench.profiled_regions(rows, [9]) == []           # more steps than the run has


def test_traffic_reported_only_for_the_recorded_sources(tmp_path, monkeypatch):
    rec = {"sources_sha256": "abc", "workloads": {"gpt2_b1": {"kernels": {
        "k_attn_o<64, 1, 4, false, 0>": {"fetch_bytes": 100, "write_bytes": 7}}}}}
    (tmp_path / "profiles").mkdir()
    (tmp_path / "profiles" / "hbm_traffic.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_sources_sha256", lambda: "abc")
    assert bench.measured_traffic("k_attn_o<64, 1>", "gpt2_b1") == 107
    assert bench.measured_traffic("k_attn_o<64, 1>", "gpt2_b32") is None
    assert bench.measured_traffic("k_gemv<0, 3>", "gpt2_b1") is None
    monkeypatch.setattr(bench, "kernel_sources_sha256", lambda: "changed")
    assert bench.measured_traffic("k_attn_o<64, 1>", "gpt2_b1") is None
