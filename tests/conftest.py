import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

FULLSIZE_TESTS = {"test_c3_gpt2_stress_full_context": "gpt2_stress", "test_c4_gpt2_batch32_fp32": "gpt2_b32",
                  "test_c4_gpt2_batch32_bf16": "gpt2_b32_bf16", "test_c5_llama_paged_batch8": "llama_b8",
                  "test_c4_gpt2_batch32_kv_bf16": "gpt2_b32_kv16"}


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; calls the HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def pytest_collection_modifyitems(config, items):
    # GPU tests never pass silently on a machine without a GPU: they fail if the
    # library or the device is missing (see tests/gpu_util.py). Nothing is skipped here.
    pass


def pytest_collection_finish(session):
    # Whole-row oracle generations of the selected full-size tests start now, in
    # worker processes, and run while the other tests use the GPU.
    wanted = []
    for item in session.items:
        name = getattr(item, "originalname", item.name)
        if name in FULLSIZE_TESTS and FULLSIZE_TESTS[name] not in wanted:
            wanted.append(FULLSIZE_TESTS[name])
    if wanted:
        from tests import live_oracle
        live_oracle.start(wanted)


def pytest_sessionfinish(session, exitstatus):
    from tests import live_oracle
    live_oracle.stop()


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    # The parity record of every end-to-end GPU test that ran: flips, logit
    # differences and token checksums, GPU against oracle.
    from tests import gpu_util
    if not gpu_util.RECORDS:
        return
    tr = terminalreporter
    tr.write_sep("-", "decode parity record (GPU vs oracle)")
    for r in gpu_util.RECORDS:
        tr.write_line(gpu_util.format_record(r))
