import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_addoption(parser):
    parser.addoption("--kda-checked", action="store_true", default=False,
                     help="run every test on the checked build (libkda_checked.so, device-side bounds checks) "
                          "and fail the session if any check fired")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built libkda")
    config.addinivalue_line("markers", "slow: takes tens of seconds on the CPU")
    if config.getoption("--kda-checked"):
        import linear_attention_sequence_gate_amd as kda
        kda.LIB_PATH = kda.CHECKED_LIB_PATH


def pytest_sessionfinish(session, exitstatus):
    if not session.config.getoption("--kda-checked"):
        return
    import torch
    import linear_attention_sequence_gate_amd as kda
    if not torch.cuda.is_available():
        return
    bits = kda.device_check_bits()
    print(f"\nchecked build: device check bits after the session {bits:#x}", flush=True)
    if bits:
        session.exitstatus = 1
