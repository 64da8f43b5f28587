"""Shared pytest setup: the ``gpu`` marker and small conversion helpers."""
import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


def bits(t):
    """bf16 torch tensor (CPU) -> numpy uint16 bit patterns, strides kept."""
    import torch
    assert t.dtype == torch.bfloat16 and t.device.type == "cpu"
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_rne(x: np.ndarray) -> np.ndarray:
    """float64 -> nearest bf16 (ties to even) via fp32, as float64."""
    f = np.asarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lower = u & 0xFFFF
    upper = u >> 16
    up = (lower > 0x8000) | ((lower == 0x8000) & ((upper & 1) == 1))
    upper = (upper + up.astype(np.uint64)) & 0xFFFF
    return (upper.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


@pytest.fixture(scope="session")
def orc():
    import oracle
    return oracle
