"""Shared test helpers.  GPU tests are marked ``gpu``; everything else runs on CPU."""
import os
import sys

import numpy as np
import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the HIP library")
    config.addinivalue_line("markers", "slow: long-running full-size case")


def u16(t: torch.Tensor) -> np.ndarray:
    """bf16 torch tensor (any device) -> numpy uint16 bit patterns."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def bf16_from_u16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)


def f64(a: np.ndarray) -> np.ndarray:
    """uint16 bf16 bit patterns -> float64."""
    return (np.ascontiguousarray(a).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def ulp_diff(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Distance in bf16 units-in-the-last-place between two uint16 arrays."""
    def key(x):
        x = x.astype(np.int32)
        return np.where(x & 0x8000, 0x8000 - (x & 0x7FFF), 0x8000 + (x & 0x7FFF))
    return np.abs(key(a) - key(b))


def row_rel_err(got: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """Per-row max|got-ref| / max|ref| (0 for all-zero reference rows that match)."""
    g, r = f64(got), f64(ref)
    err = np.abs(g - r).max(axis=-1)
    scale = np.abs(r).max(axis=-1)
    return np.where(scale > 0, err / np.where(scale > 0, scale, 1), err)


@pytest.fixture(scope="session")
def orc():
    import oracle
    oracle.lib()
    return oracle
