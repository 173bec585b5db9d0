"""Helpers for the GPU tests: device copies of generator arrays and the
comparison rule (max |gpu - oracle| over every compared element)."""
import sys

import numpy as np
import pytest
import torch

import gqa_inputs as gi

TOL = {"f32": 1e-5, "bf16": 2e-2}


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")


def say(*parts):
    print("[gpu-test]", *parts, flush=True)
    sys.stdout.flush()


def dev(arr: np.ndarray, dtype: str) -> torch.Tensor:
    """Device tensor holding exactly the generator's values."""
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(arr)).cuda()


def decode_tensors(inp: gi.DecodeInputs):
    dt = inp.cfg.dtype
    return (dev(inp.q, dt), dev(inp.k_cache, dt), dev(inp.v_cache, dt),
            torch.from_numpy(inp.seq_lens).cuda())


def max_err(got: np.ndarray, ref: np.ndarray) -> float:
    got = np.asarray(got, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), "non-finite GPU output"
    return float(np.max(np.abs(got - ref))) if got.size else 0.0
