"""Shared helpers of the GPU parity tests."""
import os

import numpy as np
import pytest
import torch

FP32_TOL = 2e-4   # max|err| / max|ref| for fp32 paths
FP16_TOL = 2e-2   # for fp16-operand contraction paths
# bfloat16-operand paths: the error of a rounded-operand contraction scales
# with the operands' unit roundoff, 8x larger for bfloat16 (2^-8) than for
# fp16 (2^-11); the fp16 paths measure <= 1.3e-3 against the oracle at the
# full Qwen3-4B shape, so bfloat16 is expected near 1e-2, and 5e-2 bounds it
# with margin.
BF16_TOL = 5e-2


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def host(t):
    return t.detach().float().cpu().double().numpy() if t.dtype != torch.float64 else t.detach().cpu().numpy()


def rel_err(gpu, ref):
    g = host(gpu) if isinstance(gpu, torch.Tensor) else np.asarray(gpu, np.float64)
    r = np.asarray(ref, np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    denom = np.max(np.abs(r))
    if denom == 0.0:
        return float(np.max(np.abs(g)))
    return float(np.max(np.abs(g - r)) / denom)


# Every comparison made through check(): (test id, tensor name, error, tolerance).
# The test session prints the worst ratio per test at its end (conftest.py).
PARITY_LOG = []


def check(name, gpu, ref, tol, report=None):
    e = rel_err(gpu, ref)
    if report is not None:
        report[name] = e
    test = os.environ.get("PYTEST_CURRENT_TEST", "?").split(" ")[0]
    PARITY_LOG.append((test, name, e, tol))
    assert e <= tol, f"{name}: max|err|/max|ref| = {e:.3e} > {tol:.1e}"
    return e


def announce(msg):
    print(msg, flush=True)
