"""Shared helpers for the GPU parity tests (imported only by tests marked gpu)."""

import sys

import numpy as np
import torch

import attention_causal_gqa_amd as A

# Tolerances: max |gpu - oracle| over all compared elements, in fp64.
TOL_F32 = 1e-4   # fp32 path
TOL_BF16 = 1.6e-2  # bf16 inputs, fp32 accumulation, bf16 output
TOL_LSE = 1e-3


def device():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a GPU: none is visible")
    A.load_library()  # raises if libattn.so is not built
    return torch.device("cuda:0")


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def np64(t):
    return t.detach().cpu().to(torch.float64).numpy()


def max_err(got, want, what, tol, extra=""):
    """Assert max |got - want| <= tol; on failure report the worst element."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (got.shape, want.shape)
    if got.size == 0:
        return 0.0
    both_inf = np.isinf(got) & np.isinf(want) & (np.sign(got) == np.sign(want))
    err = np.where(both_inf, 0.0, np.abs(got - want))
    err = np.where(np.isnan(err), np.inf, err)
    worst = float(err.max())
    if not worst <= tol:
        idx = np.unravel_index(int(np.argmax(err)), err.shape)
        raise AssertionError(
            f"{what}: max err {worst:.3e} > {tol:.1e} at {idx}: got {got[idx]!r} want {want[idx]!r} {extra}")
    return worst
