"""Helpers for the GPU parity tests: device transfer, error metrics, tolerances."""
import sys

import numpy as np
import torch

# Tolerances of the parity bar: fp32 path max-abs; bf16-input / fp32-accumulate paths
# max-abs and relative L2 (||gpu - oracle|| / ||oracle||).
FP32_MAX_ABS = 1e-5
BF16_MAX_ABS = 2e-2
BF16_REL_L2 = 5e-3


def say(*a):
    """Name the case before a GPU step, flushed, so a failing run still shows it."""
    print("[case]", *a, file=sys.stderr, flush=True)


def dev(t):
    return t.contiguous().to("cuda")


def host64(t):
    return t.detach().to("cpu").to(torch.float64).numpy()


def errors(gpu, ref):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    assert np.isfinite(gpu).all(), "non-finite GPU output"
    diff = gpu - ref
    max_abs = float(np.max(np.abs(diff))) if diff.size else 0.0
    nref = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(diff)) / nref if nref > 0 else float(np.linalg.norm(diff))
    return max_abs, rel


def assert_fp32(gpu, ref, tol=FP32_MAX_ABS, what=""):
    m, r = errors(gpu, ref)
    assert m <= tol, f"{what}: max-abs {m:.3e} > {tol:.0e} (rel-L2 {r:.3e})"
    return m, r


def assert_bf16(gpu, ref, what=""):
    m, r = errors(gpu, ref)
    assert m <= BF16_MAX_ABS and r <= BF16_REL_L2, \
        f"{what}: max-abs {m:.3e} (<= {BF16_MAX_ABS}), rel-L2 {r:.3e} (<= {BF16_REL_L2})"
    return m, r
