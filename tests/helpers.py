"""Shared helpers for the parity tests."""
import numpy as np
import torch

# Tolerances on the normwise max-relative error max|x - ref| / max|ref|,
# per output tensor: fp32 inputs, and bf16 inputs with an fp32 state.
TOL_FP32 = 1e-4
TOL_BF16 = 2e-2


def relerr(x, ref):
    x = x.detach().to("cpu", torch.float64).numpy() if hasattr(x, "detach") else np.asarray(x, np.float64)
    ref = ref.detach().to("cpu", torch.float64).numpy() if hasattr(ref, "detach") else np.asarray(ref, np.float64)
    scale = np.max(np.abs(ref))
    if scale == 0:
        return float(np.max(np.abs(x)))
    return float(np.max(np.abs(x - ref)) / scale)


def tol_for(io_dtype):
    return TOL_FP32 if io_dtype == torch.float32 else TOL_BF16


def to_dev(d, device="cuda"):
    return {k: (None if v is None else v.to(device)) for k, v in d.items()}


def announce(msg):
    """Name the case before a GPU step, flushed, so a failing run says which."""
    print(f"[case] {msg}", flush=True)
