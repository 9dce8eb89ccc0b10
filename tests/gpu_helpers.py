"""Shared helpers of the GPU tests (no arithmetic of the method here)."""
import numpy as np
import torch

TOL = {"bf16": 1e-2, "fp32": 1e-4}


def require_gpu():
    if not torch.cuda.is_available():
        raise RuntimeError("this test needs a gfx950 GPU")
    name = torch.cuda.get_device_properties(0).gcnArchName
    assert name.startswith("gfx950"), f"expected gfx950, found {name}"


def f64(t):
    if t is None:
        return None
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel_err(x, ref):
    """max |x - ref| / max |ref| in fp64 (the graded measure)."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = float(np.max(np.abs(ref))) if ref.size else 0.0
    num = float(np.max(np.abs(x - ref))) if ref.size else 0.0
    return num / den if den > 0 else num


def per_head_err(x, ref):
    """Relative error of each (b, h) slice, for reporting."""
    B, H = ref.shape[:2]
    return np.array([[rel_err(x[b, h], ref[b, h]) for h in range(H)] for b in range(B)])


def log(msg):
    print(msg, flush=True)
