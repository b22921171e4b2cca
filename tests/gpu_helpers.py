"""Shared helpers of the GPU parity tests (no layer arithmetic here)."""
import numpy as np
import pytest

import synth

# Relative-error bars: max|gpu - oracle| / max|oracle| per tensor.
TOL = {"bf16": 2e-2, "f32": 1e-4}


def need_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")


def rel_err(a, ref) -> float:
    a = np.asarray(a, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = float(np.max(np.abs(ref))) if ref.size else 0.0
    num = float(np.max(np.abs(a - ref))) if ref.size else 0.0
    return num / den if den > 0 else num


def dev(a, dtype):
    """fp32 numpy -> CUDA tensor in `dtype` (exact for bf16-grid values)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    td = torch.bfloat16 if dtype == "bf16" else torch.float32
    return t.to(device="cuda", dtype=td)


def host(t) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def gpu_weights(inp, dtype):
    return {n: dev(inp[n], dtype) for n in synth.PARAM_NAMES}


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)
