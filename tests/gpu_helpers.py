"""Shared helpers of the GPU parity tests (no layer arithmetic here): the
error measures, NaN-poisoned guarded buffers and host/device copies."""
import numpy as np
import pytest

import synth

# Tensor-wide bars (the workload definition's max relative error): bf16
# configs 2e-2, fp32 configs 1e-4.
TOL = {"bf16": 2e-2, "f32": 1e-4}
# The row-local bar is LOCAL_FACTOR times the tensor-wide one: for bf16 that
# is 0.0625 = 32 units of bf16 roundoff (u = 2^-9), room for the roundings a
# value passes through on the way (A5 of the design notes: q/k/v, P, O, h,
# g/u, dS, the activation gradients) at the tail of the error distribution
# over a million elements; for fp32 3.1e-4.
LOCAL_FACTOR = 3.125
# Share of the tensor's RMS in each element's local scale: a floor under the
# row scale, so that a single ill-conditioned value (a dot product that
# cancels, silu' near its zero for one token) is held to the noise of its
# inputs rather than to its own near-zero size, while a region whose values
# are 10x or more below the tensor's largest (the last keys of a causal dK)
# still has a scale of its own.
BETA = 0.1

# Poison byte: 0xFF fills bf16 and fp32 buffers with NaN (all-ones exponent
# and mantissa), so any output element a kernel fails to write, and any
# workspace element read before it is written, shows up as a NaN.
POISON = 0xFF
GUARD_BYTES = 64 * 1024


def need_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")


def rel_err(a, ref) -> float:
    """max|a - ref| / max|ref| over the whole tensor."""
    a = np.asarray(a, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = float(np.max(np.abs(ref))) if ref.size else 0.0
    num = float(np.max(np.abs(a - ref))) if ref.size else 0.0
    return num / den if den > 0 else num


def local_err(a, ref, row_len=None) -> float:
    """Largest element-wise ratio
        |a - ref| / (|ref| + rms(row of ref) + BETA rms(ref)).

    Rows are runs of `row_len` consecutive elements of the flattened tensor
    (default: the last axis) -- a token's features, a key's heads, an output
    row of a weight gradient.  Unlike ``rel_err`` this does not let a
    tensor's largest values hide errors in a region of small ones (the last
    keys of a causal dK, a sequence's first rows, a weight row that sees few
    tokens): each element is held to its own row's scale."""
    a = np.asarray(a, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if ref.size == 0:
        return 0.0
    n = ref.shape[-1] if row_len is None else row_len
    a2, r2 = a.reshape(-1, n), ref.reshape(-1, n)
    rms = np.sqrt(np.mean(r2 * r2, axis=1, keepdims=True))
    den = np.abs(r2) + rms + BETA * np.sqrt(np.mean(r2 * r2))
    num = np.abs(a2 - r2)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(den > 0, num / np.where(den > 0, den, 1.0), num)
    if np.isnan(ratio).any():
        return float("inf")
    return float(np.max(ratio))


def check(name, a, ref, tol, row_len=None, errs=None, local=True):
    """Both bars: the tensor-wide max relative error <= tol and the
    row-local element-wise bound <= LOCAL_FACTOR tol; NaN anywhere fails.
    local=False keeps only the tensor-wide bar (for outputs that are
    ill-conditioned by construction, said where it is used)."""
    a = np.asarray(a, dtype=np.float64)
    g = rel_err(a, ref)
    l = local_err(a, ref, row_len) if local else 0.0
    if not np.isfinite(a).all():
        g = l = float("inf")
    if errs is not None:
        errs[name] = g
        if local:
            errs[name + "_local"] = l
    return g <= tol and l <= LOCAL_FACTOR * tol


def assert_close(name, a, ref, tol, row_len=None, local=True):
    errs = {}
    ok = check(name, a, ref, tol, row_len, errs, local)
    assert ok, {k: f"{v:.3e}" for k, v in errs.items()}


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


class Guarded:
    """A device buffer of `shape` and `dtype` inside a larger allocation:
    GUARD_BYTES before and after it, everything filled with the poison
    byte.  ``t`` is the buffer handed to the library; ``guards_intact()``
    says whether anything was written outside it, ``finite()`` whether
    every element of it was written (no poison left)."""

    def __init__(self, shape, dtype, fill=None):
        import torch
        shape = tuple(int(s) for s in shape)
        es = torch.empty((), dtype=dtype).element_size()
        n = int(np.prod(shape)) if shape else 1
        g = GUARD_BYTES // es
        self.raw = torch.full((2 * GUARD_BYTES + n * es,), POISON, dtype=torch.uint8,
                              device="cuda")
        flat = self.raw.view(dtype)
        self.t = flat[g:g + n].view(shape)
        if fill is not None:
            self.t.copy_(fill)

    def guards_intact(self) -> bool:
        import torch
        head = self.raw[:GUARD_BYTES]
        tail = self.raw[-GUARD_BYTES:]
        return bool(torch.all(head == POISON)) and bool(torch.all(tail == POISON))

    def finite(self) -> bool:
        import torch
        t = self.t
        if t.dtype == torch.uint8:
            raise TypeError("finite() is for float buffers")
        return bool(torch.isfinite(t.float()).all())

    def check(self, name, written=True):
        assert self.guards_intact(), f"{name}: write outside the buffer"
        if written:
            assert self.finite(), f"{name}: elements left unwritten (poison) or NaN"


def guarded_bytes(n):
    """A Guarded uint8 buffer of n bytes (saved blocks, workspaces)."""
    import torch
    return Guarded((max(int(n), 1),), torch.uint8)


def saved_fields(cfg, lay):
    """(name, byte offset, shape, torch dtype) of every tensor the forward
    saves (only the fields the layout gives room for)."""
    import torch
    T, d, qd, kvd, f = cfg.T, cfg.d, cfg.h_q * cfg.d_h, cfg.h_kv * cfg.d_h, cfg.d_ffn
    act = cfg.torch_dtype
    f32 = torch.float32
    out = [("rstd1", (T,), f32), ("xn", (T, d), act), ("qkv", (T, qd + 2 * kvd), act),
           ("qk_rope", (T, qd + kvd), act),
           ("rope_cos", (cfg.L, cfg.d_h // 2), f32), ("rope_sin", (cfg.L, cfg.d_h // 2), f32),
           ("attn_o", (T, qd), act), ("lse", (cfg.B, cfg.h_q, cfg.L), f32),
           ("h", (T, d), act), ("rstd2", (T,), f32), ("hn", (T, d), act),
           ("gu", (T, 2 * f), act), ("f", (T, f), act)]
    if cfg.qk_norm:
        out += [("rstd_q", (T, cfg.h_q), f32), ("rstd_k", (T, cfg.h_kv), f32)]
    return [(n, lay[n], s, dt) for n, s, dt in out]


def view_saved(buf, off, shape, dtype):
    import torch
    es = torch.empty((), dtype=dtype).element_size()
    nbytes = int(np.prod(shape)) * es
    return buf[off:off + nbytes].view(dtype).view(shape)
