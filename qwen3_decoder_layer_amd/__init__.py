"""Python binding of libq3layer.so: one Qwen3 decoder layer (forward and
backward) on an MI355X, computed entirely by the library's HIP kernels.

The functions below have the names of the C ABI in include/q3layer.h minus
the ``q3l_`` prefix.  They only marshal arguments: tensors are torch tensors
on the GPU (PyTorch supplies device memory, streams and events), and any
buffer the caller does not pass is allocated with ``torch.empty``.  Shapes,
dtypes and sizes are checked here before a pointer crosses the C ABI.  If the
library is missing the calls raise; there is no fallback path.
"""
from __future__ import annotations

import ctypes as C
from dataclasses import dataclass, asdict

from . import _abi
from ._abi import (BWD_ACCUMULATE, BWD_DEFERRED_WEIGHT, BWD_INPUT, BWD_WEIGHT,
                   PARAMS, Q3L_BF16, Q3L_F32)

__all__ = ["LayerConfig", "Q3LError", "Exec", "MarkEvents", "validate", "saved_bytes",
           "workspace_bytes", "saved_layout", "phase_names", "layer_forward",
           "layer_backward", "rmsnorm_fwd", "rmsnorm_bwd", "rope_table",
           "qknorm_rope_fwd", "qknorm_rope_bwd", "linear_fwd", "linear_dgrad",
           "linear_wgrad", "swiglu_fwd", "swiglu_bwd", "attention_fwd",
           "attention_bwd", "attention_bwd_noalloc", "attention_fwd_block",
           "attention_merge", "attention_finish", "library", "param_shapes", "PARAMS", "BWD_INPUT",
           "BWD_WEIGHT", "BWD_ACCUMULATE", "BWD_DEFERRED_WEIGHT", "ModelConfig",
           "model_validate", "model_saved_bytes", "model_workspace_bytes",
           "model_forward", "model_backward"]


class Q3LError(RuntimeError):
    pass


def library():
    return _abi.load()


@dataclass
class LayerConfig:
    d: int
    h_q: int
    h_kv: int
    d_h: int
    d_ffn: int
    B: int
    L: int
    eps: float = 1e-6
    rope_theta: float = 1e6
    qk_norm: bool = True
    tp_partial: bool = False
    dtype: str = "bf16"          # "bf16" or "f32"

    @classmethod
    def from_dict(cls, c: dict) -> "LayerConfig":
        keys = cls.__dataclass_fields__.keys()
        return cls(**{k: c[k] for k in keys if k in c})

    def c_struct(self) -> _abi.Cfg:
        return _abi.Cfg(self.d, self.h_q, self.h_kv, self.d_h, self.d_ffn,
                        self.B, self.L, self.eps, self.rope_theta,
                        int(bool(self.qk_norm)), int(bool(self.tp_partial)),
                        Q3L_BF16 if self.dtype == "bf16" else Q3L_F32)

    @property
    def T(self):
        return self.B * self.L

    @property
    def torch_dtype(self):
        import torch
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    def as_dict(self):
        return asdict(self)


def param_shapes(cfg: LayerConfig) -> dict:
    """Shapes of the eleven parameters as the C ABI reads them."""
    qd, kvd = cfg.h_q * cfg.d_h, cfg.h_kv * cfg.d_h
    return {"in_norm": (cfg.d,), "q": (qd, cfg.d), "k": (kvd, cfg.d),
            "v": (kvd, cfg.d), "q_norm": (cfg.d_h,), "k_norm": (cfg.d_h,),
            "o": (cfg.d, qd), "post_norm": (cfg.d,), "gate": (cfg.d_ffn, cfg.d),
            "up": (cfg.d_ffn, cfg.d), "down": (cfg.d, cfg.d_ffn)}


def _check(status: int):
    if status != 0:
        msg = library().q3l_last_error().decode()
        raise Q3LError(f"{_abi.STATUS.get(status, status)}: {msg}")


def _p(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return C.c_void_p(stream.cuda_stream)


def _code(dtype) -> int:
    import torch
    if dtype in ("bf16", torch.bfloat16, Q3L_BF16):
        return Q3L_BF16
    if dtype in ("f32", torch.float32, Q3L_F32):
        return Q3L_F32
    raise ValueError(f"unsupported dtype {dtype!r}")


def _need(t, name, numel=None, dtype=None, contiguous=True, min_bytes=None):
    """Raise unless tensor t is on the GPU with the given size and dtype."""
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} has {t.numel()} elements, expected {numel}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if min_bytes is not None and t.numel() * t.element_size() < min_bytes:
        raise ValueError(f"{name} holds {t.numel() * t.element_size()} bytes, "
                         f"{min_bytes} needed")


def _nbytes(t):
    return 0 if t is None else t.numel() * t.element_size()


_HIP = None
_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000   # hipEventDisableSystemFence


def _hip():
    """The HIP runtime already loaded into the process (torch's; the library
    links against the same soname, so there is one runtime)."""
    global _HIP
    if _HIP is None:
        h = C.CDLL("libamdhip64.so.7")
        h.hipEventCreateWithFlags.argtypes = [C.POINTER(C.c_void_p), C.c_uint]
        h.hipEventDestroy.argtypes = [C.c_void_p]
        h.hipEventElapsedTime.argtypes = [C.POINTER(C.c_float), C.c_void_p, C.c_void_p]
        h.hipEventSynchronize.argtypes = [C.c_void_p]
        _HIP = h
    return _HIP


class MarkEvents:
    """n timing events for phase marks, created with
    hipEventDisableSystemFence: recording one costs no system-scope cache
    writeback, so marks between kernels change the timed work little.
    Read the times after the work has finished (elapsed())."""

    def __init__(self, n):
        import torch
        torch.cuda.init()
        hip = _hip()
        self.handles = []
        for _ in range(n):
            e = C.c_void_p()
            st = hip.hipEventCreateWithFlags(C.byref(e), _EVENT_DISABLE_SYSTEM_FENCE)
            if st != 0:
                raise Q3LError(f"hipEventCreateWithFlags failed ({st})")
            self.handles.append(e.value)

    def __len__(self):
        return len(self.handles)

    def elapsed(self, i, j):
        hip = _hip()
        if hip.hipEventSynchronize(self.handles[j]) != 0:
            raise Q3LError("hipEventSynchronize failed")
        ms = C.c_float()
        if hip.hipEventElapsedTime(C.byref(ms), self.handles[i], self.handles[j]) != 0:
            raise Q3LError("hipEventElapsedTime failed")
        return ms.value

    def __del__(self):
        try:
            hip = _hip()
            for h in self.handles:
                hip.hipEventDestroy(h)
        except Exception:  # pragma: no cover - interpreter shutdown
            pass


class Exec:
    """Execution options of layer_forward / layer_backward (q3l_exec).

    side_stream: a torch.cuda.Stream for the bf16 training forward's
    transposed copies (run beside the attention step; two events for the
    fork and join are created here).  marks: ``phase_count + 1`` timing
    events -- a MarkEvents, or a list of ``torch.cuda.Event(enable_timing=
    True)`` -- recorded by the library at the phase boundaries; read them
    back with ``phase_times()``."""

    def __init__(self, side_stream=None, marks=None):
        import torch
        self.side_stream = side_stream
        self.marks = marks if isinstance(marks, MarkEvents) else (
            list(marks) if marks else None)
        self._fork = self._join = None
        if side_stream is not None:
            self._fork, self._join = torch.cuda.Event(), torch.cuda.Event()
            # torch creates the HIP event on its first record.
            for e in (self._fork, self._join):
                e.record(side_stream)
        if self.marks and not isinstance(self.marks, MarkEvents):
            for e in self.marks:
                e.record()
        self._arr = None

    def c_struct(self) -> _abi.Exec:
        ex = _abi.Exec()
        if self.side_stream is not None:
            ex.side_stream = self.side_stream.cuda_stream
            ex.fork_event = self._fork.cuda_event
            ex.join_event = self._join.cuda_event
        if self.marks:
            hs = (self.marks.handles if isinstance(self.marks, MarkEvents)
                  else [e.cuda_event for e in self.marks])
            self._arr = (C.c_void_p * len(hs))(*hs)
            ex.marks = C.cast(self._arr, C.POINTER(C.c_void_p))
            ex.n_marks = len(self.marks)
        return ex

    def phase_times(self):
        """Milliseconds of each phase from the last call's marks."""
        if isinstance(self.marks, MarkEvents):
            return [self.marks.elapsed(i, i + 1) for i in range(len(self.marks) - 1)]
        return [a.elapsed_time(b) for a, b in zip(self.marks, self.marks[1:])]


def _exec(ex):
    return None if ex is None else C.byref(ex.c_struct())


def phase_names(backward: bool) -> list:
    lib = library()
    b = int(bool(backward))
    return [lib.q3l_phase_name(b, i).decode() for i in range(lib.q3l_phase_count(b))]


def validate(cfg: LayerConfig) -> None:
    c = cfg.c_struct()
    _check(library().q3l_validate(C.byref(c)))


def saved_bytes(cfg: LayerConfig) -> int:
    c = cfg.c_struct()
    return library().q3l_saved_bytes(C.byref(c))


def workspace_bytes(cfg: LayerConfig, backward: bool) -> int:
    c = cfg.c_struct()
    return library().q3l_workspace_bytes(C.byref(c), int(bool(backward)))


def saved_layout(cfg: LayerConfig) -> dict:
    c = cfg.c_struct()
    lay = _abi.SavedLayout()
    _check(library().q3l_saved_layout_of(C.byref(c), C.byref(lay)))
    return {n: getattr(lay, n) for n in _abi.SAVED_FIELDS}


def _weights(cfg: LayerConfig, w: dict) -> _abi.Weights:
    shapes = param_shapes(cfg)
    for n in PARAMS:
        if not cfg.qk_norm and n in ("q_norm", "k_norm") and w.get(n) is None:
            continue
        _need(w.get(n), f"weights[{n!r}]", numel=int(__import__("math").prod(shapes[n])),
              dtype=cfg.torch_dtype)
    return _abi.Weights(*[None if w.get(n) is None else w[n].data_ptr()
                          for n in PARAMS])


def _bytes(n, device):
    import torch
    return torch.empty(max(int(n), 1), dtype=torch.uint8, device=device)


def layer_forward(cfg: LayerConfig, weights: dict, x, out: dict | None = None,
                  saved=None, workspace=None, stream=None, exec=None) -> dict:
    """q3l_layer_forward.  x: [B, L, d] (or [T, d]) tensor of cfg's dtype.

    Returns {"y"} or, for tp_partial, {"attn_partial", "mlp_partial"}
    (fp32).  Pass ``saved`` (uint8, ``saved_bytes(cfg)``) to keep the
    intermediates for ``layer_backward``; ``exec`` is an optional Exec."""
    import torch
    c = cfg.c_struct()
    lib = library()
    _need(x, "x", numel=cfg.T * cfg.d, dtype=cfg.torch_dtype)
    out = dict(out or {})
    shape = (cfg.B, cfg.L, cfg.d)
    if cfg.tp_partial:
        for k in ("attn_partial", "mlp_partial"):
            if out.get(k) is None:
                out[k] = torch.empty(shape, dtype=torch.float32, device=x.device)
            _need(out[k], k, numel=cfg.T * cfg.d, dtype=torch.float32)
        o = _abi.Outputs(None, out["attn_partial"].data_ptr(),
                         out["mlp_partial"].data_ptr())
    else:
        if out.get("y") is None:
            out["y"] = torch.empty(shape, dtype=x.dtype, device=x.device)
        _need(out["y"], "y", numel=cfg.T * cfg.d, dtype=cfg.torch_dtype)
        o = _abi.Outputs(out["y"].data_ptr(), None, None)
    if saved is not None:
        _need(saved, "saved", min_bytes=saved_bytes(cfg))
    elif workspace is None:
        workspace = _bytes(workspace_bytes(cfg, False), x.device)
    if workspace is not None:
        _need(workspace, "workspace")
    w = _weights(cfg, weights)
    _check(lib.q3l_layer_forward(C.byref(c), C.byref(w), _p(x), C.byref(o),
                                 _p(saved), _p(workspace), _nbytes(workspace),
                                 _stream(stream), _exec(exec)))
    return out


def layer_backward(cfg: LayerConfig, weights: dict, x, dy, saved, dx=None,
                   grads: dict | None = None,
                   flags: int = BWD_INPUT | BWD_WEIGHT, workspace=None,
                   stream=None, exec=None):
    """q3l_layer_backward.  Returns (dx, grads) with grads a dict of fp32
    tensors shaped like the parameters.  For a split backward, pass the
    same ``workspace`` to the INPUT call and to its WEIGHT |
    DEFERRED_WEIGHT call."""
    import torch
    c = cfg.c_struct()
    lib = library()
    td = cfg.torch_dtype
    _need(x, "x", numel=cfg.T * cfg.d, dtype=td)
    _need(dy, "dy", numel=cfg.T * cfg.d, dtype=td)
    _need(saved, "saved", min_bytes=saved_bytes(cfg))
    if (flags & BWD_INPUT) and dx is None:
        dx = torch.empty_like(x)
    if dx is not None:
        _need(dx, "dx", numel=cfg.T * cfg.d, dtype=td)
    if flags & BWD_WEIGHT:
        grads = dict(grads or {})
        for n, shp in param_shapes(cfg).items():
            if grads.get(n) is None:
                grads[n] = torch.empty(shp, dtype=torch.float32, device=x.device)
            _need(grads[n], f"grads[{n!r}]", numel=int(__import__("math").prod(shp)),
                  dtype=torch.float32)
    g = _abi.Grads(*[None if not grads or grads.get(n) is None
                     else grads[n].data_ptr() for n in PARAMS])
    if workspace is None:
        workspace = _bytes(workspace_bytes(cfg, True), x.device)
    _need(workspace, "workspace")
    w = _weights(cfg, weights)
    _check(lib.q3l_layer_backward(C.byref(c), C.byref(w), _p(x), _p(dy),
                                  _p(saved), _p(dx), C.byref(g), flags,
                                  _p(workspace), _nbytes(workspace),
                                  _stream(stream), _exec(exec)))
    return dx, grads


# ---- phase-level calls --------------------------------------------------
def _rows_n(x):
    return x.numel() // x.shape[-1], x.shape[-1]


def rmsnorm_fwd(x, w, eps, y=None, rstd=None, stream=None):
    import torch
    rows, n = _rows_n(x)
    _need(x, "x")
    _need(w, "w", numel=n, dtype=x.dtype)
    y = torch.empty_like(x) if y is None else y
    rstd = (torch.empty(rows, dtype=torch.float32, device=x.device)
            if rstd is None else rstd)
    _need(y, "y", numel=x.numel(), dtype=x.dtype)
    _need(rstd, "rstd", numel=rows, dtype=torch.float32)
    _check(library().q3l_rmsnorm_fwd(_code(x.dtype), rows, n, _p(x), _p(w), eps,
                                     _p(y), _p(rstd), _stream(stream)))
    return y, rstd


def rmsnorm_bwd(dy, x, rstd, w, resid=None, dx=None, dw=None, accumulate=False,
                want_dw=True, workspace=None, stream=None):
    """dx = resid + RMSNorm adjoint; dw (+)= sum over rows (fp32)."""
    import torch
    rows, n = _rows_n(x)
    for t, name in ((dy, "dy"), (x, "x")):
        _need(t, name, numel=rows * n, dtype=x.dtype)
    _need(rstd, "rstd", numel=rows, dtype=torch.float32)
    _need(w, "w", numel=n, dtype=x.dtype)
    if resid is not None:
        _need(resid, "resid", numel=rows * n, dtype=x.dtype)
    dx = torch.empty_like(x) if dx is None else dx
    _need(dx, "dx", numel=rows * n, dtype=x.dtype)
    if want_dw and dw is None:
        dw = torch.empty(n, dtype=torch.float32, device=x.device)
    if dw is not None:
        _need(dw, "dw", numel=n, dtype=torch.float32)
    lib = library()
    nb = lib.q3l_rmsnorm_bwd_workspace_bytes(n)
    workspace = _bytes(nb, x.device) if workspace is None else workspace
    _check(lib.q3l_rmsnorm_bwd(_code(x.dtype), rows, n, _p(dy), _p(x), _p(rstd),
                               _p(w), _p(resid), _p(dx), _p(dw), int(bool(accumulate)),
                               _p(workspace), _nbytes(workspace), _stream(stream)))
    return dx, dw


def rope_table(L, d_h, theta, device="cuda", stream=None):
    """(cos, sin), each fp32 [L, d_h/2]."""
    import torch
    cos = torch.empty((L, d_h // 2), dtype=torch.float32, device=device)
    sin = torch.empty_like(cos)
    _check(library().q3l_rope_table(L, d_h, theta, _p(cos), _p(sin), _stream(stream)))
    return cos, sin


def qknorm_rope_fwd(qk, wq, wk, cos, sin, h_q, h_kv, d_h, eps=1e-6, qk_norm=True,
                    out=None, rstd_q=None, rstd_k=None, stream=None):
    """qk: [B, L, >= (h_q + h_kv) d_h] with h_q query heads then h_kv key
    heads (row stride from the tensor).  Returns (out, rstd_q, rstd_k)."""
    import torch
    B, L = qk.shape[0], qk.shape[1]
    w = (h_q + h_kv) * d_h
    out = torch.empty((B, L, w), dtype=qk.dtype, device=qk.device) if out is None else out
    rstd_q = (torch.empty((B * L, h_q), dtype=torch.float32, device=qk.device)
              if rstd_q is None else rstd_q)
    rstd_k = (torch.empty((B * L, h_kv), dtype=torch.float32, device=qk.device)
              if rstd_k is None else rstd_k)
    for t, name in ((cos, "cos"), (sin, "sin")):
        _need(t, name, numel=L * d_h // 2, dtype=torch.float32)
    _need(rstd_q, "rstd_q", numel=B * L * h_q, dtype=torch.float32)
    _need(rstd_k, "rstd_k", numel=B * L * h_kv, dtype=torch.float32)
    _check(library().q3l_qknorm_rope_fwd(
        _code(qk.dtype), B, L, h_q, h_kv, d_h, int(bool(qk_norm)), eps, _p(qk),
        qk.stride(1), _p(wq), _p(wk), _p(cos), _p(sin), _p(out), out.stride(1),
        _p(rstd_q), _p(rstd_k), _stream(stream)))
    return out, rstd_q, rstd_k


def qknorm_rope_bwd(g, pre, wq, wk, rstd_q, rstd_k, cos, sin, h_q, h_kv, d_h,
                    qk_norm=True, out=None, dwq=None, dwk=None, accumulate=False,
                    stream=None):
    """Adjoint of qknorm_rope_fwd.  Returns (out, dwq, dwk)."""
    import torch
    B, L = g.shape[0], g.shape[1]
    w = (h_q + h_kv) * d_h
    out = torch.empty((B, L, w), dtype=g.dtype, device=g.device) if out is None else out
    if qk_norm:
        dwq = torch.empty(d_h, dtype=torch.float32, device=g.device) if dwq is None else dwq
        dwk = torch.empty(d_h, dtype=torch.float32, device=g.device) if dwk is None else dwk
    lib = library()
    nb = lib.q3l_qknorm_rope_bwd_workspace_bytes(d_h)
    ws = _bytes(nb, g.device)
    _check(lib.q3l_qknorm_rope_bwd(
        _code(g.dtype), B, L, h_q, h_kv, d_h, int(bool(qk_norm)), _p(g), g.stride(1),
        _p(pre), 0 if pre is None else pre.stride(1), _p(wq), _p(wk), _p(rstd_q),
        _p(rstd_k), _p(cos), _p(sin), _p(out), out.stride(1), _p(dwq), _p(dwk),
        int(bool(accumulate)), _p(ws), nb, _stream(stream)))
    return out, dwq, dwk


def linear_fwd(a, w, resid=None, y=None, stream=None):
    import torch
    M, K = _rows_n(a)
    N = w.shape[0]
    _need(a, "a")
    _need(w, "w", numel=N * K, dtype=a.dtype)
    y = torch.empty((*a.shape[:-1], N), dtype=a.dtype, device=a.device) \
        if y is None else y
    _need(y, "y", numel=M * N, dtype=a.dtype)
    if resid is not None:
        _need(resid, "resid", numel=M * N, dtype=a.dtype)
    _check(library().q3l_linear_fwd(_code(a.dtype), M, N, K, _p(a), _p(w),
                                    _p(resid), _p(y), _stream(stream)))
    return y


def linear_dgrad(dy, w, da=None, stream=None):
    import torch
    M, N = _rows_n(dy)
    K = w.shape[1]
    _need(dy, "dy")
    _need(w, "w", numel=N * K, dtype=dy.dtype)
    da = torch.empty((*dy.shape[:-1], K), dtype=dy.dtype, device=dy.device) \
        if da is None else da
    _need(da, "da", numel=M * K, dtype=dy.dtype)
    _check(library().q3l_linear_dgrad(_code(dy.dtype), M, N, K, _p(dy), _p(w),
                                      _p(da), _stream(stream)))
    return da


def linear_wgrad(dy, a, dw=None, accumulate=False, stream=None):
    import torch
    M, N = _rows_n(dy)
    K = a.shape[-1]
    _need(dy, "dy")
    _need(a, "a", numel=M * K, dtype=dy.dtype)
    dw = torch.empty((N, K), dtype=torch.float32, device=dy.device) \
        if dw is None else dw
    _need(dw, "dw", numel=N * K, dtype=torch.float32)
    _check(library().q3l_linear_wgrad(_code(dy.dtype), M, N, K, _p(dy), _p(a),
                                      _p(dw), int(bool(accumulate)),
                                      _stream(stream)))
    return dw


def swiglu_fwd(hn, gate, up, f=None, gu=None, stream=None):
    """f = silu(hn gate^T) * (hn up^T) with the layer's fused kernel; gu
    (optional [M, 2N]) receives gate | up pre-activations."""
    import torch
    M, K = _rows_n(hn)
    N = gate.shape[0]
    _need(hn, "hn")
    _need(gate, "gate", numel=N * K, dtype=hn.dtype)
    _need(up, "up", numel=N * K, dtype=hn.dtype)
    f = torch.empty((*hn.shape[:-1], N), dtype=hn.dtype, device=hn.device) \
        if f is None else f
    _need(f, "f", numel=M * N, dtype=hn.dtype)
    if gu is not None:
        _need(gu, "gu", numel=M * 2 * N, dtype=hn.dtype)
    _check(library().q3l_swiglu_fwd(_code(hn.dtype), M, N, K, _p(hn),
                                    _p(gate), _p(up), _p(f), _p(gu),
                                    _stream(stream)))
    return f


def swiglu_bwd(df, gu, dgu=None, stream=None):
    """dg | du ([M, 2N]) from df [M, N] and g | u [M, 2N]."""
    import torch
    M, N = _rows_n(df)
    _need(df, "df")
    _need(gu, "gu", numel=M * 2 * N, dtype=df.dtype)
    dgu = torch.empty((*df.shape[:-1], 2 * N), dtype=df.dtype, device=df.device) \
        if dgu is None else dgu
    _need(dgu, "dgu", numel=M * 2 * N, dtype=df.dtype)
    _check(library().q3l_swiglu_bwd(_code(df.dtype), M, N, _p(df), _p(gu), _p(dgu),
                                    _stream(stream)))
    return dgu


def attention_fwd(q, k, v, h_q, h_kv, d_h, o=None, lse=None, stream=None):
    """q [B, L, >=h_q*d_h], k/v [B, L, >=h_kv*d_h] (row strides taken from
    the tensors; the last dim must be contiguous)."""
    import torch
    B, L = q.shape[0], q.shape[1]
    o = torch.empty((B, L, h_q * d_h), dtype=q.dtype, device=q.device) \
        if o is None else o
    lse = torch.empty((B, h_q, L), dtype=torch.float32, device=q.device) \
        if lse is None else lse
    _need(lse, "lse", numel=B * h_q * L, dtype=torch.float32)
    _check(library().q3l_attention_fwd(
        _code(q.dtype), B, L, h_q, h_kv, d_h, _p(q), q.stride(1), _p(k),
        k.stride(1), _p(v), v.stride(1), _p(o), o.stride(1), _p(lse),
        _stream(stream)))
    return o, lse


def attention_fwd_block(q, k, v, h_q, h_kv, d_h, k0, k1, m=None, l=None, acc=None,
                        stream=None):
    """Block state (m, l, acc) of attention over keys [k0, k1) (fp32)."""
    import torch
    B, L = q.shape[0], q.shape[1]
    m = torch.empty((B, h_q, L), dtype=torch.float32, device=q.device) if m is None else m
    l = torch.empty((B, h_q, L), dtype=torch.float32, device=q.device) if l is None else l
    acc = (torch.empty((B, L, h_q * d_h), dtype=torch.float32, device=q.device)
           if acc is None else acc)
    for t, name, n in ((m, "m", B * h_q * L), (l, "l", B * h_q * L),
                       (acc, "acc", B * L * h_q * d_h)):
        _need(t, name, numel=n, dtype=torch.float32)
    _check(library().q3l_attention_fwd_block(
        _code(q.dtype), B, L, h_q, h_kv, d_h, _p(q), q.stride(1), _p(k), k.stride(1),
        _p(v), v.stride(1), int(k0), int(k1), _p(m), _p(l), _p(acc), _stream(stream)))
    return m, l, acc


def attention_merge(state, state2, stream=None):
    """state := merge(state, state2) in place; states are (m, l, acc)."""
    m, l, acc = state
    m2, l2, acc2 = state2
    B, h_q, L = m.shape
    d_h = acc.shape[-1] // h_q
    for a, b, name in ((m2, m, "m2"), (l2, l, "l2"), (acc2, acc, "acc2")):
        _need(a, name, numel=b.numel(), dtype=b.dtype)
    _check(library().q3l_attention_merge(B, L, h_q, d_h, _p(m), _p(l), _p(acc), _p(m2),
                                         _p(l2), _p(acc2), _stream(stream)))
    return state


def attention_finish(state, dtype="bf16", o=None, lse=None, stream=None):
    """(o, lse) of a merged state."""
    import torch
    m, l, acc = state
    B, h_q, L = m.shape
    d_h = acc.shape[-1] // h_q
    td = torch.bfloat16 if _code(dtype) == Q3L_BF16 else torch.float32
    o = torch.empty((B, L, h_q * d_h), dtype=td, device=m.device) if o is None else o
    lse = torch.empty((B, h_q, L), dtype=torch.float32, device=m.device) if lse is None else lse
    _check(library().q3l_attention_finish(_code(dtype), B, L, h_q, d_h, _p(m), _p(l), _p(acc),
                                          _p(o), o.stride(1), _p(lse), _stream(stream)))
    return o, lse


def _like_strided(t):
    """An uninitialised tensor with t's sizes and strides (so a strided view
    gets an output of the layout the library writes)."""
    import torch
    return torch.empty_strided(t.size(), t.stride(), dtype=t.dtype, device=t.device)


def attention_bwd(q, k, v, o, dout, lse, h_q, h_kv, d_h, dq=None, dk=None,
                  dv=None, stream=None, stored_ds=True):
    """dq, dk, dv are written with q, k, v's row strides: by default they
    are allocated with the same strides.  stored_ds: give the library the
    workspace with which the bf16 backward stores dS and forms dQ from it
    (False: the minimum, with which it recomputes S and dP for dQ)."""
    B, L = q.shape[0], q.shape[1]
    dq = _like_strided(q) if dq is None else dq
    dk = _like_strided(k) if dk is None else dk
    dv = _like_strided(v) if dv is None else dv
    for a, b, name in ((dq, q, "dq"), (dk, k, "dk"), (dv, v, "dv")):
        if a.stride() != b.stride() or a.shape != b.shape:
            raise ValueError(f"{name} must have the shape and strides of its input")
    lib = library()
    n = (lib.q3l_attention_bwd_stored_ds_workspace_bytes if stored_ds
         else lib.q3l_attention_bwd_workspace_bytes)(B, L, h_q)
    ws = _bytes(n, q.device)
    _check(lib.q3l_attention_bwd(
        _code(q.dtype), B, L, h_q, h_kv, d_h, _p(q), q.stride(1), _p(k),
        k.stride(1), _p(v), v.stride(1), _p(o), o.stride(1), _p(dout),
        dout.stride(1), _p(lse), _p(dq), _p(dk), _p(dv), _p(ws), n,
        _stream(stream)))
    return dq, dk, dv


def attention_bwd_noalloc(q, k, v, o, dout, lse, h_q, h_kv, d_h, dq, dk, dv, stream=None):
    """q3l_attention_bwd_noalloc: the attention backward with the library's
    built-in scratch; the caller passes every output (nothing is allocated
    here or in the library)."""
    B, L = q.shape[0], q.shape[1]
    for a, b, name in ((dq, q, "dq"), (dk, k, "dk"), (dv, v, "dv")):
        if a is None or a.stride() != b.stride() or a.shape != b.shape:
            raise ValueError(f"{name} must be given with the shape and strides of its input")
    _check(library().q3l_attention_bwd_noalloc(
        _code(q.dtype), B, L, h_q, h_kv, d_h, _p(q), q.stride(1), _p(k),
        k.stride(1), _p(v), v.stride(1), _p(o), o.stride(1), _p(dout),
        dout.stride(1), _p(lse), _p(dq), _p(dk), _p(dv), _stream(stream)))
    return dq, dk, dv


# ---- the model around a stack of layers ----------------------------------
@dataclass
class ModelConfig:
    layer: LayerConfig
    n_layers: int
    vocab: int
    recompute: bool = False

    def c_struct(self) -> _abi.ModelCfg:
        return _abi.ModelCfg(self.layer.c_struct(), self.n_layers, self.vocab,
                             int(bool(self.recompute)))


def model_validate(mc: ModelConfig) -> None:
    c = mc.c_struct()
    _check(library().q3l_model_validate(C.byref(c)))


def model_saved_bytes(mc: ModelConfig) -> int:
    c = mc.c_struct()
    return library().q3l_model_saved_bytes(C.byref(c))


def model_workspace_bytes(mc: ModelConfig, backward: bool) -> int:
    c = mc.c_struct()
    return library().q3l_model_workspace_bytes(C.byref(c), int(bool(backward)))


def _model_weights(mc: ModelConfig, embed, final_norm, layers):
    cfg = mc.layer
    _need(embed, "embed", numel=mc.vocab * cfg.d, dtype=cfg.torch_dtype)
    _need(final_norm, "final_norm", numel=cfg.d, dtype=cfg.torch_dtype)
    if len(layers) != mc.n_layers:
        raise ValueError(f"{len(layers)} layer weight dicts for {mc.n_layers} layers")
    arr = (_abi.Weights * max(1, mc.n_layers))(*[_weights(cfg, l) for l in layers])
    return _abi.ModelWeights(embed.data_ptr(), final_norm.data_ptr(),
                             C.cast(arr, C.POINTER(_abi.Weights))), arr


def model_forward(mc: ModelConfig, embed, final_norm, layers, ids, logits=None,
                  saved=None, workspace=None, stream=None, exec=None):
    """q3l_model_forward: logits [B, L, V] of int32 token ids [B, L]."""
    import torch
    cfg = mc.layer
    _need(ids, "ids", numel=cfg.T, dtype=torch.int32)
    if logits is None:
        logits = torch.empty((cfg.B, cfg.L, mc.vocab), dtype=cfg.torch_dtype, device=ids.device)
    _need(logits, "logits", numel=cfg.T * mc.vocab, dtype=cfg.torch_dtype)
    if saved is not None:
        _need(saved, "saved", min_bytes=model_saved_bytes(mc))
    if workspace is None:
        workspace = _bytes(model_workspace_bytes(mc, False), ids.device)
    w, keep = _model_weights(mc, embed, final_norm, layers)
    c = mc.c_struct()
    _check(library().q3l_model_forward(C.byref(c), C.byref(w), _p(ids), _p(logits), _p(saved),
                                       _p(workspace), _nbytes(workspace), _stream(stream),
                                       _exec(exec)))
    del keep
    return logits


def model_backward(mc: ModelConfig, embed, final_norm, layers, ids, dlogits, saved,
                   grads=None, accumulate=False, workspace=None, stream=None):
    """q3l_model_backward: returns grads = {"embed", "final_norm", "layers":
    [per-layer dicts]} (fp32)."""
    import torch
    cfg = mc.layer
    dev = ids.device
    _need(ids, "ids", numel=cfg.T, dtype=torch.int32)
    _need(dlogits, "dlogits", numel=cfg.T * mc.vocab, dtype=cfg.torch_dtype)
    _need(saved, "saved", min_bytes=model_saved_bytes(mc))
    if grads is None:
        grads = {"embed": torch.empty((mc.vocab, cfg.d), dtype=torch.float32, device=dev),
                 "final_norm": torch.empty(cfg.d, dtype=torch.float32, device=dev),
                 "layers": [{n: torch.empty(s, dtype=torch.float32, device=dev)
                             for n, s in param_shapes(cfg).items()}
                            for _ in range(mc.n_layers)]}
    _need(grads["embed"], "grads['embed']", numel=mc.vocab * cfg.d, dtype=torch.float32)
    _need(grads["final_norm"], "grads['final_norm']", numel=cfg.d, dtype=torch.float32)
    garr = (_abi.Grads * max(1, mc.n_layers))(
        *[_abi.Grads(*[g[n].data_ptr() for n in PARAMS]) for g in grads["layers"]])
    for g in grads["layers"]:
        for n, shp in param_shapes(cfg).items():
            _need(g[n], f"grads[layers][{n!r}]", numel=int(__import__("math").prod(shp)),
                  dtype=torch.float32)
    mg = _abi.ModelGrads(grads["embed"].data_ptr(), grads["final_norm"].data_ptr(),
                         C.cast(garr, C.POINTER(_abi.Grads)))
    if workspace is None:
        workspace = _bytes(model_workspace_bytes(mc, True), dev)
    w, keep = _model_weights(mc, embed, final_norm, layers)
    c = mc.c_struct()
    _check(library().q3l_model_backward(C.byref(c), C.byref(w), _p(ids), _p(dlogits), _p(saved),
                                        C.byref(mg), BWD_ACCUMULATE if accumulate else 0,
                                        _p(workspace), _nbytes(workspace), _stream(stream)))
    del keep
    return grads
