"""Python binding of libq3layer.so: one Qwen3 decoder layer (forward and
backward) on an MI355X, computed entirely by the library's HIP kernels.

The functions below have the names of the C ABI in include/q3layer.h minus
the ``q3l_`` prefix.  They only marshal arguments: tensors are torch tensors
on the GPU (PyTorch supplies device memory and the current stream), and any
buffer the caller does not pass is allocated with ``torch.empty``.  If the
library is missing the calls raise; there is no fallback path.
"""
from __future__ import annotations

import ctypes as C
from dataclasses import dataclass, asdict

from . import _abi
from ._abi import BWD_ACCUMULATE, BWD_INPUT, BWD_WEIGHT, PARAMS, Q3L_BF16, Q3L_F32

__all__ = ["LayerConfig", "Q3LError", "validate", "saved_bytes",
           "workspace_bytes", "saved_layout", "layer_forward",
           "layer_backward", "rmsnorm_fwd", "linear_fwd", "linear_dgrad",
           "linear_wgrad", "swiglu_fwd", "attention_fwd", "attention_bwd", "library",
           "PARAMS", "BWD_INPUT", "BWD_WEIGHT", "BWD_ACCUMULATE"]


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


def _weights(w: dict) -> _abi.Weights:
    return _abi.Weights(*[None if w.get(n) is None else w[n].data_ptr()
                          for n in PARAMS])


def _bytes(n, device):
    import torch
    return torch.empty(max(int(n), 1), dtype=torch.uint8, device=device)


def layer_forward(cfg: LayerConfig, weights: dict, x, out: dict | None = None,
                  saved=None, workspace=None, stream=None) -> dict:
    """q3l_layer_forward.  x: [B, L, d] (or [T, d]) tensor of cfg's dtype.

    Returns {"y"} or, for tp_partial, {"attn_partial", "mlp_partial"}
    (fp32).  Pass ``saved`` (uint8, ``saved_bytes(cfg)``) to keep the
    intermediates for ``layer_backward``."""
    import torch
    c = cfg.c_struct()
    lib = library()
    out = dict(out or {})
    shape = (cfg.B, cfg.L, cfg.d)
    if cfg.tp_partial:
        for k in ("attn_partial", "mlp_partial"):
            if out.get(k) is None:
                out[k] = torch.empty(shape, dtype=torch.float32, device=x.device)
        o = _abi.Outputs(None, out["attn_partial"].data_ptr(),
                         out["mlp_partial"].data_ptr())
    else:
        if out.get("y") is None:
            out["y"] = torch.empty(shape, dtype=x.dtype, device=x.device)
        o = _abi.Outputs(out["y"].data_ptr(), None, None)
    ws_n = 0
    if saved is None and workspace is None:
        workspace = _bytes(workspace_bytes(cfg, False), x.device)
    if workspace is not None:
        ws_n = workspace.numel() * workspace.element_size()
    w = _weights(weights)
    _check(lib.q3l_layer_forward(C.byref(c), C.byref(w), _p(x), C.byref(o),
                                 _p(saved), _p(workspace), ws_n,
                                 _stream(stream)))
    return out


def layer_backward(cfg: LayerConfig, weights: dict, x, dy, saved, dx=None,
                   grads: dict | None = None,
                   flags: int = BWD_INPUT | BWD_WEIGHT, workspace=None,
                   stream=None):
    """q3l_layer_backward.  Returns (dx, grads) with grads a dict of fp32
    tensors shaped like the parameters."""
    import torch
    c = cfg.c_struct()
    lib = library()
    if (flags & BWD_INPUT) and dx is None:
        dx = torch.empty_like(x)
    if flags & BWD_WEIGHT:
        grads = dict(grads or {})
        for n in PARAMS:
            if grads.get(n) is None:
                grads[n] = torch.empty(weights[n].shape, dtype=torch.float32,
                                       device=x.device)
    g = _abi.Grads(*[None if not grads or grads.get(n) is None
                     else grads[n].data_ptr() for n in PARAMS])
    if workspace is None:
        workspace = _bytes(workspace_bytes(cfg, True), x.device)
    ws_n = workspace.numel() * workspace.element_size()
    w = _weights(weights)
    _check(lib.q3l_layer_backward(C.byref(c), C.byref(w), _p(x), _p(dy),
                                  _p(saved), _p(dx), C.byref(g), flags,
                                  _p(workspace), ws_n, _stream(stream)))
    return dx, grads


# ---- phase-level calls --------------------------------------------------
def rmsnorm_fwd(x, w, eps, y=None, rstd=None, stream=None):
    import torch
    rows = x.numel() // x.shape[-1]
    y = torch.empty_like(x) if y is None else y
    rstd = (torch.empty(rows, dtype=torch.float32, device=x.device)
            if rstd is None else rstd)
    _check(library().q3l_rmsnorm_fwd(_code(x.dtype), rows, x.shape[-1], _p(x),
                                     _p(w), eps, _p(y), _p(rstd),
                                     _stream(stream)))
    return y, rstd


def linear_fwd(a, w, resid=None, y=None, stream=None):
    import torch
    M, K = a.numel() // a.shape[-1], a.shape[-1]
    N = w.shape[0]
    y = torch.empty((*a.shape[:-1], N), dtype=a.dtype, device=a.device) \
        if y is None else y
    _check(library().q3l_linear_fwd(_code(a.dtype), M, N, K, _p(a), _p(w),
                                    _p(resid), _p(y), _stream(stream)))
    return y


def linear_dgrad(dy, w, da=None, stream=None):
    import torch
    M, N = dy.numel() // dy.shape[-1], dy.shape[-1]
    K = w.shape[1]
    da = torch.empty((*dy.shape[:-1], K), dtype=dy.dtype, device=dy.device) \
        if da is None else da
    _check(library().q3l_linear_dgrad(_code(dy.dtype), M, N, K, _p(dy), _p(w),
                                      _p(da), _stream(stream)))
    return da


def linear_wgrad(dy, a, dw=None, accumulate=False, stream=None):
    import torch
    M, N, K = dy.numel() // dy.shape[-1], dy.shape[-1], a.shape[-1]
    dw = torch.empty((N, K), dtype=torch.float32, device=dy.device) \
        if dw is None else dw
    _check(library().q3l_linear_wgrad(_code(dy.dtype), M, N, K, _p(dy), _p(a),
                                      _p(dw), int(bool(accumulate)),
                                      _stream(stream)))
    return dw


def swiglu_fwd(hn, gate, up, f=None, gu=None, stream=None):
    """f = silu(hn gate^T) * (hn up^T) with the layer's fused kernel; gu
    (optional [M, 2N]) receives gate | up pre-activations."""
    import torch
    M, K, N = hn.numel() // hn.shape[-1], hn.shape[-1], gate.shape[0]
    f = torch.empty((*hn.shape[:-1], N), dtype=hn.dtype, device=hn.device) \
        if f is None else f
    _check(library().q3l_swiglu_fwd(_code(hn.dtype), M, N, K, _p(hn),
                                    _p(gate), _p(up), _p(f), _p(gu),
                                    _stream(stream)))
    return f


def attention_fwd(q, k, v, h_q, h_kv, d_h, o=None, lse=None, stream=None):
    """q [B, L, >=h_q*d_h], k/v [B, L, >=h_kv*d_h] (row strides taken from
    the tensors; the last dim must be contiguous)."""
    import torch
    B, L = q.shape[0], q.shape[1]
    o = torch.empty((B, L, h_q * d_h), dtype=q.dtype, device=q.device) \
        if o is None else o
    lse = torch.empty((B, h_q, L), dtype=torch.float32, device=q.device) \
        if lse is None else lse
    _check(library().q3l_attention_fwd(
        _code(q.dtype), B, L, h_q, h_kv, d_h, _p(q), q.stride(1), _p(k),
        k.stride(1), _p(v), v.stride(1), _p(o), o.stride(1), _p(lse),
        _stream(stream)))
    return o, lse


def attention_bwd(q, k, v, o, dout, lse, h_q, h_kv, d_h, dq=None, dk=None,
                  dv=None, stream=None):
    import torch
    B, L = q.shape[0], q.shape[1]
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    lib = library()
    n = lib.q3l_attention_bwd_workspace_bytes(B, L, h_q)
    ws = _bytes(n, q.device)
    _check(lib.q3l_attention_bwd(
        _code(q.dtype), B, L, h_q, h_kv, d_h, _p(q), q.stride(1), _p(k),
        k.stride(1), _p(v), v.stride(1), _p(o), _p(dout), dout.stride(1),
        _p(lse), _p(dq), _p(dk), _p(dv), _p(ws), n, _stream(stream)))
    return dq, dk, dv
