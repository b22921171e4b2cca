"""Seeded synthetic workloads for the Qwen3 decoder layer.

This module only *draws numbers*: it holds the five workload presets (their
shapes and value distributions) and the seeded generator that fills x, the
eleven layer parameters and the upstream gradient dy.  It contains none of the
layer's arithmetic.  Both the fp64 oracle (``oracle/``) and the HIP path
(``qwen3_decoder_layer_amd``) consume what it returns; neither imports the
other.

Distributions (the layer's workloads): x ~ N(0, 1); the seven projection
weights ~ N(0, 0.02); the four RMSNorm weights 1 + N(0, 0.1); dy ~ N(0, 1).
Draw order: x, then the parameters in the order of the parameter table of the
"FSDP2 Qwen3 Decoder Layer Walkthrough" page (input_layernorm, q, k, v,
q_norm, k_norm, o, post_attention_layernorm, gate, up, down), then dy.  Values
are drawn in fp64 from ``numpy.random.Generator(PCG64(seed))``, cast to fp32,
and for bf16 workloads rounded to bf16 (round to nearest, ties to even).  The
returned fp32 arrays therefore hold exactly the values the GPU receives.
"""
from __future__ import annotations

import numpy as np

EPS = 1e-6
ROPE_THETA = 1e6

# Parameter names in the walkthrough page's parameter-table order.
PARAM_NAMES = ("in_norm", "q", "k", "v", "q_norm", "k_norm", "o",
               "post_norm", "gate", "up", "down")
NORM_PARAMS = ("in_norm", "q_norm", "k_norm", "post_norm")

# The five workloads.  `fwd_only` workloads are timed/checked forward only.
CONFIGS = {
    0: dict(name="tiny-fp32-fwd", d=512, h_q=8, h_kv=4, d_h=64, d_ffn=1024,
            B=2, L=8, dtype="f32", backward=False, tp_partial=False),
    1: dict(name="tiny-dims-bf16-fwd-L2048", d=512, h_q=8, h_kv=4, d_h=64,
            d_ffn=1024, B=8, L=2048, dtype="bf16", backward=False,
            tp_partial=False),
    2: dict(name="qwen3-8b-bf16-fwd", d=4096, h_q=32, h_kv=8, d_h=128,
            d_ffn=12288, B=4, L=4096, dtype="bf16", backward=False,
            tp_partial=False),
    3: dict(name="llama70b-tp8-share-bf16-fwd", d=8192, h_q=8, h_kv=1,
            d_h=128, d_ffn=3584, B=4, L=4096, dtype="bf16", backward=False,
            tp_partial=True),
    4: dict(name="qwen3-8b-bf16-fwd-bwd", d=4096, h_q=32, h_kv=8, d_h=128,
            d_ffn=12288, B=2, L=4096, dtype="bf16", backward=True,
            tp_partial=False),
}


def make_cfg(d, h_q, h_kv, d_h, d_ffn, B, L, dtype="bf16", tp_partial=False,
             qk_norm=True, eps=EPS, rope_theta=ROPE_THETA, name="custom",
             backward=False):
    """A workload description (plain dict) with the layer's hyper-parameters."""
    return dict(name=name, d=d, h_q=h_q, h_kv=h_kv, d_h=d_h, d_ffn=d_ffn, B=B,
                L=L, dtype=dtype, tp_partial=tp_partial, qk_norm=qk_norm,
                eps=eps, rope_theta=rope_theta, backward=backward)


def preset(idx: int) -> dict:
    c = dict(CONFIGS[idx])
    c.setdefault("qk_norm", True)
    c.setdefault("eps", EPS)
    c.setdefault("rope_theta", ROPE_THETA)
    return c


def param_shapes(cfg: dict) -> dict:
    """Shapes of the eleven parameters ([out, in] for the projections)."""
    d, qd, kvd, dh, f = (cfg["d"], cfg["h_q"] * cfg["d_h"],
                         cfg["h_kv"] * cfg["d_h"], cfg["d_h"], cfg["d_ffn"])
    return {"in_norm": (d,), "q": (qd, d), "k": (kvd, d), "v": (kvd, d),
            "q_norm": (dh,), "k_norm": (dh,), "o": (d, qd),
            "post_norm": (d,), "gate": (f, d), "up": (f, d), "down": (d, f)}


def bf16_round(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bf16 (ties to even); returns fp32."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) \
        & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """The bf16 bit patterns (uint16) of fp32 values already on the bf16 grid."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    return (u >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32)
            << np.uint32(16)).view(np.float32)


def _draw(rng, shape, mean, std, dtype):
    a = rng.standard_normal(size=shape, dtype=np.float64)
    a *= std
    a += mean
    a = a.astype(np.float32)
    return bf16_round(a) if dtype == "bf16" else a


def make_inputs(cfg: dict, seed: int, with_dy: bool | None = None) -> dict:
    """x [B, L, d], the eleven parameters and (optionally) dy [B, L, d].

    All arrays are float32 and hold exactly the values handed to the GPU
    (bf16-representable for bf16 workloads).
    """
    if with_dy is None:
        with_dy = bool(cfg.get("backward", False))
    rng = np.random.Generator(np.random.PCG64(seed))
    dt = cfg["dtype"]
    out = {"x": _draw(rng, (cfg["B"], cfg["L"], cfg["d"]), 0.0, 1.0, dt)}
    for name, shape in param_shapes(cfg).items():
        if name in NORM_PARAMS:
            out[name] = _draw(rng, shape, 1.0, 0.1, dt)
        else:
            out[name] = _draw(rng, shape, 0.0, 0.02, dt)
    if with_dy:
        out["dy"] = _draw(rng, (cfg["B"], cfg["L"], cfg["d"]), 0.0, 1.0, dt)
    return out


def preset_inputs(idx: int) -> tuple[dict, dict]:
    """The preset workload `idx` with its conventional seed 1000 + idx."""
    cfg = preset(idx)
    return cfg, make_inputs(cfg, 1000 + idx)


def make_model_inputs(cfg: dict, n_layers: int, vocab: int, seed: int) -> dict:
    """Inputs of a stack of n_layers layers with the model's ends: token ids
    [B, L] (uniform in [0, vocab), with repeats), the embedding table
    [vocab, d] ~ N(0, 1) (so embedded rows have the layer workload's x
    distribution), the final norm weight 1 + N(0, 0.1), each layer's eleven
    parameters (make_inputs with seeds seed + 1 + i, x and dy unused) and
    dlogits [B, L, vocab] ~ N(0, 1).  Values rounded like make_inputs."""
    rng = np.random.Generator(np.random.PCG64(seed))
    dt = cfg["dtype"]
    out = {"ids": rng.integers(0, vocab, size=(cfg["B"], cfg["L"]), dtype=np.int64).astype(np.int32)}
    out["embed"] = _draw(rng, (vocab, cfg["d"]), 0.0, 1.0, dt)
    out["final_norm"] = _draw(rng, (cfg["d"],), 1.0, 0.1, dt)
    out["dlogits"] = _draw(rng, (cfg["B"], cfg["L"], vocab), 0.0, 1.0, dt)
    out["layers"] = []
    for i in range(n_layers):
        li = make_inputs(cfg, seed + 1 + i)
        out["layers"].append({n: li[n] for n in PARAM_NAMES})
    return out
