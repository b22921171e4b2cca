"""ctypes mirror of include/q3layer.h (argument marshalling only).

Every struct and prototype here restates a declaration of the header; the
library itself is libq3layer.so built next to this file.
"""
from __future__ import annotations

import ctypes as C
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)),
                        "libq3layer.so")

Q3L_F32, Q3L_BF16 = 0, 1
STATUS = {0: "Q3L_OK", 1: "Q3L_EINVAL", 2: "Q3L_EUNSUPPORTED",
          3: "Q3L_EALIGN", 4: "Q3L_EHIP"}
BWD_INPUT, BWD_WEIGHT, BWD_ACCUMULATE, BWD_DEFERRED_WEIGHT = 1, 2, 4, 8

PARAMS = ("in_norm", "q", "k", "v", "q_norm", "k_norm", "o", "post_norm",
          "gate", "up", "down")


class Cfg(C.Structure):
    _fields_ = [("d", C.c_int32), ("h_q", C.c_int32), ("h_kv", C.c_int32),
                ("d_h", C.c_int32), ("d_ffn", C.c_int32), ("B", C.c_int32),
                ("L", C.c_int32), ("eps", C.c_float),
                ("rope_theta", C.c_float), ("qk_norm", C.c_int32),
                ("tp_partial", C.c_int32), ("dtype", C.c_int32)]


class Weights(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in PARAMS]


class Grads(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in PARAMS]


class Outputs(C.Structure):
    _fields_ = [("y", C.c_void_p), ("attn_partial", C.c_void_p),
                ("mlp_partial", C.c_void_p)]


SAVED_FIELDS = ("rstd1", "xn", "qkv", "qk_rope", "rstd_q", "rstd_k",
                "rope_cos", "rope_sin", "attn_o", "lse", "h", "rstd2", "hn",
                "gu", "f", "wt", "xnt", "total")


class SavedLayout(C.Structure):
    _fields_ = [(n, C.c_size_t) for n in SAVED_FIELDS]


class ModelCfg(C.Structure):
    _fields_ = [("layer", Cfg), ("n_layers", C.c_int32), ("vocab", C.c_int32),
                ("recompute", C.c_int32)]


class ModelWeights(C.Structure):
    _fields_ = [("embed", C.c_void_p), ("final_norm", C.c_void_p),
                ("layers", C.POINTER(Weights))]


class ModelGrads(C.Structure):
    _fields_ = [("embed", C.c_void_p), ("final_norm", C.c_void_p),
                ("layers", C.POINTER(Grads))]


class Exec(C.Structure):
    _fields_ = [("side_stream", C.c_void_p), ("fork_event", C.c_void_p),
                ("join_event", C.c_void_p), ("marks", C.POINTER(C.c_void_p)),
                ("n_marks", C.c_int32)]


# name -> (restype, argtypes)
_vp, _i32, _i64, _sz, _f = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t, C.c_float
PROTOTYPES = {
    "q3l_validate": (C.c_int, [C.POINTER(Cfg)]),
    "q3l_saved_layout_of": (C.c_int, [C.POINTER(Cfg), C.POINTER(SavedLayout)]),
    "q3l_saved_bytes": (_sz, [C.POINTER(Cfg)]),
    "q3l_workspace_bytes": (_sz, [C.POINTER(Cfg), C.c_int]),
    "q3l_layer_forward": (C.c_int, [C.POINTER(Cfg), C.POINTER(Weights), _vp,
                                    C.POINTER(Outputs), _vp, _vp, _sz, _vp,
                                    C.POINTER(Exec)]),
    "q3l_layer_backward": (C.c_int, [C.POINTER(Cfg), C.POINTER(Weights), _vp,
                                     _vp, _vp, _vp, C.POINTER(Grads), C.c_int,
                                     _vp, _sz, _vp, C.POINTER(Exec)]),
    "q3l_phase_count": (C.c_int, [C.c_int]),
    "q3l_phase_name": (C.c_char_p, [C.c_int, C.c_int]),
    "q3l_model_validate": (C.c_int, [C.POINTER(ModelCfg)]),
    "q3l_model_saved_bytes": (_sz, [C.POINTER(ModelCfg)]),
    "q3l_model_workspace_bytes": (_sz, [C.POINTER(ModelCfg), C.c_int]),
    "q3l_model_forward": (C.c_int, [C.POINTER(ModelCfg), C.POINTER(ModelWeights),
                                    _vp, _vp, _vp, _vp, _sz, _vp, C.POINTER(Exec)]),
    "q3l_model_backward": (C.c_int, [C.POINTER(ModelCfg), C.POINTER(ModelWeights),
                                     _vp, _vp, _vp, C.POINTER(ModelGrads), C.c_int,
                                     _vp, _sz, _vp]),
    "q3l_last_error": (C.c_char_p, []),
    "q3l_version": (C.c_int, []),
    "q3l_rmsnorm_fwd": (C.c_int, [_i32, _i64, _i32, _vp, _vp, _f, _vp, _vp,
                                  _vp]),
    "q3l_rmsnorm_bwd_workspace_bytes": (_sz, [_i32]),
    "q3l_rmsnorm_bwd": (C.c_int, [_i32, _i64, _i32, _vp, _vp, _vp, _vp, _vp,
                                  _vp, _vp, C.c_int, _vp, _sz, _vp]),
    "q3l_rope_table": (C.c_int, [_i32, _i32, _f, _vp, _vp, _vp]),
    "q3l_qknorm_rope_fwd": (C.c_int, [_i32, _i32, _i32, _i32, _i32, _i32,
                                      _i32, _f, _vp, _i64, _vp, _vp, _vp, _vp,
                                      _vp, _i64, _vp, _vp, _vp]),
    "q3l_qknorm_rope_bwd_workspace_bytes": (_sz, [_i32]),
    "q3l_qknorm_rope_bwd": (C.c_int, [_i32, _i32, _i32, _i32, _i32, _i32,
                                      _i32, _vp, _i64, _vp, _i64, _vp, _vp,
                                      _vp, _vp, _vp, _vp, _vp, _i64, _vp, _vp,
                                      C.c_int, _vp, _sz, _vp]),
    "q3l_swiglu_bwd": (C.c_int, [_i32, _i64, _i32, _vp, _vp, _vp, _vp]),
    "q3l_linear_fwd": (C.c_int, [_i32, _i64, _i32, _i32, _vp, _vp, _vp, _vp,
                                 _vp]),
    "q3l_linear_dgrad": (C.c_int, [_i32, _i64, _i32, _i32, _vp, _vp, _vp,
                                   _vp]),
    "q3l_linear_wgrad": (C.c_int, [_i32, _i64, _i32, _i32, _vp, _vp, _vp,
                                   C.c_int, _vp]),
    "q3l_swiglu_fwd": (C.c_int, [_i32, _i64, _i32, _i32, _vp, _vp, _vp, _vp,
                                 _vp, _vp]),
    "q3l_attention_fwd": (C.c_int, [_i32, _i32, _i32, _i32, _i32, _i32, _vp,
                                    _i64, _vp, _i64, _vp, _i64, _vp, _i64,
                                    _vp, _vp]),
    "q3l_attention_bwd_workspace_bytes": (_sz, [_i32, _i32, _i32]),
    "q3l_attention_bwd_stored_ds_workspace_bytes": (_sz, [_i32, _i32, _i32]),
    "q3l_attention_fwd_block": (C.c_int, [_i32, _i32, _i32, _i32, _i32, _i32,
                                          _vp, _i64, _vp, _i64, _vp, _i64, _i32,
                                          _i32, _vp, _vp, _vp, _vp]),
    "q3l_attention_merge": (C.c_int, [_i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp,
                                      _vp, _vp, _vp]),
    "q3l_attention_finish": (C.c_int, [_i32, _i32, _i32, _i32, _i32, _vp, _vp,
                                       _vp, _vp, _i64, _vp, _vp]),
    "q3l_attention_bwd_noalloc_max_rows": (_sz, []),
    "q3l_attention_bwd_noalloc": (C.c_int, [_i32, _i32, _i32, _i32, _i32, _i32,
                                            _vp, _i64, _vp, _i64, _vp, _i64, _vp,
                                            _i64, _vp, _i64, _vp, _vp, _vp, _vp,
                                            _vp]),
    "q3l_attention_bwd": (C.c_int, [_i32, _i32, _i32, _i32, _i32, _i32, _vp,
                                    _i64, _vp, _i64, _vp, _i64, _vp, _i64,
                                    _vp, _i64, _vp, _vp, _vp, _vp, _vp, _sz,
                                    _vp]),
}

_lib = None


def load(path: str = LIB_PATH):
    """Load libq3layer.so and declare every prototype.  Raises if absent:
    there is no fallback implementation."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with "
            "`python -m qwen3_decoder_layer_amd.build` (hipcc, gfx950)")
    lib = C.CDLL(path)
    for name, (res, args) in PROTOTYPES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib
