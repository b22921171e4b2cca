"""fp64 CPU oracle for the local compute of one Qwen3 decoder layer.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
link this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
path (``qwen3_decoder_layer_amd``); the only module both sides read is the
seeded input generator ``synth``.

It is a plain, slow, obviously-correct evaluation of the definitions on the
"FSDP2 Qwen3 Decoder Layer Walkthrough" page (Steps 1-10 of its forward
walkthrough and the "reverse order, local" backward), in numpy float64, with
no blocking, fusion or reordering beyond what those definitions state.

Pins (tests marked ``not gpu`` under ``tests/``) tie it to values the pages
print and to mathematical facts: the walkthrough page's parameter table, the
Megatron memory-model page's parameter-count worked example, the
state-placement page's online-softmax and tensor-parallel worked examples,
closed forms, brute force on tiny inputs, causality, GQA->MHA reduction, RoPE
norm preservation and central finite differences of the backward.

Parity unpinned: the RoPE *pairing and frequency layout* (rotate-half pairs
(i, i + d_h/2), angle t * theta^(-2i/d_h)).  The walkthrough page only says
that q and k are rotated along head_dim and defers the details to a page that
is not available; the reading taken is the rotate-half convention its call
name ``apply_rotary_pos_emb`` denotes.  Norm preservation, identity at
position 0 and the relative-position property are pinned; the pairing itself
is not.
"""
from .layer import (rmsnorm, rmsnorm_backward, linear, linear_backward,
                    rope_cos_sin, rope, rope_backward, softmax_attend,
                    causal_attention, attention, attention_backward, silu,
                    swiglu, swiglu_backward, layer_forward, layer_backward,
                    layer_forward_rows)
from .accounting import (param_counts, param_total, megatron_layer_params,
                         megatron_model_params)
from .model import model_forward, model_backward, model_param_counts
from .online_softmax import (block_state, merge_states, finish_state,
                             attention_block_state, merge_block_states)

__all__ = [
    "rmsnorm", "rmsnorm_backward", "linear", "linear_backward",
    "rope_cos_sin", "rope", "rope_backward", "softmax_attend",
    "causal_attention", "attention", "attention_backward", "silu", "swiglu",
    "swiglu_backward", "layer_forward", "layer_backward",
    "layer_forward_rows", "param_counts", "param_total",
    "megatron_layer_params", "megatron_model_params", "block_state",
    "merge_states", "finish_state", "attention_block_state",
    "merge_block_states", "model_forward", "model_backward",
    "model_param_counts",
]
