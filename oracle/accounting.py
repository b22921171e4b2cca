"""Parameter accounting for one decoder layer.

TEST INFRASTRUCTURE ONLY (see the package docstring).

* ``param_counts`` follows the walkthrough page's single-layer parameter
  table: eleven tensors, projections stored [out, in].
* ``megatron_layer_params`` is the Megatron memory-model page's parameter
  estimate (section 2.2): per layer 2*h*q*(1 + g/a) + 3*h*ffn + 2*h for GQA
  attention, SwiGLU and two RMSNorms, with q = a*d.  Qwen3's per-head
  q_norm/k_norm add 2*d, which that formula does not contain.
"""
from __future__ import annotations


def param_counts(d, h_q, h_kv, d_h, d_ffn, qk_norm=True):
    """Element count of each of the layer's parameters, by name."""
    qd, kvd = h_q * d_h, h_kv * d_h
    c = {"in_norm": d, "q": qd * d, "k": kvd * d, "v": kvd * d,
         "q_norm": d_h if qk_norm else 0, "k_norm": d_h if qk_norm else 0,
         "o": d * qd, "post_norm": d, "gate": d_ffn * d, "up": d_ffn * d,
         "down": d * d_ffn}
    return c


def param_total(d, h_q, h_kv, d_h, d_ffn, qk_norm=True):
    return sum(param_counts(d, h_q, h_kv, d_h, d_ffn, qk_norm).values())


def megatron_layer_params(h, a, g, d, ffn, qk_norm=False):
    """Per-layer terms of the memory-model page's estimate, as integers.

    attention = 2*h*q*(1 + g/a) with q = a*d, i.e. 2*h*q + 2*h*g*d exactly;
    mlp = 3*h*ffn; norms = 2*h (+ 2*d with Qwen3's q/k norms).
    """
    q = a * d
    attention = 2 * h * q + 2 * h * g * d
    mlp = 3 * h * ffn
    norms = 2 * h + (2 * d if qk_norm else 0)
    return {"attention": attention, "mlp": mlp, "norms": norms,
            "layer": attention + mlp + norms}


def megatron_model_params(h, a, g, d, ffn, n_layers, vocab, qk_norm=False):
    """Whole-model estimate: n_layers layers + final norm + tied embedding."""
    per = megatron_layer_params(h, a, g, d, ffn, qk_norm)["layer"]
    block = n_layers * per + h
    emb = vocab * h
    return {"block": block, "embedding": emb, "total": block + emb}
