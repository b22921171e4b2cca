"""fp64 evaluation of a stack of Qwen3 decoder layers with the model's two
ends, forward and backward.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The walkthrough page's "简化的 Qwen3 结构" listing gives the whole model: a
token embedding table [vocab, d], N_L decoder layers, a final RMSNorm, and an
output projection that shares the embedding's weights (tied).  Hidden
states flow from one layer into the next (the text after Steps 10-11).  The
pages stop at the logits; the loss is not part of the path, so the backward
starts from a given upstream gradient dlogits, as the layer's starts from
dy.  With tied weights the embedding table's gradient is the sum of the
output projection's weight gradient and the scattered gradients of the
embedded rows (a token that occurs several times adds all its rows).
"""
from __future__ import annotations

import numpy as np

from .layer import layer_backward, layer_forward, linear, linear_backward, rmsnorm, rmsnorm_backward


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def model_forward(cfg, n_layers, embed, final_norm, layers, ids, keep=False):
    """logits [B, L, V] of token ids [B, L] (ints in [0, V)).

    layers: a list of n_layers parameter dicts (the eleven layer tensors).
    x_0 = embed[ids]; x_{i+1} = layer_i(x_i); hf = RMSNorm(x_N; final_norm);
    logits = hf embed^T.  With keep=True also returns the layer inputs
    ("xs", x_0 .. x_N) and the final norm's hf and rstd ("hf", "rf")."""
    E = _f64(embed)
    x = E[np.asarray(ids)]
    xs = [x]
    for i in range(n_layers):
        x = layer_forward(cfg, layers[i], x)["y"]
        xs.append(x)
    hf, rf = rmsnorm(x, _f64(final_norm), cfg["eps"])
    logits = linear(hf, E)
    if keep:
        return {"logits": logits, "xs": xs, "hf": hf, "rf": rf}
    return {"logits": logits}


def model_backward(cfg, n_layers, embed, final_norm, layers, ids, dlogits):
    """Gradients of sum(logits * dlogits) w.r.t. the embedding table (tied:
    both of its uses), the final norm weight and every layer's eleven
    parameters.  Returns (d_embed [V, d], d_final_norm [d], [layer grads])."""
    c = model_forward(cfg, n_layers, embed, final_norm, layers, ids, keep=True)
    E = _f64(embed)
    dlogits = _f64(dlogits)
    # Output projection (tied): logits = hf E^T.
    dhf, dE = linear_backward(dlogits, c["hf"], E)
    # Final RMSNorm.
    dx, d_final = rmsnorm_backward(dhf, c["xs"][-1], c["rf"], _f64(final_norm))
    # Layers, last first.
    grads = [None] * n_layers
    for i in reversed(range(n_layers)):
        dx, grads[i] = layer_backward(cfg, layers[i], c["xs"][i], dx)
    # Embedding gather: scatter-add every token's row gradient.
    ids = np.asarray(ids).reshape(-1)
    rows = dx.reshape(-1, dx.shape[-1])
    for t, v in enumerate(ids):
        dE[v] += rows[t]
    return dE, d_final, grads


def model_param_counts(d, h_q, h_kv, d_h, d_ffn, n_layers, vocab, qk_norm=True):
    """Element counts of the stack's tensors: the tied embedding [vocab, d],
    n_layers times the eleven layer tensors, and the final norm [d]."""
    from .accounting import param_total
    layer = param_total(d, h_q, h_kv, d_h, d_ffn, qk_norm)
    return {"embedding": vocab * d, "layers": n_layers * layer, "final_norm": d,
            "total": vocab * d + n_layers * layer + d}
