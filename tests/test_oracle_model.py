"""Pins of the oracle's model stack (embedding, N_L layers, final RMSNorm,
tied output projection; walkthrough page, "简化的 Qwen3 结构"): the
memory-model page's parameter total, central finite differences through
every use of the tied embedding, the reduction to the model's ends when the
layers are identities, and batch independence."""
import json
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_stack_parameter_total_matches_the_memory_model_page():
    # The page's 7B example: 32 layers of h=4096, 32/8 heads of 128, ffn
    # 14336, vocab 128256, tied embedding, no q/k norms: 7,504,924,672.
    fx = json.load(open(os.path.join(GOLDEN, "megatron_7b_param_count.json")))
    i = fx["inputs"]
    c = oracle.model_param_counts(i["h"], i["a"], i["g"], i["d"], i["ffn"], i["n_layers"],
                                  i["vocab"], qk_norm=False)
    assert c["total"] == fx["total"] == 7_504_924_672
    assert c["embedding"] == fx["embedding_tied"]
    assert c["layers"] + c["final_norm"] == fx["block_with_final_ln"]


def _tiny(n_layers, seed, V=11):
    cfg = synth.make_cfg(d=16, h_q=2, h_kv=1, d_h=8, d_ffn=24, B=2, L=5, dtype="f32")
    rng = np.random.default_rng(seed)
    layers = []
    for i in range(n_layers):
        inp = synth.make_inputs(cfg, seed + 10 * i)
        layers.append({n: inp[n].astype(np.float64) for n in synth.PARAM_NAMES})
    E = rng.standard_normal((V, cfg["d"]))
    w = 1.0 + 0.1 * rng.standard_normal(cfg["d"])
    ids = np.array([[3, 7, 3, 0, 10], [7, 7, 1, 2, 3]])     # repeats on purpose
    dlog = rng.standard_normal((cfg["B"], cfg["L"], V))
    return cfg, layers, E, w, ids, dlog


def _loss(cfg, n, E, w, layers, ids, dlog):
    return float(np.sum(oracle.model_forward(cfg, n, E, w, layers, ids)["logits"] * dlog))


def test_model_backward_matches_central_differences():
    n = 2
    cfg, layers, E, w, ids, dlog = _tiny(n, 5)
    dE, dw, grads = oracle.model_backward(cfg, n, E, w, layers, ids, dlog)
    rng = np.random.default_rng(9)
    h = 1e-6

    def fd(perturb):
        return (perturb(h) - perturb(-h)) / (2 * h)

    # Tied embedding: both the gathered rows (with repeats) and the output
    # projection move.
    D = rng.standard_normal(E.shape)
    num = fd(lambda e: _loss(cfg, n, E + e * D, w, layers, ids, dlog))
    assert abs(num - np.sum(dE * D)) <= 1e-6 * max(1.0, abs(num))
    # A row of E no token uses still gets the output-projection part.
    assert not np.isin(4, ids) and np.abs(dE[4]).max() > 0
    Dw = rng.standard_normal(w.shape)
    num = fd(lambda e: _loss(cfg, n, E, w + e * Dw, layers, ids, dlog))
    assert abs(num - np.sum(dw * Dw)) <= 1e-6 * max(1.0, abs(num))
    for i, name in ((0, "q"), (1, "down"), (0, "k_norm"), (1, "in_norm")):
        Dl = rng.standard_normal(layers[i][name].shape)

        def pert(e, i=i, name=name, Dl=Dl):
            ls = [dict(l) for l in layers]
            ls[i][name] = ls[i][name] + e * Dl
            return _loss(cfg, n, E, w, ls, ids, dlog)
        num = fd(pert)
        assert abs(num - np.sum(grads[i][name] * Dl)) <= 1e-6 * max(1.0, abs(num)), (i, name)


def test_identity_layers_reduce_the_stack_to_its_ends():
    # W_o = W_down = 0 makes each layer the identity (y = x): the stack's
    # logits are those of the model without layers, RMSNorm(E[ids]) E^T.
    cfg, layers, E, w, ids, dlog = _tiny(3, 8)
    for l in layers:
        l["o"] = np.zeros_like(l["o"])
        l["down"] = np.zeros_like(l["down"])
    y3 = oracle.model_forward(cfg, 3, E, w, layers, ids)["logits"]
    y0 = oracle.model_forward(cfg, 0, E, w, [], ids)["logits"]
    assert np.allclose(y3, y0, rtol=0, atol=1e-13)
    xn, _ = oracle.rmsnorm(E[ids], w, cfg["eps"])
    assert np.allclose(y0, xn @ E.T, rtol=0, atol=1e-13)
    dE3, dw3, _ = oracle.model_backward(cfg, 3, E, w, layers, ids, dlog)
    dE0, dw0, _ = oracle.model_backward(cfg, 0, E, w, [], ids, dlog)
    assert np.allclose(dE3, dE0, atol=1e-12) and np.allclose(dw3, dw0, atol=1e-12)


def test_stack_batch_independence():
    cfg, layers, E, w, ids, dlog = _tiny(2, 3)
    y = oracle.model_forward(cfg, 2, E, w, layers, ids)["logits"]
    c1 = dict(cfg, B=1)
    for b in range(2):
        yb = oracle.model_forward(c1, 2, E, w, layers, ids[b:b + 1])["logits"]
        assert np.allclose(yb[0], y[b], rtol=0, atol=1e-12)


# ---- planted mistakes (on the CPU): the finite-difference pin catches each --
import oracle.model as OM  # noqa: E402


def _bwd_without_head_part(cfg, n, E, w, layers, ids, dlog):
    dE, dw, g = OM.__dict__["_orig_model_backward"](cfg, n, E, w, layers, ids, dlog)
    c = oracle.model_forward(cfg, n, E, w, layers, ids, keep=True)
    _, dE_head = oracle.linear_backward(np.asarray(dlog, float), c["hf"], np.asarray(E, float))
    return dE - dE_head, dw, g


def _bwd_scatter_drops_repeats(cfg, n, E, w, layers, ids, dlog):
    # the classic fancy-index update, which keeps one row per repeated token
    c = oracle.model_forward(cfg, n, E, w, layers, ids, keep=True)
    Ef = np.asarray(E, float)
    dhf, dE = oracle.linear_backward(np.asarray(dlog, float), c["hf"], Ef)
    dx, dw = oracle.rmsnorm_backward(dhf, c["xs"][-1], c["rf"], np.asarray(w, float))
    g = [None] * n
    for i in reversed(range(n)):
        dx, g[i] = oracle.layer_backward(cfg, layers[i], c["xs"][i], dx)
    flat = np.asarray(ids).reshape(-1)
    dE[flat] += dx.reshape(-1, dx.shape[-1])
    return dE, dw, g


@pytest.mark.parametrize("bad", [_bwd_without_head_part, _bwd_scatter_drops_repeats])
def test_planted_model_mistake_is_caught(monkeypatch, bad):
    monkeypatch.setitem(OM.__dict__, "_orig_model_backward", OM.model_backward)
    monkeypatch.setattr(oracle, "model_backward", bad)
    with pytest.raises(AssertionError):
        test_model_backward_matches_central_differences()
