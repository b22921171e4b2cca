"""The model around a stack of layers (q3l_model_forward / q3l_model_backward:
embedding gather, N_L layers, final RMSNorm, tied output projection) through
the C ABI against the oracle's model_forward / model_backward, on poisoned
guarded buffers; the full-recompute mode against the stored one."""
import numpy as np
import pytest

import oracle
import qwen3_decoder_layer_amd as q3
from gpu_helpers import TOL, Guarded, check, dev, guarded_bytes, host, need_gpu, say
import synth

pytestmark = pytest.mark.gpu


def _gpu_model(mc, inp):
    import torch
    dt = mc.layer.dtype
    E = dev(inp["embed"], dt)
    wf = dev(inp["final_norm"], dt)
    layers = [{n: dev(l[n], dt) for n in synth.PARAM_NAMES} for l in inp["layers"]]
    ids = torch.from_numpy(inp["ids"]).to("cuda")
    return E, wf, layers, ids


def _run(mc, inp):
    """Forward (training) + backward on guarded, poisoned buffers."""
    import torch
    cfg = mc.layer
    E, wf, layers, ids = _gpu_model(mc, inp)
    logits = Guarded((cfg.B, cfg.L, mc.vocab), cfg.torch_dtype)
    saved = guarded_bytes(q3.model_saved_bytes(mc))
    fws = guarded_bytes(q3.model_workspace_bytes(mc, False))
    q3.model_forward(mc, E, wf, layers, ids, logits=logits.t, saved=saved.t, workspace=fws.t)
    torch.cuda.synchronize()
    logits.check("logits")
    assert saved.guards_intact() and fws.guards_intact()
    gE = Guarded((mc.vocab, cfg.d), torch.float32)
    gf = Guarded((cfg.d,), torch.float32)
    gl = [{n: Guarded(s, torch.float32) for n, s in q3.param_shapes(cfg).items()}
          for _ in range(mc.n_layers)]
    bws = guarded_bytes(q3.model_workspace_bytes(mc, True))
    q3.model_backward(mc, E, wf, layers, ids, dev(inp["dlogits"], cfg.dtype), saved.t,
                      grads={"embed": gE.t, "final_norm": gf.t,
                             "layers": [{n: g.t for n, g in l.items()} for l in gl]},
                      workspace=bws.t)
    torch.cuda.synchronize()
    assert bws.guards_intact()
    gE.check("d_embed"), gf.check("d_final_norm")
    res = {"logits": host(logits.t), "d_embed": host(gE.t), "d_final_norm": host(gf.t)}
    for i, l in enumerate(gl):
        for n, g in l.items():
            g.check(f"layer{i}.d_{n}")
            res[f"layer{i}.d_{n}"] = host(g.t)
    return res


def _oracle(mc, cfg_d, inp):
    p = [{n: l[n] for n in synth.PARAM_NAMES} for l in inp["layers"]]
    y = oracle.model_forward(cfg_d, mc.n_layers, inp["embed"], inp["final_norm"], p,
                             inp["ids"])["logits"]
    dE, dw, grads = oracle.model_backward(cfg_d, mc.n_layers, inp["embed"], inp["final_norm"],
                                          p, inp["ids"], inp["dlogits"])
    ref = {"logits": y, "d_embed": dE, "d_final_norm": dw}
    for i, g in enumerate(grads):
        for n in synth.PARAM_NAMES:
            ref[f"layer{i}.d_{n}"] = g[n]
    return ref


STACKS = [
    # layer shape, n_layers, vocab
    (dict(d=256, h_q=4, h_kv=2, d_h=64, d_ffn=256, B=2, L=37, dtype="f32"), 2, 120),
    (dict(d=256, h_q=4, h_kv=2, d_h=64, d_ffn=512, B=2, L=100, dtype="bf16"), 3, 520),
    (dict(d=512, h_q=8, h_kv=2, d_h=128, d_ffn=1024, B=1, L=130, dtype="bf16"), 2, 1000),
    (dict(d=256, h_q=4, h_kv=2, d_h=64, d_ffn=256, B=1, L=20, dtype="bf16"), 0, 64),
]


@pytest.mark.parametrize("shape,n_layers,vocab", STACKS,
                         ids=lambda v: "-".join(f"{k}{x}" for k, x in v.items())
                         if isinstance(v, dict) else str(v))
def test_model_stack_against_oracle(shape, n_layers, vocab):
    need_gpu()
    say(f"model stack {shape} n_layers={n_layers} vocab={vocab}")
    cfg_d = synth.make_cfg(**shape)
    mc = q3.ModelConfig(q3.LayerConfig.from_dict(cfg_d), n_layers, vocab)
    inp = synth.make_model_inputs(cfg_d, n_layers, vocab, 2024 + n_layers)
    res = _run(mc, inp)
    ref = _oracle(mc, cfg_d, inp)
    tol = TOL[cfg_d["dtype"]]
    errs = {}
    ok = all([check(k, res[k], ref[k], tol, errs=errs) for k in ref])
    print({k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    assert ok, {k: v for k, v in errs.items() if not v <= tol}


def test_recompute_mode_is_bitwise_the_stored_one():
    """Keeping only the layer inputs and recomputing each layer's forward in
    the backward gives bitwise the gradients of the stored-activation run,
    from a saved block a fraction of the size."""
    need_gpu()
    say("model stack recompute vs stored")
    cfg_d = synth.make_cfg(d=256, h_q=4, h_kv=2, d_h=64, d_ffn=512, B=2, L=100, dtype="bf16")
    inp = synth.make_model_inputs(cfg_d, 3, 520, 7)
    lc = q3.LayerConfig.from_dict(cfg_d)
    stored = _run(q3.ModelConfig(lc, 3, 520, recompute=False), inp)
    mc_r = q3.ModelConfig(lc, 3, 520, recompute=True)
    rec = _run(mc_r, inp)
    for k in stored:
        assert np.array_equal(stored[k], rec[k]), k
    assert q3.model_saved_bytes(mc_r) * 3 < q3.model_saved_bytes(q3.ModelConfig(lc, 3, 520))


def test_model_backward_is_deterministic_and_accumulates():
    need_gpu()
    import torch
    say("model stack determinism")
    cfg_d = synth.make_cfg(d=256, h_q=4, h_kv=2, d_h=64, d_ffn=256, B=2, L=64, dtype="bf16")
    mc = q3.ModelConfig(q3.LayerConfig.from_dict(cfg_d), 2, 64)   # small vocab: many repeats
    inp = synth.make_model_inputs(cfg_d, 2, 64, 11)
    E, wf, layers, ids = _gpu_model(mc, inp)
    saved = torch.empty(q3.model_saved_bytes(mc), dtype=torch.uint8, device="cuda")
    q3.model_forward(mc, E, wf, layers, ids, saved=saved)
    dl = dev(inp["dlogits"], "bf16")
    g1 = q3.model_backward(mc, E, wf, layers, ids, dl, saved)
    e1 = g1["embed"].clone()
    g2 = q3.model_backward(mc, E, wf, layers, ids, dl, saved)
    assert torch.equal(g2["embed"], e1)
    q3.model_backward(mc, E, wf, layers, ids, dl, saved, grads=g2, accumulate=True)
    assert torch.allclose(g2["embed"], 2 * e1, rtol=1e-6, atol=1e-6)
