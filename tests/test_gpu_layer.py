"""Whole-layer parity of the HIP path (q3l_layer_forward / q3l_layer_backward
through the C ABI) against the fp64 oracle on the same seeded inputs."""
import os

import numpy as np
import pytest

import oracle
import qwen3_decoder_layer_amd as q3
from gpu_helpers import TOL, dev, gpu_weights, host, need_gpu, rel_err, say
import synth

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def run_layer(cfg_d, inp, backward=False, flags=None):
    import torch
    cfg = q3.LayerConfig.from_dict(cfg_d)
    W = gpu_weights(inp, cfg.dtype)
    x = dev(inp["x"], cfg.dtype)
    saved = (torch.empty(q3.saved_bytes(cfg), dtype=torch.uint8, device="cuda")
             if backward else None)
    out = q3.layer_forward(cfg, W, x, saved=saved)
    res = {k: host(v) for k, v in out.items()}
    if backward:
        dy = dev(inp["dy"], cfg.dtype)
        dx, grads = q3.layer_backward(cfg, W, x, dy, saved,
                                      flags=flags or (q3.BWD_INPUT | q3.BWD_WEIGHT))
        if dx is not None:
            res["dx"] = host(dx)
        for k, v in (grads or {}).items():
            res["d_" + k] = host(v)
    torch.cuda.synchronize()
    return res, saved, cfg


def check_against_oracle(cfg_d, inp, res, tol, backward):
    ref = oracle.layer_forward(cfg_d, {n: inp[n] for n in synth.PARAM_NAMES},
                               inp["x"])
    errs = {}
    for k, v in ref.items():
        errs[k] = rel_err(res[k], v)
    if backward:
        dx, grads = oracle.layer_backward(
            cfg_d, {n: inp[n] for n in synth.PARAM_NAMES}, inp["x"], inp["dy"])
        errs["dx"] = rel_err(res["dx"], dx)
        for n in synth.PARAM_NAMES:
            if not cfg_d.get("qk_norm", True) and n in ("q_norm", "k_norm"):
                continue
            errs["d_" + n] = rel_err(res["d_" + n], grads[n])
    print({k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, bad


def test_config0_tiny_fp32_forward():
    need_gpu()
    say("preset 0 forward (fp32)")
    cfg, inp = synth.preset_inputs(0)
    res, _, _ = run_layer(cfg, inp)
    check_against_oracle(cfg, inp, res, TOL["f32"], False)


def test_config0_tiny_fp32_forward_backward():
    need_gpu()
    say("preset 0 dims forward+backward (fp32)")
    cfg = synth.preset(0)
    inp = synth.make_inputs(cfg, 1000, with_dy=True)
    res, _, _ = run_layer(cfg, inp, backward=True)
    check_against_oracle(cfg, inp, res, TOL["f32"], True)


SMALL = [
    dict(d=256, h_q=4, h_kv=2, d_h=64, d_ffn=520, B=2, L=37, dtype="f32"),
    dict(d=256, h_q=4, h_kv=2, d_h=64, d_ffn=520, B=2, L=200, dtype="bf16"),
    dict(d=512, h_q=8, h_kv=2, d_h=128, d_ffn=1024, B=1, L=300, dtype="bf16"),
    dict(d=384, h_q=6, h_kv=2, d_h=64, d_ffn=776, B=3, L=129, dtype="bf16",
         qk_norm=False),
    dict(d=256, h_q=2, h_kv=2, d_h=128, d_ffn=256, B=1, L=1, dtype="bf16"),
    # Widest rows the norms take (8192: four 8-element chunks per thread in
    # the bf16 RMSNorm backward) and a width whose last chunks overhang the
    # workgroup (2560), both at token counts that leave partial row groups.
    dict(d=8192, h_q=4, h_kv=1, d_h=128, d_ffn=384, B=1, L=70, dtype="bf16"),
    dict(d=2560, h_q=4, h_kv=2, d_h=64, d_ffn=512, B=2, L=45, dtype="bf16"),
]


@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "-".join(
    f"{k}{v}" for k, v in s.items()))
def test_small_layer_forward_backward(shape):
    need_gpu()
    say(f"layer fwd+bwd {shape}")
    cfg = synth.make_cfg(**shape)
    inp = synth.make_inputs(cfg, 77, with_dy=True)
    res, _, _ = run_layer(cfg, inp, backward=True)
    check_against_oracle(cfg, inp, res, TOL[cfg["dtype"]], True)


def test_small_tp_partial_forward():
    need_gpu()
    say("tp_partial forward small")
    cfg = synth.make_cfg(d=512, h_q=4, h_kv=1, d_h=128, d_ffn=448, B=2, L=130,
                         dtype="bf16", tp_partial=True)
    inp = synth.make_inputs(cfg, 5)
    res, _, _ = run_layer(cfg, inp)
    check_against_oracle(cfg, inp, res, TOL["bf16"], False)


def test_saved_intermediates():
    """The tensors the forward saves match the oracle's intermediates."""
    need_gpu()
    import torch
    say("saved intermediates")
    cfg = synth.make_cfg(d=512, h_q=8, h_kv=2, d_h=128, d_ffn=640, B=2,
                         L=100, dtype="bf16")
    inp = synth.make_inputs(cfg, 9, with_dy=True)
    res, saved, c = run_layer(cfg, inp, backward=True)
    lay = q3.saved_layout(c)
    ref = oracle.layer_forward(cfg, {n: inp[n] for n in synth.PARAM_NAMES},
                               inp["x"], keep=True)
    T, d, qd, kvd, f = c.T, c.d, c.h_q * c.d_h, c.h_kv * c.d_h, c.d_ffn

    def view(name, shape, dt):
        nbytes = int(np.prod(shape)) * (2 if dt == torch.bfloat16 else 4)
        return host(saved[lay[name]:lay[name] + nbytes].view(dt).view(shape))

    bf = torch.bfloat16
    checks = {
        "rstd1": (view("rstd1", (T,), torch.float32), ref["r1"].reshape(T)),
        "xn": (view("xn", (T, d), bf), ref["xn"].reshape(T, d)),
        "lse": (view("lse", (c.B, c.h_q, c.L), torch.float32), ref["LSE"]),
        "attn_o": (view("attn_o", (T, qd), bf), ref["O"].reshape(T, qd)),
        "h": (view("h", (T, d), bf), ref["h"].reshape(T, d)),
        "hn": (view("hn", (T, d), bf), ref["hn"].reshape(T, d)),
        "f": (view("f", (T, f), bf), ref["f"].reshape(T, f)),
    }
    qkr = view("qk_rope", (T, qd + kvd), bf)
    checks["q_rope"] = (qkr[:, :qd], ref["qr"].reshape(T, qd))
    checks["k_rope"] = (qkr[:, qd:], ref["kr"].reshape(T, kvd))
    gu = view("gu", (T, 2 * f), bf)
    checks["gate"] = (gu[:, :f], ref["g"].reshape(T, f))
    checks["up"] = (gu[:, f:], ref["u"].reshape(T, f))
    errs = {k: rel_err(a, b) for k, (a, b) in checks.items()}
    print({k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    assert all(v <= TOL["bf16"] for v in errs.values()), errs

    # The transposed copies the bf16 forward leaves for the backward are
    # exact: the weights as [in, out] (down; gate | up; o; q | k | v, each
    # region 256-byte aligned) and xn^T with its padding columns zero.
    def region(off, shape):
        nbytes = int(np.prod(shape)) * 2
        return host(saved[off:off + nbytes].view(bf).view(shape))

    def up(n):
        return (n + 255) // 256 * 256

    wt, nqkv = lay["wt"], qd + 2 * kvd
    o_down = wt
    o_gu = o_down + up(f * d * 2)
    o_o = o_gu + up(d * 2 * f * 2)
    o_qkv = o_o + up(qd * d * 2)
    W = {n: np.asarray(inp[n], dtype=np.float64) for n in ("down", "gate", "up", "o", "q", "k", "v")}
    assert np.array_equal(region(o_down, (f, d)), W["down"].T)
    gut = region(o_gu, (d, 2 * f))
    assert np.array_equal(gut[:, :f], W["gate"].T) and np.array_equal(gut[:, f:], W["up"].T)
    assert np.array_equal(region(o_o, (qd, d)), W["o"].T)
    qkvt = region(o_qkv, (d, nqkv))
    assert np.array_equal(qkvt[:, :qd], W["q"].T)
    assert np.array_equal(qkvt[:, qd:qd + kvd], W["k"].T)
    assert np.array_equal(qkvt[:, qd + kvd:], W["v"].T)
    Tp = (T + 7) // 8 * 8
    xnt = region(lay["xnt"], (d, Tp))
    assert np.array_equal(xnt[:, :T], view("xn", (T, d), bf).T)
    assert not xnt[:, T:].any()


def test_backward_flags_and_accumulate():
    need_gpu()
    import torch
    say("backward flags")
    cfg = synth.make_cfg(d=256, h_q=4, h_kv=2, d_h=64, d_ffn=256, B=1, L=64,
                         dtype="bf16")
    inp = synth.make_inputs(cfg, 3, with_dy=True)
    c = q3.LayerConfig.from_dict(cfg)
    W = gpu_weights(inp, "bf16")
    x, dy = dev(inp["x"], "bf16"), dev(inp["dy"], "bf16")
    saved = torch.empty(q3.saved_bytes(c), dtype=torch.uint8, device="cuda")
    q3.layer_forward(c, W, x, saved=saved)
    dx, g1 = q3.layer_backward(c, W, x, dy, saved)
    g1 = {k: v.clone() for k, v in g1.items()}
    # ACCUMULATE adds a second copy.
    _, g2 = q3.layer_backward(c, W, x, dy, saved, grads={k: v.clone() for k, v in g1.items()},
                              flags=q3.BWD_INPUT | q3.BWD_WEIGHT | q3.BWD_ACCUMULATE)
    for k in g1:
        assert torch.allclose(g2[k], 2 * g1[k], rtol=1e-5, atol=1e-6), k
    # INPUT only: grads untouched.
    sentinel = {k: torch.full_like(v, 7.0) for k, v in g1.items()}
    dx2, g3 = q3.layer_backward(c, W, x, dy, saved, grads=sentinel, flags=q3.BWD_INPUT)
    assert torch.equal(dx2, dx)
    for k in sentinel:
        assert torch.all(sentinel[k] == 7.0), k
    # WEIGHT only: dx untouched.
    dxs = torch.full_like(dx, 3.0)
    _, g4 = q3.layer_backward(c, W, x, dy, saved, dx=dxs, flags=q3.BWD_WEIGHT)
    assert torch.all(dxs == 3.0)
    for k in g1:
        assert torch.equal(g4[k], g1[k]), k


def test_forward_is_deterministic():
    need_gpu()
    import torch
    say("determinism")
    cfg = synth.make_cfg(d=512, h_q=8, h_kv=2, d_h=128, d_ffn=1024, B=2,
                         L=256, dtype="bf16")
    inp = synth.make_inputs(cfg, 4)
    c = q3.LayerConfig.from_dict(cfg)
    W = gpu_weights(inp, "bf16")
    x = dev(inp["x"], "bf16")
    y1 = q3.layer_forward(c, W, x)["y"].clone()
    y2 = q3.layer_forward(c, W, x)["y"]
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


# ---- full-size workloads -------------------------------------------------
def test_preset1_full_forward():
    """Tiny dims at B=8, L=2048 in bf16: every output against the full oracle."""
    need_gpu()
    say("preset 1 full forward")
    cfg, inp = synth.preset_inputs(1)
    res, _, _ = run_layer(cfg, inp)
    check_against_oracle(cfg, inp, res, TOL["bf16"], False)


def _sampled_rows_check(idx):
    cfg, inp = synth.preset_inputs(idx)
    res, _, _ = run_layer(cfg, inp)
    p = {n: inp[n] for n in synth.PARAM_NAMES}
    L = cfg["L"]
    rng = np.random.default_rng(idx)
    rows = np.unique(np.concatenate([[0, 1, 63, 64, 127, 128, L // 2, L - 2, L - 1],
                                     rng.integers(0, L, 7)]))
    errs = {}
    for b in (0, cfg["B"] - 1):
        ref = oracle.layer_forward_rows(cfg, p, inp["x"][b], rows)
        for k, v in ref.items():
            den = np.max(np.abs(v))
            e = np.max(np.abs(res[k][b, rows] - v)) / den
            errs[f"{k}[b={b}]"] = e
    print({k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    assert all(v <= TOL["bf16"] for v in errs.values()), errs


def test_preset2_qwen3_8b_forward_sampled_rows():
    need_gpu()
    say("preset 2 forward, sampled rows")
    _sampled_rows_check(2)


def test_preset3_tp_share_forward_sampled_rows():
    need_gpu()
    say("preset 3 forward, sampled rows")
    _sampled_rows_check(3)


def test_preset4_qwen3_8b_forward_backward_golden():
    """Full-size forward+backward against stored fp64 oracle samples
    (tests/golden/make_oracle_samples.py)."""
    need_gpu()
    import sys
    sys.path.insert(0, GOLDEN)
    import make_oracle_samples as mk
    say("preset 4 forward+backward vs oracle samples")
    gold = np.load(os.path.join(GOLDEN, os.path.basename(mk.OUT)))
    cfg, inp = synth.preset_inputs(4)
    res, _, _ = run_layer(cfg, inp, backward=True)
    errs = {}
    for name in mk.TENSORS:
        key = name if name in ("y", "dx") else "d_" + name
        a = res[key].ravel()
        assert a.size == int(gold[f"{name}_size"])
        idx = mk.sample_indices(name, a.size)
        errs[name] = float(np.max(np.abs(a[idx] - gold[f"{name}_val"]))
                           / float(gold[f"{name}_maxabs"]))
        # the GPU tensor's own scale agrees with the oracle's
        errs[name + "_maxabs"] = abs(np.max(np.abs(a)) / float(gold[f"{name}_maxabs"]) - 1)
    print({k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    assert all(v <= TOL["bf16"] for v in errs.values()), errs


def test_other_stream_and_graph_replay():
    """The forward forks work to the library's second stream and joins it
    back: results on another caller stream and from a replayed HIP graph of
    forward + backward are bitwise those of the eager default-stream run."""
    need_gpu()
    import torch
    say("caller stream / graph replay")
    cfg = synth.make_cfg(d=256, h_q=4, h_kv=2, d_h=64, d_ffn=512, B=2, L=96,
                         dtype="bf16")
    inp = synth.make_inputs(cfg, 21, with_dy=True)
    c = q3.LayerConfig.from_dict(cfg)
    W = gpu_weights(inp, "bf16")
    x, dy = dev(inp["x"], "bf16"), dev(inp["dy"], "bf16")
    saved = torch.empty(q3.saved_bytes(c), dtype=torch.uint8, device="cuda")
    ws = torch.empty(q3.workspace_bytes(c, True), dtype=torch.uint8, device="cuda")
    y = torch.empty_like(x)
    dx = torch.empty_like(x)
    grads = {n: torch.empty(W[n].shape, dtype=torch.float32, device="cuda")
             for n in synth.PARAM_NAMES}

    def step(stream):
        q3.layer_forward(c, W, x, out={"y": y}, saved=saved, stream=stream)
        q3.layer_backward(c, W, x, dy, saved, dx=dx, grads=grads, workspace=ws,
                          stream=stream)

    def snapshot():
        return [t.clone() for t in [y, dx] + [grads[n] for n in synth.PARAM_NAMES]]

    step(torch.cuda.current_stream())
    torch.cuda.synchronize()
    ref = snapshot()

    side = torch.cuda.Stream()
    for t in [y, dx] + list(grads.values()):
        t.zero_()
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        step(side)
    side.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(snapshot(), ref))

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(torch.cuda.current_stream())
    for rep in range(3):
        for t in [y, dx] + list(grads.values()):
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = snapshot()
        assert all(torch.equal(a, b) for a, b in zip(got, ref)), f"replay {rep}"
        step(torch.cuda.current_stream())   # eager work between replays
        torch.cuda.synchronize()
