"""Whole-layer parity of the HIP path (q3l_layer_forward / q3l_layer_backward
through the C ABI) against the fp64 oracle on the same seeded inputs.

Outputs, the saved block and both workspaces are NaN-poisoned buffers
between guard bands: every output element and every saved tensor must be
written, nothing outside a buffer may be, and nothing may be read from a
workspace before it is written (a poisoned read would leave NaNs)."""
import os

import numpy as np
import pytest

import oracle
import qwen3_decoder_layer_amd as q3
from gpu_helpers import (BETA, LOCAL_FACTOR, TOL, Guarded, check, dev, gpu_weights,
                         guarded_bytes, host, need_gpu, saved_fields, say, view_saved)
import synth

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def run_layer(cfg_d, inp, backward=False, flags=None, side_stream=False):
    import torch
    cfg = q3.LayerConfig.from_dict(cfg_d)
    td = cfg.torch_dtype
    W = gpu_weights(inp, cfg.dtype)
    x = dev(inp["x"], cfg.dtype)
    shape = (cfg.B, cfg.L, cfg.d)
    if cfg.tp_partial:
        outs = {k: Guarded(shape, torch.float32) for k in ("attn_partial", "mlp_partial")}
    else:
        outs = {"y": Guarded(shape, td)}
    saved = guarded_bytes(q3.saved_bytes(cfg)) if backward else None
    fws = None if backward else guarded_bytes(q3.workspace_bytes(cfg, False))
    ex = q3.Exec(side_stream=torch.cuda.Stream()) if side_stream else None
    q3.layer_forward(cfg, W, x, out={k: g.t for k, g in outs.items()},
                     saved=None if saved is None else saved.t,
                     workspace=None if fws is None else fws.t, exec=ex)
    torch.cuda.synchronize()
    res = {}
    for k, g in outs.items():
        g.check(k)
        res[k] = host(g.t)
    if fws is not None:
        assert fws.guards_intact(), "forward workspace overrun"
    if backward:
        assert saved.guards_intact(), "saved block overrun"
        lay = q3.saved_layout(cfg)
        for name, off, shp, dt in saved_fields(cfg, lay):
            assert bool(torch.isfinite(view_saved(saved.t, off, shp, dt).float()).all()), \
                f"saved {name} not fully written"
        dy = dev(inp["dy"], cfg.dtype)
        flags = flags or (q3.BWD_INPUT | q3.BWD_WEIGHT)
        dx = Guarded(shape, td) if flags & q3.BWD_INPUT else None
        grads = ({n: Guarded(s, torch.float32) for n, s in q3.param_shapes(cfg).items()}
                 if flags & q3.BWD_WEIGHT else None)
        if grads is not None and not cfg.qk_norm:
            for n in ("q_norm", "k_norm"):
                grads[n].t.zero_()
        bws = guarded_bytes(q3.workspace_bytes(cfg, True))
        q3.layer_backward(cfg, W, x, dy, saved.t, dx=None if dx is None else dx.t,
                          grads=None if grads is None else {k: g.t for k, g in grads.items()},
                          flags=flags, workspace=bws.t)
        torch.cuda.synchronize()
        assert bws.guards_intact(), "backward workspace overrun"
        if dx is not None:
            dx.check("dx")
            res["dx"] = host(dx.t)
        for k, g in (grads or {}).items():
            g.check("d_" + k)
            res["d_" + k] = host(g.t)
    return res, (None if saved is None else saved.t), cfg


def check_against_oracle(cfg_d, inp, res, tol, backward):
    ref = oracle.layer_forward(cfg_d, {n: inp[n] for n in synth.PARAM_NAMES},
                               inp["x"])
    errs = {}
    ok = True
    for k, v in ref.items():
        ok &= check(k, res[k], v, tol, errs=errs)
    if backward:
        dx, grads = oracle.layer_backward(
            cfg_d, {n: inp[n] for n in synth.PARAM_NAMES}, inp["x"], inp["dy"])
        ok &= check("dx", res["dx"], dx, tol, errs=errs)
        # With a handful of tokens a projection gradient is an outer product
        # of a few rounded activation rows -- nothing sums the rounding over
        # tokens, and a row whose activation value cancels to near zero
        # keeps a relative error a row-local scale cannot bound: such
        # gradients are held to the tensor-wide bar only.
        few = cfg_d["B"] * cfg_d["L"] < 8
        for n in synth.PARAM_NAMES:
            if not cfg_d.get("qk_norm", True) and n in ("q_norm", "k_norm"):
                continue
            # Rows of a projection gradient are its output features; a norm
            # weight's gradient is one row.
            ok &= check("d_" + n, res["d_" + n], grads[n], tol, errs=errs,
                        local=not (few and n not in synth.NORM_PARAMS))
    print({k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    assert ok, {k: v for k, v in errs.items() if not v <= tol}


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


def test_small_layer_with_side_stream():
    """The training forward with the caller's second stream (transposed
    copies beside the attention step) gives the same results."""
    need_gpu()
    say("layer fwd+bwd with a side stream")
    cfg = synth.make_cfg(d=512, h_q=8, h_kv=2, d_h=128, d_ffn=1024, B=2, L=130,
                         dtype="bf16")
    inp = synth.make_inputs(cfg, 78, with_dy=True)
    res, _, _ = run_layer(cfg, inp, backward=True, side_stream=True)
    check_against_oracle(cfg, inp, res, TOL["bf16"], True)
    res2, _, _ = run_layer(cfg, inp, backward=True, side_stream=False)
    for k in res:
        assert np.array_equal(res[k], res2[k]), k


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
        return host(view_saved(saved, lay[name], shape, dt))

    bf = torch.bfloat16
    checks = {
        "rstd1": (view("rstd1", (T,), torch.float32), ref["r1"].reshape(1, T)),
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
    errs = {}
    ok = all([check(k, a.reshape(b.shape), b, TOL["bf16"], errs=errs)
              for k, (a, b) in checks.items()])
    print({k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    assert ok, errs

    # The transposed copy the bf16 forward leaves for the backward is exact:
    # xn^T with its padding columns zero.  (The weights are read by the
    # backward as they are: the wt region is empty.)
    def region(off, shape):
        return host(view_saved(saved, off, shape, bf))

    assert lay["wt"] == lay["xnt"]
    Tp = (T + 7) // 8 * 8
    xnt = region(lay["xnt"], (d, Tp))
    assert np.array_equal(xnt[:, :T], view("xn", (T, d), bf).T)
    assert not xnt[:, T:].any()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_backward_flags_and_accumulate(dtype):
    need_gpu()
    import torch
    say(f"backward flags {dtype}")
    cfg = synth.make_cfg(d=256, h_q=4, h_kv=2, d_h=64, d_ffn=256, B=1, L=70,
                         dtype=dtype)
    inp = synth.make_inputs(cfg, 3, with_dy=True)
    c = q3.LayerConfig.from_dict(cfg)
    W = gpu_weights(inp, dtype)
    x, dy = dev(inp["x"], dtype), dev(inp["dy"], dtype)
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
    ws = torch.full((q3.workspace_bytes(c, True),), 0xFF, dtype=torch.uint8, device="cuda")
    dx2, g3 = q3.layer_backward(c, W, x, dy, saved, grads=sentinel, flags=q3.BWD_INPUT,
                                workspace=ws)
    assert torch.equal(dx2, dx)
    for k in sentinel:
        assert torch.all(sentinel[k] == 7.0), k
    # ... then the deferred weight-gradient half on the same workspace:
    # bitwise the gradients of the one-call backward, dx untouched.
    dxs = torch.full_like(dx, 3.0)
    _, g5 = q3.layer_backward(c, W, x, dy, saved, dx=dxs,
                              flags=q3.BWD_WEIGHT | q3.BWD_DEFERRED_WEIGHT, workspace=ws)
    assert torch.all(dxs == 3.0)
    for k in g1:
        assert torch.equal(g5[k], g1[k]), k
    # ... and accumulated.
    _, g6 = q3.layer_backward(c, W, x, dy, saved, grads={k: v.clone() for k, v in g1.items()},
                              flags=q3.BWD_WEIGHT | q3.BWD_DEFERRED_WEIGHT | q3.BWD_ACCUMULATE,
                              workspace=ws)
    for k in g1:
        assert torch.equal(g6[k], g2[k]), k
    # WEIGHT only, not deferred: the whole chain, dx untouched.
    _, g4 = q3.layer_backward(c, W, x, dy, saved, dx=dxs, flags=q3.BWD_WEIGHT)
    assert torch.all(dxs == 3.0)
    for k in g1:
        assert torch.equal(g4[k], g1[k]), k


def test_phase_marks():
    """The caller's timing events are recorded at every phase boundary of a
    forward and a backward call, in order."""
    need_gpu()
    import torch
    say("phase marks")
    cfg = synth.make_cfg(d=512, h_q=8, h_kv=2, d_h=128, d_ffn=1024, B=2, L=256,
                         dtype="bf16")
    inp = synth.make_inputs(cfg, 6, with_dy=True)
    c = q3.LayerConfig.from_dict(cfg)
    W = gpu_weights(inp, "bf16")
    x, dy = dev(inp["x"], "bf16"), dev(inp["dy"], "bf16")
    saved = torch.empty(q3.saved_bytes(c), dtype=torch.uint8, device="cuda")
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    exf = q3.Exec(side_stream=torch.cuda.Stream(),
                  marks=[torch.cuda.Event(enable_timing=True)
                         for _ in range(len(q3.phase_names(False)) + 1)])
    exb = q3.Exec(marks=[torch.cuda.Event(enable_timing=True)
                         for _ in range(len(q3.phase_names(True)) + 1)])
    start.record()
    q3.layer_forward(c, W, x, saved=saved, exec=exf)
    q3.layer_backward(c, W, x, dy, saved, exec=exb)
    end.record()
    torch.cuda.synchronize()
    tf, tb = exf.phase_times(), exb.phase_times()
    total = start.elapsed_time(end)
    assert len(tf) == len(q3.phase_names(False)) and len(tb) == len(q3.phase_names(True))
    assert all(t >= 0 for t in tf + tb)
    assert 0 < sum(tf) + sum(tb) <= total * 1.01 + 0.05
    names = q3.phase_names(False)
    assert tf[names.index("F5 attention")] > 0 and tf[names.index("F8-F9 gate/up gemm + swiglu")] > 0


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
    """Full-size forward, checked on whole output rows of every sequence: one
    seeded row in each 64-row tile plus the sequence's first and last rows,
    each recomputed by the oracle on its own."""
    cfg, inp = synth.preset_inputs(idx)
    res, _, _ = run_layer(cfg, inp)
    p = {n: inp[n] for n in synth.PARAM_NAMES}
    L = cfg["L"]
    rng = np.random.default_rng(idx)
    errs = {}
    ok = True
    for b in range(cfg["B"]):
        tiles = np.arange(0, L, 64)
        rows = np.unique(np.concatenate(
            [[0, 1, L - 1], tiles + rng.integers(0, 64, tiles.size)]).clip(0, L - 1))
        ref = oracle.layer_forward_rows(cfg, p, inp["x"][b], rows)
        for k, v in ref.items():
            ok &= check(f"{k}[b={b}]", res[k][b, rows], v, TOL["bf16"], errs=errs)
    print({k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    assert ok, {k: v for k, v in errs.items() if not v <= TOL["bf16"]}


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
    (tests/golden/make_oracle_samples.py): one element of every 32 x 64
    block of y, dx and each projection gradient, the norm-weight gradients
    whole, each against both bars (the row-local one with the oracle's row
    RMS; reported divided by LOCAL_FACTOR, so both compare to the same
    number)."""
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
        m = mk.as_matrix(name, res[key])
        assert tuple(m.shape) == tuple(gold[f"{name}_shape"])
        r, c = mk.sample_indices(name, m.shape)
        got, ref = m[r, c], gold[f"{name}_val"].astype(np.float64)
        rowrms = gold[f"{name}_rowrms"].astype(np.float64)
        scale = np.abs(ref) + rowrms[r] + BETA * np.sqrt(np.mean(rowrms ** 2))
        diff = np.abs(got - ref)
        errs[name] = float(np.max(diff) / float(gold[f"{name}_maxabs"]))
        errs[name + "_local"] = float(np.max(diff / scale)) / LOCAL_FACTOR
        # the GPU tensor's own row scales agree with the oracle's
        g_rms = np.sqrt(np.mean(m * m, axis=1))
        errs[name + "_rowrms"] = float(np.max(np.abs(g_rms / gold[f"{name}_rowrms"] - 1)))
        assert np.isfinite(m).all(), name
    print({k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    assert all(v <= TOL["bf16"] for v in errs.values()), errs


def test_other_stream_and_graph_replay():
    """Forward (with the caller's second stream) + backward on another
    caller stream and as a replayed HIP graph are bitwise the eager
    default-stream run."""
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
    ex = q3.Exec(side_stream=torch.cuda.Stream())

    def step(stream, exec_=None):
        q3.layer_forward(c, W, x, out={"y": y}, saved=saved, stream=stream, exec=exec_)
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
        step(side, ex)
    side.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(snapshot(), ref))

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(torch.cuda.current_stream(), ex)
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
