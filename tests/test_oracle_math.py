"""Pins of the oracle to mathematics: closed forms, brute force on tiny
inputs, invariants and finite differences."""
import math

import numpy as np
import pytest

import oracle
import synth


def tiny_cfg(**kw):
    base = dict(d=64, h_q=4, h_kv=2, d_h=16, d_ffn=96, B=2, L=6,
                dtype="f32")
    base.update(kw)
    return synth.make_cfg(**base)


def inputs(cfg, seed=3):
    return synth.make_inputs(cfg, seed, with_dy=True)


def params(inp):
    return {k: inp[k] for k in synth.PARAM_NAMES}


# --- RMSNorm (walkthrough page, Step 1 formula) -----------------------------
def test_rmsnorm_closed_form_constant_vector():
    eps = 1e-6
    w = np.linspace(0.5, 1.5, 8)
    for c in (0.0, 1e-4, 0.3, -2.0, 7.5):
        y, r = oracle.rmsnorm(np.full(8, c), w, eps)
        assert np.allclose(y, c / math.sqrt(c * c + eps) * w, rtol=1e-15,
                           atol=1e-300)
        assert math.isclose(r, 1 / math.sqrt(c * c + eps), rel_tol=1e-15)


def test_rmsnorm_brute_force_and_scale_invariance():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((3, 5))
    w = rng.standard_normal(5)
    y, _ = oracle.rmsnorm(x, w, 1e-6)
    for i in range(3):
        ss = 0.0
        for j in range(5):
            ss += x[i, j] * x[i, j]
        den = math.sqrt(ss / 5 + 1e-6)
        for j in range(5):
            assert math.isclose(y[i, j], x[i, j] / den * w[j], rel_tol=1e-13)
    y2, _ = oracle.rmsnorm(10.0 * x, w, 1e-6)
    assert np.allclose(y, y2, rtol=1e-5)


def test_qk_norm_unit_weight_rms():
    """With w = 1 each head vector's RMS after the norm is sqrt(ms/(ms+eps))."""
    rng = np.random.default_rng(2)
    q = rng.standard_normal((2, 3, 4, 16)) * 1e-3
    y, _ = oracle.rmsnorm(q, np.ones(16), 1e-6)
    ms = np.mean(q * q, axis=-1)
    rms = np.sqrt(np.mean(y * y, axis=-1))
    assert np.allclose(rms, np.sqrt(ms / (ms + 1e-6)), rtol=1e-13)


# --- RoPE (walkthrough page, Step 4) ----------------------------------------
def test_rope_properties():
    rng = np.random.default_rng(4)
    L, dh = 50, 16
    cos, sin = oracle.rope_cos_sin(L, dh, 1e6)
    u = rng.standard_normal((1, L, 3, dh))
    r = oracle.rope(u, cos, sin)
    # Per-head norm preserved.
    assert np.allclose(np.linalg.norm(r, axis=-1), np.linalg.norm(u, axis=-1),
                       rtol=1e-13)
    # Position 0 is the identity.
    assert np.array_equal(r[:, 0], u[:, 0])
    # <R_m q, R_n k> depends on m - n only.
    q = rng.standard_normal(dh)
    k = rng.standard_normal(dh)
    Q = oracle.rope(np.broadcast_to(q, (1, L, 1, dh)).copy(), cos, sin)[0, :, 0]
    K = oracle.rope(np.broadcast_to(k, (1, L, 1, dh)).copy(), cos, sin)[0, :, 0]
    for delta in (0, 1, 7):
        dots = [Q[m] @ K[m - delta] for m in range(delta, L)]
        assert np.allclose(dots, dots[0], rtol=1e-10, atol=1e-12)
    # The backward is the adjoint.
    g = rng.standard_normal(u.shape)
    assert math.isclose(np.sum(r * g),
                        np.sum(u * oracle.rope_backward(g, cos, sin)),
                        rel_tol=1e-12)


# --- attention (walkthrough page, Step 5) -----------------------------------
def brute_attention(q, k, v):
    """Pure-Python loops: softmax(q.k / sqrt(d_h)) over keys s <= t, GQA by
    repeat_interleave (q head j -> kv head j // G)."""
    B, L, hq, dh = q.shape
    G = hq // k.shape[2]
    O = np.zeros_like(q)
    lse = np.zeros((B, hq, L))
    for b in range(B):
        for j in range(hq):
            g = j // G
            for t in range(L):
                sc = []
                for s in range(t + 1):
                    dot = 0.0
                    for c in range(dh):
                        dot += q[b, t, j, c] * k[b, s, g, c]
                    sc.append(dot / math.sqrt(dh))
                m = max(sc)
                ex = [math.exp(x - m) for x in sc]
                den = sum(ex)
                lse[b, j, t] = m + math.log(den)
                for c in range(dh):
                    O[b, t, j, c] = sum(ex[s] * v[b, s, g, c]
                                        for s in range(t + 1)) / den
    return O, lse


def test_attention_brute_force():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((2, 5, 4, 4))
    k = rng.standard_normal((2, 5, 2, 4))
    v = rng.standard_normal((2, 5, 2, 4))
    O, lse = oracle.attention(q, k, v)
    Ob, lseb = brute_attention(q, k, v)
    assert np.allclose(O, Ob, rtol=1e-12, atol=1e-13)
    assert np.allclose(lse, lseb, rtol=1e-12, atol=1e-13)


def test_gqa_equals_mha_with_repeat_interleave():
    rng = np.random.default_rng(6)
    q = rng.standard_normal((1, 7, 6, 8))
    k = rng.standard_normal((1, 7, 2, 8))
    v = rng.standard_normal((1, 7, 2, 8))
    O, lse = oracle.attention(q, k, v)
    O2, lse2 = oracle.attention(q, np.repeat(k, 3, axis=2),
                                np.repeat(v, 3, axis=2))
    assert np.allclose(O, O2, rtol=1e-14, atol=1e-14)
    assert np.allclose(lse, lse2, rtol=1e-14, atol=1e-14)
    # h_kv = h_q is plain multi-head attention: head j uses kv head j.
    kf = rng.standard_normal((1, 7, 6, 8))
    vf = rng.standard_normal((1, 7, 6, 8))
    O3, _ = oracle.attention(q, kf, vf)
    for j in range(6):
        Oj, _ = oracle.attention(q[:, :, j:j + 1], kf[:, :, j:j + 1],
                                 vf[:, :, j:j + 1])
        assert np.allclose(O3[:, :, j], Oj[:, :, 0], rtol=1e-14, atol=1e-14)


def test_attention_special_cases():
    rng = np.random.default_rng(8)
    # L = 1: the only visible key is itself, O = v.
    q = rng.standard_normal((2, 1, 4, 8))
    k = rng.standard_normal((2, 1, 2, 8))
    v = rng.standard_normal((2, 1, 2, 8))
    O, lse = oracle.attention(q, k, v)
    assert np.allclose(O, np.repeat(v, 2, axis=2), rtol=1e-15, atol=0)
    # q = 0: uniform weights, O_t = mean(v_0..v_t) and lse = log(t + 1).
    L = 9
    q = np.zeros((1, L, 4, 8))
    k = rng.standard_normal((1, L, 2, 8))
    v = rng.standard_normal((1, L, 2, 8))
    O, lse = oracle.attention(q, k, v)
    csum = np.cumsum(v, axis=1) / np.arange(1, L + 1)[None, :, None, None]
    assert np.allclose(O, np.repeat(csum, 2, axis=2), rtol=1e-13, atol=1e-14)
    assert np.allclose(lse[0, 0], np.log(np.arange(1, L + 1)), atol=1e-14)


# --- layer-level invariants -------------------------------------------------
def test_causality_of_whole_layer():
    cfg = tiny_cfg(L=10)
    inp = inputs(cfg)
    p = params(inp)
    x = inp["x"].astype(np.float64)
    y = oracle.layer_forward(cfg, p, x)["y"]
    for t in (0, 4, 8):
        x2 = x.copy()
        x2[:, t + 1:] += np.random.default_rng(t).standard_normal(
            x2[:, t + 1:].shape)
        y2 = oracle.layer_forward(cfg, p, x2)["y"]
        assert np.array_equal(y[:, :t + 1], y2[:, :t + 1])
        if t + 1 < cfg["L"]:
            assert not np.allclose(y[:, t + 1:], y2[:, t + 1:])


def test_batch_independence():
    cfg = tiny_cfg(B=3)
    inp = inputs(cfg)
    p = params(inp)
    y = oracle.layer_forward(cfg, p, inp["x"])["y"]
    for b in range(3):
        cb = dict(cfg, B=1)
        yb = oracle.layer_forward(cb, p, inp["x"][b:b + 1])["y"]
        assert np.allclose(y[b:b + 1], yb, rtol=1e-14, atol=1e-14)


def test_zero_weight_special_cases():
    cfg = tiny_cfg()
    inp = inputs(cfg)
    x = inp["x"].astype(np.float64)
    dy = inp["dy"].astype(np.float64)
    # W_gate = 0: silu(0) = 0 so the MLP adds nothing: y = h.
    p = params(inp)
    p["gate"] = np.zeros_like(p["gate"])
    out = oracle.layer_forward(cfg, p, x, keep=True)
    assert np.array_equal(out["y"], out["h"])
    # W_down = 0: y = h as well.
    p = params(inp)
    p["down"] = np.zeros_like(p["down"])
    out = oracle.layer_forward(cfg, p, x, keep=True)
    assert np.array_equal(out["y"], out["h"])
    # W_o = W_down = 0: the layer is the identity and dx = dy.
    p["o"] = np.zeros_like(p["o"])
    out = oracle.layer_forward(cfg, p, x)
    assert np.array_equal(out["y"], x)
    dx, grads = oracle.layer_backward(cfg, p, x, dy)
    assert np.array_equal(dx, dy)
    for name in ("in_norm", "q", "k", "v", "q_norm", "k_norm", "post_norm",
                 "gate", "up"):
        assert not np.any(grads[name]), name


def test_rows_evaluation_matches_full_forward():
    for tp in (False, True):
        cfg = tiny_cfg(L=23, B=2, tp_partial=tp)
        inp = inputs(cfg)
        p = params(inp)
        full = oracle.layer_forward(cfg, p, inp["x"])
        rows = np.array([0, 5, 22, 11])
        for b in range(2):
            part = oracle.layer_forward_rows(cfg, p, inp["x"][b], rows)
            for key, val in part.items():
                assert np.allclose(val, full[key][b, rows], rtol=1e-13,
                                   atol=1e-13), key


def test_tp_decomposition_of_layer_share():
    """One TP rank's share (heads and d_ffn split, o/down rows) emits partial
    sums; summing the ranks' partials reproduces the unsplit projections."""
    cfg = tiny_cfg(h_q=4, h_kv=2, L=7)
    inp = inputs(cfg)
    p = params(inp)
    x = inp["x"]
    full = oracle.layer_forward(cfg, p, x, keep=True)
    dh, f = cfg["d_h"], cfg["d_ffn"]
    a_sum = 0
    m_sum = 0
    for r in range(2):       # TP = 2: 2 q heads and 1 kv head per rank
        pr = dict(p)
        pr["q"] = p["q"][r * 2 * dh:(r + 1) * 2 * dh]
        pr["k"] = p["k"][r * dh:(r + 1) * dh]
        pr["v"] = p["v"][r * dh:(r + 1) * dh]
        pr["o"] = p["o"][:, r * 2 * dh:(r + 1) * 2 * dh]
        pr["gate"] = p["gate"][r * f // 2:(r + 1) * f // 2]
        pr["up"] = p["up"][r * f // 2:(r + 1) * f // 2]
        pr["down"] = p["down"][:, r * f // 2:(r + 1) * f // 2]
        cr = dict(cfg, h_q=2, h_kv=1, d_ffn=f // 2, tp_partial=True)
        part = oracle.layer_forward(cr, pr, x, keep=True)
        a_sum = a_sum + part["attn_partial"]
        # MLP partials of the unsplit h: feed the full layer's h.
        pr_h = oracle.rmsnorm(full["h"], p["post_norm"], cfg["eps"])[0]
        m_sum = m_sum + oracle.linear(
            oracle.swiglu(oracle.linear(pr_h, pr["gate"]),
                          oracle.linear(pr_h, pr["up"])), pr["down"])
    assert np.allclose(a_sum, full["a"], rtol=1e-12, atol=1e-13)
    assert np.allclose(m_sum, full["m"], rtol=1e-12, atol=1e-13)


# --- backward: central finite differences (fp64) ----------------------------
def _loss(cfg, p, x, dy):
    return float(np.sum(oracle.layer_forward(cfg, p, x)["y"] * dy))


@pytest.mark.parametrize("qk_norm", [True, False])
def test_backward_finite_differences_tiny(qk_norm):
    cfg = tiny_cfg(qk_norm=qk_norm)
    inp = inputs(cfg, seed=11)
    p = {k: v.astype(np.float64) for k, v in params(inp).items()}
    x = inp["x"].astype(np.float64)
    dy = inp["dy"].astype(np.float64)
    dx, grads = oracle.layer_backward(cfg, p, x, dy)
    rng = np.random.default_rng(12)
    h = 1e-5
    names = ["x"] + list(synth.PARAM_NAMES)
    if not qk_norm:
        names = [n for n in names if n not in ("q_norm", "k_norm")]
    for name in names:
        base = x if name == "x" else p[name]
        dirn = rng.standard_normal(base.shape)
        g = dx if name == "x" else grads[name]

        def shifted(sgn):
            if name == "x":
                return _loss(cfg, p, x + sgn * h * dirn, dy)
            q = dict(p)
            q[name] = p[name] + sgn * h * dirn
            return _loss(cfg, q, x, dy)

        fd = (shifted(1) - shifted(-1)) / (2 * h)
        an = float(np.sum(g * dirn))
        assert abs(fd - an) <= 1e-6 * max(abs(an), 1e-3), (name, fd, an)


def test_backward_finite_differences_config0_shapes():
    """The walkthrough page's own tiny layer (d=512, 8/4 heads, d_h=64,
    d_ffn=1024, B=2, L=8) at its preset inputs."""
    cfg, inp = synth.preset_inputs(0)
    inp = synth.make_inputs(cfg, 1000, with_dy=True)
    p = {k: inp[k].astype(np.float64) for k in synth.PARAM_NAMES}
    x = inp["x"].astype(np.float64)
    dy = inp["dy"].astype(np.float64)
    dx, grads = oracle.layer_backward(cfg, p, x, dy)
    rng = np.random.default_rng(0)
    h = 1e-5
    for name in ["x"] + list(synth.PARAM_NAMES):
        base = x if name == "x" else p[name]
        dirn = rng.standard_normal(base.shape)
        g = dx if name == "x" else grads[name]
        if name == "x":
            fp = _loss(cfg, p, x + h * dirn, dy)
            fm = _loss(cfg, p, x - h * dirn, dy)
        else:
            q1, q2 = dict(p), dict(p)
            q1[name] = p[name] + h * dirn
            q2[name] = p[name] - h * dirn
            fp, fm = _loss(cfg, q1, x, dy), _loss(cfg, q2, x, dy)
        fd = (fp - fm) / (2 * h)
        an = float(np.sum(g * dirn))
        assert abs(fd - an) <= 1e-6 * max(abs(an), 1e-3), (name, fd, an)


def test_data_parallel_gradient_sum():
    """Weight gradients of a batch equal the sum of its shards' gradients;
    dx of each shard is its slice of the batch's dx."""
    cfg = tiny_cfg(B=4)
    inp = inputs(cfg)
    p = params(inp)
    dx, grads = oracle.layer_backward(cfg, p, inp["x"], inp["dy"])
    acc = {k: 0 for k in grads}
    for lo in (0, 2):
        c2 = dict(cfg, B=2)
        dx2, g2 = oracle.layer_backward(c2, p, inp["x"][lo:lo + 2],
                                        inp["dy"][lo:lo + 2])
        assert np.allclose(dx2, dx[lo:lo + 2], rtol=1e-12, atol=1e-13)
        for k in g2:
            acc[k] = acc[k] + g2[k]
    for k in grads:
        assert np.allclose(acc[k], grads[k], rtol=1e-12, atol=1e-12), k
