"""fp64 evaluation of one Qwen3 decoder layer, forward and backward.

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the
product path.

Every function works on numpy float64 arrays.  Layouts follow the
walkthrough page: activations are [B, L, features]; projection weights are
[out, in] (``nn.Linear`` without bias, "Decoder Layer 的结构" listing), and
head j of a projection output occupies features j*d_h ... (j+1)*d_h - 1 (the
``.view(B, L, h, d_h)`` of Step 2).
"""
from __future__ import annotations

import numpy as np


# --------------------------------------------------------------------------
# RMSNorm -- walkthrough page, Step 1 (formula), Step 3 (per-head q/k norm)
# and Step 8 (post-attention norm).
# --------------------------------------------------------------------------
def rmsnorm(x, w, eps):
    """y_i = x_i / sqrt(mean_j x_j^2 + eps) * w_i over the last axis.

    Returns (y, r) with r = 1 / sqrt(mean(x^2) + eps) (one per vector).
    """
    ms = np.mean(x * x, axis=-1, keepdims=True)
    r = 1.0 / np.sqrt(ms + eps)
    return x * r * w, r[..., 0]


def rmsnorm_backward(dy, x, r, w):
    """Adjoint of ``rmsnorm`` (chain rule through y = x * r(x) * w).

    With xhat = x * r and g = dy * w:
      dx = r * (g - xhat * mean(g * xhat))      (d r / d x_j = -r^3 x_j / n)
      dw = sum over every leading index of dy * xhat
    """
    r = r[..., None]
    xhat = x * r
    g = dy * w
    dx = r * (g - xhat * np.mean(g * xhat, axis=-1, keepdims=True))
    dw = np.sum((dy * xhat).reshape(-1, x.shape[-1]), axis=0)
    return dx, dw


# --------------------------------------------------------------------------
# Bias-free linear layers -- walkthrough page, Steps 2, 6 and 9 (x @ W.T).
# --------------------------------------------------------------------------
def linear(x, W):
    """y = x @ W.T with W stored [out, in]."""
    return x @ W.T


def linear_backward(dy, x, W):
    """dx = dy @ W and dW = dy.T @ x summed over every token."""
    dx = dy @ W
    dW = dy.reshape(-1, dy.shape[-1]).T @ x.reshape(-1, x.shape[-1])
    return dx, dW


# --------------------------------------------------------------------------
# RoPE -- walkthrough page, Step 4.  Reading (parity unpinned as to the
# pairing): rotate-half pairs (i, i + d_h/2), angle t * theta^(-2i/d_h) for
# token position t = 0 .. L-1 within each sequence.
# --------------------------------------------------------------------------
def rope_cos_sin(L, d_h, theta):
    """cos / sin tables [L, d_h/2] of the rotation angles."""
    half = d_h // 2
    inv_freq = float(theta) ** (-(2.0 * np.arange(half, dtype=np.float64))
                                / d_h)
    ang = np.arange(L, dtype=np.float64)[:, None] * inv_freq[None, :]
    return np.cos(ang), np.sin(ang)


def rope(u, cos, sin):
    """Rotate u [B, L, h, d_h]: pair (a_i, b_i) = (u_i, u_{i+d_h/2}) becomes
    (a cos - b sin, b cos + a sin) with the angle of its position and i."""
    half = u.shape[-1] // 2
    a, b = u[..., :half], u[..., half:]
    c = cos[None, :, None, :]
    s = sin[None, :, None, :]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def rope_backward(g, cos, sin):
    """Adjoint of ``rope``: each 2x2 rotation is orthogonal, so its adjoint is
    the rotation by the opposite angle."""
    return rope(g, cos, -sin)


# --------------------------------------------------------------------------
# Causal GQA attention -- walkthrough page, Step 5: K/V repeated with
# repeat_interleave(dim=2, repeats=h_q/h_kv), so q head j reads kv head
# j // (h_q/h_kv); softmax(Q K^T / sqrt(d_h) + causal_mask) V, mask keeping
# key positions s <= t.
# --------------------------------------------------------------------------
def softmax_attend(scores, V):
    """softmax over the last axis of `scores` (entries of -inf are excluded),
    applied to V.  Returns (out, lse) with lse = log sum exp(scores)."""
    m = np.max(scores, axis=-1, keepdims=True)
    e = np.exp(scores - m)
    l = np.sum(e, axis=-1, keepdims=True)
    return (e / l) @ V, (m + np.log(l))[..., 0]


def causal_attention(q_rows, q_pos, K, V, d_h):
    """Attention of query vectors q_rows [n, d_h] at positions q_pos [n] over
    keys/values K, V [L_k, d_h] of the same sequence (key s visible iff
    s <= position)."""
    S = (q_rows @ K.T) / np.sqrt(d_h)
    visible = np.arange(K.shape[0])[None, :] <= np.asarray(q_pos)[:, None]
    S = np.where(visible, S, -np.inf)
    return softmax_attend(S, V)


def attention(q, k, v):
    """q [B, L, h_q, d_h], k/v [B, L, h_kv, d_h] -> O [B, L, h_q, d_h] and
    LSE [B, h_q, L] (natural-log sum of exp of the scaled, masked scores)."""
    B, L, hq, dh = q.shape
    G = hq // k.shape[2]
    O = np.empty_like(q)
    LSE = np.empty((B, hq, L))
    pos = np.arange(L)
    for b in range(B):
        for j in range(hq):
            g = j // G
            O[b, :, j, :], LSE[b, j, :] = causal_attention(
                q[b, :, j, :], pos, k[b, :, g, :], v[b, :, g, :], dh)
    return O, LSE


def attention_backward(dO, q, k, v):
    """Gradients of ``attention`` w.r.t. q, k, v (textbook softmax adjoint).

    Per (b, q head j, kv head g = j // G): P = softmax(S) is recomputed,
    dV_g += P^T dO, dP = dO V^T, dS = P * (dP - rowsum(P * dP)),
    dQ = dS K / sqrt(d_h), dK_g += dS^T Q / sqrt(d_h).  The kv-head sums over
    the G q heads are the adjoint of repeat_interleave.
    """
    B, L, hq, dh = q.shape
    G = hq // k.shape[2]
    scale = 1.0 / np.sqrt(dh)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    visible = np.tril(np.ones((L, L), dtype=bool))
    for b in range(B):
        for j in range(hq):
            g = j // G
            Q, K, V = q[b, :, j, :], k[b, :, g, :], v[b, :, g, :]
            S = np.where(visible, (Q @ K.T) * scale, -np.inf)
            e = np.exp(S - np.max(S, axis=-1, keepdims=True))
            P = e / np.sum(e, axis=-1, keepdims=True)
            G_o = dO[b, :, j, :]
            dv[b, :, g, :] += P.T @ G_o
            dP = G_o @ V.T
            dS = P * (dP - np.sum(P * dP, axis=-1, keepdims=True))
            dq[b, :, j, :] = (dS @ K) * scale
            dk[b, :, g, :] += (dS.T @ Q) * scale
    return dq, dk, dv


# --------------------------------------------------------------------------
# SwiGLU MLP -- walkthrough page, Step 9: down(silu(gate(x)) * up(x)).
# --------------------------------------------------------------------------
def silu(z):
    return z / (1.0 + np.exp(-z))


def swiglu(g, u):
    return silu(g) * u


def swiglu_backward(df, g, u):
    """f = g * sigma(g) * u:  df/dg = u * sigma(g) * (1 + g (1 - sigma(g))),
    df/du = silu(g)."""
    s = 1.0 / (1.0 + np.exp(-g))
    return df * u * s * (1.0 + g * (1.0 - s)), df * g * s


# --------------------------------------------------------------------------
# The whole layer -- walkthrough page, Steps 1-10 ("Decoder Layer 的结构").
# --------------------------------------------------------------------------
def _f64(a):
    return np.asarray(a, dtype=np.float64)


def _heads(cfg):
    return cfg["h_q"], cfg["h_kv"], cfg["d_h"]


def layer_forward(cfg, p, x, keep=False):
    """Forward of one decoder layer on x [B, L, d].

    Returns a dict.  Normally {"y"}; with cfg["tp_partial"] (one tensor-
    parallel rank's share, the all-reduce replaced by the identity) it is
    {"attn_partial", "mlp_partial"} with h = x + attn_partial feeding the MLP.
    With keep=True every intermediate is included as well.
    """
    p = {k: _f64(v) for k, v in p.items()}
    x = _f64(x)
    B, L, _ = x.shape
    hq, hkv, dh = _heads(cfg)
    eps = cfg["eps"]
    # Step 1: input RMSNorm.
    xn, r1 = rmsnorm(x, p["in_norm"], eps)
    # Step 2: projections, viewed as heads.
    q0 = linear(xn, p["q"]).reshape(B, L, hq, dh)
    k0 = linear(xn, p["k"]).reshape(B, L, hkv, dh)
    v = linear(xn, p["v"]).reshape(B, L, hkv, dh)
    # Step 3: Qwen3 per-head q_norm / k_norm (shared [d_h] weights).
    if cfg.get("qk_norm", True):
        qn, rq = rmsnorm(q0, p["q_norm"], eps)
        kn, rk = rmsnorm(k0, p["k_norm"], eps)
    else:
        qn, rq, kn, rk = q0, None, k0, None
    # Step 4: RoPE.
    cos, sin = rope_cos_sin(L, dh, cfg["rope_theta"])
    qr, kr = rope(qn, cos, sin), rope(kn, cos, sin)
    # Step 5: causal GQA attention.
    O, LSE = attention(qr, kr, v)
    O2 = O.reshape(B, L, hq * dh)
    # Steps 6-7: o_proj and residual.
    a = linear(O2, p["o"])
    h = x + a
    # Step 8: post-attention RMSNorm.
    hn, r2 = rmsnorm(h, p["post_norm"], eps)
    # Step 9: SwiGLU MLP.
    g = linear(hn, p["gate"])
    u = linear(hn, p["up"])
    f = swiglu(g, u)
    m = linear(f, p["down"])
    # Step 10: residual.
    out = {}
    if cfg.get("tp_partial", False):
        out["attn_partial"] = a
        out["mlp_partial"] = m
    else:
        out["y"] = h + m
    if keep:
        out.update(dict(x=x, xn=xn, r1=r1, q0=q0, k0=k0, v=v, qn=qn, kn=kn,
                        rq=rq, rk=rk, cos=cos, sin=sin, qr=qr, kr=kr, O=O,
                        LSE=LSE, a=a, h=h, hn=hn, r2=r2, g=g, u=u, f=f, m=m))
    return out


def layer_backward(cfg, p, x, dy):
    """Gradients of sum(y * dy) w.r.t. x and the eleven parameters.

    The walkthrough page's backward runs "each operator's backward in reverse
    order, locally"; this is the chain rule through Steps 10 -> 1.  Weight
    gradients are summed over every token of the batch.  Returns
    (dx, grads) with grads keyed by parameter name.
    """
    assert not cfg.get("tp_partial", False)
    c = layer_forward(cfg, p, x, keep=True)
    p = {k: _f64(v) for k, v in p.items()}
    dy = _f64(dy)
    B, L, d = dy.shape
    hq, hkv, d_h = _heads(cfg)
    grads = {}
    # Step 10 residual: dy reaches both h and the MLP output.
    # Step 9: down, SwiGLU, gate/up.
    df, grads["down"] = linear_backward(dy, c["f"], p["down"])
    dg, du = swiglu_backward(df, c["g"], c["u"])
    dhn_g, grads["gate"] = linear_backward(dg, c["hn"], p["gate"])
    dhn_u, grads["up"] = linear_backward(du, c["hn"], p["up"])
    # Step 8: post-attention RMSNorm; Step 7: residual.
    dh_n, grads["post_norm"] = rmsnorm_backward(dhn_g + dhn_u, c["h"], c["r2"],
                                                p["post_norm"])
    d_hidden = dy + dh_n
    # Step 6: o_proj.
    dO2, grads["o"] = linear_backward(d_hidden, c["O"].reshape(B, L, hq * d_h),
                                      p["o"])
    # Step 5: attention.
    dqr, dkr, dv = attention_backward(dO2.reshape(B, L, hq, d_h), c["qr"],
                                      c["kr"], c["v"])
    # Step 4: RoPE.
    dqn = rope_backward(dqr, c["cos"], c["sin"])
    dkn = rope_backward(dkr, c["cos"], c["sin"])
    # Step 3: q/k norm.
    if cfg.get("qk_norm", True):
        dq0, grads["q_norm"] = rmsnorm_backward(dqn, c["q0"], c["rq"],
                                                p["q_norm"])
        dk0, grads["k_norm"] = rmsnorm_backward(dkn, c["k0"], c["rk"],
                                                p["k_norm"])
    else:
        dq0, dk0 = dqn, dkn
        grads["q_norm"] = np.zeros(d_h)
        grads["k_norm"] = np.zeros(d_h)
    # Step 2: projections.
    dxn_q, grads["q"] = linear_backward(dq0.reshape(B, L, hq * d_h), c["xn"],
                                        p["q"])
    dxn_k, grads["k"] = linear_backward(dk0.reshape(B, L, hkv * d_h), c["xn"],
                                        p["k"])
    dxn_v, grads["v"] = linear_backward(dv.reshape(B, L, hkv * d_h), c["xn"],
                                        p["v"])
    # Step 1: input RMSNorm, plus the attention residual.
    dx_n, grads["in_norm"] = rmsnorm_backward(dxn_q + dxn_k + dxn_v, c["x"],
                                              c["r1"], p["in_norm"])
    return d_hidden + dx_n, grads


def layer_forward_rows(cfg, p, x_seq, rows):
    """Forward outputs of ONE sequence x_seq [L, d] at token positions `rows`.

    The same Steps 1-10 as ``layer_forward``, evaluated only where needed:
    position t reads keys/values of positions 0..t, so k and v are computed
    for positions 0..max(rows) and everything else for `rows` alone.  Used to
    check full-size outputs on a sample of tokens.  Returns a dict with the
    same keys as ``layer_forward`` (rows in the given order).
    """
    p = {k: _f64(v) for k, v in p.items()}
    rows = np.asarray(rows)
    hq, hkv, dh = _heads(cfg)
    eps = cfg["eps"]
    G = hq // hkv
    last = int(rows.max()) + 1
    xs = _f64(x_seq[:last])
    xn, _ = rmsnorm(xs, p["in_norm"], eps)
    k0 = linear(xn, p["k"]).reshape(1, last, hkv, dh)
    v = linear(xn, p["v"]).reshape(1, last, hkv, dh)
    q0 = linear(xn[rows], p["q"]).reshape(1, len(rows), hq, dh)
    if cfg.get("qk_norm", True):
        q0, _ = rmsnorm(q0, p["q_norm"], eps)
        k0, _ = rmsnorm(k0, p["k_norm"], eps)
    cos, sin = rope_cos_sin(last, dh, cfg["rope_theta"])
    kr = rope(k0, cos, sin)[0]
    qr = rope(q0, cos[rows], sin[rows])[0]
    O = np.empty((len(rows), hq, dh))
    for j in range(hq):
        O[:, j, :], _ = causal_attention(qr[:, j, :], rows, kr[:, j // G, :],
                                         v[0, :, j // G, :], dh)
    a = linear(O.reshape(len(rows), hq * dh), p["o"])
    h = xs[rows] + a
    hn, _ = rmsnorm(h, p["post_norm"], eps)
    m = linear(swiglu(linear(hn, p["gate"]), linear(hn, p["up"])), p["down"])
    if cfg.get("tp_partial", False):
        return {"attn_partial": a, "mlp_partial": m}
    return {"y": h + m}
