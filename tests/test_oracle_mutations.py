"""Plant plausible mistakes in the oracle (on the CPU) and check that at least
one pin catches each: evidence that the pins constrain every part of it."""
import numpy as np
import pytest

import oracle
import oracle.layer as L
import test_oracle_math as M
import test_oracle_pins as P


def _no_eps_rmsnorm(x, w, eps):
    return L.__dict__["_orig_rmsnorm"](x, w, 0.0)


def _sum_rmsnorm(x, w, eps):
    r = 1.0 / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)
    return x * r * w, r[..., 0]


def _mod_gqa_attention(q, k, v):
    B, Lq, hq, dh = q.shape
    hkv = k.shape[2]
    O = np.empty_like(q)
    LSE = np.empty((B, hq, Lq))
    pos = np.arange(Lq)
    for b in range(B):
        for j in range(hq):
            O[b, :, j], LSE[b, j] = L.causal_attention(
                q[b, :, j], pos, k[b, :, j % hkv], v[b, :, j % hkv], dh)
    return O, LSE


def _strict_causal(q_rows, q_pos, K, V, d_h):
    S = (q_rows @ K.T) / np.sqrt(d_h)
    vis = np.arange(K.shape[0])[None, :] <= np.asarray(q_pos)[:, None] - 1
    vis[:, 0] = True
    return L.softmax_attend(np.where(vis, S, -np.inf), V)


def _wrong_scale(q_rows, q_pos, K, V, d_h):
    S = (q_rows @ K.T) / d_h
    vis = np.arange(K.shape[0])[None, :] <= np.asarray(q_pos)[:, None]
    return L.softmax_attend(np.where(vis, S, -np.inf), V)


def _swiglu_bwd_dropped_term(df, g, u):
    s = 1.0 / (1.0 + np.exp(-g))
    return df * u * s, df * g * s


def _linear_bwd_transposed(dy, x, W):
    dx = dy @ W
    dW = x.reshape(-1, x.shape[-1]).T @ dy.reshape(-1, dy.shape[-1])
    return dx, dW


def _rope_bwd_not_adjoint(g, cos, sin):
    return L.rope(g, cos, sin)


def _rmsnorm_bwd_no_mean(dy, x, r, w):
    r = r[..., None]
    dx = r * dy * w
    dw = np.sum((dy * x * r).reshape(-1, x.shape[-1]), axis=0)
    return dx, dw


def _attn_bwd_no_D(dO, q, k, v):
    B, Lq, hq, dh = q.shape
    G = hq // k.shape[2]
    sc = 1.0 / np.sqrt(dh)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    vis = np.tril(np.ones((Lq, Lq), dtype=bool))
    for b in range(B):
        for j in range(hq):
            g = j // G
            Q, K, V = q[b, :, j], k[b, :, g], v[b, :, g]
            S = np.where(vis, Q @ K.T * sc, -np.inf)
            P = np.exp(S - S.max(-1, keepdims=True))
            P /= P.sum(-1, keepdims=True)
            dv[b, :, g] += P.T @ dO[b, :, j]
            dS = P * (dO[b, :, j] @ V.T)
            dq[b, :, j] = dS @ K * sc
            dk[b, :, g] += dS.T @ Q * sc
    return dq, dk, dv


def _rope_wrong_pairs(u, cos, sin):
    # adjacent-pair (interleaved) rotation with the SAME angle table but the
    # imaginary part negated: a wrong sign as well as a different pairing.
    a, b = u[..., 0::2], u[..., 1::2]
    c, s = cos[None, :, None, :], sin[None, :, None, :]
    out = np.empty_like(u)
    out[..., 0::2] = a * c + b * s
    out[..., 1::2] = b * c + a * s
    return out


MUTATIONS = [
    ("rmsnorm", _sum_rmsnorm, M.test_rmsnorm_closed_form_constant_vector),
    ("rmsnorm", _no_eps_rmsnorm, M.test_rmsnorm_closed_form_constant_vector),
    ("attention", _mod_gqa_attention,
     M.test_gqa_equals_mha_with_repeat_interleave),
    ("causal_attention", _strict_causal, M.test_attention_brute_force),
    ("causal_attention", _wrong_scale, M.test_attention_brute_force),
    ("swiglu_backward", _swiglu_bwd_dropped_term,
     lambda: M.test_backward_finite_differences_tiny(True)),
    ("linear_backward", _linear_bwd_transposed,
     P.test_tp_toy_linear_conventions),
    ("rope_backward", _rope_bwd_not_adjoint, M.test_rope_properties),
    ("rmsnorm_backward", _rmsnorm_bwd_no_mean,
     lambda: M.test_backward_finite_differences_tiny(True)),
    ("attention_backward", _attn_bwd_no_D,
     lambda: M.test_backward_finite_differences_tiny(False)),
    ("rope", _rope_wrong_pairs, M.test_rope_properties),
]


@pytest.mark.parametrize("name,bad,check", MUTATIONS,
                         ids=[f"{m[0]}:{m[1].__name__}" for m in MUTATIONS])
def test_planted_mistake_is_caught(monkeypatch, name, bad, check):
    monkeypatch.setitem(L.__dict__, "_orig_rmsnorm", L.rmsnorm)
    monkeypatch.setattr(L, name, bad)
    if hasattr(oracle, name):
        monkeypatch.setattr(oracle, name, bad)
    with pytest.raises((AssertionError, ValueError, FloatingPointError)):
        with np.errstate(all="ignore"):
            check()
