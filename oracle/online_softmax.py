"""Block-wise (online) softmax state and its merge rule.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The state-placement page (section 4.2, ring attention) keeps, for one query
and one block of keys, three quantities: the block's largest score m, the
denominator part l = sum exp(s_k - m) and the numerator part
acc = sum exp(s_k - m) v_k.  Two states are merged by rescaling each one's
l and acc by exp(m_i - m_new), m_new = max(m_1, m_2), and adding.  The final
output is acc / l and log-sum-exp is m + log l.  Flash attention's tile loop
is the same merge applied tile by tile.
"""
from __future__ import annotations

import numpy as np


def block_state(scores, V):
    """(m, l, acc) of one block: scores [n], V [n, dv]."""
    s = np.asarray(scores, dtype=np.float64)
    m = float(np.max(s))
    w = np.exp(s - m)
    return m, float(np.sum(w)), w @ np.asarray(V, dtype=np.float64)


def merge_states(a, b):
    ma, la, acca = a
    mb, lb, accb = b
    m = max(ma, mb)
    fa, fb = np.exp(ma - m), np.exp(mb - m)
    return m, la * fa + lb * fb, acca * fa + accb * fb


def finish_state(st):
    """(output, log-sum-exp) of a (merged) state."""
    m, l, acc = st
    return acc / l, m + np.log(l)


def attention_block_state(q, k, v, k0, k1):
    """The state (m, l, acc) of causal GQA attention restricted to the keys
    s in [k0, k1), for every query: q [B, L, h_q, d_h], k/v [B, L, h_kv,
    d_h]; key s is visible to query t iff k0 <= s < k1 and s <= t (the
    causal rule of the walkthrough page's Step 5), q head j reads kv head
    j // (h_q / h_kv), scores are q.k / sqrt(d_h).  m is the largest visible
    score, l = sum exp(score - m), acc = sum exp(score - m) v.  A query with
    no visible key gets (-inf, 0, 0).  Returns m, l [B, h_q, L] and acc
    [B, L, h_q, d_h]."""
    B, L, hq, dh = q.shape
    G = hq // k.shape[2]
    m = np.full((B, hq, L), -np.inf)
    l = np.zeros((B, hq, L))
    acc = np.zeros((B, L, hq, dh))
    s_idx = np.arange(L)[None, :]
    t_idx = np.arange(L)[:, None]
    visible = (s_idx >= k0) & (s_idx < k1) & (s_idx <= t_idx)
    for b in range(B):
        for j in range(hq):
            g = j // G
            S = (q[b, :, j, :] @ k[b, :, g, :].T) / np.sqrt(dh)
            S = np.where(visible, S, -np.inf)
            rows = visible.any(axis=1)
            mb = np.where(rows, S.max(axis=1), -np.inf)
            w = np.where(visible, np.exp(S - np.where(rows, mb, 0.0)[:, None]), 0.0)
            m[b, j] = mb
            l[b, j] = w.sum(axis=1)
            acc[b, :, j, :] = w @ v[b, :, g, :]
    return m, l, acc


def merge_block_states(a, b):
    """``merge_states`` applied to every query of two attention_block_state
    results (a (-inf, 0, 0) state drops out)."""
    ma, la, acca = a
    mb, lb, accb = b
    mn = np.maximum(ma, mb)
    with np.errstate(invalid="ignore"):
        fa = np.where(ma == -np.inf, 0.0, np.exp(ma - mn))
        fb = np.where(mb == -np.inf, 0.0, np.exp(mb - mn))
    fa_t = np.transpose(fa, (0, 2, 1))[..., None]
    fb_t = np.transpose(fb, (0, 2, 1))[..., None]
    return mn, la * fa + lb * fb, acca * fa_t + accb * fb_t
