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
