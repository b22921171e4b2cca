"""Attention over a block of keys, exporting the unnormalised state (m, l,
acc), and the merge of such states (the parallelism page, section 4.2, ring
attention), through the C ABI against the oracle's attention_block_state /
merge_block_states and the whole-sequence attention."""
import json
import os

import numpy as np
import pytest

import oracle
import qwen3_decoder_layer_amd as q3
from gpu_helpers import TOL, Guarded, assert_close, dev, host, need_gpu, say
import synth

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _f32():
    import torch
    return torch.float32


def _state(dtype, q, k, v, hq, hkv, dh, k0, k1):
    B, L = q.shape[0], q.shape[1]
    m, l = Guarded((B, hq, L), _f32()), Guarded((B, hq, L), _f32())
    acc = Guarded((B, L, hq * dh), _f32())
    q3.attention_fwd_block(q, k, v, hq, hkv, dh, k0, k1, m=m.t, l=l.t, acc=acc.t)
    for g, n in ((m, "m"), (l, "l"), (acc, "acc")):
        assert g.guards_intact(), n
    assert not bool(np.isnan(host(m.t)).any()) and bool(np.isfinite(host(l.t)).all())
    assert bool(np.isfinite(host(acc.t)).all())
    return m.t, l.t, acc.t


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_page_example_through_the_kernel(dtype):
    """One head, keys scoring [1, 0 | 2, 0] for the query at position 3:
    merged, the printed output (1.000, 0.693) with l = 1.639."""
    need_gpu()
    say(f"block attention, page example {dtype}")
    fx = json.load(open(os.path.join(GOLDEN, "online_softmax_example.json")))
    scores = np.array(fx["scores_blocks"][0] + fx["scores_blocks"][1], dtype=np.float32)
    L, dh = 4, 64
    q = np.zeros((1, L, dh), np.float32); q[0, :, 0] = 8.0
    k = np.zeros((1, L, dh), np.float32); k[0, :, 0] = scores
    v = np.zeros((1, L, dh), np.float32); v[0, :, :2] = np.array(fx["values"])
    gq, gk, gv = dev(q, dtype), dev(k, dtype), dev(v, dtype)
    a = _state(dtype, gq, gk, gv, 1, 1, dh, 0, 2)
    b = _state(dtype, gq, gk, gv, 1, 1, dh, 2, 4)
    assert host(a[0])[0, 0, 3] == pytest.approx(1.0, abs=1e-6)
    assert host(b[0])[0, 0, 3] == pytest.approx(2.0, abs=1e-6)
    assert host(b[0])[0, 0, 0] == -np.inf and host(b[1])[0, 0, 0] == 0.0
    q3.attention_merge(a, b)
    o, lse = q3.attention_finish(a, dtype=dtype)
    # bf16: the probabilities are rounded to bf16 before the product with V
    # (relative 2^-9); fp32: the page's print precision.
    tol = 2e-3 if dtype == "bf16" else fx["print_precision"]
    assert np.allclose(host(o)[0, 3, :2], fx["printed"]["output"], atol=tol)
    assert host(a[1])[0, 0, 3] == pytest.approx(fx["printed"]["merged_l"],
                                                abs=fx["print_precision"])
    assert host(a[0])[0, 0, 3] == pytest.approx(2.0, abs=1e-6)


CASES = [
    # B, L, h_q, h_kv, d_h, key-block cuts (ragged, not tile-aligned)
    (2, 200, 8, 2, 128, [0, 37, 128, 200]),
    (1, 131, 4, 2, 64, [0, 64, 65, 131]),
    (1, 300, 3, 1, 64, [0, 150, 300]),
]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("B,L,hq,hkv,dh,cuts", CASES)
def test_block_states_and_merge(dtype, B, L, hq, hkv, dh, cuts):
    need_gpu()
    say(f"block attention {dtype} B={B} L={L} hq={hq} hkv={hkv} dh={dh} cuts={cuts}")
    rng = np.random.default_rng(L + hq)

    def r(shape):
        a = rng.standard_normal(shape).astype(np.float32)
        return synth.bf16_round(a) if dtype == "bf16" else a
    q, k, v = r((B, L, hq, dh)), r((B, L, hkv, dh)), r((B, L, hkv, dh))
    q64, k64, v64 = (t.astype(np.float64) for t in (q, k, v))
    gq, gk, gv = (dev(t.reshape(B, L, -1), dtype) for t in (q, k, v))
    states = []
    for k0, k1 in zip(cuts, cuts[1:]):
        st = _state(dtype, gq, gk, gv, hq, hkv, dh, k0, k1)
        m_ref, l_ref, acc_ref = oracle.attention_block_state(q64, k64, v64, k0, k1)
        m, l, acc = (host(t) for t in st)
        empty = m_ref == -np.inf
        assert np.array_equal(m == -np.inf, empty), (k0, k1)
        assert not l[empty].any()
        assert not acc.reshape(B, L, hq, dh).transpose(0, 2, 1, 3)[empty].any()
        assert np.max(np.abs(m[~empty] - m_ref[~empty])) <= 1e-3 * max(1.0, np.max(np.abs(m_ref[~empty])))
        assert_close("l", l[~empty], l_ref[~empty], TOL[dtype], row_len=1)
        assert_close("acc", acc.reshape(B, L, hq, dh), acc_ref, TOL[dtype])
        states.append(st)
    O_ref, lse_ref = oracle.attention(q64, k64, v64)
    o_full, lse_full = q3.attention_fwd(gq, gk, gv, hq, hkv, dh)
    for order in (states, states[::-1]):
        st = tuple(t.clone() for t in order[0])
        for other in order[1:]:
            q3.attention_merge(st, other)
        o, lse = q3.attention_finish(st, dtype=dtype)
        assert_close("o", host(o), O_ref.reshape(B, L, -1), TOL[dtype])
        assert np.max(np.abs(host(lse) - lse_ref)) <= 1e-3 * max(1.0, np.max(np.abs(lse_ref)))
        # against the whole-sequence kernel on the same inputs
        assert_close("o_vs_fwd", host(o), host(o_full), TOL[dtype])
