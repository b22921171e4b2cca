"""Per-step parity of the HIP kernels against the fp64 oracle, through the
C ABI's phase-level entry points, at sizes with several tiles and ragged
tails."""
import numpy as np
import pytest

import oracle
import qwen3_decoder_layer_amd as q3
from gpu_helpers import TOL, dev, host, need_gpu, rel_err, say
import synth

pytestmark = pytest.mark.gpu


def _rand(rng, shape, scale=1.0, dtype="bf16"):
    a = (rng.standard_normal(shape) * scale).astype(np.float32)
    return synth.bf16_round(a) if dtype == "bf16" else a


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("rows,n", [(37, 520), (1000, 4096), (5, 8192)])
def test_rmsnorm_fwd(dtype, rows, n):
    need_gpu()
    say(f"rmsnorm_fwd {dtype} rows={rows} n={n}")
    rng = np.random.default_rng(rows + n)
    x = _rand(rng, (rows, n), 1.0, dtype)
    w = (1.0 + rng.standard_normal(n) * 0.1).astype(np.float32)
    if dtype == "bf16":
        w = synth.bf16_round(w)
    y, rstd = q3.rmsnorm_fwd(dev(x, dtype), dev(w, dtype), 1e-6)
    ref, rref = oracle.rmsnorm(x.astype(np.float64), w.astype(np.float64), 1e-6)
    assert rel_err(host(y), ref) <= TOL[dtype]
    assert rel_err(host(rstd), rref) <= 1e-5


# The last two select 192-row tiles for the forward product (2 rounds of
# 192 x 256 tiles beat 1.5 rounds of 256 x 256), one of them ragged.
LIN_SHAPES = [(300, 264, 136), (4100, 4096, 520), (64, 1024, 4096), (6144, 4096, 64),
              (6100, 4040, 72)]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("M,N,K", LIN_SHAPES)
def test_linear_fwd_dgrad_wgrad(dtype, M, N, K):
    need_gpu()
    if dtype == "f32" and M * N * K > 2e8:
        pytest.skip("fp32 correctness path is for small shapes")
    say(f"linear {dtype} M={M} N={N} K={K}")
    rng = np.random.default_rng(M + N + K)
    a = _rand(rng, (M, K), 1.0, dtype)
    w = _rand(rng, (N, K), 0.02, dtype)
    r = _rand(rng, (M, N), 1.0, dtype)
    dy = _rand(rng, (M, N), 1.0, dtype)
    a64, w64 = a.astype(np.float64), w.astype(np.float64)
    y = q3.linear_fwd(dev(a, dtype), dev(w, dtype))
    assert rel_err(host(y), oracle.linear(a64, w64)) <= TOL[dtype]
    y2 = q3.linear_fwd(dev(a, dtype), dev(w, dtype), resid=dev(r, dtype))
    assert rel_err(host(y2), r + oracle.linear(a64, w64)) <= TOL[dtype]
    da_ref, dw_ref = oracle.linear_backward(dy.astype(np.float64), a64, w64)
    da = q3.linear_dgrad(dev(dy, dtype), dev(w, dtype))
    assert rel_err(host(da), da_ref) <= TOL[dtype]
    dw = q3.linear_wgrad(dev(dy, dtype), dev(a, dtype))
    assert rel_err(host(dw), dw_ref) <= TOL[dtype]
    # accumulate adds into the existing fp32 buffer
    q3.linear_wgrad(dev(dy, dtype), dev(a, dtype), dw=dw, accumulate=True)
    assert rel_err(host(dw), 2 * dw_ref) <= TOL[dtype]


ATTN_CASES = [
    # B, L, h_q, h_kv, d_h
    (2, 200, 8, 2, 128),     # GQA 4:1, ragged L
    (1, 131, 4, 2, 64),      # GQA 2:1
    (1, 96, 2, 2, 64),       # MHA
    (1, 77, 8, 1, 128),      # GQA 8:1
    (2, 1, 4, 2, 128),       # single token
    (1, 300, 3, 1, 64),      # G = 3
]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("B,L,hq,hkv,dh", ATTN_CASES)
def test_attention_fwd_bwd(dtype, B, L, hq, hkv, dh):
    need_gpu()
    say(f"attention {dtype} B={B} L={L} hq={hq} hkv={hkv} dh={dh}")
    rng = np.random.default_rng(B * 1000 + L + hq + dh)
    q = _rand(rng, (B, L, hq, dh), 1.0, dtype)
    k = _rand(rng, (B, L, hkv, dh), 1.0, dtype)
    v = _rand(rng, (B, L, hkv, dh), 1.0, dtype)
    do = _rand(rng, (B, L, hq, dh), 1.0, dtype)
    q64, k64, v64 = (t.astype(np.float64) for t in (q, k, v))
    O_ref, lse_ref = oracle.attention(q64, k64, v64)
    gq = dev(q.reshape(B, L, hq * dh), dtype)
    gk = dev(k.reshape(B, L, hkv * dh), dtype)
    gv = dev(v.reshape(B, L, hkv * dh), dtype)
    o, lse = q3.attention_fwd(gq, gk, gv, hq, hkv, dh)
    assert rel_err(host(o).reshape(O_ref.shape), O_ref) <= TOL[dtype]
    assert np.max(np.abs(host(lse) - lse_ref)) <= 1e-3 * max(1.0, np.max(np.abs(lse_ref)))
    dq_ref, dk_ref, dv_ref = oracle.attention_backward(do.astype(np.float64), q64, k64, v64)
    dq, dk, dv = q3.attention_bwd(gq, gk, gv, o, dev(do.reshape(B, L, hq * dh), dtype),
                                  lse, hq, hkv, dh)
    assert rel_err(host(dq).reshape(dq_ref.shape), dq_ref) <= TOL[dtype]
    assert rel_err(host(dk).reshape(dk_ref.shape), dk_ref) <= TOL[dtype]
    assert rel_err(host(dv).reshape(dv_ref.shape), dv_ref) <= TOL[dtype]


def test_attention_strided_views():
    """q/k/v read from column slices of one [T, q+k+v] buffer (the layer's
    layout)."""
    need_gpu()
    import torch
    say("attention strided views")
    B, L, hq, hkv, dh = 2, 150, 8, 2, 128
    rng = np.random.default_rng(5)
    qkv = _rand(rng, (B, L, (hq + 2 * hkv) * dh), 1.0)
    g = dev(qkv, "bf16")
    qd, kvd = hq * dh, hkv * dh
    o, lse = q3.attention_fwd(g[..., :qd], g[..., qd:qd + kvd], g[..., qd + kvd:], hq, hkv, dh)
    qq = qkv[..., :qd].reshape(B, L, hq, dh).astype(np.float64)
    kk = qkv[..., qd:qd + kvd].reshape(B, L, hkv, dh).astype(np.float64)
    vv = qkv[..., qd + kvd:].reshape(B, L, hkv, dh).astype(np.float64)
    O_ref, _ = oracle.attention(qq, kk, vv)
    assert rel_err(host(o).reshape(O_ref.shape), O_ref) <= TOL["bf16"]
    torch.cuda.synchronize()


# Logits whose scale grows along the sequence: the log-sum-exp of the last
# rows reaches 55-75 in log2 units, against under 10 for the first. The
# kernels' running maximum then moves many times within a row and the partial
# output and row sum are rescaled each time (the block-state merge of the
# online softmax, state-placement page, section 4.2); the result must still be
# the one-pass softmax of the oracle. A CPU emulation of the kernels' bf16
# roundings on these inputs stays within 5e-3 of the oracle.
GROWING = [
    # q scale, growth of the key scale from the first to the last position
    (1.0, 10.0),
    (3.0, 4.0),
]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("qs,kgrow", GROWING, ids=["keys-growing", "sharp-growing"])
def test_attention_growing_logits(dtype, qs, kgrow):
    need_gpu()
    B, L, hq, hkv, dh = 1, 400, 4, 2, 128
    say(f"attention growing logits {dtype} qs={qs} kgrow={kgrow} B={B} L={L}")
    rng = np.random.default_rng(11)
    ramp = (1.0 + kgrow * np.arange(L) / L)[None, :, None, None]
    q = _rand(rng, (B, L, hq, dh), qs, dtype)
    k = (rng.standard_normal((B, L, hkv, dh)) * ramp).astype(np.float32)
    k = synth.bf16_round(k) if dtype == "bf16" else k
    v = _rand(rng, (B, L, hkv, dh), 1.0, dtype)
    do = _rand(rng, (B, L, hq, dh), 1.0, dtype)
    q64, k64, v64 = (t.astype(np.float64) for t in (q, k, v))
    O_ref, lse_ref = oracle.attention(q64, k64, v64)
    # The inputs must reach the regime this test is for.
    assert np.max(lse_ref) * np.log2(np.e) > 50.0
    gq = dev(q.reshape(B, L, hq * dh), dtype)
    gk = dev(k.reshape(B, L, hkv * dh), dtype)
    gv = dev(v.reshape(B, L, hkv * dh), dtype)
    o, lse = q3.attention_fwd(gq, gk, gv, hq, hkv, dh)
    assert rel_err(host(o).reshape(O_ref.shape), O_ref) <= TOL[dtype]
    assert np.max(np.abs(host(lse) - lse_ref)) <= 1e-3 * max(1.0, np.max(np.abs(lse_ref)))
    dq_ref, dk_ref, dv_ref = oracle.attention_backward(do.astype(np.float64), q64, k64, v64)
    dq, dk, dv = q3.attention_bwd(gq, gk, gv, o, dev(do.reshape(B, L, hq * dh), dtype),
                                  lse, hq, hkv, dh)
    assert rel_err(host(dq).reshape(dq_ref.shape), dq_ref) <= TOL[dtype]
    assert rel_err(host(dk).reshape(dk_ref.shape), dk_ref) <= TOL[dtype]
    assert rel_err(host(dv).reshape(dv_ref.shape), dv_ref) <= TOL[dtype]
