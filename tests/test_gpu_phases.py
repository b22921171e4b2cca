"""Per-step parity of the HIP kernels against the fp64 oracle, through the
C ABI's phase-level entry points, at sizes with several tiles and ragged
tails.  Every output is a NaN-poisoned buffer between guard bands: each
element must be written, nothing outside it may be, and the result must meet
both the tensor-wide and the row-local bar."""
import numpy as np
import pytest

import oracle
import qwen3_decoder_layer_amd as q3
from gpu_helpers import TOL, Guarded, assert_close, dev, host, local_err, need_gpu, say
import synth

pytestmark = pytest.mark.gpu


def _rand(rng, shape, scale=1.0, dtype="bf16"):
    a = (rng.standard_normal(shape) * scale).astype(np.float32)
    return synth.bf16_round(a) if dtype == "bf16" else a


def _td(dtype):
    import torch
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def _f32():
    import torch
    return torch.float32


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
    y, rstd = Guarded((rows, n), _td(dtype)), Guarded((rows,), _f32())
    q3.rmsnorm_fwd(dev(x, dtype), dev(w, dtype), 1e-6, y=y.t, rstd=rstd.t)
    y.check("y"), rstd.check("rstd")
    ref, rref = oracle.rmsnorm(x.astype(np.float64), w.astype(np.float64), 1e-6)
    assert_close("y", host(y.t), ref, TOL[dtype])
    assert_close("rstd", host(rstd.t), rref, 1e-5, row_len=rows)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("rows,n,resid", [(37, 520, True), (1000, 4096, False),
                                          (5, 8192, True), (4099, 2560, True)])
def test_rmsnorm_bwd(dtype, rows, n, resid):
    """RMSNorm adjoint (walkthrough page, backward of Steps 1 and 8): dx with
    the residual gradient added, and the weight gradient summed over rows."""
    need_gpu()
    import torch
    say(f"rmsnorm_bwd {dtype} rows={rows} n={n} resid={resid}")
    rng = np.random.default_rng(rows * 7 + n)
    x = _rand(rng, (rows, n), 1.0, dtype)
    dy = _rand(rng, (rows, n), 1.0, dtype)
    r = _rand(rng, (rows, n), 1.0, dtype)
    w = (1.0 + rng.standard_normal(n) * 0.1).astype(np.float32)
    if dtype == "bf16":
        w = synth.bf16_round(w)
    x64, w64 = x.astype(np.float64), w.astype(np.float64)
    _, r_ref = oracle.rmsnorm(x64, w64, 1e-6)
    # The forward's rstd, as the layer's saved block holds it (fp32).
    rstd = dev(r_ref.astype(np.float32), "f32")
    dx_ref, dw_ref = oracle.rmsnorm_backward(dy.astype(np.float64), x64, r_ref, w64)
    if resid:
        dx_ref = dx_ref + r
    dx, dw = Guarded((rows, n), _td(dtype)), Guarded((n,), _f32())
    q3.rmsnorm_bwd(dev(dy, dtype), dev(x, dtype), rstd, dev(w, dtype),
                   resid=dev(r, dtype) if resid else None, dx=dx.t, dw=dw.t)
    dx.check("dx"), dw.check("dw")
    assert_close("dx", host(dx.t), dx_ref, TOL[dtype])
    assert_close("dw", host(dw.t), dw_ref, TOL[dtype])
    # accumulate adds into dw
    before = dw.t.clone()
    q3.rmsnorm_bwd(dev(dy, dtype), dev(x, dtype), rstd, dev(w, dtype), dx=dx.t, dw=dw.t,
                   accumulate=True)
    torch.cuda.synchronize()
    assert_close("dw2", host(dw.t), 2 * host(before), 1e-6)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("B,L,hq,hkv,dh,qk_norm", [
    (2, 77, 8, 2, 128, True), (1, 131, 4, 4, 64, True), (3, 5, 6, 2, 64, False)])
def test_qknorm_rope_fwd_bwd(dtype, B, L, hq, hkv, dh, qk_norm):
    """Walkthrough page Steps 3-4 (per-head q_norm / k_norm, then RoPE) and
    their adjoint, against the oracle's rmsnorm / rope / rope_backward."""
    need_gpu()
    say(f"qknorm_rope {dtype} B={B} L={L} hq={hq} hkv={hkv} dh={dh} qk_norm={qk_norm}")
    rng = np.random.default_rng(B * 100 + L + dh)
    W = (hq + hkv) * dh
    qk = _rand(rng, (B, L, W), 1.0, dtype)
    g = _rand(rng, (B, L, W), 1.0, dtype)
    wq = (1.0 + rng.standard_normal(dh) * 0.1).astype(np.float32)
    wk = (1.0 + rng.standard_normal(dh) * 0.1).astype(np.float32)
    if dtype == "bf16":
        wq, wk = synth.bf16_round(wq), synth.bf16_round(wk)
    theta = 1e6
    cos_g, sin_g = q3.rope_table(L, dh, theta)
    cos, sin = oracle.rope_cos_sin(L, dh, theta)
    assert_close("cos", host(cos_g), cos, 1e-6)
    assert_close("sin", host(sin_g), sin, 1e-6)
    q64 = qk[..., :hq * dh].reshape(B, L, hq, dh).astype(np.float64)
    k64 = qk[..., hq * dh:].reshape(B, L, hkv, dh).astype(np.float64)
    if qk_norm:
        qn, rq = oracle.rmsnorm(q64, wq.astype(np.float64), 1e-6)
        kn, rk = oracle.rmsnorm(k64, wk.astype(np.float64), 1e-6)
    else:
        qn, kn, rq, rk = q64, k64, None, None
    ref = np.concatenate([oracle.rope(qn, cos, sin).reshape(B, L, -1),
                          oracle.rope(kn, cos, sin).reshape(B, L, -1)], axis=-1)
    out = Guarded((B, L, W), _td(dtype))
    rsq, rsk = Guarded((B * L, hq), _f32()), Guarded((B * L, hkv), _f32())
    gqk = dev(qk, dtype)
    gwq, gwk = dev(wq, dtype), dev(wk, dtype)
    q3.qknorm_rope_fwd(gqk, gwq, gwk, cos_g, sin_g, hq, hkv, dh, qk_norm=qk_norm,
                       out=out.t, rstd_q=rsq.t, rstd_k=rsk.t)
    out.check("out")
    assert_close("out", host(out.t), ref, TOL[dtype], row_len=dh)
    if qk_norm:
        rsq.check("rstd_q"), rsk.check("rstd_k")
        assert_close("rstd_q", host(rsq.t), rq.reshape(B * L, hq), 1e-5)
        assert_close("rstd_k", host(rsk.t), rk.reshape(B * L, hkv), 1e-5)
    # Backward: rotate g back, then the per-head RMSNorm adjoint.
    gq = g[..., :hq * dh].reshape(B, L, hq, dh).astype(np.float64)
    gk = g[..., hq * dh:].reshape(B, L, hkv, dh).astype(np.float64)
    dqn = oracle.rope_backward(gq, cos, sin)
    dkn = oracle.rope_backward(gk, cos, sin)
    if qk_norm:
        dq_ref, dwq_ref = oracle.rmsnorm_backward(dqn, q64, rq, wq.astype(np.float64))
        dk_ref, dwk_ref = oracle.rmsnorm_backward(dkn, k64, rk, wk.astype(np.float64))
    else:
        dq_ref, dk_ref = dqn, dkn
    dref = np.concatenate([dq_ref.reshape(B, L, -1), dk_ref.reshape(B, L, -1)], axis=-1)
    dout = Guarded((B, L, W), _td(dtype))
    dwq, dwk = Guarded((dh,), _f32()), Guarded((dh,), _f32())
    q3.qknorm_rope_bwd(dev(g, dtype), gqk if qk_norm else None, gwq, gwk,
                       rsq.t if qk_norm else None, rsk.t if qk_norm else None, cos_g, sin_g,
                       hq, hkv, dh, qk_norm=qk_norm, out=dout.t,
                       dwq=dwq.t if qk_norm else None, dwk=dwk.t if qk_norm else None)
    dout.check("dqk")
    assert_close("dqk", host(dout.t), dref, TOL[dtype], row_len=dh)
    if qk_norm:
        dwq.check("dwq"), dwk.check("dwk")
        assert_close("dwq", host(dwq.t), dwq_ref, TOL[dtype])
        assert_close("dwk", host(dwk.t), dwk_ref, TOL[dtype])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("M,N", [(300, 264), (4100, 1032), (1, 8)])
def test_swiglu_bwd(dtype, M, N):
    """SwiGLU adjoint (walkthrough page, Step 9)."""
    need_gpu()
    say(f"swiglu_bwd {dtype} M={M} N={N}")
    rng = np.random.default_rng(M + 3 * N)
    df = _rand(rng, (M, N), 1.0, dtype)
    gu = _rand(rng, (M, 2 * N), 2.0, dtype)
    dg_ref, du_ref = oracle.swiglu_backward(df.astype(np.float64),
                                            gu[:, :N].astype(np.float64),
                                            gu[:, N:].astype(np.float64))
    dgu = Guarded((M, 2 * N), _td(dtype))
    q3.swiglu_bwd(dev(df, dtype), dev(gu, dtype), dgu=dgu.t)
    dgu.check("dgu")
    out = host(dgu.t)
    assert_close("dg", out[:, :N], dg_ref, TOL[dtype])
    assert_close("du", out[:, N:], du_ref, TOL[dtype])


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
    ga, gw = dev(a, dtype), dev(w, dtype)
    y = Guarded((M, N), _td(dtype))
    q3.linear_fwd(ga, gw, y=y.t)
    y.check("y")
    assert_close("y", host(y.t), oracle.linear(a64, w64), TOL[dtype])
    y2 = Guarded((M, N), _td(dtype))
    q3.linear_fwd(ga, gw, resid=dev(r, dtype), y=y2.t)
    y2.check("y+r")
    assert_close("y+r", host(y2.t), r + oracle.linear(a64, w64), TOL[dtype])
    da_ref, dw_ref = oracle.linear_backward(dy.astype(np.float64), a64, w64)
    da = Guarded((M, K), _td(dtype))
    q3.linear_dgrad(dev(dy, dtype), gw, da=da.t)
    da.check("da")
    assert_close("da", host(da.t), da_ref, TOL[dtype])
    dw = Guarded((N, K), _f32())
    q3.linear_wgrad(dev(dy, dtype), ga, dw=dw.t)
    dw.check("dw")
    assert_close("dw", host(dw.t), dw_ref, TOL[dtype])
    # accumulate adds into the existing fp32 buffer
    q3.linear_wgrad(dev(dy, dtype), ga, dw=dw.t, accumulate=True)
    assert_close("dw2", host(dw.t), 2 * dw_ref, TOL[dtype])


ATTN_CASES = [
    # B, L, h_q, h_kv, d_h
    (2, 200, 8, 2, 128),     # GQA 4:1, ragged L
    (1, 131, 4, 2, 64),      # GQA 2:1
    (1, 96, 2, 2, 64),       # MHA
    (1, 77, 8, 1, 128),      # GQA 8:1
    (2, 1, 4, 2, 128),       # single token
    (1, 300, 3, 1, 64),      # G = 3
]


def _attn_check(dtype, q, k, v, do, o, lse, dq, dk, dv, local_dqk=True):
    """Oracle comparison of one attention forward + backward; row-local
    scales are per token (all heads of the token's row).  local_dqk=False
    holds dq and dk to the tensor-wide bar only (their row-local errors are
    printed)."""
    B, L, hq, dh = q.shape
    q64, k64, v64 = (t.astype(np.float64) for t in (q, k, v))
    O_ref, lse_ref = oracle.attention(q64, k64, v64)
    assert_close("o", host(o).reshape(B, L, -1), O_ref.reshape(B, L, -1), TOL[dtype])
    assert np.max(np.abs(host(lse) - lse_ref)) <= 1e-3 * max(1.0, np.max(np.abs(lse_ref)))
    dq_ref, dk_ref, dv_ref = oracle.attention_backward(do.astype(np.float64), q64, k64, v64)
    for name, a, ref in (("dq", dq, dq_ref), ("dk", dk, dk_ref), ("dv", dv, dv_ref)):
        a2, r2 = host(a).reshape(B, L, -1), ref.reshape(B, L, -1)
        loc = local_dqk or name == "dv"
        if not loc:
            print(f"{name}: local {local_err(a2, r2):.3e} (not asserted)", flush=True)
        assert_close(name, a2, r2, TOL[dtype], local=loc)


def _attn_run(dtype, q, k, v, do, stored_ds=True):
    """Attention forward + backward on guarded, poisoned outputs (bf16:
    the stored-dS form, or with stored_ds=False the recomputing one)."""
    B, L, hq, dh = q.shape
    hkv = k.shape[2]
    gq = dev(q.reshape(B, L, hq * dh), dtype)
    gk = dev(k.reshape(B, L, hkv * dh), dtype)
    gv = dev(v.reshape(B, L, hkv * dh), dtype)
    o, lse = Guarded((B, L, hq * dh), _td(dtype)), Guarded((B, hq, L), _f32())
    q3.attention_fwd(gq, gk, gv, hq, hkv, dh, o=o.t, lse=lse.t)
    o.check("o"), lse.check("lse")
    dq = Guarded((B, L, hq * dh), _td(dtype))
    dk, dv = Guarded((B, L, hkv * dh), _td(dtype)), Guarded((B, L, hkv * dh), _td(dtype))
    q3.attention_bwd(gq, gk, gv, o.t, dev(do.reshape(B, L, hq * dh), dtype), lse.t, hq, hkv,
                     dh, dq=dq.t, dk=dk.t, dv=dv.t, stored_ds=stored_ds)
    dq.check("dq"), dk.check("dk"), dv.check("dv")
    return o.t, lse.t, dq.t, dk.t, dv.t


def _same_bits(a, b, what):
    import torch
    assert torch.equal(a, b), f"{what}: the two backward forms differ"


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
    res = _attn_run(dtype, q, k, v, do)
    _attn_check(dtype, q, k, v, do, *res)
    if dtype == "bf16":
        # dQ from the stored dS and dQ from a recomputation: the same bits.
        alt = _attn_run(dtype, q, k, v, do, stored_ds=False)
        for name, a, b in zip(("dq", "dk", "dv"), res[2:], alt[2:]):
            _same_bits(a, b, name)


@pytest.mark.parametrize("B,L", [(2, 4096), (1, 11586)], ids=["qwen3-8b", "ds-past-4GiB"])
def test_attention_backward_forms_full_size(B, L):
    """The Qwen3-8B attention shape in full (B=2, L=4096, 32 q heads on 8 kv
    heads, d_h=128, inside the layer's [T, q|k|v] buffer), and one sequence
    long enough that the stored dS passes 4 GiB (32-bit byte offsets would
    wrap): dQ from the stored dS and dQ from a recomputation of S and dP,
    every element of dq, dk and dv bitwise equal (the layer tests compare
    the first shape with the oracle on sampled rows)."""
    need_gpu()
    import torch
    hq, hkv, dh = 32, 8, 128
    say(f"attention backward forms, B={B} L={L} hq={hq} hkv={hkv} dh={dh}")
    n = (L + 31) // 32
    if L > 4096:
        assert B * hq * n * (n + 1) // 2 * 2048 > 4 << 30
    qd, kvd = hq * dh, hkv * dh
    g = torch.Generator(device="cuda").manual_seed(4096)
    qkv = torch.randn(B, L, qd + 2 * kvd, device="cuda", generator=g).to(torch.bfloat16)
    do = torch.randn(B, L, qd, device="cuda", generator=g).to(torch.bfloat16)
    gq, gk, gv = qkv[..., :qd], qkv[..., qd:qd + kvd], qkv[..., qd + kvd:]
    o, lse = q3.attention_fwd(gq, gk, gv, hq, hkv, dh)
    outs = []
    for stored in (True, False):
        grad = torch.full_like(qkv, float("nan"))
        q3.attention_bwd(gq, gk, gv, o, do, lse, hq, hkv, dh, dq=grad[..., :qd],
                         dk=grad[..., qd:qd + kvd], dv=grad[..., qd + kvd:], stored_ds=stored)
        outs.append(grad)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(outs[0].float()).all())
    _same_bits(outs[0], outs[1], "dq|dk|dv")


def test_attention_strided_views():
    """q/k/v read from column slices of one [T, q+k+v] buffer (the layer's
    layout), forward and backward; dq/dk/dv are written with the same row
    strides into slices of one gradient buffer, whose other columns stay
    untouched."""
    need_gpu()
    import torch
    say("attention strided views")
    B, L, hq, hkv, dh = 2, 150, 8, 2, 128
    rng = np.random.default_rng(5)
    qd, kvd = hq * dh, hkv * dh
    qkv = _rand(rng, (B, L, qd + 2 * kvd), 1.0)
    do = _rand(rng, (B, L, qd), 1.0)
    g = dev(qkv, "bf16")
    gq, gk, gv = g[..., :qd], g[..., qd:qd + kvd], g[..., qd + kvd:]
    # o inside a wider buffer as well (its own row stride).
    ob = Guarded((B, L, qd + 64), torch.bfloat16)
    o = ob.t[..., :qd]
    lse = Guarded((B, hq, L), torch.float32)
    q3.attention_fwd(gq, gk, gv, hq, hkv, dh, o=o, lse=lse.t)
    ob.check("o", written=False), lse.check("lse")
    assert bool(torch.isfinite(o.float()).all())
    assert not bool(torch.isfinite(ob.t[..., qd:].float()).any())
    grad = Guarded((B, L, qd + 2 * kvd), torch.bfloat16)
    dq, dk, dv = q3.attention_bwd(gq, gk, gv, o, dev(do, "bf16"), lse.t, hq, hkv, dh,
                                  dq=grad.t[..., :qd], dk=grad.t[..., qd:qd + kvd],
                                  dv=grad.t[..., qd + kvd:])
    grad.check("dqkv")
    q = qkv[..., :qd].reshape(B, L, hq, dh)
    k = qkv[..., qd:qd + kvd].reshape(B, L, hkv, dh)
    v = qkv[..., qd + kvd:].reshape(B, L, hkv, dh)
    _attn_check("bf16", q, k, v, do.reshape(B, L, hq, dh), o, lse.t, dq, dk, dv)
    # A strided view with a contiguous gradient buffer is refused.
    with pytest.raises(ValueError):
        q3.attention_bwd(gq, gk, gv, o, dev(do, "bf16"), lse.t, hq, hkv, dh,
                         dq=torch.empty_like(o))


# Logits whose scale grows along the sequence: the log-sum-exp of the last
# rows reaches 55-75 in log2 units, against under 10 for the first. The
# kernels' running maximum then moves many times within a row and the partial
# output and row sum are rescaled each time (the block-state merge of the
# online softmax, parallelism page, section 4.2); the result must still be
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
    _, lse_ref = oracle.attention(q.astype(np.float64), k.astype(np.float64),
                                  v.astype(np.float64))
    # The inputs must reach the regime this test is for.
    assert np.max(lse_ref) * np.log2(np.e) > 50.0
    # Most rows here have (nearly) one-hot probabilities, so their dS =
    # P (dP - D) is a difference of nearly equal numbers, D = rowsum(dO O)
    # taken from the bf16-rounded O: dq and dk rows are then set by the
    # rounding of O, not by the kernels, and only the tensor-wide bar
    # applies to them in bf16.
    _attn_check(dtype, q, k, v, do, *_attn_run(dtype, q, k, v, do),
                local_dqk=(dtype == "f32"))
