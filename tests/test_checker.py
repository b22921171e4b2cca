"""The parity checker itself, on the CPU: the row-local bound used by the GPU
tests must reject a result that drops the ragged last key tile of a causal
dK/dV or zeroes one 32-row block of a GEMM output -- mistakes the tensor-wide
max relative error lets through -- and must accept results that differ from
the oracle only by bf16 rounding."""
import numpy as np

import oracle
import synth
from gpu_helpers import LOCAL_FACTOR, TOL, check, local_err, rel_err

TOL_LOCAL = LOCAL_FACTOR * TOL["bf16"]


def _rand(rng, shape, scale=1.0):
    return synth.bf16_round((rng.standard_normal(shape) * scale).astype(np.float32))


def _attention_case():
    # The seeded inputs of the GPU attention case B=1, L=131, h_q=4, h_kv=2,
    # d_h=64 (same generator and draw order as that test).
    B, L, hq, hkv, dh = 1, 131, 4, 2, 64
    rng = np.random.default_rng(B * 1000 + L + hq + dh)
    q = _rand(rng, (B, L, hq, dh))
    k = _rand(rng, (B, L, hkv, dh))
    v = _rand(rng, (B, L, hkv, dh))
    do = _rand(rng, (B, L, hq, dh))
    return [t.astype(np.float64) for t in (q, k, v, do)]


def test_local_bound_catches_a_dropped_ragged_key_tile():
    q, k, v, do = _attention_case()
    dq, dk, dv = oracle.attention_backward(do, q, k, v)
    B, L, hkv, dh = dk.shape
    for ref in (dk, dv):
        bad = ref.copy()
        bad[:, 128:131] = 0.0          # the whole ragged last key tile
        flat_ref = ref.reshape(B, L, hkv * dh)
        flat_bad = bad.reshape(B, L, hkv * dh)
        # The tensor-wide measure misses it ...
        assert rel_err(flat_bad, flat_ref) <= TOL["bf16"]
        # ... the row-local bound does not.
        assert local_err(flat_bad, flat_ref) > 2 * TOL_LOCAL
        assert not check("d", flat_bad, flat_ref, TOL["bf16"])


def test_local_bound_catches_a_zeroed_gemm_block():
    rng = np.random.default_rng(3)
    a = _rand(rng, (300, 136)).astype(np.float64)
    w = _rand(rng, (264, 136), 0.02).astype(np.float64)
    y = oracle.linear(a, w)
    bad = y.copy()
    bad[64:96, 128:192] = 0.0           # one 32-row block of one tile column
    assert not check("y", bad, y, TOL["bf16"])
    # A single wrong element at a tenth of its row's scale is caught too.
    one = y.copy()
    one[7, 11] += 0.1 * np.sqrt(np.mean(y[7] ** 2)) + 0.1 * abs(y[7, 11])
    one[7, 11] += 0.1 * np.sqrt(np.mean(y ** 2))
    assert local_err(one, y) > TOL_LOCAL


def test_local_bound_accepts_bf16_rounding():
    # The oracle's own outputs rounded to bf16 (what an exact kernel with a
    # bf16 output would give) pass with a wide margin, also in the small
    # rows of a causal dK/dV.
    q, k, v, do = _attention_case()
    for ref in oracle.attention_backward(do, q, k, v):
        flat = ref.reshape(ref.shape[0], ref.shape[1], -1)
        r16 = synth.bf16_round(flat.astype(np.float32)).astype(np.float64)
        assert local_err(r16, flat) < TOL_LOCAL / 8
        assert check("d", r16, flat, TOL["bf16"])


def test_nan_fails_the_check():
    y = np.ones((4, 8))
    bad = y.copy()
    bad[2, 3] = np.nan
    assert not check("y", bad, y, TOL["bf16"])
