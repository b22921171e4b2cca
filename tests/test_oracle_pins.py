"""Pins of the oracle to values the pages print (worked examples, tables).

Each fixture under tests/golden/ names the page and section it comes from.
"""
import json
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as fh:
        return json.load(fh)


# --- walkthrough page: single-layer parameter table -------------------------
def test_walkthrough_parameter_table():
    fx = _load("walkthrough_param_table.json")
    c = fx["config"]
    counts = oracle.param_counts(c["d"], c["h_q"], c["h_kv"], c["d_h"],
                                 c["d_ffn"])
    shapes = synth.param_shapes(dict(c))
    assert list(counts) == list(fx["per_tensor"]) == list(synth.PARAM_NAMES)
    for name, row in fx["per_tensor"].items():
        assert counts[name] == row["elements"], name
        assert list(shapes[name]) == row["shape"], name
    total = oracle.param_total(c["d"], c["h_q"], c["h_kv"], c["d_h"],
                               c["d_ffn"])
    assert total == 2_360_448
    assert round(total / 1e6, 2) == fx["total_approx_millions"]
    # fp16: two bytes per parameter.
    assert round(2 * total / 1e6, 2) == fx["fp16_bytes_approx_MB"]
    # FSDP shard: dim 0 split four ways.
    per_rank = 0
    for name, rows in fx["per_rank_shard_rows"].items():
        shape = fx["per_tensor"][name]["shape"]
        assert rows * c["dp_world"] == shape[0]
        per_rank += rows * int(np.prod(shape[1:], dtype=np.int64))
    assert per_rank * c["dp_world"] == total
    assert round(per_rank / 1e3, -1) == fx["per_rank_approx_thousands"]
    assert round(2 * per_rank / 1e6, 2) == fx["per_rank_fp16_approx_MB"]
    sent = (c["dp_world"] - 1) / c["dp_world"] * round(2 * total / 1e6, 2)
    assert round(sent, 2) == fx["allgather_sent_per_rank_approx_MB"]


# --- memory-model page: parameter formula and the 7B worked example --------
def test_megatron_7b_param_count():
    fx = _load("megatron_7b_param_count.json")
    i = fx["inputs"]
    per = oracle.megatron_layer_params(i["h"], i["a"], i["g"], i["d"],
                                       i["ffn"])
    assert per["attention"] == fx["attention_per_layer"]
    assert per["mlp"] == fx["mlp_per_layer"]
    assert per["norms"] == fx["ln_per_layer"]
    assert per["layer"] == fx["per_layer"]
    # The formula's attention term equals the sum of the four projections of
    # the eleven-tensor layout (qk_norm off: the page's model has none).
    c = oracle.param_counts(i["h"], i["a"], i["g"], i["d"], i["ffn"],
                            qk_norm=False)
    assert c["q"] == fx["Wq"] and c["k"] == fx["Wk"] and c["v"] == fx["Wv"]
    assert c["o"] == fx["Wo"]
    assert oracle.param_total(i["h"], i["a"], i["g"], i["d"], i["ffn"],
                              qk_norm=False) == fx["per_layer"]
    model = oracle.megatron_model_params(i["h"], i["a"], i["g"], i["d"],
                                         i["ffn"], i["n_layers"], i["vocab"])
    assert model["block"] == fx["block_with_final_ln"]
    assert model["embedding"] == fx["embedding_tied"]
    assert model["total"] == fx["total"]


def test_formula_plus_qk_norm_reproduces_walkthrough_table():
    # The memory-model formula with Qwen3's two [d_h] norms added gives the
    # walkthrough page's layer exactly; and the Qwen3-8B-shaped layer.
    assert oracle.megatron_layer_params(512, 8, 4, 64, 1024,
                                        qk_norm=True)["layer"] == 2_360_448
    assert oracle.param_total(4096, 32, 8, 128, 12288) == 192_946_432
    assert oracle.megatron_layer_params(4096, 32, 8, 128, 12288,
                                        qk_norm=True)["layer"] == 192_946_432


# --- state-placement page: online-softmax worked example -------------------
def test_online_softmax_worked_example():
    fx = _load("online_softmax_example.json")
    tol = fx["print_precision"]
    pr = fx["printed"]
    s1, s2 = fx["scores_blocks"]
    V = np.array(fx["values"])
    a = oracle.block_state(s1, V[:2])
    b = oracle.block_state(s2, V[2:])
    merged = oracle.merge_states(a, b)
    out, lse = oracle.finish_state(merged)
    assert np.allclose(out, pr["output"], atol=tol)
    assert merged[0] == 2.0
    assert abs(merged[1] - pr["merged_l"]) < tol
    assert abs(merged[1] * np.e ** 2 - pr["denominator"]) < 2 * tol * np.e ** 2
    # Order of blocks does not matter.
    m2 = oracle.merge_states(b, a)
    assert np.allclose(oracle.finish_state(m2)[0], out, rtol=0, atol=1e-15)
    # The plain softmax the oracle's attention uses gives the same numbers.
    scores = np.array(s1 + s2)
    o_full, lse_full = oracle.softmax_attend(scores[None, :], V)
    assert np.allclose(o_full[0], pr["output"], atol=tol)
    assert np.allclose(np.exp(scores), pr["exp_scores"], atol=tol)
    assert abs(np.exp(scores).sum() - pr["denominator"]) < tol
    w = np.exp(scores) / np.exp(scores).sum()
    assert np.allclose(w, pr["weights"], atol=tol)
    assert abs(lse_full[0] - lse) < 1e-14


def test_online_merge_equals_full_softmax_random():
    rng = np.random.default_rng(7)
    s = rng.standard_normal(37) * 3
    V = rng.standard_normal((37, 5))
    st = None
    for lo in range(0, 37, 8):
        blk = oracle.block_state(s[lo:lo + 8], V[lo:lo + 8])
        st = blk if st is None else oracle.merge_states(st, blk)
    out, lse = oracle.finish_state(st)
    ref, ref_lse = oracle.softmax_attend(s[None, :], V)
    assert np.allclose(out, ref[0], rtol=1e-13, atol=1e-13)
    assert abs(lse - ref_lse[0]) < 1e-13


# --- state-placement page: two-rank tensor-parallel toy ---------------------
def test_tp_toy_linear_conventions():
    """Z = relu(X A) B split column-then-row; the oracle's linear layers store
    W = A^T ([out, in]).  Loss = sum(Z), so dZ = 1."""
    fx = _load("tp_toy.json")
    pr = fx["printed"]
    X = np.array(fx["X"])
    A = np.array(fx["reconstructed"]["A"])
    Bm = np.array(fx["reconstructed"]["B"])
    Z_sum = 0
    dX_sum = 0
    for t in range(2):
        WA = A[:, t:t + 1].T          # column shard of A as an [out, in] weight
        WB = Bm[t:t + 1, :].T         # row shard of B as an [out, in] weight
        Y = oracle.linear(X, WA)
        R = np.maximum(Y, 0)
        Z = oracle.linear(R, WB)
        assert np.array_equal(Y, pr[f"Y_{t}"])
        assert np.array_equal(Z, pr[f"Z_{t}"])
        Z_sum = Z_sum + Z
        dZ = np.ones_like(Z)
        dR, dWB = oracle.linear_backward(dZ, R, WB)
        dY = dR * (Y > 0)
        dX, dWA = oracle.linear_backward(dY, X, WA)
        assert np.array_equal(dWB.T, pr[f"dB_{t}"])
        assert np.array_equal(dWA.T, pr[f"dA_{t}"])
        dX_sum = dX_sum + dX
    assert np.array_equal(Z_sum, pr["Z"])
    assert np.array_equal(dX_sum, pr["dX"])
    # The unsplit computation gives the same.
    Y = oracle.linear(X, A.T)
    Z = oracle.linear(np.maximum(Y, 0), Bm.T)
    assert np.array_equal(Z, pr["Z"])
    dR, dWB = oracle.linear_backward(np.ones_like(Z), np.maximum(Y, 0), Bm.T)
    dX, dWA = oracle.linear_backward(dR * (Y > 0), X, A.T)
    assert np.array_equal(dWB.T, pr["dB"])
    assert np.array_equal(dWA.T, pr["dA"])
    assert np.array_equal(dX, pr["dX"])


@pytest.mark.parametrize("a10", [0.0, 3.0, -2.5])
def test_tp_toy_outputs_do_not_depend_on_reconstruction(a10):
    """Every A consistent with the printed Y and dX gives the printed dA/dB."""
    A = np.array([[7 - 2 * a10, a10 - 1], [a10, (11 - a10) / 2]])
    X = np.array([[1.0, 2.0]])
    Y = oracle.linear(X, A.T)
    assert np.allclose(Y, [[7.0, 10.0]])
    dX, _ = oracle.linear_backward(np.array([[1.0, 2.0]]), X, A.T)
    assert np.allclose(dX, [[5.0, 11.0]])


def _page_example_tensors():
    """The page's four-key example as attention inputs: one sequence of 4
    tokens, one head, d_h = 64; the query at position 3 scores the keys
    [1, 0, 2, 0] (q = 8 e_0, k_s = score_s e_0, so q.k / sqrt(64) = score)
    and the values are the printed 2-vectors padded with zeros."""
    fx = _load("online_softmax_example.json")
    scores = np.array(fx["scores_blocks"][0] + fx["scores_blocks"][1])
    V = np.array(fx["values"])
    L, dh = 4, 64
    q = np.zeros((1, L, 1, dh)); q[0, :, 0, 0] = 8.0
    k = np.zeros((1, L, 1, dh)); k[0, :, 0, 0] = scores
    v = np.zeros((1, L, 1, dh)); v[0, :, 0, :2] = V
    return fx, q, k, v


def test_block_state_attention_on_the_page_example():
    """Blocks [0, 2) and [2, 4) of the page's example through the per-query
    block-state attention: the last query's states, merged, give the printed
    output (1.000, 0.693) and merged l = 1.639."""
    fx, q, k, v = _page_example_tensors()
    tol = fx["print_precision"]
    a = oracle.attention_block_state(q, k, v, 0, 2)
    b = oracle.attention_block_state(q, k, v, 2, 4)
    # Query 3's states are the page's two block states.
    s1, s2 = fx["scores_blocks"]
    V = np.array(fx["values"])
    for st, (sc, vv) in ((a, (s1, V[:2])), (b, (s2, V[2:]))):
        m_ref, l_ref, acc_ref = oracle.block_state(sc, vv)
        assert st[0][0, 0, 3] == m_ref
        assert abs(st[1][0, 0, 3] - l_ref) < 1e-14
        assert np.allclose(st[2][0, 3, 0, :2], acc_ref, atol=1e-14)
        assert not st[2][0, 3, 0, 2:].any()
    m, l, acc = oracle.merge_block_states(a, b)
    out = acc[0, 3, 0, :2] / l[0, 0, 3]
    assert np.allclose(out, fx["printed"]["output"], atol=tol)
    assert m[0, 0, 3] == 2.0 and abs(l[0, 0, 3] - fx["printed"]["merged_l"]) < tol
    # Query 0 sees only key 0: block [2, 4) is empty for it.
    assert b[0][0, 0, 0] == -np.inf and b[1][0, 0, 0] == 0.0 and not b[2][0, 0].any()


@pytest.mark.parametrize("cuts", [[0, 131], [0, 37, 131], [0, 64, 65, 100, 131]])
def test_block_states_merged_over_a_partition_equal_attention(cuts):
    """Merging the block states of any partition of [0, L), in any order,
    gives the one-pass softmax attention of the oracle (output and LSE)."""
    rng = np.random.default_rng(len(cuts))
    B, L, hq, hkv, dh = 2, 131, 4, 2, 64
    q = rng.standard_normal((B, L, hq, dh))
    k = rng.standard_normal((B, L, hkv, dh))
    v = rng.standard_normal((B, L, hkv, dh))
    O, LSE = oracle.attention(q, k, v)
    states = [oracle.attention_block_state(q, k, v, a, b) for a, b in zip(cuts, cuts[1:])]
    for order in (states, states[::-1]):
        st = order[0]
        for other in order[1:]:
            st = oracle.merge_block_states(st, other)
        m, l, acc = st
        assert np.allclose(acc / np.transpose(l, (0, 2, 1))[..., None], O, rtol=1e-12, atol=1e-12)
        assert np.allclose(m + np.log(l), LSE, rtol=1e-12, atol=1e-12)
