"""Write sampled fp64 oracle outputs of the full-size forward+backward
workload (Qwen3-8B-shaped layer, d=4096, 32/8 heads, d_h=128, d_ffn=12288,
B=2, L=4096, bf16 inputs, seed 1004) to oracle_samples_qwen3_8b_fwd_bwd.npz.

The oracle needs minutes for this workload, so the GPU test reads these
samples instead of re-running it.  Only ``oracle`` and ``synth`` are used:
no value here comes from the HIP path.

Every checked tensor (y and dx as [tokens, d]; the seven projection
gradients as [out, in]) is cut into blocks of BLOCK_ROWS x BLOCK_COLS and
one element per block, at a seeded position inside it, is stored -- so a
wrong or missing output tile of any GEMM or attention kernel region hits at
least one sample.  The four norm-weight gradients are stored whole.  For
each tensor the file also holds the RMS of every row (the local scale of
the element-wise bound the test applies) and the tensor's max |.| (the
denominator of the max-relative-error bar).

    python tests/golden/make_oracle_samples.py
"""
from __future__ import annotations

import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

OUT = os.path.join(HERE, "oracle_samples_qwen3_8b_fwd_bwd.npz")
PRESET = 4
BLOCK_ROWS, BLOCK_COLS = 32, 64
TENSORS = ("y", "dx") + ("in_norm", "q", "k", "v", "q_norm", "k_norm", "o",
                         "post_norm", "gate", "up", "down")


def as_matrix(name: str, a: np.ndarray) -> np.ndarray:
    """The 2-D view a tensor is sampled in: rows are tokens for y and dx,
    output features for the projection gradients; a 1-D norm-weight
    gradient is one row."""
    a = np.asarray(a)
    if a.ndim == 1:
        return a.reshape(1, -1)
    return a.reshape(-1, a.shape[-1])


def sample_indices(name: str, shape: tuple) -> tuple:
    """(rows, cols) of the stored samples of a matrix of `shape`: every
    element of a single-row tensor, else one seeded element per block."""
    R, Cn = shape
    if R == 1:
        return np.zeros(Cn, dtype=np.int64), np.arange(Cn)
    seed = 7000 + TENSORS.index(name)
    rng = np.random.Generator(np.random.PCG64(seed))
    nbr, nbc = -(-R // BLOCK_ROWS), -(-Cn // BLOCK_COLS)
    bi, bj = np.meshgrid(np.arange(nbr), np.arange(nbc), indexing="ij")
    bi, bj = bi.ravel(), bj.ravel()
    hr = np.minimum(BLOCK_ROWS, R - bi * BLOCK_ROWS)
    hc = np.minimum(BLOCK_COLS, Cn - bj * BLOCK_COLS)
    rows = bi * BLOCK_ROWS + (rng.random(bi.size) * hr).astype(np.int64)
    cols = bj * BLOCK_COLS + (rng.random(bj.size) * hc).astype(np.int64)
    return rows, cols


def main():
    import oracle
    import synth
    cfg, inp = synth.preset_inputs(PRESET)
    p = {n: inp[n] for n in synth.PARAM_NAMES}
    t0 = time.time()
    y = oracle.layer_forward(cfg, p, inp["x"])["y"]
    print(f"forward {time.time() - t0:.1f}s", flush=True)
    dx, grads = oracle.layer_backward(cfg, p, inp["x"], inp["dy"])
    print(f"backward {time.time() - t0:.1f}s", flush=True)
    full = {"y": y, "dx": dx, **grads}
    out = {}
    for name in TENSORS:
        m = as_matrix(name, np.asarray(full[name], dtype=np.float64))
        r, c = sample_indices(name, m.shape)
        out[f"{name}_val"] = m[r, c].astype(np.float32)
        out[f"{name}_rowrms"] = np.sqrt(np.mean(m * m, axis=1)).astype(np.float32)
        out[f"{name}_maxabs"] = np.array(np.max(np.abs(m)))
        out[f"{name}_shape"] = np.array(m.shape)
    np.savez_compressed(OUT, **out)
    print(f"wrote {OUT}")


if __name__ == "__main__":
    main()
