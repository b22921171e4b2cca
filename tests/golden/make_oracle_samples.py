"""Write sampled fp64 oracle outputs of the full-size forward+backward
workload (Qwen3-8B-shaped layer, d=4096, 32/8 heads, d_h=128, d_ffn=12288,
B=2, L=4096, bf16 inputs, seed 1004) to oracle_samples_qwen3_8b_fwd_bwd.npz.

The oracle needs minutes for this workload, so the GPU test reads these
samples instead of re-running it.  Only ``oracle`` and ``synth`` are used:
no value here comes from the HIP path.

For every checked tensor (y, dx and the eleven weight gradients) the file
holds the values at SAMPLE_COUNT flat indices drawn by ``sample_indices``
(seeded, so the test regenerates the same indices) and the tensor's max |.|,
which is the denominator of the relative-error bar.

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
SAMPLE_COUNT = 2048
TENSORS = ("y", "dx") + ("in_norm", "q", "k", "v", "q_norm", "k_norm", "o",
                         "post_norm", "gate", "up", "down")


def sample_indices(name: str, size: int) -> np.ndarray:
    """Seeded flat indices for tensor `name` (all of them if small)."""
    if size <= SAMPLE_COUNT:
        return np.arange(size)
    seed = 7000 + TENSORS.index(name)
    rng = np.random.Generator(np.random.PCG64(seed))
    return np.sort(rng.choice(size, size=SAMPLE_COUNT, replace=False))


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
        a = np.asarray(full[name], dtype=np.float64).ravel()
        idx = sample_indices(name, a.size)
        out[f"{name}_val"] = a[idx]
        out[f"{name}_maxabs"] = np.array(np.max(np.abs(a)))
        out[f"{name}_size"] = np.array(a.size)
    np.savez_compressed(OUT, **out)
    print(f"wrote {OUT}")


if __name__ == "__main__":
    main()
