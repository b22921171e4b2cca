"""The attention backward that allocates nothing (q3l_attention_bwd_noalloc,
its row-sum scratch in the library's fixed device array) against the
workspace entry point q3l_attention_bwd, through the C ABI: bitwise equal
results on two calls in a row, the second smaller than the first (the array
keeps the first call's contents), and oversized calls refused."""
import ctypes as C

import numpy as np
import pytest

import qwen3_decoder_layer_amd as q3
from gpu_helpers import dev, need_gpu, say
import synth

pytestmark = pytest.mark.gpu


def _case(rng, B, L, hq, hkv, dh):
    def r(shape):
        return synth.bf16_round(rng.standard_normal(shape).astype(np.float32))
    q = dev(r((B, L, hq * dh)), "bf16")
    k = dev(r((B, L, hkv * dh)), "bf16")
    v = dev(r((B, L, hkv * dh)), "bf16")
    do = dev(r((B, L, hq * dh)), "bf16")
    o, lse = q3.attention_fwd(q, k, v, hq, hkv, dh)
    return q, k, v, o, do, lse


@pytest.mark.parametrize("first,second", [
    ((2, 1000, 8, 2, 128), (1, 131, 4, 2, 64)),
    ((1, 4096, 32, 8, 128), (2, 77, 8, 1, 128)),
])
def test_noalloc_matches_workspace_entry(first, second):
    need_gpu()
    import torch
    rng = np.random.default_rng(17)
    for shape in (first, second):
        B, L, hq, hkv, dh = shape
        say(f"attention_bwd_noalloc B={B} L={L} hq={hq} hkv={hkv} dh={dh}")
        q, k, v, o, do, lse = _case(rng, *shape)
        ref = q3.attention_bwd(q, k, v, o, do, lse, hq, hkv, dh)
        out = [torch.full_like(t, float("nan")) for t in (q, k, v)]
        q3.attention_bwd_noalloc(q, k, v, o, do, lse, hq, hkv, dh, *out)
        torch.cuda.synchronize()
        for name, a, b in zip(("dq", "dk", "dv"), out, ref):
            assert torch.equal(a, b), name


def test_noalloc_refuses_sizes_beyond_its_scratch():
    need_gpu()
    lib = q3.library()
    cap = lib.q3l_attention_bwd_noalloc_max_rows()
    assert cap == 1 << 22
    buf = C.create_string_buffer(256)
    p = C.c_void_p((C.addressof(buf) + 15) // 16 * 16)
    L = cap // 8 + 64            # one sequence, 8 heads: just past the cap
    st = lib.q3l_attention_bwd_noalloc(1, 1, L, 8, 8, 64, p, 512, p, 512, p, 512, p,
                                       512, p, 512, p, p, p, p, None)
    assert st == 1 and b"scratch" in lib.q3l_last_error()
