"""Throughput of one Qwen3 decoder layer, forward + backward, on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--no-cpu-baseline]

A step is one pass of the whole hot path over one batch of synthetic input:
q3l_layer_forward (saving intermediates) then q3l_layer_backward (dx and all
eleven fp32 weight gradients), on the Qwen3-8B-shaped layer (d=4096, 32 q /
8 kv heads, d_h=128, d_ffn=12288, B=2, L=4096, bf16).  Inputs and weights
are resident in HBM before the timed region.  Rank 0 prints one JSON line.

After the timed steps it runs the same number of steps again with phase
marks: HIP events the library records on its stream at every phase
boundary.  Their medians give each phase's time and its fraction of the
matrix-core or HBM roofline ("phases"), and the in-step time of the dominant
kernel (the fused gate/up GEMM with the SwiGLU epilogue) for "roofline".  The
fp64 CPU oracle is timed on a bounded sample of the same workload as a
reported baseline.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402

METRIC = ("decoder-layer fwd+bwd tokens/s and TFLOP/s (% bf16 MFMA peak), "
          "1 MI355X")
PEAK_BF16_TFLOPS = 2516.6     # 256 CU x 2.4 GHz x 4096 dense bf16 FLOP/clk
PEAK_HBM_GBS = 8000.0
COPY_BYTES = 1 << 30          # calibration copy for the HBM byte counters

# HBM traffic of the dominant kernel from two hardware-counter passes
# (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch) over `bench.py
# --kernel-probe`, each scaled by what the same counter reads for the 1 GiB
# calibration copy.  Valid only for the kernel source it was taken on: the
# digest below is of gemm_bf16.hip, and a changed source reports null.
TRAFFIC = {"source_sha256": "52c84c34524a98f3",
           "fetch_kib": 1181001.7, "write_kib": 592221.6, "copy_fetch_kib": 524303.0,
           "copy_write_kib": 1048576.0, "bytes": 3025057346}

WORKLOADS = {
    "qwen3-8b-bf16-fwd-bwd": 4,
    "qwen3-8b-bf16-fwd": 2,
    "llama70b-tp8-share-bf16-fwd": 3,
    "tiny-dims-bf16-fwd-L2048": 1,
}


def model_flops(c: dict, backward: bool) -> dict:
    """Model FLOPs of one layer pass (attention counts causal pairs)."""
    T, d, f = c["B"] * c["L"], c["d"], c["d_ffn"]
    qd, kvd = c["h_q"] * c["d_h"], c["h_kv"] * c["d_h"]
    gemm = 2 * T * d * (qd + 2 * kvd) + 2 * T * qd * d + 2 * T * d * 2 * f \
        + 2 * T * f * d
    pairs = c["B"] * c["L"] * (c["L"] + 1) // 2
    attn = 4 * c["h_q"] * c["d_h"] * pairs
    out = {"gemm_fwd": gemm, "attn_fwd": attn}
    total = gemm + attn
    if backward:
        total += 2 * gemm + 2 * attn
        out["attn_recompute"] = 2 * c["h_q"] * c["d_h"] * pairs
    out["total"] = total
    return out


def phase_work(c: dict) -> tuple:
    """Algorithmic work of each phase of one step, keyed by the library's
    phase names: (bound, amount) with bound "mfma" (FLOPs) or "hbm" (bytes:
    one read of each input and one write of each output).  Attention counts
    causal pairs (model FLOPs: 4 h_q d_h per pair forward, twice that
    backward; the recomputed scores are not counted)."""
    T, d, f, L = c["B"] * c["L"], c["d"], c["d_ffn"], c["L"]
    qd, kvd, dh = c["h_q"] * c["d_h"], c["h_kv"] * c["d_h"], c["d_h"]
    nqkv, nqk, heads = qd + 2 * kvd, qd + kvd, c["h_q"] + c["h_kv"]
    pairs = c["B"] * L * (L + 1) // 2
    a = 2                                   # bf16 bytes
    norm_fwd = ("hbm", 2 * a * T * d + 4 * T + a * d)
    norm_bwd = ("hbm", 4 * a * T * d + 4 * T + a * d)
    fwd = {
        "F1 rmsnorm": norm_fwd,
        "F2 qkv gemm": ("mfma", 2 * T * d * nqkv),
        "F3-F4 qk-norm + rope": ("hbm", 2 * a * T * nqk + 4 * T * heads + 8 * L * dh),
        "transposes for the backward": ("hbm", 2 * a * T * d),
        "F5 attention": ("mfma", 4 * c["h_q"] * dh * pairs),
        "F6 o gemm + residual": ("mfma", 2 * T * qd * d),
        "F7 rmsnorm": norm_fwd,
        "F8-F9 gate/up gemm + swiglu": ("mfma", 2 * T * d * 2 * f),
        "F10 down gemm + residual": ("mfma", 2 * T * f * d),
    }
    bwd = {
        "B1 down dgrad gemm": ("mfma", 2 * T * d * f),
        "B2 swiglu adjoint": ("hbm", 7 * a * T * f),
        "B1 down wgrad transposes": ("hbm", 2 * a * T * d),
        "B1 down wgrad gemm": ("mfma", 2 * T * d * f),
        "B3 gate/up dgrad gemm": ("mfma", 2 * T * 2 * f * d),
        "B3 gate/up wgrad transposes": ("hbm", 0),   # none: hn read in place
        "B3 gate/up wgrad gemm": ("mfma", 2 * T * 2 * f * d),
        "B4 rmsnorm bwd": norm_bwd,
        "B5 o dgrad gemm": ("mfma", 2 * T * d * qd),
        "B5 o wgrad transposes": ("hbm", 0),   # none: both operands read in place
        "B5 o wgrad gemm": ("mfma", 2 * T * d * qd),
        "B6 attention bwd": ("mfma", 8 * c["h_q"] * dh * pairs),
        "B7 qk-norm + rope bwd": ("hbm", 3 * a * T * nqk + 4 * T * heads),
        "B8 qkv dgrad gemm": ("mfma", 2 * T * nqkv * d),
        "B8 qkv wgrad transposes": ("hbm", 2 * a * T * nqkv),
        "B8 qkv wgrad gemm": ("mfma", 2 * T * nqkv * d),
        "B9 rmsnorm bwd": norm_bwd,
    }
    return fwd, bwd


def gpu_run(cfg: dict, inp: dict, steps: int, warmup: int) -> dict:
    import torch
    import qwen3_decoder_layer_amd as q3
    lc = q3.LayerConfig.from_dict(cfg)
    bf = torch.bfloat16
    dev = "cuda"

    def up(a):
        return torch.from_numpy(a).to(device=dev, dtype=bf)

    W = {n: up(inp[n]) for n in synth.PARAM_NAMES}
    x = up(inp["x"])
    backward = cfg["backward"]
    # A training step saves the intermediates for its backward; a forward-only
    # workload runs as inference, with scratch instead (allocated here, not in
    # the timed loop).
    saved = (torch.empty(q3.saved_bytes(lc), dtype=torch.uint8, device=dev)
             if backward else None)
    fwd_ws = (None if backward else
              torch.empty(q3.workspace_bytes(lc, False), dtype=torch.uint8, device=dev))
    out = {}
    if cfg.get("tp_partial"):
        out = {k: torch.empty((lc.B, lc.L, lc.d), dtype=torch.float32, device=dev)
               for k in ("attn_partial", "mlp_partial")}
    else:
        out = {"y": torch.empty_like(x)}
    if backward:
        dy = up(inp["dy"])
        dx = torch.empty_like(x)
        grads = {n: torch.empty(W[n].shape, dtype=torch.float32, device=dev)
                 for n in synth.PARAM_NAMES}
        ws = torch.empty(q3.workspace_bytes(lc, True), dtype=torch.uint8,
                         device=dev)
    stream = torch.cuda.current_stream()
    # The training forward's transposed copy (xn^T) runs on this second stream,
    # beside the attention step (default priority, like every stream here).
    side = q3.Exec(side_stream=torch.cuda.Stream()) if backward else None
    nf, nb = len(q3.phase_names(False)), len(q3.phase_names(True))

    def marks(n):
        return q3.MarkEvents(n + 1)

    def step(exf=side, exb=None):
        q3.layer_forward(lc, W, x, out=out, saved=saved, workspace=fwd_ws, stream=stream,
                         exec=exf)
        if backward:
            q3.layer_backward(lc, W, x, dy, saved, dx=dx, grads=grads,
                              workspace=ws, stream=stream, exec=exb)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    # The same steps again with phase marks (events the library records at
    # its phase boundaries on the stream): per-phase times inside a step.
    fwd_t, bwd_t = [], []
    t1 = time.perf_counter()
    for _ in range(steps):
        exf = q3.Exec(side_stream=side.side_stream if side else None, marks=marks(nf))
        exb = q3.Exec(marks=marks(nb)) if backward else None
        step(exf, exb)
        fwd_t.append(exf)
        bwd_t.append(exb)
    torch.cuda.synchronize()
    marked_elapsed = time.perf_counter() - t1
    fwd_ms = np.median(np.array([e.phase_times() for e in fwd_t]), axis=0)
    bwd_ms = (np.median(np.array([e.phase_times() for e in bwd_t]), axis=0)
              if backward else None)
    del saved, fwd_ws
    return {"elapsed": elapsed, "marked_elapsed": marked_elapsed,
            "fwd_phase_ms": dict(zip(q3.phase_names(False), fwd_ms)),
            "bwd_phase_ms": (dict(zip(q3.phase_names(True), bwd_ms))
                             if backward else {})}


def dominant_operands(lc, gate, up):
    import torch
    bf = torch.bfloat16
    gen = torch.Generator(device=gate.device).manual_seed(7)
    hn = torch.randn((lc.T, lc.d), device=gate.device, generator=gen).to(bf)
    f = torch.empty((lc.T, lc.d_ffn), dtype=bf, device=gate.device)
    gu = torch.empty((lc.T, 2 * lc.d_ffn), dtype=bf, device=gate.device)
    return hn, f, gu


def time_dominant(lc, gate, up, stream, reps: int, between=None) -> float:
    """Average duration (ms) of the fused gate/up GEMM + SwiGLU kernel at the
    layer's shapes, with HIP events recorded on the stream it launches on.

    With `between` (one layer step), each timed launch follows a step, so
    the kernel runs under the same clock and cache conditions as inside the
    timed steps; launched back to back instead, the sustained matrix-core
    load lowers the clock and the kernel runs a few per cent slower."""
    import torch
    import qwen3_decoder_layer_amd as q3
    hn, f, gu = dominant_operands(lc, gate, up)
    for _ in range(3):
        q3.swiglu_fwd(hn, gate, up, f=f, gu=gu, stream=stream)
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(reps)]
    for ev0, ev1 in pairs:
        if between is not None:
            between()
        ev0.record(stream)
        q3.swiglu_fwd(hn, gate, up, f=f, gu=gu, stream=stream)
        ev1.record(stream)
    torch.cuda.synchronize()
    return sum(a.elapsed_time(b) for a, b in pairs) / reps


def dominant_work(T: int, d: int, f: int) -> tuple:
    """(FLOPs, algorithmic HBM bytes) of one gate/up + SwiGLU launch (bf16):
    2*T*d*(2f) multiply-adds; read hn and both weights once, write f and the
    saved g|u once."""
    return 2 * T * d * 2 * f, 2 * (T * d + 2 * f * d + T * f + 2 * T * f)


def kernel_probe(cfg: dict) -> None:
    """Short run for hardware-counter passes: a plain 1 GiB device copy (the
    calibration kernel: reads and writes exactly COPY_BYTES), then the
    dominant kernel, each a few times, then one training forward and one
    backward of the layer on one stream (every kernel of a step once)."""
    import torch
    import qwen3_decoder_layer_amd as q3
    lc = q3.LayerConfig.from_dict(cfg)
    dev = "cuda"
    src = torch.empty(COPY_BYTES // 2, dtype=torch.bfloat16, device=dev).normal_()
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    gen = torch.Generator(device=dev).manual_seed(3)
    gate = (0.02 * torch.randn((lc.d_ffn, lc.d), device=dev, generator=gen)).to(torch.bfloat16)
    up = (0.02 * torch.randn((lc.d_ffn, lc.d), device=dev, generator=gen)).to(torch.bfloat16)
    stream = torch.cuda.current_stream()
    ms = time_dominant(lc, gate, up, stream, 5)
    torch.cuda.synchronize()
    del gate, up
    inp = synth.make_inputs(cfg, 1000 + 5, with_dy=True)
    W = {n: torch.from_numpy(inp[n]).to(dev, torch.bfloat16) for n in synth.PARAM_NAMES}
    x = torch.from_numpy(inp["x"]).to(dev, torch.bfloat16)
    dy = torch.from_numpy(inp["dy"]).to(dev, torch.bfloat16)
    saved = torch.empty(q3.saved_bytes(lc), dtype=torch.uint8, device=dev)
    ws = torch.empty(q3.workspace_bytes(lc, True), dtype=torch.uint8, device=dev)
    dx = torch.empty_like(x)
    grads = {n: torch.empty(W[n].shape, dtype=torch.float32, device=dev) for n in W}
    q3.layer_forward(lc, W, x, saved=saved, stream=stream)
    q3.layer_backward(lc, W, x, dy, saved, dx=dx, grads=grads, workspace=ws, stream=stream)
    torch.cuda.synchronize()
    print(f"kernel probe: copy {COPY_BYTES} B x3, dominant kernel {ms:.3f} ms avg, "
          "then one layer step", flush=True)


def split_probe(cfg: dict) -> None:
    """One training forward, then the backward split in two calls: INPUT
    (dx; leaves the activation gradients in the workspace) and WEIGHT |
    DEFERRED_WEIGHT (the weight gradients only), each timed with HIP events
    and followed by a device synchronisation, so that a kernel trace of this
    run shows which kernels each call launches.  Prints one JSON line."""
    import torch
    import qwen3_decoder_layer_amd as q3
    lc = q3.LayerConfig.from_dict(cfg)
    inp = synth.make_inputs(cfg, 1000 + 4, with_dy=True)
    W = {n: torch.from_numpy(inp[n]).to("cuda", torch.bfloat16) for n in synth.PARAM_NAMES}
    x = torch.from_numpy(inp["x"]).to("cuda", torch.bfloat16)
    dy = torch.from_numpy(inp["dy"]).to("cuda", torch.bfloat16)
    saved = torch.empty(q3.saved_bytes(lc), dtype=torch.uint8, device="cuda")
    ws = torch.empty(q3.workspace_bytes(lc, True), dtype=torch.uint8, device="cuda")
    dx = torch.empty_like(x)
    grads = {n: torch.empty(W[n].shape, dtype=torch.float32, device="cuda") for n in W}
    calls = [("forward", lambda: q3.layer_forward(lc, W, x, saved=saved)),
             ("backward INPUT", lambda: q3.layer_backward(
                 lc, W, x, dy, saved, dx=dx, flags=q3.BWD_INPUT, workspace=ws)),
             ("backward WEIGHT|DEFERRED_WEIGHT", lambda: q3.layer_backward(
                 lc, W, x, dy, saved, grads=grads,
                 flags=q3.BWD_WEIGHT | q3.BWD_DEFERRED_WEIGHT, workspace=ws)),
             ("backward INPUT|WEIGHT", lambda: q3.layer_backward(
                 lc, W, x, dy, saved, dx=dx, grads=grads, workspace=ws))]
    for _, fn in calls:          # warm-up
        fn()
    torch.cuda.synchronize()
    times = {}
    for name, fn in calls:
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        torch.cuda.synchronize()
        times[name] = a.elapsed_time(b)
    print(json.dumps({"workload": cfg["name"], "ms": times}), flush=True)


def kernel_source_digest() -> str:
    """Digest of the dominant kernel's device code: gemm_bf16.hip and the
    helpers it includes (common.h), comments and whitespace removed, so a
    documentation edit keeps the counter figures and any code edit drops
    them."""
    import hashlib
    import re
    h = hashlib.sha256()
    for name in ("gemm_bf16.hip", "common.h"):
        text = open(os.path.join(ROOT, "qwen3_decoder_layer_amd", "csrc", name)).read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def traffic_bytes():
    """Measured HBM bytes per dominant-kernel launch, or None when no counter
    pass exists for the current kernel code."""
    if TRAFFIC is None or kernel_source_digest() != TRAFFIC["source_sha256"]:
        return None
    return TRAFFIC["bytes"]


def cpu_baseline(cfg: dict, budget_tokens: int) -> dict:
    """The fp64 oracle, untuned, on one sequence of `budget_tokens` tokens of
    the same layer (forward + backward when the workload has a backward)."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads", 1) for i in threadpool_info()),
                      default=1)
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    c = dict(cfg, B=1, L=budget_tokens)
    inp = synth.make_inputs(c, 1000 + 4, with_dy=cfg["backward"])
    p = {n: inp[n] for n in synth.PARAM_NAMES}
    t0 = time.perf_counter()
    if cfg["backward"]:
        oracle.layer_backward(c, p, inp["x"], inp["dy"])   # runs the forward too
    else:
        oracle.layer_forward(c, p, inp["x"])
    dt = time.perf_counter() - t0
    return {"value": budget_tokens / dt, "unit": "tokens/s", "cores": int(threads),
            "kind": "oracle",
            "sample": (f"1 sequence x {budget_tokens} tokens of the same layer "
                       f"(d={cfg['d']}, {cfg['h_q']}/{cfg['h_kv']} heads, "
                       f"d_ffn={cfg['d_ffn']}), numpy fp64, "
                       f"{'fwd+bwd' if cfg['backward'] else 'fwd'}, "
                       f"{dt:.1f} s")}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="qwen3-8b-bf16-fwd-bwd",
                    choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=4096,
                    help="tokens of the oracle sample (0: no CPU baseline)")
    ap.add_argument("--split-probe", action="store_true",
                    help="one forward and the backward as INPUT then "
                         "WEIGHT|DEFERRED_WEIGHT calls (for a kernel trace)")
    ap.add_argument("--kernel-probe", action="store_true",
                    help="only the calibration copy and the dominant kernel "
                         "(for hardware-counter passes)")
    args = ap.parse_args()
    if args.cpu_tokens < 0:
        ap.error("--cpu-tokens must be >= 0")
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not "
              "supported (the layer's local compute runs on a single device).",
              file=sys.stderr)
        sys.exit(2)
    if args.split_probe:
        split_probe(synth.preset(WORKLOADS[args.workload]))
        return
    if args.kernel_probe:
        kernel_probe(synth.preset(WORKLOADS[args.workload]))
        return
    cfg, inp = synth.preset_inputs(WORKLOADS[args.workload])
    res = gpu_run(cfg, inp, args.steps, args.warmup)
    fl = model_flops(cfg, cfg["backward"])
    T = cfg["B"] * cfg["L"]
    ms = res["elapsed"] / args.steps * 1e3
    tflops = fl["total"] / (ms * 1e-3) / 1e12
    fwd_work, bwd_work = phase_work(cfg)
    # The time between two of the library's marks also holds one gap between
    # the mark and the next kernel (the event's packet and the launch, about
    # 5 us here), which a kernel trace of the same phase does not count.  A
    # phase without kernels measures exactly that gap, so every phase time
    # below is its mark time less the median time of the run's empty phases
    # (kept as "ms_marks"), i.e. its kernels' time.
    empty = [t for times, work in ((res["fwd_phase_ms"], fwd_work),
                                   (res["bwd_phase_ms"], bwd_work))
             for name, t in times.items() if work[name][1] == 0]
    gap = float(np.median(empty)) if empty else 0.0
    phases = []
    for times, work in ((res["fwd_phase_ms"], fwd_work), (res["bwd_phase_ms"], bwd_work)):
        for name, tm in times.items():
            bound, amount = work[name]
            if name == "transposes for the backward" and cfg["backward"]:
                continue   # on the second stream, beside F5: no time of its own
            t = tm - gap
            if amount == 0 or t <= 0:
                continue
            if bound == "mfma":
                ach, peak, unit = amount / (t * 1e-3) / 1e12, PEAK_BF16_TFLOPS, "TFLOP/s"
            else:
                ach, peak, unit = amount / (t * 1e-3) / 1e9, PEAK_HBM_GBS, "GB/s"
            phases.append({"phase": name, "ms": round(float(t), 4),
                           "ms_marks": round(float(tm), 4), "bound": bound,
                           "work": int(amount), "achieved": round(float(ach), 1),
                           "unit": unit, "frac": round(float(ach / peak), 4)})
    dom = "F8-F9 gate/up gemm + swiglu"
    k_ms = float(res["fwd_phase_ms"][dom]) - gap
    k_flops, k_bytes = dominant_work(T, cfg["d"], cfg["d_ffn"])
    k_tflops = k_flops / (k_ms * 1e-3) / 1e12
    line = {
        "metric": METRIC,
        "value": T / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded: x, dy ~ N(0,1); projections ~ N(0,0.02); "
                "norm weights ~ 1+N(0,0.1); rounded to bf16)",
        "config": {"workload": cfg["name"], "d": cfg["d"], "h_q": cfg["h_q"],
                   "h_kv": cfg["h_kv"], "d_h": cfg["d_h"], "d_ffn": cfg["d_ffn"],
                   "B": cfg["B"], "L": cfg["L"], "tokens": T,
                   "pass": "fwd+bwd" if cfg["backward"] else "fwd",
                   "parallelism": "none (1 GPU)"},
        "tflops": tflops,
        "mfma_frac": tflops / PEAK_BF16_TFLOPS,
        "model_flops_per_step": fl["total"],
        "roofline": {"kernel": "gate/up GEMM + SwiGLU epilogue "
                               f"[{T}x{cfg['d']}] x [{2 * cfg['d_ffn']}x{cfg['d']}]^T",
                     "bound": "mfma", "achieved": k_tflops,
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": k_tflops / PEAK_BF16_TFLOPS,
                     "avg_ms": k_ms,
                     "timing": "median over the steps of the launch inside the step, "
                               "between HIP events the library records on its stream, "
                               "less the mark-to-kernel gap (phase_gap_ms)",
                     "algorithmic_bytes": k_bytes,
                     "traffic": traffic_bytes()},
        "phases": phases,
        "phase_gap_ms": round(gap, 4),
        "marked_ms_per_step": res["marked_elapsed"] / args.steps * 1e3,
    }
    if not args.no_cpu_baseline and args.cpu_tokens > 0:
        line["cpu_baseline"] = cpu_baseline(cfg, args.cpu_tokens)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
