"""Throughput of the fused attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--no-cpu-baseline]

A step is one mha_fwd call (scheduler prepass + attention kernel) over the
whole workload, inputs resident in HBM.  Default workload: bf16 causal
prefill, B=4, H=32, S=4096, D=128.  Prints one JSON line.

value      attention TFLOP/s = metric FLOPs (4*B*H*S^2*D, halved for causal)
           / mean step time over the K timed steps;
roofline   the attention kernel against the dense MFMA peak of its dtype:
           achieved = metric FLOPs per launch / mean launch duration (HIP
           events on the launch stream around each call, so it includes the
           few-microsecond prepass);
cpu_baseline  the float64 CPU oracle on a bounded sample of the same
           workload: whole (sequence, head) pairs, as many as fit in about
           10 s, rated with the same metric FLOPs.
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

import mha_inputs as mi  # noqa: E402

DEFAULT_WORKLOAD = "bf16_causal_b4_h32_s4096_d128"
METRIC = "attention fwd TFLOP/s (4·B·H·Sq·Sk·D, causal halved) and % of MFMA peak"
# MI355X dense matrix peaks (TFLOP/s) by the dtype of the products
PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "f32": 157.3}


def peak_for(inp) -> float:
    if inp.dtype == "fp8":
        # QK^T runs at the fp8 rate, PV at the bf16 rate: time-weighted peak
        dqk, dv = inp.head_dim_nope, inp.v_dim
        return (dqk + dv) / (dqk / PEAK_TFLOPS["fp8"] + dv / PEAK_TFLOPS["bf16"])
    return PEAK_TFLOPS[inp.dtype]


def cpu_baseline(inp, budget_s: float = 10.0):
    """Time the oracle (as it is) on whole (sequence, head) pairs."""
    import oracle
    from threadpoolctl import threadpool_info
    cu = inp.cu_seqlens.astype(np.int64)
    group = inp.num_heads // inp.num_kv_heads
    d = (inp.head_dim_nope + inp.head_dim_rope + inp.v_dim) / 2.0
    flops, pairs, t_used = 0.0, 0, 0.0
    for b in range(inp.batch):
        s0, s1 = int(cu[b]), int(cu[b + 1])
        L = s1 - s0
        if L == 0:
            continue
        for h in range(inp.num_heads):
            g = h // group
            sl = slice(s0, s1)
            if inp.dtype == "fp8":
                q = oracle.dequantize_per_token(inp.q[sl, h:h + 1], inp.q_scale[sl, h:h + 1])
                k = oracle.dequantize_per_token(inp.k[sl, g:g + 1], inp.k_scale[sl, g:g + 1])
            elif inp.dtype == "bf16":
                q, k = oracle.decode_bf16(inp.q[sl, h:h + 1]), oracle.decode_bf16(inp.k[sl, g:g + 1])
            else:
                q, k = inp.q[sl, h:h + 1].astype(np.float64), inp.k[sl, g:g + 1].astype(np.float64)
            v = (oracle.decode_bf16(inp.v[sl, g:g + 1]) if inp.dtype != "f32"
                 else inp.v[sl, g:g + 1].astype(np.float64))
            qr = kr = None
            if inp.q_rope is not None:
                qr = oracle.decode_bf16(inp.q_rope[sl, h:h + 1])
                kr = oracle.decode_bf16(inp.k_rope[sl, g:g + 1])
            t0 = time.perf_counter()
            oracle.mha_forward(q, k, v, np.array([0, L]), inp.causal, inp.softmax_scale,
                               q_rope=qr, k_rope=kr)
            t_used += time.perf_counter() - t0
            f = 4.0 * L * L * d
            flops += f / 2.0 if inp.causal else f
            pairs += 1
            if t_used >= budget_s:
                break
        if t_used >= budget_s:
            break
    threads = max([p.get("num_threads", 1) for p in threadpool_info()
                   if p.get("user_api") == "blas"] or [1])
    return {
        "value": flops / t_used / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"{pairs} whole (sequence, head) pairs of {inp.name} "
                   f"({pairs}/{inp.batch * inp.num_heads} of the workload), float64 numpy, "
                   f"{t_used:.1f} s; the oracle builds the full LxL score matrix, i.e. twice "
                   f"the causal metric work"),
    }


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=mi.WORKLOAD_ORDER)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=10.0)
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run a plain device-to-device copy of this many MiB (five "
                         "times), to calibrate HBM byte counters against a known size")
    a = ap.parse_args(argv)
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {a.gpus}): this path has no "
              "multi-GPU mode", file=sys.stderr)
        return 2

    import torch
    from head_attention_forward_fa_amd import mha_fwd
    from head_attention_forward_fa_amd import _native

    _native.load()  # fail loudly if the HIP library is missing
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if a.copy_probe_mib:
        n = a.copy_probe_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(f"[bench] copied {a.copy_probe_mib} MiB five times", file=sys.stderr)
        return 0
    inp = mi.workload(a.workload)
    print(f"[bench] workload {inp.name}: T={inp.total_tokens} Hq={inp.num_heads} "
          f"Hkv={inp.num_kv_heads} D={inp.head_dim_nope}+{inp.head_dim_rope}/{inp.v_dim}",
          file=sys.stderr, flush=True)

    def dev_bits(x, kind):
        if x is None:
            return None
        if kind == "bf16":
            return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)
        if kind == "fp8":
            return torch.from_numpy(x).view(torch.float8_e4m3fn).to(dev)
        return torch.from_numpy(x).to(dev)

    vk = "f32" if inp.dtype == "f32" else "bf16"
    q, k, v = dev_bits(inp.q, inp.dtype), dev_bits(inp.k, inp.dtype), dev_bits(inp.v, vk)
    qr, kr = dev_bits(inp.q_rope, vk), dev_bits(inp.k_rope, vk)
    qs = None if inp.q_scale is None else torch.from_numpy(inp.q_scale).to(dev)
    ks = None if inp.k_scale is None else torch.from_numpy(inp.k_scale).to(dev)
    cu = torch.from_numpy(inp.cu_seqlens).to(dev)
    o = torch.empty((inp.total_tokens, inp.num_heads, inp.v_dim),
                    dtype=torch.float32 if inp.dtype == "f32" else torch.bfloat16, device=dev)
    lse = torch.empty((inp.num_heads, inp.total_tokens), dtype=torch.float32, device=dev)

    def step():
        mha_fwd(q, k, v, causal=inp.causal, cu_seqlens=cu, max_seqlen=inp.max_seqlen,
                q_rope=qr, k_rope=kr, q_scale=qs, k_scale=ks,
                softmax_scale=inp.softmax_scale, out=o, lse=lse)

    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    if not (bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all())):
        print("[bench] non-finite output", file=sys.stderr)
        return 1

    stream = torch.cuda.current_stream(dev)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(a.steps)]
    t_all0 = torch.cuda.Event(enable_timing=True)
    t_all1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_all0.record(stream)
    for i in range(a.steps):
        ev[i][0].record(stream)
        step()
        ev[i][1].record(stream)
    t_all1.record(stream)
    torch.cuda.synchronize()
    total_ms = t_all0.elapsed_time(t_all1)
    launch_ms = [s.elapsed_time(e) for s, e in ev]
    ms_per_step = total_ms / a.steps
    kernel_ms = float(np.mean(launch_ms))

    flops = mi.attention_flops(inp)
    value = flops / (ms_per_step * 1e-3) / 1e12
    achieved = flops / (kernel_ms * 1e-3) / 1e12
    peak = peak_for(inp)
    print(f"[bench] {ms_per_step * 1e3:.1f} us/step, launch mean {kernel_ms * 1e3:.1f} us "
          f"(min {min(launch_ms) * 1e3:.1f}), {value:.1f} TFLOP/s, {100 * achieved / peak:.1f}% "
          f"of {peak:.0f}", file=sys.stderr, flush=True)

    cpu = None
    if not a.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        cpu = cpu_baseline(inp, a.cpu_budget)

    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"bf16": "bf16", "fp8": "fp8-e4m3 QK / bf16 PV", "f32": "f32"}[inp.dtype],
        "data": "synthetic",
        "config": {
            "workload": inp.name,
            "batch": inp.batch,
            "num_heads": inp.num_heads,
            "num_kv_heads": inp.num_kv_heads,
            "seq_len": inp.max_seqlen if len(set(inp.seqlens.tolist())) == 1 else "ragged",
            "total_tokens": inp.total_tokens,
            "head_dim_nope": inp.head_dim_nope,
            "head_dim_rope": inp.head_dim_rope,
            "v_dim": inp.v_dim,
            "causal": inp.causal,
            "parallelism": "single-gpu",
        },
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": round(peak, 1),
            "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4),
            "traffic": None,
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
