"""Throughput of the fused attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--settle-s SECONDS] [--no-cpu-baseline]

A step is one mha_fwd call (scheduler prepass + attention kernel; with
--splits N > 1 also the split merge) over the whole workload, inputs
resident in HBM.  Default workload: bf16 causal
prefill, B=4, H=32, S=4096, D=128.  Prints one JSON line.  Before the W
warm-up steps, untimed steps run for --settle-s seconds (default 0.3), so
that the part has reached its steady speed; the JSON line reports them
under "settle".

value      attention TFLOP/s = metric FLOPs (4*B*H*S^2*D, halved for causal)
           / mean step time over the K timed steps;
roofline   the attention kernel against the dense MFMA peak of its dtype:
           achieved = metric FLOPs per launch / mean duration of the attention
           kernel itself (HIP events that the library records on the launch
           stream right before and after the kernel, mha_fwd_set_kernel_events;
           the scheduler prepass is outside them); traffic = HBM bytes per
           launch from the rocprofv3 FETCH_SIZE / WRITE_SIZE summary committed
           under profiles/ for this workload, scaled by the plain-copy
           calibration recorded there, or null when the kernel sources have
           changed since those counters were taken;
cpu_baseline  the float64 CPU oracle on a bounded sample of the same
           workload: whole (sequence, head) pairs, as many as fit in about
           10 s, rated with the same metric FLOPs.

    python bench.py --op quantize [--steps K] [--warmup W]
times the per-row fp8 quantiser (mha_quantize_fp8) on the fp8 workload's Q
(32768 tokens x 32 heads x 128, bf16) and prints its own JSON line: GB/s of
algorithmic HBM bytes (input read + codes and scales written) against the
8 TB/s HBM peak, with the CPU oracle quantiser timed on sampled rows.

    python bench.py --summarize-profile DIR --workload NAME
writes profiles/<kernel>_<workload>.md from the rocprofv3 output under DIR
(trace/, pmcA/, pmcB/, pmcC/ = FETCH_SIZE, pmcD/ = WRITE_SIZE, copy_fetch/,
copy_write/ = the same two counters on --copy-probe-mib 1024).
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
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


KERNEL = "attn_fwd_mfma_kernel"      # bf16 and fp8 Q/K
KERNEL_F32 = "attn_fwd_f32_kernel"   # float32
PROFILE_DIR = os.path.join(ROOT, "profiles")
COPY_PROBE_MIB = 1024


# the sources that decide what each attention kernel and its scheduler do on
# the device (kernels.h holds the queue chunk rule; the other entry points of
# the library do not matter)
KERNEL_SOURCES = {
    KERNEL: ("attn_bf16.hip", "attn_fp8.hip", "attn_mfma.h", "common.h", "kernels.h",
             "sched.hip"),
    KERNEL_F32: ("attn_f32.hip", "common.h", "kernels.h", "sched.hip"),
}


def kernel_of(dtype: str) -> str:
    return KERNEL_F32 if dtype == "f32" else KERNEL


def kernel_sources_sha256(kernel: str = KERNEL) -> str:
    """Hash of an attention kernel's sources: a traffic figure is valid for
    these only."""
    h = hashlib.sha256()
    src = os.path.join(ROOT, "head_attention_forward_fa_amd", "csrc")
    for f in KERNEL_SOURCES[kernel]:
        h.update(f.encode())
        with open(os.path.join(src, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def profile_path(workload: str, kernel: str = KERNEL) -> str:
    return os.path.join(PROFILE_DIR, f"{kernel}_{workload}.md")


def traffic_from_profile(workload: str, kernel: str = KERNEL):
    """HBM bytes per launch recorded for the current sources, else None."""
    path = profile_path(workload, kernel)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"sources_sha256=(\w+)\s+hbm_bytes_per_launch=([0-9.e+]+)", text)
    if not m or m.group(1) != kernel_sources_sha256(kernel):
        return None
    return float(m.group(2))


class HipEvents:
    """Timing events of the HIP runtime the process already uses (the same
    library instance that PyTorch and libmha_fwd.so share)."""

    def __init__(self):
        import ctypes
        self.ct = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float),
                                                 ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self):
        ev = self.ct.c_void_p()
        if self.hip.hipEventCreate(self.ct.byref(ev)) != 0:
            raise RuntimeError("hipEventCreate failed")
        return ev

    def elapsed_ms(self, a, b) -> float:
        ms = self.ct.c_float()
        if self.hip.hipEventElapsedTime(self.ct.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def destroy(self, ev):
        self.hip.hipEventDestroy(ev)




def peak_for(inp, fast_accum: bool = False) -> float:
    # fp8 codes decoded to bfloat16 (the default) run every product at the
    # bf16 rate
    if inp.dtype == "fp8" and fast_accum:
        # the nope QK^T runs at the fp8 rate, a rope QK^T and PV at the bf16
        # rate: time-weighted peak
        dn, dr, dv = inp.head_dim_nope, inp.head_dim_rope, inp.v_dim
        return (dn + dr + dv) / (dn / PEAK_TFLOPS["fp8"] + (dr + dv) / PEAK_TFLOPS["bf16"])
    if inp.dtype == "fp8":
        return PEAK_TFLOPS["bf16"]
    return PEAK_TFLOPS[inp.dtype]


def settle_clocks(step, seconds: float):
    """Run `step` untimed until `seconds` of wall time have passed, before
    the warm-up steps.  From a fresh process the part needs about a hundred
    launches of sustained load to reach its steady speed: on the causal B4
    H32 S4096 workload, 20 instrumented steps after 5 warm-up steps averaged
    584 us (664 us falling to 531 us), and 495 us after 300 untimed steps,
    so a few warm-up steps alone would time the ramp, not the kernel.
    Returns (steps, seconds)."""
    import torch
    n, t0, marks = 0, time.perf_counter(), []
    while True:
        for _ in range(8):
            step()
        n += 8
        # keep two chunks of steps queued, so that the device never idles
        marks.append(torch.cuda.Event())
        marks[-1].record()
        if len(marks) > 2:
            marks.pop(0).synchronize()
        if time.perf_counter() - t0 >= seconds:
            torch.cuda.synchronize()
            return n, time.perf_counter() - t0


def cpu_model() -> str:
    """The host CPU's model name and logical CPU count (Linux)."""
    try:
        with open("/proc/cpuinfo") as fh:
            names = [ln.split(":", 1)[1].strip() for ln in fh if ln.startswith("model name")]
    except OSError:
        names = []
    return f"{names[0] if names else 'unknown'} ({len(names) or os.cpu_count()} logical CPUs)"


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
    blas = [p for p in threadpool_info() if p.get("user_api") == "blas"]
    threads = max([p.get("num_threads", 1) for p in blas] or [1])
    vendor = ", ".join(sorted({f"{p.get('internal_api', '?')} {p.get('version', '')}".strip()
                               for p in blas})) or "none found"
    return {
        "value": flops / t_used / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "cpu_model": cpu_model(),
        "blas": vendor,
        "kind": "oracle",
        "sample": (f"{pairs} whole (sequence, head) pairs of {inp.name} "
                   f"({pairs}/{inp.batch * inp.num_heads} of the workload), float64 numpy, "
                   f"{t_used:.1f} s; the oracle builds the full LxL score matrix, i.e. twice "
                   f"the causal metric work"),
    }


def _csv_rows(d: str, suffix: str):
    files = glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no *{suffix} under {d}")
    with open(files[0]) as fh:
        return list(csv.DictReader(fh))


def _pmc_per_dispatch(d: str, kernel_substr: str):
    """Mean per-dispatch value of every counter of the matching kernel."""
    acc = {}
    for r in _csv_rows(d, "counter_collection.csv"):
        if kernel_substr in r["Kernel_Name"]:
            acc.setdefault(r["Counter_Name"], {}).setdefault(r["Dispatch_Id"], 0.0)
            acc[r["Counter_Name"]][r["Dispatch_Id"]] += float(r["Counter_Value"])
    return {c: sum(v.values()) / len(v) for c, v in acc.items()}


def summarize_profile(prof: str, workload: str) -> str:
    """profiles/<kernel>_<workload>.md from the rocprofv3 runs under prof."""
    inp = mi.workload(workload)
    KERNEL = kernel_of(inp.dtype)  # noqa: N806 (the profiled kernel)
    stats = _csv_rows(os.path.join(prof, "trace"), "kernel_stats.csv")
    krow = next(r for r in stats if KERNEL in r["Name"])
    prow = [r for r in stats if "sched_prepass" in r["Name"]]
    crow = [r for r in stats if "combine_splits" in r["Name"]]  # split-KV merge
    avg_ns = float(krow["AverageNs"])
    a = _pmc_per_dispatch(os.path.join(prof, "pmcA"), KERNEL)
    b = _pmc_per_dispatch(os.path.join(prof, "pmcB"), KERNEL)
    fetch = _pmc_per_dispatch(os.path.join(prof, "pmcC"), KERNEL)["FETCH_SIZE"]
    write = _pmc_per_dispatch(os.path.join(prof, "pmcD"), KERNEL)["WRITE_SIZE"]
    # dst.copy_(src) of one contiguous buffer is the runtime's copyBuffer kernel
    cf = _pmc_per_dispatch(os.path.join(prof, "copy_fetch"), "copyBuffer")["FETCH_SIZE"]
    cw = _pmc_per_dispatch(os.path.join(prof, "copy_write"), "copyBuffer")["WRITE_SIZE"]
    copy_kib = COPY_PROBE_MIB * 1024.0
    f_fetch, f_write = copy_kib / cf, copy_kib / cw
    hbm = (fetch * f_fetch + write * f_write) * 1024.0
    flops = mi.attention_flops(inp)
    peak = peak_for(inp)
    algo = algorithmic_bytes(inp)
    mfma_busy = a.get("SQ_VALU_MFMA_BUSY_CYCLES", float("nan"))
    busy_cu = b.get("SQ_BUSY_CU_CYCLES", float("nan"))
    gui = a.get("GRBM_GUI_ACTIVE", float("nan"))
    bank = b.get("SQ_LDS_BANK_CONFLICT", float("nan"))
    lds_active = b.get("SQ_LDS_IDX_ACTIVE", float("nan"))
    bench_cmd = f"python3 bench.py --steps 5 --warmup 2 --no-cpu-baseline --workload {workload}"
    lines = [
        f"# {KERNEL} on {workload}",
        "",
        "rocprofv3 on one MI355X (gfx950), launched from the repository root after",
        "`cd /tmp && export TMPDIR=/tmp`; P is the profile output directory:",
        "",
        "```",
        f"rocprofv3 --kernel-trace --stats -f csv -T -d $P/trace -o run -- {bench_cmd}",
        f"rocprofv3 --pmc SQ_WAVES SQ_BUSY_CYCLES SQ_WAVE_CYCLES SQ_INSTS_VALU SQ_INSTS_MFMA "
        f"SQ_VALU_MFMA_BUSY_CYCLES SQ_ACTIVE_INST_VALU SQ_INSTS_LDS GRBM_GUI_ACTIVE -f csv -T "
        f"-d $P/pmcA -o run -- {bench_cmd}",
        f"rocprofv3 --pmc SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE SQ_WAIT_INST_LDS SQ_WAIT_ANY "
        f"SQ_WAIT_INST_ANY SQ_ACTIVE_INST_ANY SQ_ACTIVE_INST_LDS SQ_BUSY_CU_CYCLES GRBM_GUI_ACTIVE "
        f"-f csv -T -d $P/pmcB -o run -- {bench_cmd}",
        f"rocprofv3 --pmc FETCH_SIZE -f csv -T -d $P/pmcC -o run -- {bench_cmd}",
        f"rocprofv3 --pmc WRITE_SIZE -f csv -T -d $P/pmcD -o run -- {bench_cmd}",
        f"rocprofv3 --pmc FETCH_SIZE -f csv -T -d $P/copy_fetch -o run -- "
        f"python3 bench.py --copy-probe-mib {COPY_PROBE_MIB}",
        f"rocprofv3 --pmc WRITE_SIZE -f csv -T -d $P/copy_write -o run -- "
        f"python3 bench.py --copy-probe-mib {COPY_PROBE_MIB}",
        f"python3 bench.py --summarize-profile $P --workload {workload}",
        "```",
        "",
        "## Kernel trace (stats)",
        "",
        "| kernel | calls | average ns | min ns | max ns |",
        "|---|---|---|---|---|",
        f"| {KERNEL} | {krow['Calls']} | {avg_ns:.0f} | {krow['MinNs']} | {krow['MaxNs']} |",
    ]
    for name, rows in (("sched_prepass_kernel", prow), ("combine_splits_kernel", crow)):
        for r in rows:
            lines.append(f"| {name} | {r['Calls']} | {float(r['AverageNs']):.0f} | "
                         f"{r['MinNs']} | {r['MaxNs']} |")
    lines += [
        "",
        f"Attention TFLOP/s at the trace average: {flops / (avg_ns * 1e-9) / 1e12:.1f} "
        f"({100 * flops / (avg_ns * 1e-9) / 1e12 / peak:.1f}% of {peak:.0f}).",
    ]
    if crow:
        step_ns = avg_ns + sum(float(r["AverageNs"]) for r in prow + crow)
        lines.append(f"With the key splits' merge and the prepass (trace averages, no launch "
                     f"gaps): {step_ns / 1e3:.1f} us, {flops / (step_ns * 1e-9) / 1e12:.1f} "
                     f"TFLOP/s.")
    lines += [
        "",
        "## Counters (per dispatch of the attention kernel, mean)",
        "",
        "| counter | value |",
        "|---|---|",
    ]
    for k2, v in sorted({**a, **b}.items()):
        lines.append(f"| {k2} | {v:.4g} |")
    lines += [
        f"| FETCH_SIZE (KiB) | {fetch:.6g} |",
        f"| WRITE_SIZE (KiB) | {write:.6g} |",
        "",
        f"MFMA busy per SIMD: SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x GRBM_GUI_ACTIVE / 8 XCDs) "
        f"= {mfma_busy / (1024 * gui / 8):.3f} (GRBM_GUI_ACTIVE adds up the 8 XCDs; "
        f"{gui / 8 / (avg_ns * 1e-9) / 1e9:.2f} GHz effective clock over the trace average); "
        f"LDS bank conflicts: SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE = {bank / lds_active:.4f}.",
        "",
        "## HBM traffic",
        "",
        f"Plain copy of {COPY_PROBE_MIB} MiB (device-to-device copyBuffer): FETCH_SIZE reads "
        f"{cf:.6g} KiB and WRITE_SIZE {cw:.6g} KiB per dispatch, so the scale factors are "
        f"{f_fetch:.4f} (fetch) and {f_write:.4f} (write).",
        "",
        f"Attention kernel: {fetch:.6g} KiB x {f_fetch:.4f} read + {write:.6g} KiB x "
        f"{f_write:.4f} written = {hbm / 1e6:.1f} MB per launch; algorithmic bytes "
        f"{algo / 1e6:.1f} MB (ratio {hbm / algo:.3f}); {hbm / (avg_ns * 1e-9) / 1e9:.0f} GB/s.",
        "",
        f"traffic: sources_sha256={kernel_sources_sha256(KERNEL)} "
        f"hbm_bytes_per_launch={hbm:.6e}",
        "",
    ]
    os.makedirs(PROFILE_DIR, exist_ok=True)
    out = profile_path(workload, KERNEL)
    with open(out, "w") as fh:
        fh.write("\n".join(lines))
    return out


def algorithmic_bytes(inp) -> float:
    """Compulsory HBM bytes of one launch: read Q (+rope, +scales), K, V once;
    write O and LSE once."""
    T, Hq, Hkv = inp.total_tokens, inp.num_heads, inp.num_kv_heads
    eqk = {"f32": 4, "bf16": 2, "fp8": 1}[inp.dtype]
    ev = 4 if inp.dtype == "f32" else 2
    b = T * Hq * inp.head_dim_nope * eqk + T * Hkv * inp.head_dim_nope * eqk
    b += T * (Hq + Hkv) * inp.head_dim_rope * 2
    b += T * Hkv * inp.v_dim * ev
    if inp.dtype == "fp8":
        b += T * (Hq + Hkv) * 4
    b += T * Hq * inp.v_dim * ev + T * Hq * 4
    return float(b)


QUANT_WORKLOAD = "fp8_quant_bf16_t32768_h32_d128"
HBM_PEAK_GBS = 8000.0


def bench_quantize(a, lib, dev) -> int:
    """Per-row fp8 quantiser on the fp8 workload's Q tensor (bf16 rows)."""
    import torch
    from head_attention_forward_fa_amd import _native, mha_quantize_fp8

    T, H, D = 32768, 32, 128
    x_np = mi.make_rows((T, H, D), dtype="bf16", seed=11, magnitude_sigma=0.5)
    x = torch.from_numpy(x_np.view(np.int16)).view(torch.bfloat16).to(dev)
    codes = torch.empty((T, H, D), dtype=torch.uint8, device=dev)
    scales = torch.empty((T, H), dtype=torch.float32, device=dev)
    rows = T * H
    nbytes = rows * D * 2 + rows * D + rows * 4  # read x, write codes and scales
    # kernel-only durations: the library records these HIP events right
    # before and after its launch (mha_fwd_set_kernel_events)
    hip = HipEvents()
    kev = [(hip.create(), hip.create()) for _ in range(a.steps)]
    settle = None
    if a.settle_s > 0:
        n, dt = settle_clocks(lambda: mha_quantize_fp8(x, codes=codes, scales=scales), a.settle_s)
        settle = {"steps": n, "seconds": round(dt, 3)}
    for _ in range(a.warmup):
        mha_quantize_fp8(x, codes=codes, scales=scales)
    torch.cuda.synchronize()
    for e0, e1 in kev:
        _native.check(lib.mha_fwd_set_kernel_events(e0, e1))
        mha_quantize_fp8(x, codes=codes, scales=scales)
    _native.check(lib.mha_fwd_set_kernel_events(None, None))
    torch.cuda.synchronize()
    ms = [hip.elapsed_ms(e0, e1) for e0, e1 in kev]
    for e0, e1 in kev:
        hip.destroy(e0)
        hip.destroy(e1)
    mean_ms = float(np.mean(ms))
    gbs = nbytes / (mean_ms * 1e-3) / 1e9
    print(f"[bench] quantise {rows} rows x {D}: {mean_ms * 1e3:.1f} us (min {min(ms) * 1e3:.1f}), "
          f"{gbs:.0f} GB/s, {100 * gbs / HBM_PEAK_GBS:.1f}% of {HBM_PEAK_GBS:.0f}",
          file=sys.stderr, flush=True)
    cpu = None
    if not a.no_cpu_baseline:
        from oracle import quantize as oq
        flat = x_np.reshape(rows, D)
        done, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < min(a.cpu_budget, 10.0) and done < rows:
            oq.quantize_bf16_rows(flat[done:done + 65536])
            done += min(65536, rows - done)
        dt = time.perf_counter() - t0
        cpu = {"value": round(done * (D * 3 + 4) / dt / 1e9, 4), "unit": "GB/s",
               "cores": 1, "kind": "oracle",
               "sample": f"first {done} of {rows} rows (numpy, one thread)"}
    line = {
        "metric": "fp8 per-row quantisation GB/s (bf16 read + codes and scales written)",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(mean_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 -> fp8-e4m3",
        "data": "synthetic",
        "config": {"workload": QUANT_WORKLOAD, "rows": rows, "cols": D,
                   "parallelism": "single-gpu"},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None},
        "cpu_baseline": cpu,
        "settle": settle,
    }
    print(json.dumps(line), flush=True)
    return 0


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--settle-s", type=float, default=0.3,
                    help="untimed steps for this many seconds before the warm-up steps, so "
                         "that the part reaches its steady speed (0: none)")
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD,
                    choices=mi.WORKLOAD_ORDER + list(mi.EXTRA_WORKLOADS))
    ap.add_argument("--splits", type=int, default=1,
                    help="split-KV: cut every query tile's keys into this many work items "
                         "(mha_fwd_splitkv) and merge")
    ap.add_argument("--fp8-fast-accum", action="store_true",
                    help="fp8 workloads: Q K^T on the fp8 matrix instruction "
                         "(MHA_DTYPE_FP8_E4M3_FASTACC, reduced accumulation precision) instead "
                         "of the exact default")
    ap.add_argument("--op", default="attention", choices=("attention", "quantize"))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=10.0)
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run a plain device-to-device copy of this many MiB (five "
                         "times), to calibrate HBM byte counters against a known size")
    ap.add_argument("--summarize-profile", default=None,
                    help="write the profiles/ summary from rocprofv3 output under this directory")
    a = ap.parse_args(argv)
    if a.summarize_profile:
        print(summarize_profile(a.summarize_profile, a.workload))
        return 0
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {a.gpus}): this path has no "
              "multi-GPU mode", file=sys.stderr)
        return 2

    import torch
    from head_attention_forward_fa_amd import mha_fwd
    from head_attention_forward_fa_amd import _native

    lib = _native.load()  # fail loudly if the HIP library is missing
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
    if a.op == "quantize":
        return bench_quantize(a, lib, dev)
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
    part = {}
    if a.splits > 1:
        part = dict(num_splits=a.splits,
                    o_partial=torch.empty((a.splits, inp.total_tokens, inp.num_heads, inp.v_dim),
                                          dtype=torch.float32, device=dev),
                    lse_partial=torch.empty((a.splits, inp.num_heads, inp.total_tokens),
                                            dtype=torch.float32, device=dev))

    fast = bool(a.fp8_fast_accum and inp.dtype == "fp8")

    def step():
        mha_fwd(q, k, v, causal=inp.causal, cu_seqlens=cu, max_seqlen=inp.max_seqlen,
                q_rope=qr, k_rope=kr, q_scale=qs, k_scale=ks,
                softmax_scale=inp.softmax_scale, out=o, lse=lse, fp8_fast_accum=fast, **part)

    # everything the timed region needs is set up first, so that nothing but
    # launches runs between the settling, the warm-up and the timed steps
    hip = HipEvents()
    kev = [(hip.create(), hip.create()) for _ in range(a.steps)]
    stream = torch.cuda.current_stream(dev)
    t_all0 = torch.cuda.Event(enable_timing=True)
    t_all1 = torch.cuda.Event(enable_timing=True)
    settle = None
    if a.settle_s > 0:
        n, dt = settle_clocks(step, a.settle_s)
        settle = {"steps": n, "seconds": round(dt, 3)}
        print(f"[bench] clocks settled: {n} untimed steps in {dt:.2f} s", file=sys.stderr,
              flush=True)
    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    t_all0.record(stream)
    for i in range(a.steps):
        _native.check(lib.mha_fwd_set_kernel_events(kev[i][0], kev[i][1]))
        step()
    t_all1.record(stream)
    _native.check(lib.mha_fwd_set_kernel_events(None, None))
    torch.cuda.synchronize()
    total_ms = t_all0.elapsed_time(t_all1)
    kernel_ms = [hip.elapsed_ms(s0, s1) for s0, s1 in kev]
    for s0, s1 in kev:
        hip.destroy(s0)
        hip.destroy(s1)
    ms_per_step = total_ms / a.steps
    kmean = float(np.mean(kernel_ms))
    if not (bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all())):
        print("[bench] non-finite output", file=sys.stderr)
        return 1

    flops = mi.attention_flops(inp)
    value = flops / (ms_per_step * 1e-3) / 1e12
    achieved = flops / (kmean * 1e-3) / 1e12
    peak = peak_for(inp, fast)
    traffic = traffic_from_profile(inp.name + ("_fastacc" if fast else ""), kernel_of(inp.dtype))
    print(f"[bench] {ms_per_step * 1e3:.1f} us/step, attention kernel mean {kmean * 1e3:.1f} us "
          f"(min {min(kernel_ms) * 1e3:.1f}), {value:.1f} TFLOP/s, {100 * achieved / peak:.1f}% "
          f"of {peak:.0f}", file=sys.stderr, flush=True)
    print("[bench] attention kernel per timed step (us): "
          + " ".join(f"{x * 1e3:.0f}" for x in kernel_ms), file=sys.stderr, flush=True)

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
        "dtype": {"bf16": "bf16", "f32": "f32",
                  "fp8": ("fp8-e4m3 QK / bf16 PV" if fast
                          else "fp8-e4m3 Q/K decoded to bf16 for QK, bf16 PV")}[inp.dtype],
        "data": "synthetic",
        "config": {
            "workload": inp.name + ("_fastacc" if fast else ""),
            "batch": inp.batch,
            "num_heads": inp.num_heads,
            "num_kv_heads": inp.num_kv_heads,
            "seq_len": inp.max_seqlen if len(set(inp.seqlens.tolist())) == 1 else "ragged",
            "total_tokens": inp.total_tokens,
            "head_dim_nope": inp.head_dim_nope,
            "head_dim_rope": inp.head_dim_rope,
            "v_dim": inp.v_dim,
            "causal": inp.causal,
            "num_splits": a.splits,
            "parallelism": "single-gpu",
        },
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": round(peak, 1),
            "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4),
            "traffic": None if traffic is None else round(traffic),
        },
        "cpu_baseline": cpu,
        "settle": settle,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
