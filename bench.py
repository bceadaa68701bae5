#!/usr/bin/env python3
"""Throughput of the attention backward on one MI355X.

One step = one pass of the whole backward hot path over the workload:
fa_bwd_preprocess (D pre-pass, zeroes the dQ accumulator) then fa_bwd (the
KV-outer MFMA kernel with fp32-atomic dQ, then the dQ conversion; or, in
deterministic mode, the KV-outer kernel and the Q-outer dQ kernel).  Q, K, V,
dO and the forward's O and L are resident in HBM before timing starts.

Default workload: causal bf16, B=4, H=16, N=4096, d=128, sm_scale=1/sqrt(d),
Q, K, V, dO ~ N(0,1) (seeded, synthetic).  The line printed reports credited
TFLOP/s (10 d FLOPs per visible pair), the roofline of the dominant launch
(fa_bwd, timed with HIP events on the stream it runs on) against the bf16
dense MFMA peak, and the CPU oracle timed on one head of the same workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--mode atomic|deterministic]
                       [--workload NAME] [--dropout-p P] [--no-cpu-baseline] [--side-checks]
"""

import argparse
import ctypes
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # 256 CU x 2.4 GHz x 4096 dense bf16 (= fp16) FLOP/clk/CU
PEAK_HBM_GBS = 8000.0
KERNEL_SOURCES = ["flashattention_backward_pass_fa_amd/csrc/fa_kv128.hip",
                  "flashattention_backward_pass_fa_amd/csrc/fa_bwd16.hip",
                  "flashattention_backward_pass_fa_amd/csrc/fa_bwd_common.h",
                  "flashattention_backward_pass_fa_amd/csrc/fa_prep.hip",
                  "flashattention_backward_pass_fa_amd/csrc/fa_device.h",
                  "flashattention_backward_pass_fa_amd/build.py"]
TRAFFIC_FILE = "profiles/fa_bwd_{mode}_train_causal_bf16_traffic.md"
KERNELS_FILE = "profiles/fa_bwd_train_causal_bf16_kernels.md"
CLOCK_FILE = "profiles/fa_bwd_train_causal_bf16_clock.md"
PEAK_CLOCK_MHZ = 2400.0     # the clock PEAK_BF16_TFLOPS is quoted at
COPY_CALIBRATION_BYTES = 256 << 20   # one plain device copy, for HBM counter calibration


def kernel_source_hash():
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(mode):
    """HBM bytes per fa_bwd launch from the committed counter summary, if it
    was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, TRAFFIC_FILE.format(mode=mode))
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"kernel_source_hash:\s*([0-9a-f]+)", text)
    m_bytes = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_hash or not m_bytes or m_hash.group(1) != kernel_source_hash():
        return None
    return float(m_bytes.group(1))


def _profile_text(rel):
    """A committed profile summary, if it was taken on the current kernel source."""
    path = os.path.join(ROOT, rel)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"kernel_source_hash:\s*([0-9a-f]+)", text)
    return text if m_hash and m_hash.group(1) == kernel_source_hash() else None


def profiled_kernel_ms(mode):
    """Average duration (ms) of each kernel of one fa_bwd launch in the
    committed kernel-trace summary of the default workload, or None."""
    text = _profile_text(KERNELS_FILE)
    if text is None:
        return None
    names = (["dkdv_ws_kernel<128, false>", "dq_kernel<128, false>"] if mode == "deterministic"
             else ["dkdv_atomic_kernel<128>", "dq_convert_kernel"])
    out = {}
    for line in text.splitlines():
        cells = [c.strip().strip("`") for c in line.split("|")]
        if len(cells) > 4:
            for n in names:
                if cells[1].startswith(n):
                    out[n] = round(float(cells[3]) / 1000.0, 4)
    return out if len(out) == len(names) else None


def profiled_clock_mhz():
    """Shader clock under the backward's load, from the committed counter run
    (cycles over the same dispatches' durations), or None."""
    text = _profile_text(CLOCK_FILE)
    m = re.search(r"clock_mhz_under_load:\s*([0-9.]+)", text or "")
    return float(m.group(1)) if m else None


def device_max_clock_mhz(torch):
    """The peak engine clock the HIP runtime reports for device 0 (MHz)."""
    try:
        lib = ctypes.CDLL(os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so"))
        val = ctypes.c_int(0)
        if lib.hipDeviceGetAttribute(ctypes.byref(val), 5, 0) == 0:  # hipDeviceAttributeClockRate (kHz)
            return val.value / 1000.0
    except OSError:
        pass
    return None


def device_info(torch, dev):
    """Name, architecture and CU count as torch reports them."""
    p = torch.cuda.get_device_properties(dev)
    return {"name": p.name, "arch": p.gcnArchName.split(":")[0], "compute_units": p.multi_processor_count}


def cpu_baseline(w, host):
    """The fp64 oracle on one head of the workload, on this host's cores."""
    import oracle
    threads = None
    try:
        from threadpoolctl import threadpool_info
        threads = max((p.get("num_threads") or 0) for p in threadpool_info()) or None
    except Exception:
        pass
    spec = oracle.Spec(sm_scale=w.sm_scale, causal=w.causal, window_left=w.window_left,
                       window_right=w.window_right, dropout_p=w.dropout_p, seed=w.drop_seed,
                       offset=w.drop_offset)
    # heads in order until about 10 s of CPU work (at least one, at most all)
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    done = 0
    t0 = time.perf_counter()
    for b, h in heads:
        oracle.head_backward(host["q"][b, h], host["k"][b, h], host["v"][b, h],
                             host["do"][b, h], spec, b, h, chunk=512)
        done += 1
        if time.perf_counter() - t0 >= 10.0:
            break
    secs = time.perf_counter() - t0
    from flashattention_backward_pass_fa_amd.flops import credited_flops
    flops_head = credited_flops(1, 1, w.N, w.d, w.causal, w.window_left, w.window_right)
    cores = len(os.sched_getaffinity(0))
    return {"value": done * flops_head / secs / 1e12, "unit": "TFLOP/s",
            "cores": threads or cores, "kind": "oracle",
            "sample": f"{done} of {len(heads)} (b,h) heads, fp64 numpy backward with S, P, dS "
                      f"materialised, {secs:.2f} s; BLAS threads {threads}, host affinity {cores}"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--mode", choices=["atomic", "deterministic"], default="deterministic")
    ap.add_argument("--workload", default="train_causal_bf16")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--dropout-p", type=float, default=None,
                    help="override the workload's dropout probability (counter runs compare "
                         "the same shape with and without the keep mask)")
    ap.add_argument("--side-checks", action="store_true",
                    help="also time fa_fwd, the non-causal backward at the same shape and the "
                         "same tokens packed as variable-length sequences (kept out of the "
                         "default run so its kernel averages stay those of the timed backward)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (--gpus {args.gpus} requested): every (b, h) of "
              "the backward is independent, so G GPUs would each run these kernels on B*H/G heads; "
              "what is measured here is one GPU's share", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from flashattention_backward_pass_fa_amd import binding as fa
    from flashattention_backward_pass_fa_amd.flops import (algorithmic_bytes, credited_flops,
                                                          tile_fraction)
    from flashattention_backward_pass_fa_amd.inputs import WORKLOADS, make_workload_inputs

    w = WORKLOADS[args.workload]
    if args.dropout_p is not None:
        import dataclasses
        w = dataclasses.replace(w, dropout_p=args.dropout_p)
    if w.dtype not in ("bf16", "f16"):
        print("bench.py measures the 16-bit (bf16, fp16) workloads", file=sys.stderr)
        sys.exit(2)
    tdtype, code = ((torch.bfloat16, fa.FA_DTYPE_BF16) if w.dtype == "bf16"
                    else (torch.float16, fa.FA_DTYPE_F16))
    dev = torch.device("cuda:0")
    host = make_workload_inputs(w)
    t = {n: torch.from_numpy(host[n + "_bits"].view(np.int16)).view(tdtype).to(dev)
         for n in ("q", "k", "v", "do")}
    kw = dict(sm_scale=w.sm_scale, causal=w.causal, window=(w.window_left, w.window_right),
              dropout_p=w.dropout_p, seed=w.drop_seed, offset=w.drop_offset)
    o, lse = fa.forward(t["q"], t["k"], t["v"], **kw)

    def measure(mode):
        """Time `args.steps` steps of the backward in dQ mode `mode`."""
        deterministic = mode == "deterministic"
        params = fa.make_params(w.shape, code, deterministic=deterministic, **kw)
        ws_bytes = fa.fa_bwd_workspace_bytes(params)
        ws = torch.empty(max(ws_bytes // 4, 1), dtype=torch.float32, device=dev)
        ws_ptr = ctypes.c_void_p(ws.data_ptr() if ws_bytes else 0)
        delta = torch.empty(w.shape[:3], dtype=torch.float32, device=dev)
        dq, dk, dv = (torch.empty_like(t["q"]) for _ in range(3))
        T = fa.tensor_arg
        args_pre = (params, T(o), T(t["do"]), ctypes.c_void_p(delta.data_ptr()), ws_ptr)
        args_bwd = (params, T(t["q"]), T(t["k"]), T(t["v"]), T(t["do"]),
                    ctypes.c_void_p(lse.data_ptr()), ctypes.c_void_p(delta.data_ptr()),
                    T(dq), T(dk), T(dv), ws_ptr)
        stream = torch.cuda.current_stream(dev)
        st = ctypes.c_void_p(stream.cuda_stream)

        def step(ev=None):
            if ev is not None:
                ev[0].record(stream)
            s1 = fa.fa_bwd_preprocess(*args_pre, st)
            if ev is not None:
                ev[1].record(stream)
            s2 = fa.fa_bwd(*args_bwd, st)
            if ev is not None:
                ev[2].record(stream)
            if s1 or s2:
                raise RuntimeError(f"library status {s1}/{s2}")

        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)]
                  for _ in range(args.steps)]
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        wall0 = time.perf_counter()
        start.record(stream)
        for i in range(args.steps):
            step(events[i])
        end.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - wall0
        return {"ms_per_step": start.elapsed_time(end) / args.steps,
                "pre_ms": [e[0].elapsed_time(e[1]) for e in events],
                "bwd_ms": [e[1].elapsed_time(e[2]) for e in events],
                "step_ms": sorted(e[0].elapsed_time(e[2]) for e in events),
                "wall": wall, "ws_bytes": ws_bytes, "deterministic": deterministic}

    main_run = measure(args.mode)
    other_mode = "atomic" if args.mode == "deterministic" else "deterministic"
    other_run = measure(other_mode)

    def time_calls(fn, n):
        """Average ms of n calls of fn on the stream (after one untimed call)."""
        stream = torch.cuda.current_stream(dev)
        fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    # Forward (fa_fwd) on the same inputs: the pages compare the two passes'
    # FLOPs (backward ~2.5x) and speed.
    n_side = max(3, args.steps // 3)
    fwd_ms = nc_ms = None
    if args.side_checks:
        fwd_ms = time_calls(lambda: fa.forward(t["q"], t["k"], t["v"], **kw), n_side)
    # Mask tile skipping: the same backward without the causal mask (its own
    # forward for O and L), whose time should be ~2x the causal one.
    if args.side_checks and w.causal:
        kw_nc = dict(kw, causal=False)
        o_nc, lse_nc = fa.forward(t["q"], t["k"], t["v"], **kw_nc)
        nc_ms = time_calls(lambda: fa.backward(t["q"], t["k"], t["v"], o_nc, t["do"], lse_nc,
                                               deterministic=args.mode == "deterministic", **kw_nc),
                           n_side)
        del o_nc, lse_nc
    # Varlen: the same B * N tokens per head repacked as sequences of mixed
    # length (seeded, 256..N each, the last one cut to fit), with the
    # workload's mask applied per sequence; credited with those sequences'
    # visible pairs.
    vl = None
    if args.side_checks:
        from flashattention_backward_pass_fa_amd.inputs import cumulative, pack_lengths
        total = w.B * w.N
        lens = pack_lengths(total, 256, w.N, w.seed + 100)
        cu = torch.from_numpy(cumulative(lens)).to(dev)
        pk = {n: t[n].permute(0, 2, 1, 3).reshape(total, w.H, w.d).contiguous()
              for n in ("q", "k", "v", "do")}
        o_v, lse_v = fa.forward_varlen(pk["q"], pk["k"], pk["v"], cu, cu, max(lens), max(lens), **kw)
        # the same two C calls as the timed step, arguments built once
        vp = fa.make_params((len(lens), w.H, max(lens), w.d), code,
                            deterministic=args.mode == "deterministic", seqlen_k=max(lens),
                            cu_seqlens_q=cu.data_ptr(), cu_seqlens_k=cu.data_ptr(), **kw)
        v_ws_bytes = fa.fa_bwd_workspace_bytes(vp)
        v_ws = torch.empty(max(v_ws_bytes // 4, 1), dtype=torch.float32, device=dev)
        v_ws_ptr = ctypes.c_void_p(v_ws.data_ptr() if v_ws_bytes else 0)
        v_delta = torch.empty((len(lens), w.H, max(lens)), dtype=torch.float32, device=dev)
        v_out = [torch.empty_like(pk["q"]) for _ in range(3)]
        T = fa.tensor_arg
        v_pre = (vp, T(o_v), T(pk["do"]), ctypes.c_void_p(v_delta.data_ptr()), v_ws_ptr)
        v_bwd = (vp, T(pk["q"]), T(pk["k"]), T(pk["v"]), T(pk["do"]),
                 ctypes.c_void_p(lse_v.data_ptr()), ctypes.c_void_p(v_delta.data_ptr()),
                 *(T(x) for x in v_out), v_ws_ptr)
        v_st = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)

        def varlen_step():
            if fa.fa_bwd_preprocess(*v_pre, v_st) or fa.fa_bwd(*v_bwd, v_st):
                raise RuntimeError("varlen backward failed")

        vl_ms = time_calls(varlen_step, n_side)
        vl_flops = sum(credited_flops(1, w.H, n, w.d, w.causal, w.window_left, w.window_right)
                       for n in lens)
        vl = {"sequences": len(lens), "length_min_max": [min(lens), max(lens)], "tokens": total,
              "step_ms": round(vl_ms, 4), "tflops": round(vl_flops / (vl_ms * 1e-3) / 1e12, 2)}
        del pk, o_v, lse_v, v_ws, v_delta, v_out
    deterministic = main_run["deterministic"]
    ms_per_step = main_run["ms_per_step"]
    pre_ms, bwd_ms, step_ms = main_run["pre_ms"], main_run["bwd_ms"], main_run["step_ms"]
    ws_bytes, wall = main_run["ws_bytes"], main_run["wall"]

    flops = credited_flops(w.B, w.H, w.N, w.d, w.causal, w.window_left, w.window_right)
    tflops = flops / (ms_per_step * 1e-3) / 1e12
    bwd_avg = sum(bwd_ms) / len(bwd_ms)
    achieved = flops / (bwd_avg * 1e-3) / 1e12
    # the committed profile summaries cover the default workload only
    profiled = w.name == "train_causal_bf16" and args.dropout_p is None
    traffic = measured_traffic(args.mode) if profiled else None
    pre_avg = sum(pre_ms) / len(pre_ms)
    pre_bytes = 2 * w.B * w.H * w.N * w.d * 2 + 4 * w.B * w.H * w.N + ws_bytes

    line = {
        "metric": ("attention-backward TFLOP/s (bf16, causal) and % of MI355X bf16 MFMA peak"
                   if w.dtype == "bf16" else
                   "attention-backward TFLOP/s (fp16, causal) and % of MI355X fp16 MFMA peak"),
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d,
                   "causal": w.causal, "window": [w.window_left, w.window_right],
                   "dropout_p": w.dropout_p, "dq_mode": args.mode},
        "pct_of_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic,
                     "kernel": "fa_bwd launch (KV-outer MFMA kernel"
                               + (" + Q-outer dQ kernel)" if deterministic else " + dQ conversion)")},
        "kernels_ms": {"fa_bwd_preprocess": round(pre_avg, 4), "fa_bwd": round(bwd_avg, 4)},
        "preprocess_GBps": round(pre_bytes / (pre_avg * 1e-3) / 1e9, 1),
        "step_ms_min_median_p90": [round(step_ms[0], 4), round(step_ms[len(step_ms) // 2], 4),
                                   round(step_ms[int(0.9 * (len(step_ms) - 1))], 4)],
        "credited_flops": flops,
        "algorithmic_bytes": algorithmic_bytes(w.B, w.H, w.N, w.d),
        "tile_fraction_128": round(tile_fraction(w.N, w.causal, w.window_left, w.window_right, 128, 128), 6),
        "wall_s_timed": round(wall, 3),
        "other_mode": {"dq_mode": other_mode,
                       "ms_per_step": round(other_run["ms_per_step"], 4),
                       "value": round(flops / (other_run["ms_per_step"] * 1e-3) / 1e12, 2)},
        "device": device_info(torch, dev),
    }
    # The peak above is quoted at 2.4 GHz; under this load the shader clock
    # runs lower.  The device's reported peak clock, the clock the committed
    # counter run measured on these kernels, and the peak at that clock.
    max_mhz = device_max_clock_mhz(torch)
    load_mhz = profiled_clock_mhz() if profiled else None
    line["clock"] = {"device_max_mhz": max_mhz, "under_load_mhz": load_mhz,
                     "source": CLOCK_FILE if load_mhz else None}
    if load_mhz:
        peak_clk = PEAK_BF16_TFLOPS * load_mhz / PEAK_CLOCK_MHZ
        line["roofline_at_clock"] = {"peak": round(peak_clk, 1), "achieved": round(achieved, 2),
                                     "frac": round(achieved / peak_clk, 4),
                                     "value_frac": round(tflops / peak_clk, 4)}
    split = profiled_kernel_ms(args.mode) if profiled else None
    if split:
        line["kernels_ms_profiled"] = dict(split, source=KERNELS_FILE)
    fwd_flops = flops * 4 / 10  # forward: S and O products, 4 d per visible pair
    if fwd_ms is not None:
        line["forward"] = {"ms": round(fwd_ms, 4), "tflops": round(fwd_flops / (fwd_ms * 1e-3) / 1e12, 2),
                           "bwd_over_fwd_time": round(ms_per_step / fwd_ms, 3), "bwd_over_fwd_flops": 2.5}
    if nc_ms is not None:
        line["causal_skip_check"] = {"noncausal_step_ms": round(nc_ms, 4),
                                     "causal_over_noncausal_time": round(ms_per_step / nc_ms, 3),
                                     "visible_fraction": round(flops / credited_flops(w.B, w.H, w.N, w.d), 4)}
    if vl is not None:
        vl["tflops_over_fixed"] = round(vl["tflops"] / tflops, 3)
        line["varlen_check"] = vl
    # A plain copy of known size (outside the timed region): profiling runs
    # use its FETCH_SIZE / WRITE_SIZE to calibrate the HBM byte counters.
    src = torch.empty(COPY_CALIBRATION_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, host)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
