#!/usr/bin/env python3
"""Benchmark of the MI355X FP4 MoE feed-forward layer: one step = one moe_layer_forward
(router, top-K, dispatch, experts, blend) over one batch of synthetic input.

Prints ONE JSON line on stdout (logs go to stderr):
  value      whole-job MoE-layer tokens/s (inputs resident in HBM before timing)
  roofline   the dominant kernel's achieved GB/s (decode, HBM-bound) or TFLOP/s
             (prefill, MFMA-bound) against the MI355X peak, its duration measured with
             HIP events recorded on the kernel's own stream during the timed steps
  cpu_baseline  the CPU oracle timed on the host on a bounded sample of the workload

The default workload is the 4096-token prefill layer with Zipf-skewed expert loads (hidden
4096, 64 MXFP4 experts, top-6); --workload selects the others. With the default workload
the line also carries a compact entry per other workload ("other_workloads": step time,
tokens/s, the dominant kernel's roofline fraction). Steps cycle through several weight
sets and input batches so that weights are streamed from HBM rather than re-read from
the 256 MB Infinity Cache.
"""
from __future__ import annotations

import argparse
import statistics
import ctypes
import gc
import hashlib
import json
import os
import platform
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s; decode HBM GB/s & prefill MFMA TFLOP/s vs peak"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PROFILE_DIR = os.path.join(ROOT, "profiles")
HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000

DESCRIPTIONS = {
    "tiny": "Tiny MoE layer: 4 tokens, hidden 256, 8 experts, top_k=2, softmax, inter 512, NVFP4",
    "qwen3_decode_t1": "Decode, Qwen3-30B-A3B-like: 1 token, hidden 2048, 128 experts, top_k=8, "
                       "softmax renormalised, inter 768, NVFP4",
    "qwen3_decode_t8": "Decode, Qwen3-30B-A3B-like: 8 tokens, hidden 2048, 128 experts, top_k=8, "
                       "softmax renormalised, inter 768, NVFP4",
    "dsv3_decode_t32": "Decode, DeepSeek-V3-like: 32 tokens, hidden 7168, 256 experts, top_k=8, "
                       "sigmoid + correction bias, 1 shared expert, inter 2048, NVFP4",
    "prefill_zipf_t4096": "Prefill grouped GEMM: 4096 tokens, hidden 4096, 64 experts, top_k=6, "
                          "softmax with Zipf(1.1) logit bias, inter 1408, MXFP4",
    "hash_mxfp4_t512": "Hash-routed layer: 512 tokens, vocab 32768, hidden 4096, 256 experts, "
                       "top_k=6, inter 2048, MXFP4 routed + NVFP4 shared expert, RMSNorm input",
}
# weight sets cycled per step: enough distinct weights that the touched experts do not
# stay resident in the 256 MB Infinity Cache between steps
WEIGHT_SETS = {"tiny": 1, "qwen3_decode_t1": 4, "qwen3_decode_t8": 4, "dsv3_decode_t32": 1,
               "prefill_zipf_t4096": 2, "hash_mxfp4_t512": 1}
# oracle sample: tokens of one batch evaluated by the CPU oracle for the baseline
CPU_SAMPLE_TOKENS = {"tiny": 4, "qwen3_decode_t1": 1, "qwen3_decode_t8": 8,
                     "dsv3_decode_t32": 2, "prefill_zipf_t4096": 8, "hash_mxfp4_t512": 8}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def bytes_per_elem(fmt):
    """Storage bytes per weight element with its scales: NVFP4, MXFP4, FP8 (fp32 per
    128 x 128 block), BF16."""
    return [0.5 + 1.0 / 16, 0.5 + 1.0 / 32, 1.0 + 4.0 / (128 * 128), 2.0][fmt]


class HipEvents:
    """Raw HIP events through the runtime library torch already loaded."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p),
                                                     ctypes.c_uint]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float),
                                                 ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self):
        ev = ctypes.c_void_p()
        # timing-only events: no system-scope fence (cache writeback/invalidate) when the
        # event is recorded, which would otherwise be timed as part of the kernel
        if self.lib.hipEventCreateWithFlags(ctypes.byref(ev), HIP_EVENT_DISABLE_SYSTEM_FENCE) != 0:
            raise RuntimeError("hipEventCreate failed")
        return ev.value

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        if self.lib.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a),
                                        ctypes.c_void_p(b)) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def destroy(self, ev):
        self.lib.hipEventDestroy(ctypes.c_void_p(ev))


_CODE_TOKENS = re.compile(r'//[^\n]*|/\*.*?\*/|"(?:\\.|[^"\\])*"|\'(?:\\.|[^\'\\])*\'', re.S)


def _code_only(text):
    """C/C++ source without comments and with whitespace collapsed (string and character
    literals kept), so that edits of comments leave the digest unchanged."""
    text = _CODE_TOKENS.sub(lambda m: " " if m.group(0)[0] == "/" else m.group(0), text)
    return " ".join(text.split())


def source_digest():
    """Digest of the kernels' sources (comments and layout excluded)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "mixture_experts_ffn_03_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), encoding="utf-8") as fh:
            h.update(f.encode() + _code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def load_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` from rocprofv3 FETCH_SIZE/WRITE_SIZE counters
    (profiles/traffic_<workload>.json), or None if absent or taken on other sources."""
    p = os.path.join(PROFILE_DIR, f"traffic_{workload}.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        d = json.load(f)
    k = d.get("kernels", {}).get(kernel)
    if not k or d.get("source_digest") != source_digest():
        return None
    return k.get("bytes_per_launch")


def _rocprof_rows(d, suffix):
    import csv
    import glob
    rows = []
    for p in sorted(glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True)):
        with open(p) as f:
            rows.extend(csv.DictReader(f))
    if not rows:
        raise SystemExit(f"no *{suffix} under {d}")
    return rows


def summarize_trace(d, command):
    """Markdown table of a `rocprofv3 --kernel-trace --stats --output-format csv` run."""
    rows = [r for r in _rocprof_rows(d, "kernel_stats.csv") if "moe::" in r["Name"]]
    total = sum(float(r["TotalDurationNs"]) for r in rows)
    out = ["# rocprofv3 kernel statistics", "", "Command:", "", "    " + command, "",
           "Library kernels only (the input generator's torch kernels are left out); every "
           "call of the run is counted, warm-up and routing passes included.", "",
           "| kernel | calls | avg us | min us | max us | share |",
           "|---|---:|---:|---:|---:|---:|"]
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        name = r["Name"].split("(")[0]
        out.append(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                   f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                   f"{float(r['TotalDurationNs']) / total:.1%} |")
    # the routed experts' launches alone (a kernel symbol may also serve the shared expert)
    trace = [r for r in _rocprof_rows(d, "kernel_trace.csv") if "moe::" in r["Kernel_Name"]]
    trace.sort(key=lambda r: int(r["Start_Timestamp"]))
    dur = {"gate_up": [], "down": []}
    stage, stream = None, None

    def us(r):
        return (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3

    for r in trace:
        name, sid = r["Kernel_Name"], r.get("Stream_Id")
        if "k_dispatch" in name:  # (also k_topk_dispatch)
            stage, stream = 0, sid
        elif "k_dec_one_topk" in name:  # one token: the dispatch runs inside gate+up
            dur["gate_up"].append(us(r))
            stage, stream = 1, sid
        elif stage is not None and stage < 2 and sid == stream and \
                ("k_dec_" in name or "k_pre_gemm" in name):
            dur["gate_up" if stage == 0 else "down"].append(us(r))
            stage += 1
    out += ["", "Routed experts' launches only (the first two expert kernels after each dispatch "
            "build on the layer's stream; a shared expert runs on a side stream):", "",
            "| stage | launches | avg us | min us | max us |", "|---|---:|---:|---:|---:|"]
    for k, v in dur.items():
        if v:
            out.append(f"| {k} | {len(v)} | {sum(v) / len(v):.2f} | {min(v):.2f} | {max(v):.2f} |")
    return "\n".join(out) + "\n"


# the routed experts' kernels of one layer call, in launch order after the dispatch build
_ROUTED_KERNELS = {"decode": ("k_dec_", "k_dec_"),
                   "prefill": ("k_pre_gemm", "k_pre_gemm")}


def _dispatch_id(r):
    return int(next(v for k, v in r.items() if k.lower() == "dispatch_id"))


def _routed_counter(d, path):
    """Mean counter value (KiB) per dispatch of the routed gate+up and down kernels: the
    first two expert kernels after each dispatch build, or the one-token gate+up that builds
    it and the kernel after it (shared-expert launches are enqueued before the dispatch)."""
    rows = _rocprof_rows(d, "counter_collection.csv")
    per = {}
    for r in rows:  # one row per (dispatch, counter); sum over counter instances
        k = _dispatch_id(r)
        e = per.setdefault(k, [r["Kernel_Name"], 0.0])
        e[1] += float(r["Counter_Value"])
    want = _ROUTED_KERNELS[path]
    got = {"gate_up": [], "down": []}
    stage = None
    for k in sorted(per):
        name, v = per[k]
        if "k_dispatch" in name:  # (also k_topk_dispatch)
            stage = 0
        elif "k_dec_one_topk" in name:  # one token: the dispatch runs inside gate+up
            got["gate_up"].append(v)
            stage = 1
        elif stage is not None and stage < 2 and want[stage] in name:
            got["gate_up" if stage == 0 else "down"].append(v)
            stage += 1
    return {s: (sum(v) / len(v), len(v)) for s, v in got.items() if v}


def _copy_counter(d):
    rows = _rocprof_rows(d, "counter_collection.csv")
    per = {}
    for r in rows:
        k = _dispatch_id(r)
        per[k] = per.get(k, 0.0) + float(r["Counter_Value"])
    top = max(per.values())
    vals = [v for v in per.values() if v >= 0.5 * top]  # the 1 GiB copies, not small ones
    return sum(vals) / len(vals)


def summarize_traffic(d, workload, path, commands):
    """profiles/traffic_<workload>.json from four rocprofv3 --pmc runs under `d`:
    fetch/ and write/ (FETCH_SIZE, WRITE_SIZE of bench.py on the workload) and
    copy_fetch/, copy_write/ (the same counters on 1 GiB device copies). Each counter is
    scaled so that the copy kernel reads as 1 GiB fetched and 1 GiB written."""
    copy_bytes = float(1 << 30)
    f_copy, w_copy = _copy_counter(os.path.join(d, "copy_fetch")), \
        _copy_counter(os.path.join(d, "copy_write"))
    f_scale = copy_bytes / (f_copy * 1024.0)
    w_scale = copy_bytes / (w_copy * 1024.0)
    fetch = _routed_counter(os.path.join(d, "fetch"), path)
    write = _routed_counter(os.path.join(d, "write"), path)
    kernels = {}
    for s in ("gate_up", "down"):
        if s in fetch and s in write:
            fb = fetch[s][0] * 1024.0 * f_scale
            wb = write[s][0] * 1024.0 * w_scale
            kernels[f"{path}_{s}"] = {
                "fetch_kib_raw": round(fetch[s][0], 1), "write_kib_raw": round(write[s][0], 1),
                "dispatches": [fetch[s][1], write[s][1]],
                "fetch_bytes": round(fb), "write_bytes": round(wb),
                "bytes_per_launch": round(fb + wb)}
    doc = {"workload": workload, "source_digest": source_digest(),
           "copy_calibration": {"bytes": int(copy_bytes), "fetch_kib": f_copy,
                                "write_kib": w_copy, "fetch_scale": round(f_scale, 4),
                                "write_scale": round(w_scale, 4)},
           "kernels": kernels, "commands": commands}
    out = os.path.join(PROFILE_DIR, f"traffic_{workload}.json")
    os.makedirs(PROFILE_DIR, exist_ok=True)
    with open(out, "w") as f:
        json.dump(doc, f, indent=1)
    return out


DEFAULT_WORKLOAD = "prefill_zipf_t4096"


def host_cpu():
    """(logical CPUs this process may run on, CPU model string)."""
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    model = platform.processor() or "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return n, model


def cpu_baseline(spec, inp, name, seconds):
    import numpy as np
    import oracle as O
    from threadpoolctl import threadpool_info

    n_rows = min(CPU_SAMPLE_TOKENS.get(name, 4), spec.tokens)
    rows = np.arange(n_rows)

    def host(ws):
        parts = {}
        for p in ("gate", "up", "down"):
            w = getattr(ws, p)
            parts[p] = (w.fmt, w.packed.cpu().numpy(), w.scales.cpu().numpy(),
                        None if w.global_scale is None else w.global_scale.cpu().numpy())
        return parts

    f32 = lambda t: None if t is None else t.float().cpu().numpy()  # noqa: E731
    routed = host(inp.routed)
    shared = host(inp.shared) if inp.shared is not None else None
    args = dict(score=spec.score, select=spec.select, renormalize=spec.renormalize,
                logit_bias=f32(inp.logit_bias), correction_bias=f32(inp.correction_bias),
                token_ids=None if inp.token_ids is None else inp.token_ids.cpu().numpy(),
                tid2eid=None if inp.tid2eid is None else inp.tid2eid.cpu().numpy(),
                gamma=f32(inp.gamma), norm_eps=spec.norm_eps)
    x, res, rw = f32(inp.x), f32(inp.residual), f32(inp.router_w)
    done, t0 = 0, time.perf_counter()
    while True:
        cache = O.DequantCache(routed["gate"], routed["up"], routed["down"])
        sc = O.DequantCache(shared["gate"], shared["up"], shared["down"]) if shared else None
        O.layer_forward(x, res, rw, cache, spec.top_k, shared=sc, rows=rows, **args)
        done += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    nproc, model = host_cpu()
    return {"value": round(done * n_rows / el, 4), "unit": "tokens/s", "cores": threads,
            "kind": "oracle", "host_nproc": nproc, "cpu_model": model,
            "sample": f"{done} oracle evaluation(s) of {n_rows} token(s) of one batch of the "
                      f"same workload ({el:.1f} s; numpy fp64: matrix products on {threads} "
                      f"BLAS threads, weight decoding on one thread; host: {nproc} logical "
                      f"CPUs, {model})"}


def kernel_work(stage, u_mean, T, K, H, I, fmt, decode):
    """Algorithmic work of one routed launch of `stage` ("gate_up" or "down"): bytes (each
    touched expert's weights once, its input activations and its output rows; y is fp16 for
    routed prefill rows, else fp32) and flops of the T * K routed rows, with their per-unit
    notes. u_mean = mean number of touched experts."""
    bpe = bytes_per_elem(fmt)
    rows = T * K
    if stage == "gate_up":
        return (u_mean * 2 * I * H * bpe + T * H * 2 + rows * I * 2, 2 * rows * H * 2 * I,
                "2*I*H*b bytes per touched expert (b = 0.5625 NVFP4, 0.53125 MXFP4) + x in + h out",
                "4*H*I flops per routed row")
    return (u_mean * I * H * bpe + rows * I * 2 + rows * H * (4 if decode else 2), 2 * rows * H * I,
            "I*H*b bytes per touched expert + h in + y out", "2*H*I flops per routed row")


def roofline(kbytes, kflops, kernel_ms, unit_bytes="", unit_flops=""):
    """The bound of a kernel from its arithmetic intensity against the ridge of the published
    peaks (bf16 MFMA, HBM), and its achieved rate over the measured launch duration."""
    ridge = BF16_MFMA_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    if kflops / kbytes < ridge:
        achieved = kbytes / (kernel_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4)}
        per_launch, unit_note = kbytes, unit_bytes
    else:
        achieved = kflops / (kernel_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": BF16_MFMA_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / BF16_MFMA_PEAK_TFLOPS, 4)}
        per_launch, unit_note = kflops, unit_flops
    roof["per_launch"] = per_launch
    roof["per_unit"] = unit_note
    roof["arith_intensity"] = round(kflops / kbytes, 1)
    return roof


def run_workload(name, args, with_cpu=True, with_graph=True, steps=None, warmup=None):
    """Time `steps` layer calls of one workload; returns the result dict of the JSON line."""
    import torch
    import moe_synth as S
    import mixture_experts_ffn_03_amd as M

    steps = args.steps if steps is None else steps
    warmup = args.warmup if warmup is None else warmup
    spec = S.WORKLOADS[name]
    if args.tokens > 0:
        spec = S.scaled(spec, tokens=args.tokens)
    dev = "cuda"
    nsets = args.weight_sets or WEIGHT_SETS[name]
    path = {"auto": M.PATH_AUTO, "decode": M.PATH_DECODE, "prefill": M.PATH_PREFILL}[args.path]

    t_gen = time.perf_counter()
    sets = [S.make_inputs(spec, device=dev, seed=spec.seed + 101 * i) for i in range(nsets)]
    batches = [S.make_activations(spec, device=dev, seed=spec.seed + 7 + 31 * b)
               for b in range(args.batches)]
    torch.cuda.synchronize()
    log(f"[bench] {name}: {nsets} weight set(s), {args.batches} input batches generated in "
        f"{time.perf_counter() - t_gen:.1f} s")

    T, H, E, K, I = spec.tokens, spec.hidden, spec.experts, spec.top_k, spec.inter
    cfg = M.make_config(T, H, E, K, I, score_mode=spec.score, select_mode=spec.select,
                        renormalize=spec.renormalize, has_shared=spec.shared,
                        shared_inter=spec.shared_inter, pre_norm=spec.pre_norm,
                        norm_eps=spec.norm_eps, vocab=spec.vocab, path=path)
    ws = M.alloc_workspace(cfg, dev)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    routed = [M.expert_weights(s.routed) for s in sets]
    shared = [M.expert_weights(s.shared) if s.shared is not None else None for s in sets]
    ids = torch.empty((T, K), dtype=torch.int32, device=dev)

    def step(i, dbg=False):
        s, b = sets[i % nsets], batches[i % args.batches]
        M.layer_forward(cfg, b.x, s.router_w, routed[i % nsets], out, ws, norm_gamma=s.gamma,
                        logit_bias=s.logit_bias, correction_bias=s.correction_bias,
                        token_ids=b.token_ids, tid2eid=s.tid2eid, shared=shared[i % nsets],
                        residual=b.residual, dbg_ids=ids if dbg else None)

    # routing of every (weight set, batch) pair: unique experts touched per step
    period = nsets * args.batches // __import__("math").gcd(nsets, args.batches)
    uniq = []
    for i in range(period):
        step(i, dbg=True)
        torch.cuda.synchronize()
        uniq.append(S.count_unique_experts(ids, E))
    if M.get_device_error(ws) != 0:
        raise RuntimeError("device error word set during the benchmark's routing pass")

    hip = HipEvents()
    nst = M.STAGE_COUNT
    # instrumented pass (untimed): every stage boundary, to find the dominant kernel
    prof_steps = max(8, min(warmup, 64))
    evs = [[hip.create() for _ in range(nst)] for _ in range(prof_steps)]
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    arrs = []
    for i in range(prof_steps):
        arr = (ctypes.c_void_p * nst)(*evs[i])
        arrs.append(arr)
        M.set_stage_events(arr, nst)
        step(i)
    torch.cuda.synchronize()
    stage_ms = {}
    for si in range(1, nst):
        stage_ms[M.STAGE_NAMES[si]] = sum(hip.elapsed_ms(evs[i][si - 1], evs[i][si])
                                         for i in range(prof_steps)) / prof_steps
    for row in evs:
        for e in row:
            hip.destroy(e)
    kernel_stage = max(("gate_up", "down"), key=lambda k: stage_ms[k])
    ks = M.STAGE_NAMES.index(kernel_stage)

    # timed steps: HIP events around the dominant kernel only (on the layer's stream)
    kev = [(hip.create(), hip.create()) for _ in range(steps)]
    karrs = []
    for i in range(steps):
        arr = (ctypes.c_void_p * nst)()
        arr[ks - 1], arr[ks] = kev[i]
        karrs.append(arr)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(steps):
        M.set_stage_events(karrs[i], nst)
        step(warmup + i)
    end.record()
    torch.cuda.synchronize()
    ms_per_step = start.elapsed_time(end) / steps
    kernel_ms = sum(hip.elapsed_ms(a, b) for a, b in kev) / steps
    for a, b in kev:
        hip.destroy(a)
        hip.destroy(b)
    if M.get_device_error(ws) != 0:
        raise RuntimeError("device error word set during the timed steps")

    S_rows = T * K
    groups = min(E, S_rows)
    pre_ok = H % 64 == 0 and I % 64 == 0 and (not spec.shared or spec.shared_inter % 64 == 0)
    decode = (path == M.PATH_DECODE) or (path == M.PATH_AUTO and not (S_rows >= 4 * groups
                                                                       and pre_ok))

    # the same steps replayed from a HIP graph (one capture of a whole period: every weight
    # set and batch once), for decode layers of at most 32 tokens: launch gaps without the
    # host in the loop
    graph_replay = None
    if decode and T <= 32 and with_graph and not args.no_graph:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for i in range(period):
                step(i)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(period):
                step(i)
        graph.replay()
        torch.cuda.synchronize()
        reps = max(1, steps // period)
        start.record()
        for _ in range(reps):
            graph.replay()
        end.record()
        torch.cuda.synchronize()
        g_ms = start.elapsed_time(end) / (reps * period)
        if M.get_device_error(ws) != 0:
            raise RuntimeError("device error word set during the graph replays")
        graph_replay = {"ms_per_step": round(g_ms, 5), "value": round(T / (g_ms * 1e-3), 2),
                        "steps": reps * period, "steps_per_replay": period}
        del graph

    u_mean = sum(uniq[(warmup + i) % period] for i in range(steps)) / steps
    bpe = bytes_per_elem(spec.fmt)
    kbytes, kflops, unit_bytes, unit_flops = kernel_work(kernel_stage, u_mean, T, K, H, I,
                                                         spec.fmt, decode)
    roof = roofline(kbytes, kflops, kernel_ms, unit_bytes, unit_flops)
    kname = f"{'decode' if decode else 'prefill'}_{kernel_stage}"
    roof["traffic"] = load_traffic(name, kname) if args.tokens <= 0 else None
    roof["kernel"] = kname
    roof["kernel_ms"] = round(kernel_ms, 5)

    # whole-layer algorithmic work
    shared_bytes = (3 * H * spec.shared_inter * bytes_per_elem(spec.shared_fmt)) if spec.shared else 0
    layer_bytes = u_mean * 3 * H * I * bpe + shared_bytes + E * H * 2 + 3 * T * H * 2
    layer_flops = T * K * 6 * H * I + (T * 6 * H * spec.shared_inter if spec.shared else 0) + 2 * T * H * E
    tokens_per_s = T / (ms_per_step * 1e-3)
    layer_s = ms_per_step * 1e-3

    result = {
        "metric": METRIC, "value": round(tokens_per_s, 2), "unit": "tokens/s", "n_gpus": 1,
        "steps": steps, "warmup": warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "weights": ["nvfp4", "mxfp4", "fp8", "bf16"][spec.fmt],
        "data": "synthetic (seeded; random-init FP4 weights, N(0,1) bf16 activations)",
        "config": {"workload": name, "description": DESCRIPTIONS[name], "tokens": T,
                   "hidden": H, "experts": E, "top_k": K, "inter": I,
                   "path": "decode" if decode else "prefill", "weight_sets": nsets,
                   "input_batches": args.batches, "unique_experts_mean": round(u_mean, 2)},
        "layer": {"GB_per_s": round(layer_bytes / layer_s / 1e9, 1),
                  "TFLOP_per_s": round(layer_flops / layer_s / 1e12, 2),
                  "hbm_frac": round(layer_bytes / layer_s / 1e9 / HBM_PEAK_GBS, 4),
                  "mfma_frac": round(layer_flops / layer_s / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4),
                  "stage_ms": {k: round(v, 5) for k, v in stage_ms.items()}},
        "roofline": roof,
    }
    if graph_replay is not None:
        result["graph_replay"] = graph_replay
    if with_cpu and not args.no_cpu_baseline:
        log(f"[bench] timing the CPU oracle for about {args.cpu_seconds:.0f} s")
        result["cpu_baseline"] = cpu_baseline(spec, sets[0], name, args.cpu_seconds)
    del sets, batches, routed, shared, ws, out, ids
    gc.collect()
    torch.cuda.empty_cache()
    return result


def brief(r):
    """The compact entry of a workload in "other_workloads"."""
    roof = r["roofline"]
    b = {"ms_per_step": r["ms_per_step"], "value": r["value"], "unit": r["unit"],
         "path": r["config"]["path"],
         "roofline": {k: roof[k] for k in ("kernel", "bound", "achieved", "unit", "frac",
                                           "kernel_ms")},
         "layer": {k: r["layer"][k] for k in ("hbm_frac", "mfma_frac", "stage_ms")}}
    if "graph_replay" in r:
        b["graph_replay_ms_per_step"] = r["graph_replay"]["ms_per_step"]
    return b


PEAK_HBM_TBPS = 8.0          # MI355X published HBM3E bandwidth
PEAK_BF16_TFLOPS = 2500.0    # dense bf16 MFMA
PEAK_FP4_TFLOPS = 10100.0    # dense fp6/fp4 MFMA (the FP4 x FP8 probe runs at the fp8 rate)
PEAK_FP8_TFLOPS = 5000.0


def microbench(M, torch):
    """Achievable rates of the paths the kernels use (moe_probe_* entry points): streaming
    read of 16 MB .. 512 MB regions rotated through a 2 GiB pool (so that the 256 MB Infinity
    Cache does not serve a repeat), and the MFMA probes at one and two blocks per CU, each
    with the shader clock it sustained (its s_memtime cycles over the event time)."""
    res = {"metric": "microbench", "read": [], "mfma": []}
    pool = torch.empty(2 << 30, dtype=torch.uint8, device="cuda")
    pool.fill_(1)
    sink = torch.zeros(M.PROBE_READ_BLOCKS, dtype=torch.float32, device="cuda")
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for mb in (16, 84, 200, 512):
        n = mb << 20
        regions = max(1, pool.numel() // n)
        times = []
        for rep in range(3 * regions + 2):
            src = pool[(rep % regions) * n:(rep % regions) * n + n]
            ev0.record()
            M.probe_stream_read(src, sink)
            ev1.record()
            ev1.synchronize()
            if rep >= 2:
                times.append(ev0.elapsed_time(ev1) * 1e-3)
        best, med = min(times), statistics.median(times)
        res["read"].append({"MB": mb, "TBps_best": round(n / best / 1e12, 3),
                            "TBps_median": round(n / med / 1e12, 3),
                            "frac_of_8TBps": round(n / med / 1e12 / PEAK_HBM_TBPS, 3)})
        log(f"[microbench] read {mb} MB: {res['read'][-1]}")
    names = {0: ("bf16 32x32x16", 32768, PEAK_BF16_TFLOPS),
             1: ("scaled fp4 x fp8 32x32x64", 131072, PEAK_FP8_TFLOPS),
             2: ("mxfp4 decode + bf16 32x32x16 (GEMM step mix)", 32768, PEAK_BF16_TFLOPS)}
    for kind, (name, flop, peak) in names.items():
        for bpc in (1, 2):
            blocks = M.probe_mfma_blocks(bpc)
            msink = torch.zeros(blocks, dtype=torch.float32, device="cuda")
            cyc = torch.zeros(blocks, dtype=torch.int64, device="cuda")
            iters = 4096
            M.probe_mfma(kind, 64, bpc, msink, cyc)  # warm up
            ts = []
            for _ in range(5):
                ev0.record()
                M.probe_mfma(kind, iters, bpc, msink, cyc)
                ev1.record()
                ev1.synchronize()
                ts.append(ev0.elapsed_time(ev1) * 1e-3)
            t = statistics.median(ts)
            flops = blocks * 4 * iters * 8 * flop
            tf = flops / t / 1e12
            entry = {"kind": name, "blocks_per_cu": bpc, "TFLOPs": round(tf, 1),
                     "frac_of_published": round(tf / peak, 3)}
            if bpc == 1:
                # one block per CU: every block runs for the whole launch, so its cycles over
                # the launch time give the clock (with two, a block's lifetime is not the
                # launch's)
                clock = float(cyc.double().mean().item()) / t / 1e9
                entry["clock_GHz"] = round(clock, 3)
                entry["frac_at_that_clock"] = round(tf / (peak * clock / 2.4), 3)
            res["mfma"].append(entry)
            log(f"[microbench] mfma: {res['mfma'][-1]}")
    print(json.dumps(res), flush=True)


def wait_split(M, torch, workload):
    """Where the routed MXFP4 grouped GEMMs' waves spend their K loop, from a library built with
    MOE_PRE_WAIT_SPLIT=1 MOE_PRE_PERSIST=0 (passed with --lib): per step, the stage-load wait,
    the barrier, and the rest (the stage's LDS reads, decode and MFMA issue), summed over every
    wave of the routed launches of three layer calls."""
    import numpy as np
    lib = M.load_library()
    if not hasattr(lib, "moe_debug_prefill_wait_split"):
        raise SystemExit("--wait-split needs --lib of a build with MOE_PRE_WAIT_SPLIT=1 "
                         "MOE_PRE_PERSIST=0")
    fn = lib.moe_debug_prefill_wait_split
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p]
    import moe_synth as S
    spec = S.WORKLOADS[workload]
    inp = S.make_inputs(spec, device="cuda")
    cfg = M.make_config(spec.tokens, spec.hidden, spec.experts, spec.top_k, spec.inter,
                        score_mode=spec.score, select_mode=spec.select,
                        renormalize=spec.renormalize, has_shared=spec.shared,
                        shared_inter=spec.shared_inter, pre_norm=spec.pre_norm,
                        norm_eps=spec.norm_eps, vocab=spec.vocab)
    ws = M.alloc_workspace(cfg, "cuda")
    out = torch.empty_like(inp.x)
    shared = M.expert_weights(inp.shared) if inp.shared is not None else None

    def call():
        M.layer_forward(cfg, inp.x, inp.router_w, M.expert_weights(inp.routed), out, ws,
                        norm_gamma=inp.gamma, logit_bias=inp.logit_bias,
                        correction_bias=inp.correction_bias, token_ids=inp.token_ids,
                        tid2eid=inp.tid2eid, shared=shared, residual=inp.residual)
        torch.cuda.synchronize()

    raw = np.zeros((2, 8192, 4, 4), np.uint64)
    call()
    fn(raw.ctypes.data)  # (clears the sums of the warm-up call)
    acc = np.zeros_like(raw, dtype=np.float64)
    for _ in range(3):
        call()
        if fn(raw.ctypes.data) != 0:
            raise SystemExit("moe_debug_prefill_wait_split failed")
        acc += raw.astype(np.float64)
    res = {"metric": "wait_split", "workload": workload, "kernels": {}}
    for k, name in enumerate(("gate_up", "down")):
        v = acc[k][acc[k][:, 0, 3] > 0]
        if not len(v):
            continue
        loop, load, bar, n = (v[:, :, i].sum() for i in range(4))
        res["kernels"][name] = {"blocks": int(len(v)), "steps_per_wave": round(n / len(v) / 4 / 3, 1),
                                "load_wait": round(load / loop, 3), "barrier": round(bar / loop, 3),
                                "rest": round(1 - (load + bar) / loop, 3),
                                "cycles_per_step": round(loop / n)}
    print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=sorted(DESCRIPTIONS))
    ap.add_argument("--tokens", type=int, default=0,
                    help="run the workload's layer at this many tokens (e.g. 2 or 3 for a "
                         "multi-token verify step); 0 = the workload's own")
    ap.add_argument("--weight-sets", type=int, default=0, help="0 = workload default")
    ap.add_argument("--batches", type=int, default=8)
    ap.add_argument("--path", default="auto", choices=["auto", "decode", "prefill"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-others", action="store_true",
                    help="with the default workload, skip the entries of the other workloads")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the HIP-graph replay timing (decode layers of at most 32 tokens)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--lib", default=None,
                    help="path of the HIP library to load (default: the package's in-tree build)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run 8 device-to-device copies of 1 GiB (a copy kernel of known "
                         "size, to scale the FETCH_SIZE / WRITE_SIZE counters) and exit")
    ap.add_argument("--summarize-trace", metavar="DIR",
                    help="print a kernel table of a rocprofv3 --stats csv output dir and exit")
    ap.add_argument("--summarize-traffic", metavar="DIR",
                    help="write the workload's HBM traffic file from rocprofv3 --pmc runs in "
                         "DIR/{fetch,write,copy_fetch,copy_write} and exit")
    ap.add_argument("--microbench", action="store_true",
                    help="only measure the achievable rates (streaming read, MFMA probes with "
                         "their sustained clock) and print them as one JSON line")
    ap.add_argument("--wait-split", action="store_true",
                    help="with --lib of a MOE_PRE_WAIT_SPLIT=1 MOE_PRE_PERSIST=0 build: where the "
                         "routed MXFP4 grouped GEMMs' waves spend their K loop (one JSON line)")
    ap.add_argument("--command", action="append", default=[],
                    help="command line recorded in a summary (repeatable)")
    args = ap.parse_args()
    if args.summarize_trace:
        print(summarize_trace(args.summarize_trace, " ; ".join(args.command)), end="")
        return
    if args.summarize_traffic:
        path = "prefill" if args.workload in ("prefill_zipf_t4096", "hash_mxfp4_t512") \
            else "decode"
        print(summarize_traffic(args.summarize_traffic, args.workload, path, args.command))
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        if int(os.environ.get("RANK", "0")) == 0:
            print(f"bench.py measures one GPU only: the library has no multi-GPU path "
                  f"(asked for --gpus {args.gpus}, WORLD_SIZE={world}).", file=sys.stderr)
        sys.exit(2)

    import torch
    import mixture_experts_ffn_03_amd as M

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        src = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(8):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("[bench] copy calibration: 8 copies of 1073741824 bytes")
        return
    if args.lib:
        M.load_library(args.lib)
    else:
        M.load_library()
    if args.microbench:
        microbench(M, torch)
        return
    if args.wait_split:
        wait_split(M, torch, args.workload)
        return
    result = run_workload(args.workload, args)
    if args.workload == DEFAULT_WORKLOAD and args.tokens <= 0 and not args.no_others:
        others = {}
        for name in ("qwen3_decode_t1", "qwen3_decode_t8", "dsv3_decode_t32",
                     "hash_mxfp4_t512"):
            others[name] = brief(run_workload(name, args, with_cpu=False))
            log(f"[bench] {name}: {others[name]['ms_per_step']} ms/step")
        result["other_workloads"] = others
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
