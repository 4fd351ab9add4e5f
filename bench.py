"""Benchmark of one MoE layer forward on one MI355X (libmoe, HIP).

A step is one pass of the whole path over one batch of synthetic tokens, with every input and
weight resident in HBM:  route -> permute -> routed gate/up -> routed down -> combine on the
main stream, with the shared expert's gate/up and down inside the routed launches at decode
sizes and on a second stream that joins before combine at prefill sizes.

The headline `value` is tokens/s of the DeepSeek-V3-shaped decode layer (T=16, 256 experts,
top-8, FP8 block-scaled weights).  The same line carries the 4096-token prefill layer under
"prefill", the same layer in the opt-in FP8 activation mode under "prefill_a8" (its gate/up
roofline against the FP8 MFMA peak), the decode layer with 4-bit MXFP4 expert weights under
"decode_mxfp4", the prefill layer with MXFP4 expert weights under "prefill_mxfp4" (bf16
activations) and "prefill_mxfp4_a8" (FP8 activations, W4A8), with --ep-ranks G rank 0's share of the decode and
prefill layers under expert parallelism over G ranks under "ep_rank_share" (collectives
excluded), the roofline of the dominant kernel (the routed gate/up projection: its launch
duration from HIP events around back-to-back launches on the main stream, plus the average of
the per-step brackets inside the layer) and the CPU oracle timed on a bounded sample on the
host.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload dsv3_decode] [--no-cpu]
                    [--prefill dsv3_prefill] [--a8 dsv3_prefill] [--mxfp4 dsv3_decode]
                    [--mxfp4-prefill dsv3_prefill] [--w4a8 dsv3_prefill] [--ep-ranks 0]
                    [--extra tiny,dsv3_long_zipf,dsv3_long_zipf/fp8/fp8,...] [--vendor-ref]

Every workload is timed over the same --steps layer steps.  "extra" holds, by default, the tiny
layer and the two MFMA-bound prefill layers (T = 32768 with Zipf routing, and Kimi-K2 at
T = 8192) with bf16 activations and in the FP8-activation mode (FP8 and MXFP4 weights), each with
its gate/up roofline against the peak of its own operand type.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
FP8_PEAK_TFLOPS = 5000.0  # MI355X dense fp8 MFMA
MALL_BYTES = 256 << 20  # MI355X last-level (Infinity) cache
METRIC = "MoE-layer tokens/s at T=16 and T=4096; % of HBM BW / FP8 MFMA peak"
# the tiny layer, and the two layers where the expert GEMMs are MFMA-bound (the long Zipf-routed
# prefill and Kimi-K2) with bf16 and with FP8 activations, FP8 and MXFP4 weights
DEFAULT_EXTRA = ("tiny,dsv3_long_zipf,dsv3_long_zipf/fp8/fp8,dsv3_long_zipf/mxfp4/fp8,"
                 "kimi_k2,kimi_k2/fp8/fp8,kimi_k2/mxfp4/fp8")


# ------------------------------------------------------------------ algorithmic accounting

def matrix_bytes(H: int, I: int, wdtype: str = "fp8") -> int:
    """Bytes of one H x I projection matrix with its scales: FP8 (+ fp32 per 128x128 block),
    bf16, or MXFP4 (half a byte a weight + one E8M0 byte per 32)."""
    if wdtype == "fp8":
        return H * I + (H // 128) * (I // 128) * 4
    if wdtype == "mxfp4":
        return H * I // 2 + H * I // 32
    return H * I * 2


def expert_bytes(H: int, I: int, wdtype: str = "fp8") -> int:
    """Bytes of one expert's three projection matrices with their scales."""
    return 3 * matrix_bytes(H, I, wdtype)


def gate_up_bytes(T: int, k: int, H: int, I: int, touched: int, wdtype: str = "fp8") -> int:
    """Algorithmic bytes of the routed gate/up launch: the gate and up weights of every touched
    expert once, every token's activation row once, and the bf16 intermediate h written once."""
    return touched * 2 * matrix_bytes(H, I, wdtype) + T * H * 2 + T * k * I * 2


def gate_up_a8_bytes(T: int, k: int, H: int, I: int, touched: int, wdtype: str = "fp8") -> int:
    """Algorithmic bytes of the FP8-activation gate/up launch: the touched experts' gate and up
    weights (+ scales) once, every token's FP8 codes and exponent row once, h written once."""
    w = 2 * matrix_bytes(H, I, wdtype)
    pitch = (H // 128 + 15) // 16 * 16
    return touched * w + T * (H + pitch) + T * k * I * 2


def gate_up_flops(T: int, k: int, H: int, I: int) -> int:
    return 2 * 2 * T * k * H * I


def layer_bytes(T, H, I, E, k, touched, wdtype="fp8", shared=True) -> int:
    """Algorithmic bytes of the layer: touched experts' weights + the shared expert's, x read,
    out written, router scores read, top-k ids and weights."""
    eb = expert_bytes(H, I, wdtype)
    return touched * eb + (eb if shared else 0) + 2 * T * H * 2 + T * E * 4 + T * k * 8


def layer_flops(T, H, I, k, shared=True) -> int:
    """2 FLOP per weight per token row over the three matrices (routed rows + shared rows)."""
    return (T * k + (T if shared else 0)) * 6 * H * I


# ------------------------------------------------------------------ counter-derived traffic

def kernel_sources(kernel: str) -> list:
    """Sources (relative to the repository root) of the translation unit a libmoe gate/up kernel
    is compiled in, with the headers it includes: moe_ffn.hip (GEMV kernels and the launches),
    moe_gemm.hip (bf16-activation GEMM, with the launch choice of moe_gemm_wide.hip's 160 x 512
    tiles), moe_gemm_a8.hip (FP8-activation GEMM, and the launch choice of the W4A8 GEMM in
    moe_gemm_w4a8.hip) or moe_gemm_w4.hip (MXFP4 weights, bf16 activations)."""
    if "gemv_kernel" in kernel:
        names = ["moe_device.h", "moe_ffn.h", "moe_ffn.hip", "moe_host.h", "moe_lds.h"]
    elif "gemm_a8_kernel" in kernel:
        names = ["moe_device.h", "moe_ffn.h", "moe_gemm_a8.hip", "moe_host.h", "moe_lds.h"]
    elif "gemm_w4a8_kernel" in kernel:
        names = ["moe_device.h", "moe_ffn.h", "moe_gemm_a8.hip", "moe_gemm_w4a8.hip", "moe_host.h",
                 "moe_lds.h"]
    elif "gemm_fp8_wide_kernel" in kernel:
        names = ["moe_device.h", "moe_ffn.h", "moe_ffn.hip", "moe_gemm.hip", "moe_gemm_wide.hip",
                 "moe_host.h", "moe_lds.h"]
    elif "gemm_w4_kernel" in kernel:
        names = ["moe_device.h", "moe_ffn.h", "moe_gemm_w4.hip", "moe_host.h", "moe_lds.h"]
    else:
        names = ["moe_device.h", "moe_ffn.h", "moe_ffn.hip", "moe_gemm.hip", "moe_host.h",
                 "moe_lds.h"]
    # build.py holds the compile flags (some per file), so it is part of what the kernel is
    return sorted(os.path.join("routed_expert_grouped_amd", "csrc", n) for n in names) + \
        [os.path.join("include", "libmoe.h"), os.path.join("routed_expert_grouped_amd", "build.py")]


def source_digest(files) -> str:
    h = hashlib.sha256()
    for f in files:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return h.hexdigest()[:16]


def counter_traffic(workload: str):
    """HBM bytes per launch of the gate/up kernel from the committed rocprofv3 counter summary,
    or None when there is none or the kernel's sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"gate_up_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    files = rec.get("source_files") or []
    if not files or any(not os.path.exists(os.path.join(ROOT, f)) for f in files):
        return None
    if rec.get("source_digest") != source_digest(files):
        return None
    return rec.get("traffic_bytes")


# ------------------------------------------------------------------ profiler summaries
# rocprofv3 writes per-dispatch CSV rows; these turn them into the short records under
# profiles/ (the counter traffic that `roofline.traffic` reads, and text summaries).

GATE_UP_RE = (r"moe::(gemv_kernel<\d+, 1, true|gemm_kernel<(true|false), 1, true|"
              r"gemm_fp8_wide_kernel<1, true|gemm_fp8_q256_kernel<1, true|gemm_a8_kernel<1, true|"
              r"gemm_w4_kernel<1, true|gemm_w4a8_kernel<1, true)")
SIMDS = 1024  # MI355X: 256 CUs x 4 SIMDs
XCDS = 8


def _csv_rows(d, suffix):
    import csv
    import glob

    rows = []
    for f in sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True)):
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    return rows


def pmc_per_kernel(d):
    """{kernel name: {"dispatches": n, counter: mean per dispatch}} from a --pmc run's CSV."""
    acc = {}
    for r in _csv_rows(d, "counter_collection.csv"):
        k = r["Kernel_Name"]
        e = acc.setdefault(k, {"_disp": {}})
        if r.get("Start_Timestamp") and r.get("End_Timestamp"):
            e["_disp"][r["Dispatch_Id"]] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        else:
            e["_disp"][r["Dispatch_Id"]] = 0
        e.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    out = {}
    for k, e in acc.items():
        disp = e.pop("_disp")
        out[k] = {"dispatches": len(disp), "duration_ns": sum(disp.values()) / len(disp),
                  **{c: sum(v) / len(v) for c, v in e.items()}}
    return out


def summarize_traffic(key, fetch_dir, write_dir, commands):
    """profiles/gate_up_<key>_traffic.json from one FETCH_SIZE and one WRITE_SIZE run of one
    workload (bench.py --only ... --copy-probe-mib 1024): the routed gate/up kernel's KiB per
    dispatch, each scaled by the known bytes of the 1 GiB device copy over what the same counter
    read for it."""
    import re

    fetch = pmc_per_kernel(fetch_dir)

    def probe_copies(d, counter):
        # the device copies of the 1 GiB probe: the copy kernel's largest dispatches (the same
        # kernel also serves the run's small host <-> device copies)
        vals = [float(r["Counter_Value"]) for r in _csv_rows(d, "counter_collection.csv")
                if "copyBuffer" in r["Kernel_Name"] and r["Counter_Name"] == counter]
        if not vals:
            raise SystemExit(f"no copy kernel in the {counter} run (use --copy-probe-mib 1024)")
        big = [v for v in vals if v >= 0.9 * max(vals)]
        return sum(big) / len(big)

    copy_f = probe_copies(fetch_dir, "FETCH_SIZE")
    copy_w = probe_copies(write_dir, "WRITE_SIZE")
    probe = 1 << 30
    ff, wf = probe / 1024 / copy_f, probe / 1024 / copy_w
    gu = [k for k in fetch if re.search(GATE_UP_RE, k)]
    if len(gu) != 1:
        raise SystemExit(f"expected one routed gate/up kernel, found {gu}")
    k = gu[0]

    def routed_only(d, counter):
        # the routed gate/up launches alone: at decode sizes the layer's own launch also carries
        # the shared expert's tiles, on extra workgroups, so only the smallest grid is kept
        rows = [r for r in _csv_rows(d, "counter_collection.csv")
                if r["Kernel_Name"] == k and r["Counter_Name"] == counter]
        g = min(int(r["Grid_Size"]) for r in rows)
        vals = [float(r["Counter_Value"]) for r in rows if int(r["Grid_Size"]) == g]
        return sum(vals) / len(vals), len(vals)

    fk, nd = routed_only(fetch_dir, "FETCH_SIZE")
    wk, _ = routed_only(write_dir, "WRITE_SIZE")
    rec = dict(copy_probe_bytes=probe, copy_fetch_kib=copy_f, copy_write_kib=copy_w,
               fetch_factor=ff, write_factor=wf, kernel=k, dispatches=nd,
               fetch_kib=fk, write_kib=wk,
               traffic_bytes=int(round(fk * 1024 * ff + wk * 1024 * wf)),
               source_files=kernel_sources(k), source_digest=source_digest(kernel_sources(k)),
               commands=commands,
               note="counters in KiB per dispatch, averaged over the kernel's dispatches with the "
                    "smallest grid (the routed launch alone); each scaled by (known bytes of a 1 GiB "
                    "device copy) / (what the same counter read for that copy)")
    path = os.path.join(ROOT, "profiles", f"gate_up_{key}_traffic.json")
    json.dump(rec, open(path, "w"), indent=1)
    return path


def summarize_stats(stats_csv_dir, out, header):
    """A text table of rocprofv3 --stats kernel statistics (libmoe kernels)."""
    rows = _csv_rows(stats_csv_dir, "kernel_stats.csv")
    rows = [r for r in rows if "moe::" in r["Name"]]
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    lines = [header, "", "kernel" + " " * 58 + "calls     avg_us     min_us     max_us  total_%"]
    for r in rows:
        name = r["Name"] if len(r["Name"]) <= 62 else r["Name"][:59] + "..."
        lines.append(f"{name:62s} {int(r['Calls']):7d} {float(r['AverageNs']) / 1e3:10.2f} "
                     f"{float(r['MinNs']) / 1e3:10.2f} {float(r['MaxNs']) / 1e3:10.2f} "
                     f"{float(r['Percentage']):8.2f}")
    open(out, "w").write("\n".join(lines) + "\n")
    return out


def summarize_pmc(out, header, runs):
    """A text summary of counter runs: for each (label, directory), the libmoe kernels' counters
    per dispatch and the derived figures (MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES over all SIMDs /
    (GRBM_GUI_ACTIVE per XCD x 1024 SIMDs); MFMA FLOP = MOPS x 512; TA/TD busy over GUI cycles)."""
    lines = [header, ""]
    for label, d in runs:
        lines.append(f"== {label}  ({d})")
        for k, v in sorted(pmc_per_kernel(d).items(), key=lambda kv: kv[0]):
            if "moe::" not in k:
                continue
            lines.append(f"  {k}   [{v['dispatches']} dispatches]")
            gui = v.get("GRBM_GUI_ACTIVE")
            per_xcd = gui / XCDS if gui else None
            for c in sorted(c for c in v if c != "dispatches"):
                lines.append(f"      {c:36s} {v[c]:.6g}")
            if per_xcd and v.get("duration_ns", 0) > 50e3:  # (short dispatches: too few cycles)
                lines.append(f"      -> duration {v['duration_ns'] / 1e3:.1f} us under the counters; "
                             f"clock {per_xcd / v['duration_ns']:.2f} GHz")
            if per_xcd and "SQ_VALU_MFMA_BUSY_CYCLES" in v:
                lines.append(f"      -> MFMA busy {100 * v['SQ_VALU_MFMA_BUSY_CYCLES'] / (per_xcd * SIMDS):.1f}%"
                             f" of {per_xcd:.0f} cycles")
            for c, what in (("SQ_INSTS_VALU_MFMA_MOPS_BF16", "bf16"), ("SQ_INSTS_VALU_MFMA_MOPS_F8", "fp8")):
                if v.get(c):
                    lines.append(f"      -> {what} MFMA FLOP per dispatch {v[c] * 512:.4g}")
            if per_xcd and v.get("SQ_INSTS_MFMA") and v.get("SQ_INSTS_VALU"):
                lines.append(f"      -> VALU instructions per MFMA {v['SQ_INSTS_VALU'] / v['SQ_INSTS_MFMA']:.2f}")
            for c in ("TA_BUSY_avr", "TD_TD_BUSY_sum", "TCP_PENDING_STALL_CYCLES_sum",
                      "TCP_TCP_TA_DATA_STALL_CYCLES_sum"):
                if per_xcd and c in v:
                    lines.append(f"      -> {c} / GUI cycles {v[c] / per_xcd:.3g}")
            if v.get("TCP_TCC_READ_REQ_sum") and "TCP_TCC_READ_REQ_LATENCY_sum" in v:
                lines.append(f"      -> L1->L2 read latency "
                             f"{v['TCP_TCC_READ_REQ_LATENCY_sum'] / v['TCP_TCC_READ_REQ_sum']:.0f} cycles")
            if v.get("SQ_INSTS_MFMA") and "SQ_VALU_MFMA_COEXEC_CYCLES" in v and per_xcd:
                lines.append(f"      -> MFMA/VALU co-execution {100 * v['SQ_VALU_MFMA_COEXEC_CYCLES'] / (per_xcd * SIMDS):.1f}% of SIMD cycles")
        lines.append("")
    open(out, "w").write("\n".join(lines) + "\n")
    return out


# ------------------------------------------------------------------ timing

def time_layer(layer, steps: int, warmup: int, act: str = "bf16"):
    import torch

    import routed_expert_grouped_amd as moe

    L = moe.MoeLayer(layer.T, layer.H, layer.I, layer.E, layer.k, layer.experts, layer.shared,
                     layer.score_fn, layer.renorm, act=act)
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        L.forward(layer.scores, layer.x)
    torch.cuda.synchronize()
    # the timed region: exactly `steps` layer steps back to back, between one event pair, with
    # nothing else on the stream (each timing event recorded between kernels costs GPU time)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record(stream)
    for _ in range(steps):
        L.forward(layer.scores, layer.x)
    t1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t0.elapsed_time(t1)
    # a second, separate pass for the per-step distribution: an event at every step boundary and
    # a bracket around the routed gate/up launch (the FP8 mode runs both phases in one call, so
    # it has none)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)] if act == "bf16" else [None] * steps
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]  # step boundaries
    torch.cuda.synchronize()
    marks[0].record(stream)
    for i in range(steps):
        L.forward(layer.scores, layer.x, gate_up_events=ev[i])
        marks[i + 1].record(stream)
    torch.cuda.synchronize()
    step_ms = sorted(marks[i].elapsed_time(marks[i + 1]) for i in range(steps))
    gu_ms = [e[0].elapsed_time(e[1]) for e in ev if e is not None]
    # The same routed gate/up launch, `steps` times back to back on the same stream between one
    # event pair: the average launch duration without the per-step event latency that the
    # brackets above add (the weights read per launch are far larger than the caches, so a
    # repeat gets no help from them).
    if act == "fp8":  # the FP8-code gate/up launch on the layer's quantised x
        codes, exps = moe.moe_quantize_act(layer.x)
        launch = lambda: moe.moe_expert_gate_up_a8(codes, exps, layer.k, L.perm, L.offsets, L.w,
                                                   L.h, stream)
    else:
        launch = lambda: moe.moe_expert_gate_up(layer.x, layer.k, L.perm, L.offsets, L.w, L.h,
                                                stream)
    launch()
    torch.cuda.synchronize()
    k0 = torch.cuda.Event(enable_timing=True)
    k1 = torch.cuda.Event(enable_timing=True)
    k0.record(stream)
    for _ in range(steps):
        launch()
    k1.record(stream)
    torch.cuda.synchronize()
    counts = L.counts.cpu().numpy()
    # the same layer captured into a HIP graph and replayed `steps` times
    graph_ms = None
    if act == "bf16":
        L.capture(layer.scores, layer.x)
        L.replay()
        torch.cuda.synchronize()
        g0 = torch.cuda.Event(enable_timing=True)
        g1 = torch.cuda.Event(enable_timing=True)
        g0.record(stream)
        for _ in range(steps):
            L.replay()
        g1.record(stream)
        torch.cuda.synchronize()
        graph_ms = g0.elapsed_time(g1) / steps
    pick = lambda f: step_ms[min(steps - 1, int(round(f * (steps - 1))))]
    return dict(total_ms=total_ms, wall_s=wall, gate_up_ms=k0.elapsed_time(k1) / steps,
                step_ms=dict(median=pick(0.5), p10=pick(0.1), p90=pick(0.9)), graph_ms=graph_ms,
                gate_up_ms_in_layer=sum(gu_ms) / len(gu_ms) if gu_ms else None, counts=counts)


def run_rank_share(layer, G: int, rank: int, steps: int, warmup: int):
    """One rank's share of the layer under expert parallelism over G ranks (route + permute of
    all tokens, the rank's E/G routed experts on their assignments, the local partial reduction,
    the shared expert on the rank's T/G token rows), timed per step with HIP events.  The
    collectives that would join the ranks are not part of this single-GPU build."""
    import torch

    import routed_expert_grouped_amd as moe

    T, H, I, E, k = layer.T, layer.H, layer.I, layer.E, layer.k
    e0, e1, t0, t1 = rank * E // G, (rank + 1) * E // G, rank * T // G, (rank + 1) * T // G
    R = moe.MoeRankShare(T, H, I, E, k, layer.experts, layer.shared, e0, e1, t0, t1,
                         layer.score_fn, layer.renorm)
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        R.forward(layer.scores, layer.x)
    torch.cuda.synchronize()
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    marks[0].record(stream)
    for i in range(steps):
        R.forward(layer.scores, layer.x)
        marks[i + 1].record(stream)
    torch.cuda.synchronize()
    total_ms = marks[0].elapsed_time(marks[-1])
    step_ms = sorted(marks[i].elapsed_time(marks[i + 1]) for i in range(steps))
    pick = lambda f: step_ms[min(steps - 1, int(round(f * (steps - 1))))]
    counts = R.counts.cpu().numpy()[e0:e1]
    touched = int((counts > 0).sum())
    wd = layer.experts.wdtype
    # the local experts' and the shared expert's weights, x and the partial output once, the
    # router scores and the top-k ids and weights
    nbytes = (touched + 1) * expert_bytes(H, I, wd) + 2 * T * H * 2 + T * E * 4 + T * k * 8
    ms = total_ms / steps
    return dict(ranks=G, rank=rank, experts=[e0, e1], shared_tokens=[t0, t1],
                local_assignments=int(counts.sum()), touched_local_experts=touched,
                ms_per_step=round(ms, 4),
                step_ms={q: round(pick(f), 4) for q, f in (("median", 0.5), ("p10", 0.1), ("p90", 0.9))},
                algorithmic_bytes=nbytes, hbm_frac=round(nbytes / (ms * 1e-3) / (HBM_PEAK_GBS * 1e9), 4),
                tokens_per_s_at_G_ranks_without_collectives=round(T / (ms * 1e-3), 1))


def read_probe(gib: int = 4, steps: int = 10):
    """Read rate of plain HBM read kernels (libmoe_probe.so: 16-byte loads, nothing written) over a
    `gib` GiB buffer: grid-stride, one contiguous chunk per workgroup, or rows of 7168 bytes read
    in 128-byte columns across 8 rows per instruction (the decode weight stream's shape); the best
    of the patterns and a few grid sizes is the measured ceiling the decode kernels' achieved
    bandwidth is also set against."""
    import ctypes

    import torch

    from routed_expert_grouped_amd import build as b

    if not os.path.exists(b.PROBE_OUT):
        return None
    lib = ctypes.CDLL(b.PROBE_OUT)
    lib.moe_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_int,
                                   ctypes.c_int, ctypes.c_void_p]
    lib.moe_probe_read.restype = ctypes.c_int
    nbytes = gib << 30
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    out = torch.zeros(1, dtype=torch.int32, device="cuda")
    st = torch.cuda.current_stream()
    best = None
    for pattern, wgs in [(pt, w) for pt in (0, 1, 2) for w in (2048, 4096, 8192, 16384)]:
        call = lambda: lib.moe_probe_read(ctypes.c_void_p(buf.data_ptr()), nbytes,
                                          ctypes.c_void_p(out.data_ptr()), wgs, pattern,
                                          ctypes.c_void_p(st.cuda_stream))
        if call() != 0:
            return None
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(st)
        for _ in range(steps):
            call()
        e1.record(st)
        torch.cuda.synchronize()
        read = nbytes if pattern < 2 else (nbytes // 7168 // 32) * 32 * 7168  # whole row groups
        gbs = read / (e0.elapsed_time(e1) / steps * 1e-3) / 1e9
        if best is None or gbs > best["GBps"]:
            best = dict(GBps=round(gbs, 1), bytes=read, workgroups=wgs,
                        pattern=("strided", "blocked", "rows of 7168 bytes")[pattern])
    del buf
    return best


def vendor_reference(steps: int = 10):
    """Reference rates of the vendor GEMM library (hipBLASLt through torch) at the expert shapes,
    for context only: dense operands, no grouping or gather, and per-tensor instead of per-block
    scales for FP8.  Nothing in the layer path uses them."""
    import torch

    dev, st = "cuda", torch.cuda.current_stream()

    def tm(fn):
        fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(st)
        for _ in range(steps):
            fn()
        e1.record(st)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    g = torch.Generator(device=dev).manual_seed(0)
    out = {}
    # one DeepSeek-V3 prefill gate/up at T = 4096 as 256 dense per-expert GEMMs of 128 rows
    a = torch.randn((256, 128, 7168), device=dev, generator=g, dtype=torch.bfloat16)
    b = torch.randn((256, 7168, 4096), device=dev, generator=g, dtype=torch.bfloat16).contiguous()
    ms = tm(lambda: torch.bmm(a, b))
    fl = 2 * 256 * 128 * 7168 * 4096
    out["bf16_bmm_256x128x7168x4096"] = dict(ms=round(ms, 4), tflops=round(fl / ms / 1e9, 1),
                                             bf16_frac=round(fl / ms / 1e9 / BF16_PEAK_TFLOPS, 4))
    del a, b
    # one large dense GEMM: 32768 rows (the long prefill's assignments) x 7168 x 4096
    a = torch.randn((32768, 7168), device=dev, generator=g, dtype=torch.bfloat16)
    w = torch.randn((4096, 7168), device=dev, generator=g, dtype=torch.bfloat16)
    fl = 2 * 32768 * 7168 * 4096
    ms = tm(lambda: a @ w.t())
    out["bf16_mm_32768x7168x4096"] = dict(ms=round(ms, 4), tflops=round(fl / ms / 1e9, 1),
                                          bf16_frac=round(fl / ms / 1e9 / BF16_PEAK_TFLOPS, 4))
    a8, w8 = a.to(torch.float8_e4m3fn), w.to(torch.float8_e4m3fn)
    one = torch.ones((), device=dev)
    ms = tm(lambda: torch._scaled_mm(a8, w8.t(), scale_a=one, scale_b=one, out_dtype=torch.bfloat16))
    out["fp8_scaled_mm_per_tensor_32768x7168x4096"] = dict(
        ms=round(ms, 4), tflops=round(fl / ms / 1e9, 1),
        fp8_frac=round(fl / ms / 1e9 / FP8_PEAK_TFLOPS, 4))
    return out


def cpu_baseline(layer, rows, n_threads: int):
    """The oracle (its per-token form, as it stands) on `rows` of the same layer, wall-clock on
    the host (inputs copied first)."""
    import numpy as np

    import oracle
    import routed_expert_grouped_amd as moe

    ids, _ = moe.moe_route(layer.scores, layer.k, layer.score_fn, layer.renorm)
    used = sorted(set(ids.cpu().numpy()[rows].ravel().tolist()))
    slot = np.full(layer.E, -1, np.int32)
    slot[used] = np.arange(len(used), dtype=np.int32)
    import dataclasses

    host = dataclasses.replace(layer, scores=layer.scores.cpu(), x=layer.x.cpu(),
                               experts=layer.experts.select(used), shared=layer.shared.to("cpu"))
    oracle.lib()
    t = time.perf_counter()
    oracle.moe_layer(host, rows=rows, expert_slot=slot, n_threads=n_threads)
    dt = time.perf_counter() - t
    return dt, oracle.max_threads(n_threads)


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor()


def run_workload(name: str, steps: int, warmup: int, seed: int = 0, act: str = "bf16",
                 layer=None, wdtype=None):
    import synth

    if layer is None:
        over = {} if wdtype is None else {"wdtype": wdtype}
        layer = synth.make_layer(name, seed=seed, device="cuda", **over)
    wd = layer.experts.wdtype
    r = time_layer(layer, steps, warmup, act)
    T, H, I, E, k = layer.T, layer.H, layer.I, layer.E, layer.k
    touched = int((r["counts"] > 0).sum())
    ms = r["total_ms"] / steps
    lb = layer_bytes(T, H, I, E, k, touched, wd)
    lf = layer_flops(T, H, I, k)
    a8 = act == "fp8"
    gb = gate_up_a8_bytes(T, k, H, I, touched, wd) if a8 else gate_up_bytes(T, k, H, I, touched, wd)
    gf = gate_up_flops(T, k, H, I)
    gu_s = r["gate_up_ms"] * 1e-3
    bw = gb / gu_s / 1e9
    tf = gf / gu_s / 1e12
    mfma_peak = FP8_PEAK_TFLOPS if a8 else BF16_PEAK_TFLOPS  # the contraction's own operand type
    bound = "hbm" if gb / (HBM_PEAK_GBS * 1e9) >= gf / (mfma_peak * 1e12) else "mfma"
    if bound == "hbm":
        roof = dict(bound="hbm", achieved=round(bw, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(bw / HBM_PEAK_GBS, 4))
    else:
        roof = dict(bound="mfma", achieved=round(tf, 1), peak=mfma_peak, unit="TFLOP/s",
                    frac=round(tf / mfma_peak, 4))
    if lb < MALL_BYTES:  # the whole layer stays in the caches: launch-bound, no roofline claim
        roof = dict(bound="launch", note="layer fits the on-chip caches; launch-bound")
    roof.update(traffic=counter_traffic(name + ("_a8" if a8 else "") +
                                        ("_mxfp4" if wd == "mxfp4" else "")),
                kernel="gate_up_a8 (routed, FP8 activations)" if a8 else "gate_up (routed)",
                kernel_ms=round(r["gate_up_ms"], 4),
                kernel_ms_in_layer=(None if r["gate_up_ms_in_layer"] is None
                                    else round(r["gate_up_ms_in_layer"], 4)),
                algorithmic_bytes=gb, algorithmic_flops=gf)
    res = dict(
        workload=name, weights=wd, activations=act, T=T, H=H, I=I, E=E, k=k,
        tokens_per_s=T * steps / (r["total_ms"] * 1e-3), ms_per_step=ms,
        step_ms={q: round(v, 4) for q, v in r["step_ms"].items()},
        graph_ms_per_step=None if r["graph_ms"] is None else round(r["graph_ms"], 4),
        tokens_per_s_median=T / (r["step_ms"]["median"] * 1e-3),
        touched_experts=touched, layer_bytes=lb, layer_flops=lf,
        layer_hbm_frac=round(lb / (ms * 1e-3) / (HBM_PEAK_GBS * 1e9), 4),
        layer_bf16_mfma_frac=round(lf / (ms * 1e-3) / (BF16_PEAK_TFLOPS * 1e12), 4),
        layer_fp8_mfma_frac=round(lf / (ms * 1e-3) / (FP8_PEAK_TFLOPS * 1e12), 4),
        roofline=roof, wall_s=r["wall_s"])
    return layer, res


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="dsv3_decode")
    ap.add_argument("--prefill", default="dsv3_prefill", help="second workload ('' to skip)")
    ap.add_argument("--a8", default="dsv3_prefill",
                    help="workload also run in the FP8 activation mode ('' to skip)")
    ap.add_argument("--mxfp4", default="dsv3_decode",
                    help="workload also run with 4-bit MXFP4 expert weights ('' to skip)")
    ap.add_argument("--mxfp4-prefill", default="dsv3_prefill",
                    help="workload also run with MXFP4 weights and bf16 activations ('' to skip)")
    ap.add_argument("--w4a8", default="dsv3_prefill",
                    help="workload also run with MXFP4 weights and FP8 activations ('' to skip)")
    ap.add_argument("--extra", default=DEFAULT_EXTRA,
                    help="comma-separated further workloads to report under 'extra', each "
                         "name[/weights[/activations]] ('' to skip)")
    ap.add_argument("--ep-ranks", type=int, default=0,
                    help="also time rank 0's share of the decode and prefill layers under expert "
                         "parallelism over this many ranks (off by default: its smaller launches "
                         "of the same kernels would mix into a profile of the default run)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--vendor-ref", action="store_true",
                    help="also report the vendor GEMM library's rates at the expert shapes "
                         "(context only; off by default)")
    ap.add_argument("--cpu-threads", type=int, default=int(os.environ.get("OMP_NUM_THREADS", "0") or 0))
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="first run a plain device copy of this many MiB 5 times (a known-size "
                         "kernel that calibrates the HBM byte counters of a profiler run)")
    ap.add_argument("--only", default="",
                    help="run just this workload (name[/weights[/activations]]) and print its "
                         "result: the form the counter runs under a profiler use")
    ap.add_argument("--summarize-traffic", nargs=3, metavar=("KEY", "FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/gate_up_KEY_traffic.json from two rocprofv3 --pmc runs "
                         "(FETCH_SIZE, WRITE_SIZE) of `--only` and exit (no GPU)")
    ap.add_argument("--summarize-pmc", nargs="+", metavar="ARG",
                    help="OUT HEADER LABEL=DIR ...: write a text summary of --pmc runs and exit")
    ap.add_argument("--summarize-stats", nargs=3, metavar=("DIR", "OUT", "HEADER"),
                    help="write a text table of a --stats run's kernel statistics and exit")
    ap.add_argument("--command", action="append", default=[],
                    help="with --summarize-traffic: the profiler commands, recorded in the file")
    a = ap.parse_args(argv)
    if a.summarize_traffic:
        print(summarize_traffic(*a.summarize_traffic, commands=a.command))
        return 0
    if a.summarize_pmc:
        out, header, *runs = a.summarize_pmc
        print(summarize_pmc(out, header, [tuple(r.rsplit("=", 1)) for r in runs]))
        return 0
    if a.summarize_stats:
        print(summarize_stats(*a.summarize_stats))
        return 0
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        return 2

    import torch

    torch.cuda.set_device(0)
    if a.copy_probe_mib:
        src = torch.empty(a.copy_probe_mib << 18, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if a.only:
        parts = a.only.split("/")
        import synth

        over = {} if len(parts) < 2 else {"wdtype": parts[1]}
        lay = synth.make_layer(parts[0], seed=0, device="cuda", **over)
        _, r = run_workload(parts[0], a.steps, a.warmup,
                            act=parts[2] if len(parts) > 2 else "bf16", layer=lay)
        print(json.dumps({"only": a.only, **{k: (round(v, 4) if isinstance(v, float) else v)
                                               for k, v in r.items()}}))
        return 0
    probe = read_probe()
    layer, main_res = run_workload(a.workload, a.steps, a.warmup)
    if probe and main_res["roofline"]["unit"] == "GB/s":
        main_res["roofline"].update(read_probe_GBps=probe["GBps"], frac_of_read_probe=round(
            main_res["roofline"]["achieved"] / probe["GBps"], 4))
    cpu = None
    if not a.no_cpu:
        rows = list(range(layer.T))  # the decode layer has 16 tokens: the sample is all of them
        dt, threads = cpu_baseline(layer, rows, a.cpu_threads)
        cpu = dict(value=round(len(rows) / dt, 3), unit="tokens/s", cores=threads, kind="oracle",
                   sample=f"{len(rows)} tokens of the {a.workload} layer (all experts they select "
                          f"+ shared), {dt:.2f} s wall", cpu=cpu_model())
        # one thread: the tiny layer whole, and 4 tokens of the decode layer
        import synth

        single = {}
        tiny = synth.make_layer("tiny", seed=0, device="cuda")
        for name, lay, rws in (("tiny", tiny, list(range(tiny.T))), (a.workload, layer, [0, 1, 2, 3])):
            dt1, th1 = cpu_baseline(lay, rws, 1)
            single[name] = dict(value=round(len(rws) / dt1, 3), unit="tokens/s", cores=th1,
                                sample=f"{len(rws)} tokens of the {name} layer, {dt1:.3f} s wall")
        cpu["single_thread"] = single
        del tiny
    ep = {}
    if a.ep_ranks:
        ep[a.workload] = run_rank_share(layer, a.ep_ranks, 0, a.steps, a.warmup)
    del layer
    mx = None
    if a.mxfp4:
        torch.cuda.empty_cache()
        _, mx = run_workload(a.mxfp4, a.steps, a.warmup, wdtype="mxfp4")
    # every further workload is timed over the same `steps` layer steps as the headline one
    S, W = a.steps, a.warmup
    prefill = a8 = None
    if a.prefill:
        torch.cuda.empty_cache()
        player, prefill = run_workload(a.prefill, S, W)
        if not a.no_cpu:  # the oracle on a bounded sample of the prefill layer
            rows = list(range(0, player.T, max(1, player.T // 64)))[:64]
            dt, threads = cpu_baseline(player, rows, a.cpu_threads)
            prefill["cpu_baseline"] = dict(
                value=round(len(rows) / dt, 3), unit="tokens/s", cores=threads, kind="oracle",
                sample=f"{len(rows)} evenly spaced tokens of the {a.prefill} layer (all experts "
                       f"they select + shared), {dt:.2f} s wall")
        if a.ep_ranks:
            ep[a.prefill] = run_rank_share(player, a.ep_ranks, 0, S, W)
        if a.a8 == a.prefill:  # same layer, FP8 activations
            _, a8 = run_workload(a.a8, S, W, act="fp8", layer=player)
        del player
    if a.a8 and a8 is None:
        torch.cuda.empty_cache()
        _, a8 = run_workload(a.a8, S, W, act="fp8")
    mxp = w4 = None
    if a.mxfp4_prefill:
        torch.cuda.empty_cache()
        mlayer, mxp = run_workload(a.mxfp4_prefill, S, W, wdtype="mxfp4")
        if a.w4a8 == a.mxfp4_prefill:  # same layer, FP8 activations
            _, w4 = run_workload(a.w4a8, S, W, act="fp8", layer=mlayer)
        del mlayer
    if a.w4a8 and w4 is None:
        torch.cuda.empty_cache()
        _, w4 = run_workload(a.w4a8, S, W, act="fp8", wdtype="mxfp4")
    extra = {}
    specs = [w for w in a.extra.split(",") if w]
    layers = {}
    for spec in specs:
        # name[/weights][/activations]: e.g. dsv3_long_zipf, kimi_k2/fp8/fp8, dsv3_long_zipf/mxfp4/fp8
        parts = spec.split("/")
        name, wd = parts[0], (parts[1] if len(parts) > 1 else None)
        act = parts[2] if len(parts) > 2 else "bf16"
        import synth

        key = (name, wd or synth.CONFIGS[name]["wdtype"])
        if key not in layers:  # a layer is drawn once for all of its modes
            layers.clear()
            torch.cuda.empty_cache()
            over = {} if wd is None else {"wdtype": wd}
            layers[key] = synth.make_layer(name, seed=0, device="cuda", **over)
        _, r = run_workload(name, S, W, act=act, layer=layers[key])
        extra[spec] = {k: (round(v, 4) if isinstance(v, float) else v) for k, v in r.items()}
    layers.clear()
    vref = None
    if a.vendor_ref:
        torch.cuda.empty_cache()
        vref = vendor_reference()
    line = {
        "metric": METRIC,
        "value": round(main_res["tokens_per_s"], 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(main_res["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": a.workload, **{d: main_res[d] for d in ("T", "H", "I", "E", "k")},
                   "weights": "fp8_e4m3fn, fp32 128x128 block scales",
                   "activations": "bf16", "accumulate": "fp32", "shared_experts": 1,
                   "parallelism": "none (1 GPU)"},
        "roofline": main_res["roofline"],
        "cpu_baseline": cpu,
        "layer": {k: main_res[k] for k in ("touched_experts", "layer_bytes", "layer_flops",
                                           "layer_hbm_frac", "layer_bf16_mfma_frac",
                                           "layer_fp8_mfma_frac", "step_ms",
                                           "tokens_per_s_median", "graph_ms_per_step")},
        "prefill": None if prefill is None else {
            k: (round(v, 4) if isinstance(v, float) else v) for k, v in prefill.items()},
        "prefill_a8": None if a8 is None else {
            k: (round(v, 4) if isinstance(v, float) else v) for k, v in a8.items()},
        "decode_mxfp4": None if mx is None else {
            k: (round(v, 4) if isinstance(v, float) else v) for k, v in mx.items()},
        "ep_rank_share": ep or None,
        "extra": extra or None,
        "prefill_mxfp4": None if mxp is None else {
            k: (round(v, 4) if isinstance(v, float) else v) for k, v in mxp.items()},
        "prefill_mxfp4_a8": None if w4 is None else {
            k: (round(v, 4) if isinstance(v, float) else v) for k, v in w4.items()},
        "vendor_reference": vref,
        "hbm_read_probe": probe,
    }
    print(json.dumps(line))
    return 0


if __name__ == "__main__":
    sys.exit(main())
