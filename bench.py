"""Benchmark: packed gated-delta-rule prefill tokens/s per layer on one MI355X.

Default workload: a chat wave of 32 prompts x 1,024 tokens packed into one
pass (16 qk / 32 v heads, d = 128, bf16 q/k/v, fp32 gates and state, chunk
64, checkpoint every 256 tokens).  A step is one gdn_prefill_packed call on
that pack (the chunked scan with its checkpoint writes to device memory),
with the inputs resident in HBM.  The other rows of the path are timed in the
same run as legs: the conv at the same shape, the checkpoint copy on its own
stream, the decode batch and the mixed pass, and the long-prompt and ragged
packs.

Prints ONE JSON line on stdout.  ``--gpus N`` with N > 1 exits: the
benchmark runs on one GPU.
"""
from __future__ import annotations

import argparse
import json
import multiprocessing as mp
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
MFMA_F16_PEAK_TFLOPS = 2500.0   # dense fp16 / bf16 MFMA
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
CSRC = os.path.join(ROOT, "gated_deltanet_prefill_varlen_amd", "csrc")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ------------------------------------------------------- algorithmic work --

def prefill_alg_bytes(p, n_ckpt: int, init_nonzero: bool) -> int:
    """Bytes the method must move: q, k, v, g, beta in, out out, the final
    state per prompt (+ the initial state when given), and each checkpoint."""
    e = 2 if p.dtype == "bf16" else 4
    per_tok = (2 * p.Hqk * p.dk + p.Hv * p.dv) * e + 2 * p.Hv * 4 + p.Hv * p.dv * e
    state = p.Hv * p.dv * p.dk * 4
    return p.n_tokens * per_tok + p.n_seqs * state * (2 if init_nonzero else 1) + n_ckpt * state


def kernel_chunk(p) -> int:
    """Tokens per chunk the scan runs: min(chunk, 32) (a 64-token chunk's end
    state is the same quantity as two 32-token chunks')."""
    return min(p.chunk, 32)


def prefill_alg_flops(p) -> float:
    """Chunked form at the executed chunk C, per token per value head:
    2C(3dk + 2dv) + 6 dk dv + C^2/3."""
    C, dk, dv = kernel_chunk(p), p.dk, p.dv
    return p.n_tokens * p.Hv * (2 * C * (3 * dk + 2 * dv) + 6 * dk * dv + C * C / 3)


def step_min_bytes(p, n_ckpt: int) -> int:
    """The fewest bytes one pass of the whole step can move (conv fused into
    the scan, checkpoints written once into the pool): the pre-conv rows x in
    (as many bytes as q, k, v), g and beta in, out, the final states and each
    checkpoint once, the conv weights, each prompt's conv state and the conv
    window at each checkpoint.  The same bytes are the algorithmic bytes of
    one launch of the scan with the conv fused into its loads."""
    C = 2 * p.Hqk * p.dk + p.Hv * p.dv
    return (prefill_alg_bytes(p, n_ckpt, p.init is not None) + C * 4 * 4 +
            (p.n_seqs + n_ckpt) * 3 * C * 2)


# The C entry points' host-side validation: no device or launch code.
HOST_ONLY_SOURCES = ("gdn_api.hip",)


def csrc_digest() -> str:
    """sha256 over the device and launch sources (names and bytes, sorted by
    name): every file of csrc/ except the host-only validation of the entry
    points, which changes no kernel and no launch."""
    import hashlib
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name in HOST_ONLY_SOURCES:
            continue
        h.update(name.encode())
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload: str):
    """HBM bytes per launch of the prefill kernel on this workload from the
    committed counter runs (FETCH_SIZE and WRITE_SIZE, each scaled by what the
    counter reads for a copy of known size), or None when there is no record
    or the kernel sources changed since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("csrc_sha256") != csrc_digest():
        return None
    w = rec.get("workloads", {}).get(workload)
    return None if w is None else float(w["hbm_bytes_per_launch"])


# ------------------------------------------------- profile summaries (host) --

PREFILL_GRIDS = {786432: "chat", 98304: "long", 196608: "ragged"}   # work-items: workgroups x 768


def _csv_rows(d: str, suffix: str):
    import csv
    import glob
    files = sorted(glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True))
    if not files:
        raise SystemExit(f"no *{suffix} under {d}")
    with open(files[0]) as f:
        return list(csv.DictReader(f))


def summarize_profiles(prof_dir: str) -> dict:
    """Summaries of a rocprofv3 run set of this script: prof_dir/trace (kernel
    trace with stats), prof_dir/FETCH_SIZE and prof_dir/WRITE_SIZE (one
    counter each).  Prefill dispatches are told apart by grid size (chat wave,
    long prompts, ragged pack) and by kernel variant (the conv fused or not);
    the counters, in KiB per dispatch, are scaled by what they read for the
    device-pool checkpoint copy of the same run (96 items of 2 MiB read and
    written).  Writes profiles/traffic.json for the current kernel sources
    and returns the tables."""
    import collections
    def pref(name):
        if "pipelined_prefill_kernel<128, 128, false>" in name:
            return ""
        if "pipelined_prefill_kernel<128, 128, true>" in name:
            return "conv_fused_"
        return None
    # kernel trace: durations per (kernel, grid)
    tr = collections.defaultdict(list)
    for r in _csv_rows(os.path.join(prof_dir, "trace"), "kernel_trace.csv"):
        grid = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])
        tr[(r["Kernel_Name"], grid)].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    stats = _csv_rows(os.path.join(prof_dir, "trace"), "kernel_stats.csv")
    # counters
    cnt = {}
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        agg = collections.defaultdict(list)
        for r in _csv_rows(os.path.join(prof_dir, c), "counter_collection.csv"):
            agg[(r["Kernel_Name"], int(r["Grid_Size"]))].append(float(r["Counter_Value"]))
        cnt[c] = {k: (len(v), sum(v) / len(v)) for k, v in agg.items()}
    copies = [k for k in cnt["WRITE_SIZE"] if "snapshot_copy_kernel" in k[0]]
    ck = max(copies, key=lambda k: k[1])              # the device pool: most workgroups
    true_kib = 96 * 2 * 1024
    ff = true_kib / cnt["FETCH_SIZE"][ck][1]
    wf = true_kib / cnt["WRITE_SIZE"][ck][1]
    work = {}
    for (name, grid), (n, fk) in cnt["FETCH_SIZE"].items():
        pf = pref(name)
        if pf is None or grid not in PREFILL_GRIDS:
            continue
        wk = cnt["WRITE_SIZE"].get((name, grid), (0, float("nan")))[1]
        durs = tr.get((name, grid), [])
        work[pf + PREFILL_GRIDS[grid]] = {
            "fetch_kib": fk, "write_kib": wk, "hbm_bytes_per_launch": (fk * ff + wk * wf) * 1024,
            "dispatches": n, "trace_dispatches": len(durs),
            "trace_avg_us": statistics.fmean(durs) if durs else None}
    rec = {"csrc_sha256": csrc_digest(), "fetch_factor": ff, "write_factor": wf,
           "copy_kib_true": float(true_kib), "copy_fetch_kib": cnt["FETCH_SIZE"][ck][1],
           "copy_write_kib": cnt["WRITE_SIZE"][ck][1], "workloads": work}
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(rec, f, indent=1)
    top = sorted(stats, key=lambda r: -float(r["TotalDurationNs"]))[:10]
    return {"traffic": rec, "kernel_stats_top": [
        {"kernel": r["Name"], "calls": int(r["Calls"]), "avg_us": float(r["AverageNs"]) / 1e3,
         "min_us": float(r["MinNs"]) / 1e3, "max_us": float(r["MaxNs"]) / 1e3,
         "percent": float(r["Percentage"])} for r in top]}


def summarize_overlap(trace_dir: str) -> dict:
    """Kernels of the path on different hardware queues whose [start, end)
    intervals intersect, from a kernel trace of `--overlap-only`: per pair of
    (kernel, grid work-items), the count, the summed overlap and the summed
    duration of the shorter kernel; plus the mixed pass's steady-state loop
    (prefill pack and decode batch dispatches in it: start gap and span)."""
    import collections
    rows = _csv_rows(trace_dir, "kernel_trace.csv")
    ev = []
    for r in rows:
        n = r["Kernel_Name"]
        grid = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])
        kind = ("prefill" if "pipelined_prefill_kernel" in n else "decode" if "decode_kernel" in n
                else "copy" if "snapshot_copy_kernel" in n else None)
        if kind:
            ev.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), f"{kind}({grid})", r["Queue_Id"]))
    ev.sort()
    pairs = collections.defaultdict(lambda: [0, 0.0, 0.0])
    mixed = []
    for i, a in enumerate(ev):
        for b in ev[i + 1:]:
            if b[0] >= a[1]:
                break
            if a[3] == b[3]:
                continue
            key = " + ".join(sorted((a[2], b[2])))
            ov = (min(a[1], b[1]) - b[0]) / 1e3
            pairs[key][0] += 1
            pairs[key][1] += ov
            pairs[key][2] += min(a[1] - a[0], b[1] - b[0]) / 1e3
            if {a[2].split("(")[0], b[2].split("(")[0]} == {"prefill", "decode"}:
                mixed.append({"gap_us": (b[0] - a[0]) / 1e3, "span_us": (max(a[1], b[1]) - a[0]) / 1e3,
                              "first_us": (a[1] - a[0]) / 1e3, "second_us": (b[1] - b[0]) / 1e3,
                              "first": a[2]})
    med = lambda k: statistics.median(m[k] for m in mixed) if mixed else None
    return {"pairs": {k: {"count": v[0], "overlap_us": v[1], "shorter_us": v[2],
                          "share": v[1] / v[2] if v[2] else None} for k, v in pairs.items()},
            "mixed_pass_pairs": len(mixed),
            "mixed_pass_median": {k: med(k) for k in ("gap_us", "span_us", "first_us", "second_us")}}


def summarize_sq(prof_dir: str) -> dict:
    """SQ counter summaries of the prefill kernel per workload, from
    prof_dir/sq_<run>_p<k> (several counter passes of `--no-legs --workload
    <workload>` runs; run "chat" with `--step two-launch` for the scan alone,
    "chatfused" for the chat wave's fused scan): medians over the workload's
    prefill dispatches, per workgroup and chunk, and busy and wait fractions.
    The wave-cycle counters count 4-cycle units; GRBM_GUI_ACTIVE is summed
    over the 8 XCDs."""
    import collections
    import glob
    import workloads as W
    packs = {"chat": W.chat_wave(seed=0), "long": W.long_prompts(seed=0), "ragged": W.ragged_pack(seed=0)}
    out = {}
    runs = (("chat", "chat", "false"), ("conv_fused_chat", "chatfused", "true"),
            ("long", "long", "false"), ("ragged", "ragged", "false"))
    for key, run, variant in runs:
        w = key.replace("conv_fused_", "")
        p = packs[w]
        grid = {"chat": 786432, "long": 98304, "ragged": 196608}[w]
        vals = collections.defaultdict(list)
        times = []
        kname = f"pipelined_prefill_kernel<128, 128, {variant}>"
        for d in sorted(x for x in glob.glob(os.path.join(prof_dir, f"sq_{run}_p*")) if os.path.isdir(x)):
            for r in _csv_rows(d, "counter_collection.csv"):
                if kname in r["Kernel_Name"] and int(r["Grid_Size"]) == grid:
                    vals[r["Counter_Name"]].append(float(r["Counter_Value"]))
                    if r["Counter_Name"] == "GRBM_GUI_ACTIVE":
                        times.append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        if not vals:
            continue
        m = {k: statistics.median(v) for k, v in vals.items()}
        wgs = p.n_seqs * p.Hv
        lens = np.diff(p.cu_seqlens)
        chunks = int(sum((int(L) + 31) // 32 for L in lens)) * p.Hv
        cycles = m["GRBM_GUI_ACTIVE"] / 8
        simds = 1024
        used = min(wgs, 256) * 4
        t_us = statistics.median(times)
        per = {k: m[k] / chunks for k in ("SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS", "SQ_INSTS_SALU",
                                          "SQ_INSTS_VMEM_RD", "SQ_INSTS_VMEM_WR") if k in m}
        out[key] = {
            "workgroups": wgs, "chunks": chunks, "dispatches": len(times), "dispatch_us": t_us,
            "clock_GHz": cycles / t_us / 1e3,
            "per_workgroup_chunk": per,
            "cycles_per_chunk_interval": cycles / (chunks / min(wgs, 256)) if wgs else None,
            "valu_busy_all_simds": 4 * m["SQ_ACTIVE_INST_VALU"] / (simds * cycles),
            "valu_busy_used_simds": 4 * m["SQ_ACTIVE_INST_VALU"] / (used * cycles),
            "mfma_busy_used_simds": m["SQ_VALU_MFMA_BUSY_CYCLES"] / (used * cycles),
            "waves_per_simd_all": 4 * m["SQ_WAVE_CYCLES"] / (simds * cycles),
            "waves_per_simd_used": 4 * m["SQ_WAVE_CYCLES"] / (used * cycles),
            "wait_any_frac": m["SQ_WAIT_ANY"] / m["SQ_WAVE_CYCLES"],
            "wait_lds_frac": m["SQ_WAIT_INST_LDS"] / m["SQ_WAVE_CYCLES"],
            "lds_bank_conflict_frac": m["SQ_LDS_BANK_CONFLICT"] / m["SQ_LDS_IDX_ACTIVE"],
            "raw_medians": m}
    return out


# --------------------------------------------------------------- GPU legs --

class Timer:
    """HIP events on one stream around each launch; returns per-launch ms.
    The launches (each after the optional cache flush, outside its events)
    are queued back to back with no host wait between them, as a serving
    loop issues them, and the events are read once the last has completed."""

    def __init__(self, torch, stream):
        self.torch, self.stream = torch, stream

    def run(self, fn, reps: int, flush=None):
        t = self.torch
        evs = []
        for _ in range(reps):
            if flush is not None:
                with t.cuda.stream(self.stream):
                    flush()
            a, b = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
            a.record(self.stream)
            fn()
            b.record(self.stream)
            evs.append((a, b))
        evs[-1][1].synchronize()
        return [a.elapsed_time(b) for a, b in evs]


def make_flush(torch, dev):
    buf = torch.empty(1 << 28, dtype=torch.float32, device=dev)   # 1 GiB > 256 MB MALL

    def flush():
        buf.fill_(1.0)
    return flush


def io_t(torch, a, dtype):
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16)).view(torch.bfloat16).to("cuda:0")
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda:0")


def f32_t(torch, a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda:0")


def i32_t(torch, a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to("cuda:0")


class DevPack:
    """A pack resident in HBM with its output buffers; ``run`` is one
    gdn_prefill_packed call."""

    def __init__(self, torch, gdn, p, ck):
        self.gdn, self.p = gdn, p
        self.ck = np.asarray(ck, dtype=np.int32)
        self.cu = i32_t(torch, p.cu_seqlens)
        self.q, self.k, self.v = (io_t(torch, a, p.dtype) for a in (p.q, p.k, p.v))
        self.g, self.beta = f32_t(torch, p.g), f32_t(torch, p.beta)
        self.init = None if p.init is None else f32_t(torch, p.init)
        self.ck_d = i32_t(torch, self.ck) if len(self.ck) else None
        odt = torch.bfloat16 if p.dtype == "bf16" else torch.float32
        self.out = torch.empty((p.n_tokens, p.Hv, p.dv), dtype=odt, device="cuda:0")
        self.final = torch.empty((p.n_seqs, p.Hv, p.dv, p.dk), dtype=torch.float32, device="cuda:0")
        self.ckbuf = (torch.empty((len(self.ck), p.Hv, p.dv, p.dk), dtype=torch.float32, device="cuda:0")
                      if len(self.ck) else None)
        self.shape = gdn.make_shape(p.Hqk, p.Hv, p.dk, p.dv, p.chunk,
                                    gdn.GDN_BF16 if p.dtype == "bf16" else gdn.GDN_F32, scale=p.scale)

    def run(self, stream=None):
        self.gdn.gdn_prefill_packed(self.shape, self.cu, self.p.cu_seqlens, self.q, self.k, self.v,
                                    self.g, self.beta, self.init, self.ck_d,
                                    self.ck if len(self.ck) else None, self.out, self.final, self.ckbuf,
                                    stream=stream)


def bench_prefill(torch, gdn, p, steps, warmup, stream, flush, label):
    ck = gdn.gdn_plan_checkpoints(p.cu_seqlens, p.block)
    dp = DevPack(torch, gdn, p, ck)
    with torch.cuda.stream(stream):
        for _ in range(warmup):
            dp.run(stream=stream)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        times = Timer(torch, stream).run(lambda: dp.run(stream=stream), steps, flush)
        wall_ms = (time.perf_counter() - t0) * 1e3
    torch.cuda.synchronize()
    med = statistics.median(times)
    B = prefill_alg_bytes(p, len(ck), p.init is not None)
    F = prefill_alg_flops(p)
    t_roof = max(B / (HBM_PEAK_GBS * 1e9), F / (MFMA_F16_PEAK_TFLOPS * 1e12))
    res = {
        "workload": label, "tokens": p.n_tokens, "prompts": p.n_seqs, "checkpoints": int(len(ck)),
        "ms_median": med, "ms_mean": statistics.fmean(times),
        "ms_p10": float(np.percentile(times, 10)), "ms_p90": float(np.percentile(times, 90)),
        "tokens_per_s": p.n_tokens / (med * 1e-3), "alg_bytes": B, "alg_flops": F,
        "achieved_GBs": B / (med * 1e-3) / 1e9, "roofline_frac": t_roof / (med * 1e-3),
        "wall_ms_timed": wall_ms,
    }
    del dp
    return res, times


def conv_alg_bytes(T: int, N: int, C: int, n_ckpt: int, e: int = 2) -> int:
    """Bytes the conv must move: x in, y out, weights, each prompt's conv state
    (last three inputs) and the three-input window at each checkpoint."""
    return 2 * T * C * e + C * 4 * 4 + (N + n_ckpt) * 3 * C * e


def bench_layer_step(torch, gdn, p, steps, warmup, stream, label, fused=False):
    """One step is one pass of the whole hot path over the chat wave: the
    packed conv1d + SiLU from the pre-conv rows x into one [T, conv_dim]
    tensor (with the prompts' conv states and the conv windows at the
    checkpoints), the scan reading q, k, v as column views of it (checkpoints
    into a device buffer, final states), and the copy of those checkpoints
    into a device pool.  Steps run as a model's consecutive layers would:
    each step's copy goes on a copy stream right after its scan (an event
    from the scan), so it reads the checkpoints while the memory-side cache
    still holds them and runs beside the next step's conv; two checkpoint
    buffers alternate, and a step waits, ahead of its conv, for the copy
    that last read its scan's buffer (the copy of two steps before).  The timed region is the K steps
    queued back to back between two device synchronisations, the last step's
    copy joined before its closing event.  Inside it only the scan carries
    events (its own time, for its roofline); a second region of K steps with
    events around each conv as well gives the breakdown (each event pair
    costs a few microseconds, so that region is not the headline).  With
    ``fused`` the conv and the scan are one gdn_prefill_conv_packed call (the
    conv in the scan's loads; the same conv states and windows), timed as
    "scan"."""
    T, N = p.n_tokens, p.n_seqs
    C = 2 * p.Hqk * p.dk + p.Hv * p.dv
    ck = gdn.gdn_plan_checkpoints(p.cu_seqlens, p.block)
    n_ck = len(ck)
    x = io_t(torch, p.x, p.dtype)
    w = f32_t(torch, p.conv_w)
    y = torch.empty_like(x)
    conv_state = torch.empty((N, 3, C), dtype=x.dtype, device="cuda:0")
    conv_ckpt = torch.empty((n_ck, 3, C), dtype=x.dtype, device="cuda:0")
    cu_d, ck_d = i32_t(torch, p.cu_seqlens), i32_t(torch, ck)
    g, beta = f32_t(torch, p.g), f32_t(torch, p.beta)
    qv, kv, vv = y[:, :p.Hqk * p.dk], y[:, p.Hqk * p.dk:2 * p.Hqk * p.dk], y[:, 2 * p.Hqk * p.dk:]
    out = torch.empty((T, p.Hv, p.dv), dtype=x.dtype, device="cuda:0")
    final = torch.empty((N, p.Hv, p.dv, p.dk), dtype=torch.float32, device="cuda:0")
    ckbufs = [torch.empty((n_ck, p.Hv, p.dv, p.dk), dtype=torch.float32, device="cuda:0") for _ in range(2)]
    pool_slots = n_ck + 32
    pool = torch.empty((pool_slots, p.Hv, p.dv, p.dk), dtype=torch.float32, device="cuda:0")
    slots = np.random.default_rng(0).permutation(pool_slots)[:n_ck].astype(np.int64)
    slots_d = torch.from_numpy(slots).to("cuda:0")
    each = p.Hv * p.dv * p.dk * 4
    shape = gdn.make_shape(p.Hqk, p.Hv, p.dk, p.dv, p.chunk,
                           gdn.GDN_BF16 if p.dtype == "bf16" else gdn.GDN_F32, scale=p.scale,
                           q_tok_stride=C, k_tok_stride=C, v_tok_stride=C)
    cstream = torch.cuda.Stream()
    scan_done = [torch.cuda.Event(), torch.cuda.Event()]
    copy_done = [torch.cuda.Event(), torch.cuda.Event()]

    def run(n, rec=None, conv_events=False):
        for i in range(n):
            b = i % 2
            e = rec[i] if rec else None
            # the copy that last read this step's checkpoint buffer (two steps
            # back; it ran beside the previous conv, so this wait is already
            # met: placed ahead of the conv it keeps the conv-to-scan edge free
            # of a cross-stream wait)
            stream.wait_event(copy_done[b])
            if e and conv_events:
                e[0].record(stream)
            if not fused:
                gdn.gdn_conv1d_silu_packed(shape, cu_d, p.cu_seqlens, x, w, y, None, conv_state, ck_d, ck,
                                           conv_ckpt, stream=stream)
            if e and conv_events:
                e[1].record(stream)
            if e:
                e[2].record(stream)
            if fused:
                gdn.gdn_prefill_conv_packed(shape, cu_d, p.cu_seqlens, x, w, g, beta, None, ck_d, ck, out,
                                            final, ckbufs[b], conv_state_out=conv_state,
                                            conv_ckpt=conv_ckpt, stream=stream)
            else:
                gdn.gdn_prefill_packed(shape, cu_d, p.cu_seqlens, qv, kv, vv, g, beta, None, ck_d, ck,
                                       out, final, ckbufs[b], stream=stream)
            # one event marks the scan's end, for its timing and for the copy
            done = e[3] if e else scan_done[b]
            done.record(stream)
            gdn.gdn_snapshot_copy(ckbufs[b], n_ck, each, pool, slots_d, slots, pool_slots,
                                  wait_event=done, copy_stream=cstream, done_event=copy_done[b])
        stream.wait_event(copy_done[(n - 1) % 2])

    def region(conv_events):
        rec = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        start.record(stream)
        run(steps, rec, conv_events)
        end.record(stream)
        end.synchronize()
        torch.cuda.synchronize()
        return rec, start.elapsed_time(end), (time.perf_counter() - t0) * 1e3

    with torch.cuda.stream(stream):
        run(warmup)
        rec, region_ms, wall_ms = region(False)
        rec_b, region_b_ms, _ = region(True)
    per_step = region_ms / steps
    spacing = [rec[i][2].elapsed_time(rec[i + 1][2]) for i in range(steps - 1)]
    scan_ms = [c.elapsed_time(d) for a, b, c, d in rec]
    conv_ms = [a.elapsed_time(b) for a, b, c, d in rec_b]
    scan_b_ms = [c.elapsed_time(d) for a, b, c, d in rec_b]
    B_scan = prefill_alg_bytes(p, n_ck, p.init is not None)
    B_conv = conv_alg_bytes(T, N, C, n_ck)
    B_copy = 2 * n_ck * each
    F = prefill_alg_flops(p)
    exact = bool(torch.equal(pool[slots_d], ckbufs[(steps - 1) % 2]) and torch.equal(ckbufs[0], ckbufs[1]))
    return {
        "workload": label, "tokens": T, "prompts": N, "checkpoints": int(n_ck),
        "ms_per_step": per_step, "region_ms": region_ms, "region_wall_ms": wall_ms,
        "tokens_per_s": T / (per_step * 1e-3),
        "step_spacing_ms_median": statistics.median(spacing) if spacing else per_step,
        "step_spacing_ms_p10": float(np.percentile(spacing, 10)) if spacing else per_step,
        "step_spacing_ms_p90": float(np.percentile(spacing, 90)) if spacing else per_step,
        "scan_ms_median": statistics.median(scan_ms), "scan_ms_mean": statistics.fmean(scan_ms),
        "breakdown_region": {"ms_per_step": region_b_ms / steps,
                             "conv_ms_median": statistics.median(conv_ms),
                             "scan_ms_median": statistics.median(scan_b_ms)},
        "scan_alg_bytes": B_scan, "scan_alg_flops": F,
        "step_alg_bytes": (step_min_bytes(p, n_ck) + B_copy) if fused else B_scan + B_conv + B_copy,
        "step_min_bytes": step_min_bytes(p, n_ck),
        "copy_exact": exact,
    }


def bench_conv_fused_packs(torch, gdn, stream, flush, reps, W):
    """Scan and conv per pack: the conv kernel, the scan on its output, both
    in turn, and the scan with the conv fused into its loads (one call, the
    same conv states and windows), for the chat wave, the long prompts and
    the ragged pack (each with its conv inputs)."""
    packs = {"chat": W.chat_wave(seed=0, with_conv=True),
             "long": W.make_pack("long_4x8192_conv", [8192] * 4, 16, 32, 128, 128, 64, 1024,
                                 with_conv=True, conv_std=0.5),
             "ragged": W.make_pack("ragged_8_conv", W._ragged_lengths(), 16, 32, 128, 128, 64, 256,
                                   with_conv=True, conv_std=0.5, init_std=0.1)}
    res = {}
    for name, p in packs.items():
        T, N, C = p.n_tokens, p.n_seqs, 2 * p.Hqk * p.dk + p.Hv * p.dv
        ck = gdn.gdn_plan_checkpoints(p.cu_seqlens, p.block)
        n_ck = len(ck)
        x, w = io_t(torch, p.x, "bf16"), f32_t(torch, p.conv_w)
        y = torch.empty_like(x)
        st = torch.empty((N, 3, C), dtype=torch.bfloat16, device="cuda:0")
        cck = torch.empty((max(n_ck, 1), 3, C), dtype=torch.bfloat16, device="cuda:0")
        cu, ckd = i32_t(torch, p.cu_seqlens), i32_t(torch, ck)
        g, beta = f32_t(torch, p.g), f32_t(torch, p.beta)
        init = None if p.init is None else f32_t(torch, p.init)
        out = torch.empty((T, p.Hv, p.dv), dtype=torch.bfloat16, device="cuda:0")
        fin = torch.empty((N, p.Hv, p.dv, p.dk), dtype=torch.float32, device="cuda:0")
        ckb = torch.empty((max(n_ck, 1), p.Hv, p.dv, p.dk), dtype=torch.float32, device="cuda:0")
        sh = gdn.make_shape(p.Hqk, p.Hv, p.dk, p.dv, p.chunk, q_tok_stride=C, k_tok_stride=C,
                            v_tok_stride=C)
        Hd = p.Hqk * p.dk

        def conv():
            gdn.gdn_conv1d_silu_packed(sh, cu, p.cu_seqlens, x, w, y, None, st, ckd, ck, cck, stream=stream)

        def scan():
            gdn.gdn_prefill_packed(sh, cu, p.cu_seqlens, y[:, :Hd], y[:, Hd:2 * Hd], y[:, 2 * Hd:], g, beta,
                                   init, ckd, ck, out, fin, ckb, stream=stream)

        def both():
            conv()
            scan()

        def fused():
            gdn.gdn_prefill_conv_packed(sh, cu, p.cu_seqlens, x, w, g, beta, init, ckd, ck, out, fin, ckb,
                                        conv_state_out=st, conv_ckpt=cck, stream=stream)
        r = {"tokens": T, "prompts": N}
        with torch.cuda.stream(stream):
            for lab, fn in (("conv_ms", conv), ("scan_ms", scan), ("conv_then_scan_ms", both),
                            ("fused_ms", fused)):
                for _ in range(3):
                    fn()
                torch.cuda.synchronize()
                r[lab] = statistics.median(Timer(torch, stream).run(fn, reps, flush))
        r["fused_vs_two_launches"] = r["fused_ms"] / r["conv_then_scan_ms"]
        res[name] = r
        del x, y, out, fin, ckb
    return res


def bench_conv(torch, gdn, stream, flush, reps):
    T, Hqk, Hv, d = 32768, 16, 32, 128
    C = 2 * Hqk * d + Hv * d
    cu = np.arange(0, T + 1, 1024, dtype=np.int32)
    x = torch.randn((T, C), device="cuda:0").to(torch.bfloat16)
    w = torch.randn((C, 4), device="cuda:0") * 0.5
    y = torch.empty_like(x)
    st = torch.empty((len(cu) - 1, 3, C), dtype=torch.bfloat16, device="cuda:0")
    shape = gdn.make_shape(Hqk, Hv, d, d, 64)
    cu_d = i32_t(torch, cu)
    fn = lambda: gdn.gdn_conv1d_silu_packed(shape, cu_d, cu, x, w, y, None, st, stream=stream)
    fn()
    times = Timer(torch, stream).run(fn, reps, flush)
    med = statistics.median(times)
    B = 2 * T * C * 2 + st.numel() * 2 + w.numel() * 4
    return {"workload": "conv1d_silu 32x1024 tokens x 8192 ch bf16", "ms_median": med,
            "achieved_GBs": B / (med * 1e-3) / 1e9, "roofline_frac": B / (med * 1e-3) / 1e9 / HBM_PEAK_GBS}


def bench_snapshot(torch, gdn, stream, flush, reps):
    n, Hv, d = 96, 32, 128
    src = torch.randn((n, Hv, d, d), device="cuda:0")
    pool = torch.empty((n + 32, Hv, d, d), device="cuda:0")
    slots = np.random.default_rng(0).permutation(n + 32)[:n].astype(np.int64)
    slots_d = torch.from_numpy(slots).to("cuda:0")
    each = Hv * d * d * 4
    fn = lambda: gdn.gdn_snapshot_copy(src, n, each, pool, slots_d, slots, n + 32, copy_stream=stream)
    fn()
    times = Timer(torch, stream).run(fn, reps, flush)
    med = statistics.median(times)
    B = 2 * n * each
    ok = bool(torch.equal(pool[slots_d], src))
    return {"workload": "checkpoint copy 96 x 2 MiB device pool", "ms_median": med,
            "achieved_GBs": B / (med * 1e-3) / 1e9, "roofline_frac": B / (med * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "exact": ok}


def _pinned_device_address(t) -> int:
    """Device address of a pinned host tensor (hipHostGetDevicePointer)."""
    import ctypes
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipHostGetDevicePointer.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_void_p, ctypes.c_uint]
    d = ctypes.c_void_p()
    rc = hip.hipHostGetDevicePointer(ctypes.byref(d), ctypes.c_void_p(t.data_ptr()), 0)
    if rc != 0 or not d.value:
        raise RuntimeError(f"hipHostGetDevicePointer returned {rc}")
    return d.value


def bench_prefix_cache(torch, gdn, stream, flush, reps):
    """Checkpoint gather into a pinned host pool allocated once (device writes
    over the host link), then the H2D restore of 32 states into init_state."""
    n, Hv, d = 96, 32, 128
    src = torch.randn((n, Hv, d, d), device="cuda:0")
    pool = torch.zeros((n + 32, Hv, d, d), dtype=torch.float32, pin_memory=True)
    addr = _pinned_device_address(pool)
    slots = np.random.default_rng(0).permutation(n + 32)[:n].astype(np.int64)
    slots_d = torch.from_numpy(slots).to("cuda:0")
    each = Hv * d * d * 4
    fn = lambda: gdn.gdn_snapshot_copy(src, n, each, addr, slots_d, slots, n + 32, copy_stream=stream)
    fn()
    torch.cuda.synchronize()
    ok = bool(torch.equal(pool[torch.from_numpy(slots[:4])], src[:4].cpu()))
    t_copy = statistics.median(Timer(torch, stream).run(fn, reps, flush))
    init = torch.empty((32, Hv, d, d), dtype=torch.float32, device="cuda:0")
    rs = torch.from_numpy(slots[:32])

    def restore():
        for i in range(32):
            init[i].copy_(pool[int(rs[i])], non_blocking=True)
    with torch.cuda.stream(stream):
        restore()
    torch.cuda.synchronize()
    ok = ok and bool(torch.equal(init[:2].cpu(), pool[rs[:2]]))
    with torch.cuda.stream(stream):
        t_rest = statistics.median(Timer(torch, stream).run(restore, reps))
    return {"workload": "prefix cache: 96 x 2 MiB checkpoints to a pinned host pool; 32 x 2 MiB restored",
            "copy_ms": t_copy, "copy_GBs": n * each / (t_copy * 1e-3) / 1e9,
            "restore_ms": t_rest, "restore_GBs": 32 * each / (t_rest * 1e-3) / 1e9, "exact": ok}


def bench_decode(torch, gdn, stream, flush, reps):
    import workloads as W
    d = W.decode_batch(seed=0, batch=32, pool=64)
    q, k, v = (io_t(torch, a, "bf16") for a in (d.q, d.k, d.v))
    g, b = f32_t(torch, d.g), f32_t(torch, d.beta)
    st = f32_t(torch, d.state)
    slot = i32_t(torch, d.slot)
    out = torch.empty((32, 32, 128), dtype=torch.bfloat16, device="cuda:0")
    shape = gdn.make_shape(16, 32, 128, 128, 64)
    fn = lambda: gdn.gdn_decode_step(shape, q, k, v, g, b, st, slot, d.slot, out, stream=stream)
    fn()
    times = Timer(torch, stream).run(fn, reps, flush)
    med = statistics.median(times)
    B = 32 * 32 * 128 * 128 * 4 * 2 + 32 * (2 * 16 * 128 * 2 + 32 * 128 * 2 * 2 + 32 * 8)
    return {"workload": "decode 32 seqs x 32 heads, fp32 state in place", "ms_median": med,
            "achieved_GBs": B / (med * 1e-3) / 1e9, "roofline_frac": B / (med * 1e-3) / 1e9 / HBM_PEAK_GBS}


def bench_decode_conv(torch, gdn, stream, flush, reps):
    """The decode batch with the short conv applied in the decode kernel:
    q, k, v are the conv's inputs, each slot's conv window supplies the
    history and is moved on by a second launch."""
    import workloads as W
    d = W.decode_batch(seed=0, batch=32, pool=64)
    C = 2 * 16 * 128 + 32 * 128
    rng = np.random.default_rng(1)
    x = torch.from_numpy(W.f32_to_bf16_bits(rng.standard_normal((32, C)).astype(np.float32))).view(torch.bfloat16).to("cuda:0")
    w = f32_t(torch, (0.5 * rng.standard_normal((C, 4))).astype(np.float32))
    cs = torch.from_numpy(W.f32_to_bf16_bits(rng.standard_normal((64, 3, C)).astype(np.float32))).view(torch.bfloat16).to("cuda:0")
    g, b = f32_t(torch, d.g), f32_t(torch, d.beta)
    st, slot = f32_t(torch, d.state), i32_t(torch, d.slot)
    out = torch.empty((32, 32, 128), dtype=torch.bfloat16, device="cuda:0")
    shape = gdn.make_shape(16, 32, 128, 128, 64, q_tok_stride=C, k_tok_stride=C, v_tok_stride=C)
    nq = 16 * 128
    fn = lambda: gdn.gdn_decode_step(shape, x[:, :nq], x[:, nq:2 * nq], x[:, 2 * nq:], g, b, st, slot, d.slot,
                                     out, conv_w=w, conv_state=cs, stream=stream)
    fn()
    times = Timer(torch, stream).run(fn, reps, flush)
    med = statistics.median(times)
    B = 32 * 32 * 128 * 128 * 4 * 2 + 32 * (C * 2 + 2 * 3 * C * 2 + 32 * 128 * 2 + 32 * 8) + C * 16
    return {"workload": "decode 32 seqs x 32 heads with the conv (windows in a slot pool)", "ms_median": med,
            "achieved_GBs": B / (med * 1e-3) / 1e9, "roofline_frac": B / (med * 1e-3) / 1e9 / HBM_PEAK_GBS}


def bench_decode_tokens(torch, gdn, stream, flush, reps):
    """Speculative verification: 32 sequences x 4 tokens, the state after each
    token kept (snapshots), pool rows advanced by 4 tokens."""
    import workloads as W
    B, n = 32, 4
    ds = [W.decode_batch(seed=10 + i, batch=B) for i in range(n)]
    cat = lambda key: np.stack([getattr(d, key) for d in ds], axis=1).reshape((B * n,) + getattr(ds[0], key).shape[1:])
    q, k, v = (io_t(torch, cat(a), "bf16") for a in ("q", "k", "v"))
    g, b = f32_t(torch, cat("g")), f32_t(torch, cat("beta"))
    st, slot = f32_t(torch, ds[0].state), i32_t(torch, ds[0].slot)
    out = torch.empty((B * n, 32, 128), dtype=torch.bfloat16, device="cuda:0")
    snaps = torch.empty((B, n, 32, 128, 128), dtype=torch.float32, device="cuda:0")
    shape = gdn.make_shape(16, 32, 128, 128, 64)
    fn = lambda: gdn.gdn_decode_tokens(shape, n, q, k, v, g, b, st, slot, ds[0].slot, out, snaps, stream=stream)
    fn()
    times = Timer(torch, stream).run(fn, reps, flush)
    med = statistics.median(times)
    each = 32 * 128 * 128 * 4
    B_alg = B * each * (2 + n) + B * n * (2 * 16 * 128 * 2 + 32 * 128 * 2 * 2 + 32 * 8)
    return {"workload": "decode 32 seqs x 4 tokens x 32 heads, state kept after every token",
            "ms_median": med, "achieved_GBs": B_alg / (med * 1e-3) / 1e9,
            "roofline_frac": B_alg / (med * 1e-3) / 1e9 / HBM_PEAK_GBS}


def bench_mixed(torch, gdn, stream, flush, reps):
    import workloads as W
    pack, d = W.mixed_step(seed=0)
    dp = DevPack(torch, gdn, pack, [])
    q, k, v = (io_t(torch, a, "bf16") for a in (d.q, d.k, d.v))
    g, b = f32_t(torch, d.g), f32_t(torch, d.beta)
    st, slot = f32_t(torch, d.state), i32_t(torch, d.slot)
    out = torch.empty((32, 32, 128), dtype=torch.bfloat16, device="cuda:0")
    shape = gdn.make_shape(16, 32, 128, 128, 64)

    def fn():
        dp.run(stream=stream)
        gdn.gdn_decode_step(shape, q, k, v, g, b, st, slot, d.slot, out, stream=stream)
    fn()
    times = Timer(torch, stream).run(fn, reps, flush)
    med = statistics.median(times)
    toks = pack.n_tokens + d.batch
    return {"workload": f"mixed pass: {pack.n_tokens} prefill tokens ({pack.n_seqs} prompts) + 32 decodes",
            "ms_median": med, "tokens_per_s": toks / (med * 1e-3)}


def bench_overlap(torch, gdn, stream, flush, reps):
    """Work on its own streams overlapping: (a) the mixed pass, prefill pack on
    one stream and the decode batch on another, against each alone; (b) the
    checkpoint copy of one layer on a copy stream while the next layer's scan
    runs, against the same launches serialised on one stream (device pool,
    and pinned host pool over the host link)."""
    import workloads as W
    sA, sB = stream, torch.cuda.Stream()

    def joined(fa, fb, b_first=False):
        """fa on sA and fb on sB from a common start (fb enqueued first when
        b_first), sA waiting for sB at the end."""
        def run():
            e0 = torch.cuda.Event()
            e0.record(sA)
            sB.wait_event(e0)
            if b_first:
                fb()
                fa()
            else:
                fa()
                fb()
            e1 = torch.cuda.Event()
            e1.record(sB)
            sA.wait_event(e1)
        return run

    med = lambda fn, st: statistics.median(Timer(torch, st).run(fn, reps, flush))
    out = {}
    # (a) mixed pass
    pack, d = W.mixed_step(seed=0)
    dp = DevPack(torch, gdn, pack, [])
    q, k, v = (io_t(torch, a, "bf16") for a in (d.q, d.k, d.v))
    g, b = f32_t(torch, d.g), f32_t(torch, d.beta)
    st, slot = f32_t(torch, d.state), i32_t(torch, d.slot)
    o = torch.empty((32, 32, 128), dtype=torch.bfloat16, device="cuda:0")
    shape = gdn.make_shape(16, 32, 128, 128, 64)
    pre = lambda: dp.run(stream=sA)
    dec_a = lambda: gdn.gdn_decode_step(shape, q, k, v, g, b, st, slot, d.slot, o, stream=sA)
    dec_b = lambda: gdn.gdn_decode_step(shape, q, k, v, g, b, st, slot, d.slot, o, stream=sB)
    t_p, t_d = med(pre, sA), med(dec_a, sA)
    t_serial = med(lambda: (pre(), dec_a()), sA)
    t_two = med(joined(pre, dec_b), sA)
    out["mixed_pass"] = {"prefill_ms": t_p, "decode_ms": t_d, "one_stream_ms": t_serial,
                         "two_streams_ms": t_two, "overlap_saved_ms": t_serial - t_two}
    # K passes back to back as a serving loop issues them (one cache flush
    # ahead of the region, none between passes): one stream; two streams
    # joined after every pass (the next pass starts when both parts ended);
    # two streams each running its part of every pass, joined once at the end
    K = 50

    def region(body):
        torch.cuda.synchronize()
        with torch.cuda.stream(sA):
            flush()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(sA)
        body()
        b.record(sA)
        b.synchronize()
        return a.elapsed_time(b) / K

    def fork():
        e = torch.cuda.Event()
        e.record(sA)
        sB.wait_event(e)

    def join():
        e = torch.cuda.Event()
        e.record(sB)
        sA.wait_event(e)

    def loop_one():
        for _ in range(K):
            pre()
            dec_a()

    def loop_joined_each():
        for _ in range(K):
            fork()
            pre()
            dec_b()
            join()

    def loop_joined_once():
        fork()
        for _ in range(K):
            pre()
            dec_b()
        join()
    steady = {}
    for name, body in (("prefill_only_ms", lambda: [pre() for _ in range(K)]),
                       ("decode_only_ms", lambda: [dec_a() for _ in range(K)]),
                       ("one_stream_ms", loop_one), ("two_streams_joined_each_pass_ms", loop_joined_each),
                       ("two_streams_joined_once_ms", loop_joined_once)):
        region(body)
        steady[name] = statistics.median(region(body) for _ in range(3))
    steady["saved_joined_each_pass"] = 1 - steady["two_streams_joined_each_pass_ms"] / steady["one_stream_ms"]
    steady["saved_joined_once"] = 1 - steady["two_streams_joined_once_ms"] / steady["one_stream_ms"]
    out["mixed_pass"]["steady_state_per_pass"] = steady
    del dp
    # (b) checkpoint copy beside the next layer's scan
    p = W.chat_wave(seed=0)
    ck = gdn.gdn_plan_checkpoints(p.cu_seqlens, p.block)
    l1, l2 = DevPack(torch, gdn, p, ck), DevPack(torch, gdn, p, ck)
    n, each = len(ck), p.Hv * p.dv * p.dk * 4
    slots = np.random.default_rng(0).permutation(n + 32)[:n].astype(np.int64)
    slots_d = torch.from_numpy(slots).to("cuda:0")
    dev_pool = torch.empty((n + 32, p.Hv, p.dv, p.dk), dtype=torch.float32, device="cuda:0")
    host_pool = torch.empty((n + 32, p.Hv, p.dv, p.dk), dtype=torch.float32, pin_memory=True)
    host_addr = _pinned_device_address(host_pool)
    for name, dst in (("device_pool", dev_pool), ("host_pool", host_addr)):
        copy_a = lambda: gdn.gdn_snapshot_copy(l1.ckbuf, n, each, dst, slots_d, slots, n + 32,
                                               copy_stream=sA)
        copy_b = lambda: gdn.gdn_snapshot_copy(l1.ckbuf, n, each, dst, slots_d, slots, n + 32,
                                               copy_stream=sB)
        scan1, scan2 = (lambda: l1.run(stream=sA)), (lambda: l2.run(stream=sA))
        t_copy = med(copy_a, sA)
        t_serial = med(lambda: (scan1(), copy_a(), scan2()), sA)

        def overlapped():   # as an engine would: the copy enqueued before the next scan
            scan1()
            joined(scan2, copy_b, b_first=True)()
        t_two = med(overlapped, sA)
        out[f"copy_beside_next_scan_{name}"] = {"copy_ms": t_copy, "one_stream_ms": t_serial,
                                                "copy_stream_ms": t_two, "overlap_saved_ms": t_serial - t_two}
    del l1, l2
    return out


# ------------------------------------------------------------ CPU oracle --

def _oracle_one_prompt(args):
    from threadpoolctl import threadpool_limits
    with threadpool_limits(1):
        import oracle as O
        q, k, v, g, b, x, w = args
        t = time.perf_counter()
        if x is not None:   # the whole path: conv1d+SiLU first, q, k, v are its column blocks
            y = O.conv1d_silu_packed(x, w, [0, x.shape[0]])[0]
            L, nq, nv = x.shape[0], q.shape[1] * q.shape[2], v.shape[1] * v.shape[2]
            q = y[:, :nq].reshape(q.shape)
            k = y[:, nq:2 * nq].reshape(k.shape)
            v = y[:, 2 * nq:2 * nq + nv].reshape(v.shape)
        O.prefill_recurrent(q, k, v, g, b, [0, q.shape[0]])
        return time.perf_counter() - t


def cpu_baseline(p, n_prompts: int):
    """The fp64 oracle, untouched, on the first n_prompts prompts of the pack,
    one process per prompt (one BLAS thread each)."""
    import oracle as O
    cores = len(os.sched_getaffinity(0))
    procs = min(cores, n_prompts)
    jobs = []
    for s in range(n_prompts):
        sl = slice(int(p.cu_seqlens[s]), int(p.cu_seqlens[s + 1]))
        x = None if p.x is None else O.to_f64(p.x[sl], p.dtype)
        w = None if p.conv_w is None else p.conv_w.astype(np.float64)
        jobs.append((O.to_f64(p.q[sl], p.dtype), O.to_f64(p.k[sl], p.dtype), O.to_f64(p.v[sl], p.dtype),
                     p.g[sl].astype(np.float64), p.beta[sl].astype(np.float64), x, w))
    ctx = mp.get_context("spawn")
    t0 = time.perf_counter()
    with ctx.Pool(procs) as pool:
        per = pool.map(_oracle_one_prompt, jobs)
        pool.close()   # workers leave by themselves (the context's exit would signal them)
        pool.join()
    wall = time.perf_counter() - t0
    toks = sum(j[0].shape[0] for j in jobs)
    cpu_model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu_model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": toks / wall, "unit": "tokens/s/layer", "cores": procs, "kind": "oracle",
            "sample": f"{n_prompts} of the 32 prompts ({toks} tokens, all 32 heads), fp64 "
                      + ("conv1d+SiLU then " if p.x is not None else "")
                      + f"token-by-token recurrence, one process per prompt; wall {wall:.1f} s; {cpu_model}",
            "cpu_seconds": float(sum(per))}


# ------------------------------------------------------------------ main --

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-legs", action="store_true", help="time only the headline step")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-prompts", type=int, default=32)
    ap.add_argument("--workload", default="chat", choices=["chat", "long", "ragged"])
    ap.add_argument("--step", default="fused", choices=["fused", "two-launch"],
                    help="chat wave: the conv fused into the scan's loads (one launch; the faster here) "
                         "or the conv kernel then the scan; the other one is timed as a leg")
    ap.add_argument("--summarize-profiles", metavar="DIR",
                    help="summarize a rocprofv3 run set of this script (no GPU) and exit")
    ap.add_argument("--overlap-only", action="store_true",
                    help="run only the stream-overlap leg (for a rocprofv3 timeline)")
    args = ap.parse_args()
    if args.summarize_profiles:
        d = args.summarize_profiles
        res = summarize_profiles(d) if os.path.isdir(os.path.join(d, "FETCH_SIZE")) else {}
        if any(n.startswith("sq_") for n in os.listdir(d)):
            res["sq"] = summarize_sq(d)
        if os.path.isdir(os.path.join(d, "overlap")):
            res["overlap"] = summarize_overlap(os.path.join(d, "overlap"))
        print(json.dumps(res, indent=1))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: one GPU only (the path would shard by value-head groups with no exchange "
              "between GPUs; multi-GPU runs are not implemented). Use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import gated_deltanet_prefill_varlen_amd as gdn
    import workloads as W

    gdn.load()
    dev = "cuda:0"
    torch.cuda.set_device(0)
    stream = torch.cuda.Stream()
    flush = make_flush(torch, dev)

    makers = {"chat": (W.chat_wave, "chat wave 32 x 1,024 tokens"),
              "long": (W.long_prompts, "long prompts 4 x 8,192 tokens"),
              "ragged": (W.ragged_pack, "ragged 8 prompts <= 8,192 tokens, prefix-cache init")}
    if args.overlap_only:
        print(json.dumps({"overlap": bench_overlap(torch, gdn, stream, flush, 10)}), flush=True)
        return
    fn, label = makers[args.workload]
    log(f"[bench] generating {label}")
    p = fn(seed=0, with_conv=True) if args.workload == "chat" else fn(seed=0)
    torch.cuda.synchronize()
    t_wall0 = time.perf_counter()
    fused = args.workload == "chat" and args.step == "fused"
    step_labels = {True: ": conv1d+SiLU fused into the scan's loads (one launch, checkpoints), checkpoint "
                         "copy on its own stream",
                   False: ": conv1d+SiLU, scan with checkpoints, checkpoint copy on its own stream"}
    if args.workload == "chat":
        log(f"[bench] timing headline step ({'conv fused into the scan' if fused else 'conv, scan'}, "
            "checkpoint copy)")
        label += step_labels[fused]
        step = bench_layer_step(torch, gdn, p, args.steps, args.warmup, stream, label, fused=fused)
        # the dominant launch: the fused scan moves the step's fewest bytes (x
        # in place of q, k, v, plus the conv weights, states and windows)
        head = {"workload": label, "ms_median": step["ms_per_step"], "tokens_per_s": step["tokens_per_s"],
                "ms_p10": step["step_spacing_ms_p10"], "ms_p90": step["step_spacing_ms_p90"],
                "checkpoints": step["checkpoints"],
                "alg_bytes": step["step_min_bytes"] if fused else step["scan_alg_bytes"],
                "alg_flops": step["scan_alg_flops"],
                "scan_ms_mean": step["scan_ms_mean"], "step": step}
    else:
        log("[bench] timing headline step (scan)")
        head, _ = bench_prefill(torch, gdn, p, args.steps, args.warmup, stream, flush, label)
        head["scan_ms_mean"] = head["ms_mean"]
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall0
    scan_ach = head["alg_bytes"] / (head["scan_ms_mean"] * 1e-3) / 1e9
    log(f"[bench] headline: {head['ms_median']:.3f} ms per step, {head['tokens_per_s']/1e6:.2f} M tok/s; "
        f"scan {head['scan_ms_mean']:.3f} ms, {scan_ach / HBM_PEAK_GBS * 100:.1f}% of the HBM roofline")

    legs = {}
    if not args.no_legs:
        for name, f in (("conv", bench_conv), ("snapshot_copy", bench_snapshot),
                        ("prefix_cache_host", bench_prefix_cache), ("decode", bench_decode),
                        ("decode_conv", bench_decode_conv),
                        ("decode_tokens", bench_decode_tokens),
                        ("mixed", bench_mixed), ("overlap", bench_overlap)):
            log(f"[bench] leg {name}")
            legs[name] = f(torch, gdn, stream, flush, 10)
        if args.workload == "chat":
            other = "step_two_launches" if fused else "step_conv_fused"
            log(f"[bench] leg {other}")
            o = bench_layer_step(torch, gdn, p, args.steps, args.warmup, stream,
                                 makers["chat"][1] + step_labels[not fused], fused=not fused)
            o["vs_headline_step"] = o["ms_per_step"] / head["ms_median"]
            # the unfused scan's own roofline inside its step
            sb = o["scan_alg_bytes"] if fused else step["scan_alg_bytes"]
            sm = o["scan_ms_mean"] if fused else step["scan_ms_mean"]
            o["scan_roofline"] = {"kernel": "pipelined_prefill_kernel<128,128,false>", "alg_bytes_per_launch": sb,
                                  "launch_ms_mean": sm, "achieved_GBs": sb / (sm * 1e-3) / 1e9,
                                  "frac": sb / (sm * 1e-3) / 1e9 / HBM_PEAK_GBS,
                                  "traffic": measured_traffic("chat")}
            legs[other] = o
            log("[bench] leg conv_fused_packs")
            legs["conv_fused_packs"] = bench_conv_fused_packs(torch, gdn, stream, flush, 10, W)
            log("[bench] leg scan_only")
            legs["scan_only"], _ = bench_prefill(torch, gdn, p, args.steps, args.warmup, stream, flush,
                                                 makers["chat"][1] + ", scan alone (dense q, k, v)")
        for wname in ("long", "ragged"):
            if wname == args.workload:
                continue
            log(f"[bench] leg {wname}")
            wp = makers[wname][0](seed=0)
            legs[wname], _ = bench_prefill(torch, gdn, wp, 5, 1, stream, flush, makers[wname][1])
            del wp

    cpu = None
    if not args.no_cpu:
        log("[bench] CPU oracle baseline")
        cpu = cpu_baseline(p, args.cpu_prompts)

    mean_s = head["scan_ms_mean"] * 1e-3
    achieved = head["alg_bytes"] / mean_s / 1e9
    line = {
        "metric": "packed GDN prefill tokens/s/layer (32x1K pack) + % of MFMA/HBM roofline",
        "value": head["tokens_per_s"],
        "unit": "tokens/s/layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_median"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 in/out, fp16 MFMA operands, fp32 accumulation and state",
        "data": "synthetic (seeded; shapes of the pages' chat waves)",
        "config": {"workload": head["workload"], "tokens": p.n_tokens, "prompts": p.n_seqs,
                   "qk_heads": p.Hqk, "v_heads": p.Hv, "head_dim": p.dk, "chunk": p.chunk,
                   "kernel_chunk": kernel_chunk(p),
                   "checkpoint_block": p.block, "checkpoints": head["checkpoints"],
                   "timing": ("K steps queued back to back between two device synchronisations, "
                              "each step's checkpoint copy on its own stream right after its scan, "
                              "beside the next step's " + ("fused scan" if fused else "conv") +
                              ", the last copy joined; ms_per_step = HIP-event time of the "
                              "region / K" if args.workload == "chat" else
                              "median of per-launch HIP-event times on the launch stream; 1 GiB "
                              "cache flush before each launch, outside the events"),
                   "wall_s_timed_region": (head["step"]["region_wall_ms"] * 1e-3 if head.get("step")
                                           else head["wall_ms_timed"] * 1e-3),
                   "wall_s_all_legs_of_headline": t_wall},
        "step": head.get("step"),
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": measured_traffic(("conv_fused_" if fused else "") + args.workload),
                     "kernel": ("pipelined_prefill_kernel<128,128,true> (the conv in its loads)" if fused
                                else "pipelined_prefill_kernel<128,128,false>"),
                     "alg_bytes_per_launch": head["alg_bytes"],
                     "launch_ms_mean": head["scan_ms_mean"],
                     "mfma_alg_tflops": head["alg_flops"] / mean_s / 1e12},
        "step_roofline": ({"bound": "hbm", "alg_bytes_min": head["step"]["step_min_bytes"],
                           "achieved": head["step"]["step_min_bytes"] / (head["ms_median"] * 1e-3) / 1e9,
                           "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": head["step"]["step_min_bytes"] / (head["ms_median"] * 1e-3) / 1e9
                           / HBM_PEAK_GBS,
                           "note": "whole step (conv, scan, checkpoint copy) against the fewest bytes "
                                   "one pass can move: x, g, beta in, out, final states and "
                                   "checkpoints once, conv weights, states and windows"}
                          if head.get("step") else None),
        "cpu_baseline": cpu,
        "legs": legs,
        "step_ms_p10_p90": [head["ms_p10"], head["ms_p90"]],
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
