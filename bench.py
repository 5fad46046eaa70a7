#!/usr/bin/env python3
"""Throughput of the KDA state-update hot path on one MI355X.

One step is one pass of the whole path over the large decode batch (L=1, H=64
heads, B=512 requests, q=8 tokens, FP32 state of 512 slots x 64 heads x 64 KiB
= 2 GiB, about 5% no-op rows):

  1. the sampler's accepted counts land in the commit-length buffer (a 2 KiB
     device copy),
  2. kda_fused_replay_verify: replay each request's pending tokens from its
     records into its page, verify the 8-token window, rewrite the records,
  3. kda_defer_commit: the accepted counts become the pending counts,
  4. kda_flush_plan + kda_commit (FP32, in place, record rows): fold the pending
     replays into the checkpoints (the flush path).

All inputs are synthetic (seeded generators in ``workloads``) and resident in
HBM before timing; the records the first step replays come from a verify of a
prior window. W untimed warm-up steps, then K timed steps between device
synchronisations. Kernel durations come from HIP events recorded on the stream
the kernels are launched on: around the fused launch on the even timed steps
and around the commit on the odd ones (both on every step when K = 1). Each
pair of events costs the step the overlap of one kernel's drain with the next
one's start, about 4 us, so the step carries one pair, not one per kernel.

Printed: one JSON line. ``value`` is the step's state bandwidth: algorithmic
state bytes (pages read + pages written, from the actual plan) per second.
``roofline`` is the fused kernel's algorithmic bytes per launch over its mean
event-timed duration, against 8 TB/s. ``cpu_baseline`` times the FP64 oracle on
a sample of the same step on the host cores.

Variants of the step: --state-dtype bf16, --gated-output, --conv (with
--conv-layout), --gate-proj. --workload commit|fused|align|verify|decay times
one kernel alone on its own workload instead; before each of those launches,
outside its events, a 1 GiB scratch read evicts the 256 MB MALL (--no-evict to
skip), and ``value`` is the kernel's state rate (its total rate when it moves
no state).
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, AMD's published figure
K = V = 128


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--workload",
                    choices=("large_decode", "commit", "fused", "align", "verify", "decay"),
                    default="large_decode",
                    help="large_decode (default): the whole step on the large decode batch; "
                         "commit / fused / align: that kernel alone on the BF16 commit, "
                         "fused replay+verify and 8-layer align commit workloads; verify: "
                         "the stock verify alone on the large decode batch (pool type from "
                         "--state-dtype); decay: kda_decay on the large decode batch's raw "
                         "gates")
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the oracle timing (profiling runs)")
    ap.add_argument("--cpu-requests", type=int, default=512,
                    help="requests of the batch the CPU baseline runs (all 64 heads each)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="the CPU baseline repeats its step until this much wall time passed")
    ap.add_argument("--gated-output", action="store_true",
                    help="run the fused step with the gated RMSNorm output stage on")
    ap.add_argument("--state-dtype", choices=("f32", "bf16"), default="f32",
                    help="element type of the state pool (the workload's is f32; bf16 "
                         "rounds the same pool to BF16 and commits in BF16)")
    ap.add_argument("--conv", action="store_true",
                    help="run the fused step with its convolution prologue (q, k, v from "
                         "packed pre-activations and a window pool)")
    ap.add_argument("--conv-layout", choices=("dim_first", "window_major"), default="window_major",
                    help="window pool layout with --conv: [slot][3HK][RQ+2] (each channel's "
                         "window contiguous) or [slot][RQ+2][3HK] (each window entry a "
                         "contiguous row of channels)")
    ap.add_argument("--gate-proj", action="store_true",
                    help="compute raw_g in the step with kda_gate_projection (F_A a column "
                         "slice of packed projection rows, F_B [H*128, 128])")
    ap.add_argument("--no-evict", action="store_true",
                    help="with --workload commit|fused|align|verify: do not read the 1 GiB "
                         "scratch buffer before each launch (which evicts the 256 MB MALL "
                         "outside the timed events)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also time a plain 2 GiB device copy (streaming ceiling)")
    ap.add_argument("--trace-summary", metavar="CSV",
                    help="no GPU run: summarise a rocprofv3 kernel-trace or counter-collection "
                         "CSV of a run of this script (per kernel: launches, then the mean "
                         "duration and counters of the last --steps launches, i.e. the timed "
                         "steps without the warm-up ones)")
    return ap.parse_args()


def trace_summary(path, last):
    """Per-kernel figures from a rocprofv3 CSV of a run of this script: a
    --kernel-trace CSV gives durations, a --pmc counter-collection CSV gives
    counter values per dispatch. Reported: all launches, and the mean (min,
    max for durations) over the last `last` launches of each kernel (the run's
    timed steps, without its warm-up launches)."""
    import csv
    disp = {}  # kernel -> {dispatch id: {"t": (t0, t1), counter: value}}
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            name = row.get("Kernel_Name") or row.get("KernelName") or row.get("Name")
            did = row.get("Dispatch_Id") or row.get("Correlation_Id")
            rec = disp.setdefault(name, {}).setdefault(did, {})
            rec["t"] = (int(row.get("Start_Timestamp")), int(row.get("End_Timestamp")))
            if row.get("Counter_Name"):
                c = row["Counter_Name"]
                rec[c] = rec.get(c, 0.0) + float(row["Counter_Value"])
    out = {}
    for name, recs in disp.items():
        order = sorted(recs.values(), key=lambda r: r["t"][0])
        tail = order[-last:]
        d = [(r["t"][1] - r["t"][0]) / 1e3 for r in order]
        dt = d[-last:]
        o = {"launches": len(d), "all_mean_us": round(sum(d) / len(d), 2),
             "timed_launches": len(dt), "timed_mean_us": round(sum(dt) / len(dt), 2),
             "timed_min_us": round(min(dt), 2), "timed_max_us": round(max(dt), 2)}
        counters = sorted({k for r in tail for k in r if k != "t"})
        if counters:
            o["counters_timed_mean"] = {c: round(sum(r.get(c, 0.0) for r in tail) / len(tail), 1)
                                        for c in counters}
        out[name] = o
    return out


def strip_comments(text):
    """C++ source without its comments, blank lines and indentation (string and
    character literals kept), so that the digest below follows the code and
    not its prose."""
    out, i, n = [], 0, len(text)
    while i < n:
        ch = text[i]
        if text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            if j < 0:
                raise ValueError("unterminated block comment")
            out.append(" ")
            i = j + 2
        elif ch in "\"'":
            j = i + 1
            while j < n and text[j] != ch:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        else:
            out.append(ch)
            i += 1
    lines = (line.strip() for line in "".join(out).splitlines())
    return "\n".join(line for line in lines if line)


def source_digest(paths):
    """Digest of the code (comments excluded) of the given source files: the
    key under which profiles/traffic.json holds a kernel's measured traffic."""
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), encoding="utf-8") as f:
            h.update(strip_comments(f.read()).encode())
    return h.hexdigest()[:16]


FUSED_SOURCES = ["spec_decode_amd/csrc/fused.hip", "spec_decode_amd/csrc/verify_kernel.h",
                 "spec_decode_amd/csrc/kda_device.h"]
COMMIT_SOURCES = ["spec_decode_amd/csrc/commit.hip", "spec_decode_amd/csrc/kda_device.h"]
CONV_SOURCES = FUSED_SOURCES + ["spec_decode_amd/csrc/fused_conv.hip",
                                "spec_decode_amd/csrc/fused_conv_packed.hip",
                                "spec_decode_amd/csrc/fused_conv_window_major.hip"]


def fused_variant(args):
    """Key in profiles/traffic.json and source files of the fused launch that a
    large-decode run times: the default, or its variant."""
    parts = []
    if args.state_dtype == "bf16":
        parts.append("bf16")
    if args.gated_output:
        parts.append("gated")
    if args.conv:
        parts.append("conv_" + args.conv_layout)
    if args.gate_proj:
        parts.append("gate_proj")
    key = "/".join(["fused_replay_verify/large_decode"] + parts)
    return key, (CONV_SOURCES if args.conv else FUSED_SOURCES)


def measured_traffic(name, digest):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when the kernel changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f).get(name)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_digest") != digest:
        return None
    return rec.get("hbm_bytes_per_launch")


# ----------------------------------------------------------------- accounting

def spread(ms):
    """Median and 90th percentile (nearest rank) of per-launch times in ms."""
    xs = sorted(ms)
    return {"median_ms": round(xs[(len(xs) - 1) // 2], 4),
            "p90_ms": round(xs[min(len(xs) - 1, -(-9 * len(xs) // 10) - 1)], 4)}


def fused_bytes(slots, rows, pending, T, RQ, H, null_slot=0, gated=False, es=4, conv=False):
    """Algorithmic bytes of one fused launch: (state bytes, total bytes). The
    gated output stage reads q*256 B of gates per live item; es is the state
    element size. With the convolution prologue, q, k, v are read as the same
    bytes of pre-activations, plus each live item's windows (3*128 channels,
    the 3 taps read, q + 2 values written, BF16) and the weights once."""
    page = V * K * es
    state = total = 0
    for b in range(len(slots)):
        if slots[b] <= null_slot:
            total += H * T * V * 2  # zero outputs
            continue
        r = int(rows[b])
        n = min(max(int(pending[r]), 0), RQ) if r >= 0 else 0
        s = page + (page if n > 0 else 0)
        t = s + n * (V * 4 + 2 * K * 2)            # old records read
        t += (T * (V * 4 + 2 * K * 2)) if r >= 0 else 0  # new records written
        t += T * (3 * K * 2 + V * 2) + T * 2        # q, k, raw_g, v, raw_beta
        t += T * V * 2                              # o
        t += T * V * 2 if gated else 0              # gate
        t += (3 * K * 3 * 2 + 3 * K * (T + 2) * 2) if conv else 0  # windows
        state += H * s
        total += H * t
    if conv:
        total += 3 * 4 * H * K * 2 + 3 * H * K * 2  # convolution weights and bias
    return state, total


def commit_bytes(slots, lens, rows, H, Q, null_slot=0, es=4):
    """Algorithmic bytes of one in-place commit launch: (state, total)."""
    page = V * K * es
    state = total = 0
    for b in range(len(slots)):
        n = int(lens[b])
        r = int(rows[b])
        if not (n > 0 and slots[b] > null_slot and r >= 0):
            continue
        n = min(n, Q)
        state += H * 2 * page
        total += H * (2 * page + n * (V * 4 + 2 * K * 2))
    return state, total


def simulate_plan(slots, rows, pending0, accepted, steps, q, null_slot=0):
    """Per step: (pending the fused step replays, flush commit lengths)."""
    pending = pending0.copy()
    out = []
    for _ in range(steps):
        fused_pending = pending.copy()
        for b in range(len(slots)):  # defer
            r = int(rows[b])
            if r >= 0 and slots[b] > null_slot:
                pending[r] = accepted[b]
        lens = [0] * len(slots)
        for b in range(len(slots)):  # flush plan
            r = int(rows[b])
            n = int(pending[r]) if r >= 0 else 0
            n = min(max(n, 0), q)
            lens[b] = n if (slots[b] > null_slot and n > 0) else 0
        out.append((fused_pending, lens))
    return out


# ----------------------------------------------------------------- CPU baseline

def cpu_baseline(host, H, T, RQ, n_req, lb, bf16=False, min_seconds=10.0):
    """The FP64 oracle on the first n_req live requests (all heads) of the same
    step: fused replay+verify, then the in-place commit of the accepted tokens.
    Reports state GB/s of that sample (the same accounting as the GPU line)."""
    import numpy as np
    import oracle

    slots, rows = host["slots"], host["rows"]
    pick = [b for b in range(len(slots)) if slots[b] > 0 and rows[b] >= 0][:n_req]
    B = len(pick)
    page = H * V * K
    # A compact copy: request j owns slot j + 1 and record row j.
    state = np.zeros((B + 1) * page, np.uint16 if bf16 else np.float32)
    for j, b in enumerate(pick):
        state[(j + 1) * page:(j + 2) * page] = host["state_pages"][b]
    sl = np.arange(1, B + 1, dtype=np.int32)
    rr = np.arange(B, dtype=np.int32)
    corr = np.ascontiguousarray(host["corr"][rows[pick]])
    kg = np.ascontiguousarray(host["kg"][rows[pick]])
    pend = np.ascontiguousarray(host["pending"][rows[pick]]).astype(np.int32)
    acc = np.ascontiguousarray(host["accepted"][pick]).astype(np.int32)
    tok = np.concatenate([np.arange(b * T, (b + 1) * T) for b in pick])
    win = {k: np.ascontiguousarray(v[tok]) for k, v in host["win"].items()}
    out = np.zeros((B * T, H * V), np.uint16)
    threads = oracle.default_threads()
    oracle._load()

    def one_step():
        oracle.fused_replay_verify(heads=H, tokens=T, batch=B, q=win["q"], k=win["k"],
                                   v=win["v"], raw_g=win["raw_g"], raw_beta=win["raw_beta"],
                                   a_log=host["a_log"], dt_bias=host["dt_bias"], lower_bound=lb,
                                   state=state, state_slot_stride=page, state_indices=sl,
                                   corr=corr, kg=kg, record_tokens=RQ, record_rows=rr,
                                   pending=pend, out=out, threads=threads)
        lens = acc.copy()
        pending2 = pend.copy()
        oracle.defer(sl, lens, rr, pending2)
        fl, fin, _, _ = oracle.flush_plan(sl, rr, pending2, T)
        oracle.commit(heads=H, window=RQ, batch=B, state_bf16=bf16, state_layers=[state],
                      state_slot_strides=[page], corr_layers=[corr],
                      corr_row_strides=[H * RQ * V], kg_layers=[kg],
                      kg_row_strides=[H * RQ * 2 * K], a_log=host["a_log"][None, :],
                      dt_bias=host["dt_bias"][None, :], sources=fin, commit_lens=fl,
                      destinations=fin, record_rows=rr, lower_bound=lb, threads=threads)
        return fl

    # Repeat the same step (the records stay, the pages evolve) until about
    # min_seconds of host time have passed, so that the figure is not noise.
    t0 = time.perf_counter()
    reps = 0
    while True:
        fl = one_step()
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds or reps >= 64:
            break
    es = 2 if bf16 else 4
    fs, _ = fused_bytes(sl, rr, pend, T, RQ, H, es=es)
    cs, _ = commit_bytes(sl, fl, rr, H, RQ, es=es)
    return {
        "value": round(reps * (fs + cs) / dt / 1e9, 3),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"fused replay+verify then defer/flush/in-place commit of {B} of the "
                   f"{len(slots)} requests (all {H} heads, {B * H} items), FP64, repeated "
                   f"{reps} times: {dt:.2f} s wall"),
        "items_per_s": round(reps * B * H / dt, 1),
    }


def sampled_cpu_baseline(run, n_items, state_bytes, seconds=2.0):
    """The oracle on bounded random samples of a single-kernel workload's
    (layer, request, head) items, on every core the process may use and on one
    thread. run(items, threads) runs it on the given flattened item ids (host
    inputs snapshotted before any GPU launch); state_bytes(items) gives their
    algorithmic state bytes. Each sample doubles until it takes about
    `seconds` of wall time; a sample that covers the whole workload sooner is
    run again until that much time has passed."""
    import numpy as np
    import oracle

    oracle._load()
    rng = np.random.default_rng(0)
    res = {}
    for label, threads in (("all", oracle.default_threads()), ("one", 1)):
        size = min(n_items, 64)
        while True:
            items = np.sort(rng.choice(n_items, size, replace=False)).astype(np.int64)
            reps = 0
            t0 = time.perf_counter()
            while True:
                run(items, threads)
                reps += 1
                dt = time.perf_counter() - t0
                if dt >= seconds or size < n_items:
                    break
            if dt >= seconds or size == n_items:
                break
            size = min(n_items, max(2 * size, int(size * seconds / max(dt, 1e-3))))
        res[label] = (threads, size, reps, dt, state_bytes(items))

    def rates(r):
        threads, size, reps, dt, sb = r
        return reps * sb / dt / 1e9, reps * size / dt

    (gbs, ips), (gbs1, ips1) = rates(res["all"]), rates(res["one"])
    threads, size, reps, dt, _ = res["all"]
    _, size1, reps1, dt1, _ = res["one"]
    return {
        "value": round(gbs, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
        "sample": (f"{size} of the workload's {n_items} items, drawn at random, FP64, "
                   f"{reps} pass(es): {dt:.2f} s wall on {threads} threads; {size1} items, "
                   f"{reps1} pass(es): {dt1:.2f} s on one thread"),
        "items_per_s": round(ips, 1),
        "single_thread": {"value": round(gbs1, 3), "unit": "GB/s", "items_per_s": round(ips1, 1)},
    }


def host_bits(t):
    """Host copy of a device or host tensor: BF16 as uint16 bits, others as is."""
    import torch
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view("uint16").copy()
    return t.numpy().copy()


def _commit_cpu_runner(H, B, Q, states, slot_strides, corrs, kgs, a_log, dt_bias, src, lens,
                       dst, bnd, blen, lb):
    """Host snapshots of a commit workload's BF16 pools and records and the
    oracle over a subset of its items: (run, state_bytes) for
    sampled_cpu_baseline."""
    import oracle

    L = len(states)
    h_st = [host_bits(t) for t in states]
    h_co = [host_bits(t) for t in corrs]
    h_kg = [host_bits(t) for t in kgs]
    h_al, h_db = host_bits(a_log), host_bits(dt_bias)
    page_bytes = V * K * 2

    def run(sel, threads):
        oracle.commit(heads=H, window=Q, batch=B, state_bf16=True, state_layers=h_st,
                      state_slot_strides=slot_strides, corr_layers=h_co,
                      corr_row_strides=[H * Q * V] * L, kg_layers=h_kg,
                      kg_row_strides=[H * Q * 2 * K] * L, a_log=h_al, dt_bias=h_db,
                      sources=src, commit_lens=lens, destinations=dst, boundaries=bnd,
                      boundary_lens=blen, lower_bound=lb, items=sel, threads=threads)

    def state_bytes(sel):
        tot = 0
        for it in sel:
            b = (int(it) // H) % B  # item id (l * B + b) * H + h
            if min(int(lens[b]), Q) > 0 and src[b] > 0 and dst[b] > 0:
                tot += 2 * page_bytes + (page_bytes if bnd is not None and bnd[b] > 0
                                         and blen[b] > 0 else 0)
        return tot

    return run, state_bytes


def _verify_cpu_runner(fused, H, B, T, RQ, state, slots, rows, pend_row, corr, kg, a_log,
                       dt_bias, lb, win):
    """Host snapshots of a stock-verify or fused workload's inputs and the oracle
    over a subset of its items: (run, state_bytes) for sampled_cpu_baseline."""
    import numpy as np
    import oracle

    h = {n: host_bits(getattr(win, n)) for n in ("q", "k", "v", "raw_g", "raw_beta")}
    h.update(state=host_bits(state), corr=host_bits(corr), kg=host_bits(kg),
             a_log=host_bits(a_log), dt_bias=host_bits(dt_bias),
             slots=host_bits(slots).astype(np.int32), rows=host_bits(rows).astype(np.int32))
    pend = None if pend_row is None else host_bits(pend_row).astype(np.int32)
    out = np.zeros((B * T, H * V), np.uint16)
    page = H * V * K
    page_bytes = V * K * h["state"].itemsize

    def run(sel, threads):
        args = dict(heads=H, tokens=T, batch=B, q=h["q"], k=h["k"], v=h["v"], raw_g=h["raw_g"],
                    raw_beta=h["raw_beta"], a_log=h["a_log"], dt_bias=h["dt_bias"],
                    lower_bound=lb, state=h["state"], state_slot_stride=page,
                    state_indices=h["slots"], corr=h["corr"], kg=h["kg"], record_tokens=RQ,
                    record_rows=h["rows"], out=out, items=sel, threads=threads)
        if fused:
            oracle.fused_replay_verify(pending=pend, **args)
        else:
            oracle.verify(**args)

    def state_bytes(sel):
        tot = 0
        for it in sel:
            b = int(it) // H
            if h["slots"][b] <= 0:
                continue
            tot += page_bytes  # the page read
            r = h["rows"][b]
            if fused and r >= 0 and min(int(pend[r]), RQ) > 0:
                tot += page_bytes  # S_n written back
        return tot

    return run, state_bytes


# ----------------------------------------------------------------- single-kernel workloads

def bench_kernel_workload(args):
    """Times one kernel on its own workload (W warm-up launches, K timed) and
    prints the same JSON contract: value = algorithmic state bytes per second."""
    import numpy as np
    import torch

    sys.path.insert(0, ROOT)
    import spec_decode_amd as kda
    import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    i32 = lambda t: t.to(dev)
    cpu_run = cpu_bytes = None  # the oracle on a sample of the workload (not for decay)
    if args.workload in ("commit", "align"):
        w = W.config1(device=dev) if args.workload == "commit" else W.config3(device=dev)
        a = w.arrays
        L, H, B, Q = w.layers, w.heads, w.batch, w.tokens
        states = [a["state"]] if L == 1 else [a[f"state{l}"] for l in range(L)]
        corrs = [a["corr"].to(dev)] if L == 1 else [a[f"corr{l}"].to(dev) for l in range(L)]
        kgs = [a["kg"].to(dev)] if L == 1 else [a[f"kg{l}"].to(dev) for l in range(L)]
        bnd = a.get("boundaries")
        blen = a.get("boundary_lens")
        call = dict(heads=H, window=Q, batch=B, state_dtype=kda.KDA_STATE_BF16,
                    state_addrs=[t.data_ptr() for t in states], state_slot_strides=w.slot_strides,
                    corr_addrs=[t.data_ptr() for t in corrs], corr_row_strides=[H * Q * V] * L,
                    kg_addrs=[t.data_ptr() for t in kgs], kg_row_strides=[H * Q * 2 * K] * L,
                    a_log=a["a_log"].to(dev), dt_bias=a["dt_bias"].to(dev),
                    sources=i32(a["sources"]), commit_lens=i32(a["commit_lens"]),
                    destinations=i32(a["destinations"]),
                    boundaries=None if bnd is None else i32(bnd),
                    boundary_lens=None if blen is None else i32(blen), lower_bound=w.lower_bound)
        launch = lambda: kda.kda_commit(**call)
        src, dst = a["sources"].numpy(), a["destinations"].numpy()
        lens = a["commit_lens"].numpy()
        bn = None if bnd is None else bnd.numpy()
        bl = None if blen is None else blen.numpy()
        page = V * K * 2
        st = tot = 0
        for b in range(B):
            n = min(int(lens[b]), Q)
            if not (n > 0 and src[b] > 0 and dst[b] > 0):
                continue
            s_b = 2 * page + (page if bn is not None and bn[b] > 0 and bl[b] > 0 else 0)
            st += L * H * s_b
            tot += L * H * (s_b + n * (V * 4 + 2 * K * 2))
        items = L * B * H
        if not args.no_cpu_baseline:
            cpu_run, cpu_bytes = _commit_cpu_runner(
                H, B, Q, states, list(w.slot_strides), corrs, kgs, a["a_log"], a["dt_bias"],
                src, lens, dst, bn, bl, w.lower_bound)
        name = "kda_commit (BF16)" if L == 1 else "kda_commit (BF16, align, 8 layers)"
        workload = ("commit: L=1 H=32 B=64 window 4, BF16 pool of 256 slots, src -> dst"
                    if L == 1 else
                    "align_commit: L=8 H=32 B=256 window 8, BF16 pools of 641 slots, "
                    "128 boundary stores")
        dtype = "f32"
    elif args.workload == "decay":
        w = W.config4(device=dev)
        a = w.arrays
        H, B, T = w.heads, w.batch, w.tokens
        raw_g = w.windows["new"].raw_g.to(dev)  # [B*T, H, 128] BF16
        a_log, dt_bias = a["a_log"][0].contiguous().to(dev), a["dt_bias"][0].contiguous().to(dev)
        del a["state"]
        torch.cuda.empty_cache()
        out = torch.empty(raw_g.shape, dtype=torch.float32, device=dev)
        launch = lambda: kda.kda_decay(raw_g, a_log, dt_bias, w.lower_bound, out)
        n = raw_g.numel()
        st = 0  # no state bytes: value is the total rate
        tot = n * 2 + n * 4 + H * 4 + H * K * 4  # BF16 in, FP32 out, parameters
        items = B * H
        name = "kda_decay"
        workload = ("decay: the large decode batch's new raw gates, 4096 tokens x 64 heads x 128 "
                    "channels, BF16 -> FP32")
        dtype = "f32"
    elif args.workload == "verify":
        w = W.config4(device=dev)
        a = w.arrays
        H, B, T, RQ = w.heads, w.batch, w.tokens, w.record_tokens
        bf16 = args.state_dtype == "bf16"
        state = a.pop("state")
        if bf16:
            state = state.to(torch.bfloat16)
            torch.cuda.empty_cache()
        slots, rows = i32(a["state_indices"]), i32(a["record_rows"])
        corr, kg = a["corr"].to(dev), a["kg"].to(dev)
        a_log, dt_bias = a["a_log"][0].contiguous().to(dev), a["dt_bias"][0].contiguous().to(dev)
        new = w.windows["new"].to(dev)
        out = torch.empty((B * T, H * V), dtype=torch.bfloat16, device=dev)
        if not args.no_cpu_baseline:
            cpu_run, cpu_bytes = _verify_cpu_runner(
                False, H, B, T, RQ, state, a["state_indices"], a["record_rows"], None, corr, kg,
                a_log, dt_bias, w.lower_bound, new)
        launch = lambda: kda.kda_verify(
            heads=H, tokens=T, batch=B, q=new.q, k=new.k, v=new.v, raw_g=new.raw_g,
            raw_beta=new.raw_beta, a_log=a_log, dt_bias=dt_bias, lower_bound=w.lower_bound,
            state=state, state_slot_stride=H * V * K, state_indices=slots, corr=corr, kg=kg,
            record_tokens=RQ, record_rows=rows, out=out)
        # The stock verify moves the fused step's bytes with no replay: pages
        # read, inputs, o and the new records.
        st, tot = fused_bytes(a["state_indices"].numpy(), a["record_rows"].numpy(),
                              np.zeros(B, np.int32), T, RQ, H, es=2 if bf16 else 4)
        items = B * H
        name = f"kda_verify ({'BF16' if bf16 else 'FP32'})"
        workload = ("verify: the large decode batch, L=1 H=64 K=V=128 B=512 q=8, "
                    f"{'BF16' if bf16 else 'FP32'} state 512 slots, ~5% no-op rows; the stock "
                    "verify alone (reads the pages, writes o and the records)")
        dtype = "f32"
    else:  # fused
        w = W.config2(device=dev)
        a = w.arrays
        H, B, T, RQ = w.heads, w.batch, w.tokens, w.record_tokens
        state = a["state"]
        slots, rows = i32(a["state_indices"]), i32(a["record_rows"])
        corr, kg = a["corr"].to(dev), a["kg"].to(dev)
        pend_row = torch.zeros(B, dtype=torch.int32)
        pend_row[a["record_rows"].long()] = a["pending"]
        pending = i32(pend_row)
        a_log, dt_bias = a["a_log"][0].contiguous().to(dev), a["dt_bias"][0].contiguous().to(dev)
        new, prior = w.windows["new"].to(dev), w.windows["prior"].to(dev)
        out = torch.empty((B * T, H * V), dtype=torch.bfloat16, device=dev)
        if not args.no_cpu_baseline:
            # the generator's records (before the prior-window verify rewrites them)
            cpu_run, cpu_bytes = _verify_cpu_runner(
                True, H, B, T, RQ, state, a["state_indices"], a["record_rows"], pend_row, corr,
                kg, a_log, dt_bias, w.lower_bound, new)
        kda.kda_verify(heads=H, tokens=T, batch=B, q=prior.q, k=prior.k, v=prior.v,
                       raw_g=prior.raw_g, raw_beta=prior.raw_beta, a_log=a_log, dt_bias=dt_bias,
                       lower_bound=w.lower_bound, state=state, state_slot_stride=H * V * K,
                       state_indices=slots, corr=corr, kg=kg, record_tokens=RQ,
                       record_rows=rows, out=out)
        launch = lambda: kda.kda_fused_replay_verify(
            heads=H, tokens=T, batch=B, q=new.q, k=new.k, v=new.v, raw_g=new.raw_g,
            raw_beta=new.raw_beta, a_log=a_log, dt_bias=dt_bias, lower_bound=w.lower_bound,
            state=state, state_slot_stride=H * V * K, state_indices=slots, corr=corr, kg=kg,
            record_tokens=RQ, record_rows=rows, pending=pending, out=out)
        st, tot = fused_bytes(a["state_indices"].numpy(), a["record_rows"].numpy(),
                              pend_row.numpy(), T, RQ, H)
        items = B * H
        name = "kda_fused_replay_verify (FP32)"
        workload = "fused: L=1 H=32 B=128 q=4, FP32 pool of 256 slots, pending 0..4"
        dtype = "f32"
    # Before every launch (outside its events) a 1 GiB scratch read evicts the
    # 256 MB MALL, which would otherwise hold much of the smaller workloads. A
    # read leaves clean lines; a write would leave dirty ones whose write-back
    # fell into the timed launch.
    scratch = None
    if not args.no_evict:
        scratch = torch.zeros(1 << 28, dtype=torch.float32, device=dev)
        evict_sum = torch.empty((), dtype=torch.float32, device=dev)

    def evict():
        if scratch is not None:
            torch.sum(scratch, 0, out=evict_sum)

    torch.cuda.synchronize()
    for _ in range(args.warmup):
        evict()
        launch()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        evict()
        ev[2 * i].record()
        launch()
        ev[2 * i + 1].record()
    torch.cuda.synchronize()
    ms = [ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(args.steps)]
    mean_ms = sum(ms) / len(ms)
    achieved = tot / (mean_ms * 1e-3) / 1e9
    # over the timed launches alone; a kernel with no state bytes reports its total rate
    value = (st if st else tot) / (mean_ms * 1e-3) / 1e9
    result = {
        "metric": "state GB/s (% of HBM peak) + (req,head) items/s, KDA commit & fused verify",
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(mean_ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": dtype,
        "data": "synthetic", "config": {"workload": workload, "kernel": name,
                                        "mall_evicted": scratch is not None},
        "library": os.path.relpath(kda.library_path(), ROOT),
        "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "items_per_s": round(items / (mean_ms * 1e-3), 1),
        "kernels": {name: {"mean_ms": round(mean_ms, 4), "min_ms": round(min(ms), 4),
                           **spread(ms),
                           "state_gbs": round(st / (mean_ms * 1e-3) / 1e9, 1),
                           "total_gbs": round(achieved, 1)}},
        "roofline": {"kernel": name, "bound": "hbm", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None, "algorithmic_bytes_per_launch": int(tot)},
    }
    if cpu_run is not None:
        scratch = None
        torch.cuda.empty_cache()
        result["cpu_baseline"] = sampled_cpu_baseline(cpu_run, items, cpu_bytes)
    print(json.dumps(result), flush=True)


# ----------------------------------------------------------------- main

def main():
    args = parse_args()
    if args.trace_summary:
        for name, rec in sorted(trace_summary(args.trace_summary, args.steps).items(),
                                key=lambda kv: -kv[1]["timed_mean_us"]):
            print(json.dumps({"kernel": name, **rec}))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the path "
              "shards by request or head with no collective: run one process per GPU)",
              file=sys.stderr)
        sys.exit(2)
    if args.steps < 1:
        sys.exit("--steps must be >= 1")
    if args.workload != "large_decode":
        bench_kernel_workload(args)
        return
    import numpy as np
    import torch

    sys.path.insert(0, ROOT)
    import spec_decode_amd as kda
    import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = W.config4(device=dev)
    H, B, T, RQ = w.heads, w.batch, w.tokens, w.record_tokens
    page = H * V * K
    lb = w.lower_bound
    a = w.arrays
    bf16 = args.state_dtype == "bf16"
    es = 2 if bf16 else 4
    state = a.pop("state")
    if bf16:
        state = state.to(torch.bfloat16)
        torch.cuda.empty_cache()
    slots = a["state_indices"].to(dev)
    rows = a["record_rows"].to(dev)
    pending = a["pending"].to(dev)
    accepted = a["accepted"].to(dev)
    a_log = a["a_log"][0].contiguous().to(dev)
    dt_bias = a["dt_bias"][0].contiguous().to(dev)
    corr = a["corr"].to(dev)
    kg = a["kg"].to(dev)
    new = w.windows["new"].to(dev)
    prior = w.windows["prior"].to(dev)
    out = torch.empty((B * T, H * V), dtype=torch.bfloat16, device=dev)
    gate = norm_w = None
    norm_eps = 1e-5
    if args.gated_output:
        gate, norm_w, norm_eps = W.draw_output_stage(W._gen(4 + 200), B, T, H)
        gate, norm_w = gate.to(dev), norm_w.to(dev)
    conv = None
    if args.conv:
        cv = W.draw_conv_inputs(W._gen(4 + 300), B, T, H, RQ, w.slots)
        hk3 = 3 * H * K
        window = cv.window  # [slots, 3HK, RQ + 2]
        if args.conv_layout == "window_major":
            window = window.transpose(1, 2).contiguous()
            strides = (hk3 * (RQ + 2), 1, hk3)
        else:
            strides = (hk3 * (RQ + 2), RQ + 2, 1)
        conv = dict(x=cv.x.to(dev), pitch=cv.pitch, weight=cv.weight.to(dev),
                    bias=cv.bias.to(dev), pool=window.to(dev).reshape(-1), strides=strides)
    gp = None
    if args.gate_proj:
        hk = H * K
        pitch = (4 * hk + 128 + H + 7) // 8 * 8
        packed = conv["x"] if conv is not None else W.bf16(
            W.normal(W._gen(4 + 500), (B * T, pitch))).to(dev)
        gp = dict(f_a=packed[:, 4 * hk:], pitch=packed.shape[1],
                  f_b=W.draw_gate_factors(W._gen(4 + 501), 1, H, exact=False)[1].to(dev),
                  raw_g=torch.empty((B * T, H, K), dtype=torch.bfloat16, device=dev))
    raw_g = new.raw_g if gp is None else gp["raw_g"]
    commit_lens = torch.empty(B, dtype=torch.int32, device=dev)
    flush = [torch.empty(B, dtype=torch.int32, device=dev) for _ in range(4)]

    # The records the first step replays: a verify of the prior window.
    kda.kda_verify(heads=H, tokens=T, batch=B, q=prior.q, k=prior.k, v=prior.v,
                   raw_g=prior.raw_g, raw_beta=prior.raw_beta, a_log=a_log, dt_bias=dt_bias,
                   lower_bound=lb, state=state, state_slot_stride=page, state_indices=slots,
                   corr=corr, kg=kg, record_tokens=RQ, record_rows=rows, out=out)
    torch.cuda.synchronize()

    host = None
    if not args.no_cpu_baseline:
        sl_h = slots.cpu().numpy()
        host = dict(slots=sl_h, rows=rows.cpu().numpy(), pending=pending.cpu().numpy(),
                    accepted=accepted.cpu().numpy(), a_log=a_log.cpu().numpy(),
                    dt_bias=dt_bias.cpu().numpy(), corr=corr.cpu().numpy(),
                    kg=kg.cpu().view(torch.int16).numpy().view(np.uint16),
                    win={n: getattr(new, n).cpu().view(torch.int16).numpy().view(np.uint16)
                         for n in ("q", "k", "v", "raw_g", "raw_beta")})
        pick = [b for b in range(B) if sl_h[b] > 0][: args.cpu_requests + 32]
        pages = state.view(torch.int16) if bf16 else state
        host["state_pages"] = {
            b: pages[int(sl_h[b]) * page:(int(sl_h[b]) + 1) * page].cpu().numpy().view(
                np.uint16 if bf16 else np.float32)
            for b in pick}

    state_stride = page
    commit_args = dict(heads=H, window=RQ, batch=B,
                       state_dtype=kda.KDA_STATE_BF16 if bf16 else kda.KDA_STATE_F32,
                       state_addrs=[state.data_ptr()], state_slot_strides=[state_stride],
                       corr_addrs=[corr.data_ptr()], corr_row_strides=[H * RQ * V],
                       kg_addrs=[kg.data_ptr()], kg_row_strides=[H * RQ * 2 * K],
                       a_log=a_log, dt_bias=dt_bias, sources=flush[1], commit_lens=flush[0],
                       destinations=flush[1], record_rows=rows, lower_bound=lb)

    total = args.warmup + args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(total)]

    # Timed step j brackets the fused launch (and the gate projection) with
    # events when j is even, the commit when j is odd; both when only one step
    # is timed. Warm-up steps record none.
    def times_fused(i):
        j = i - args.warmup
        return j >= 0 and (j % 2 == 0 or args.steps == 1)

    def times_commit(i):
        j = i - args.warmup
        return j >= 0 and (j % 2 == 1 or args.steps == 1)

    def step(i):
        e = ev[i]
        tf, tc = times_fused(i), times_commit(i)
        commit_lens.copy_(accepted)
        if gp is not None:
            if tf:
                e[4].record()
            kda.kda_gate_projection(tokens=B * T, heads=H, f_a=gp["f_a"],
                                    f_a_row_stride=gp["pitch"], f_b=gp["f_b"],
                                    raw_g=gp["raw_g"])
        if tf:
            e[0].record()
        if conv is None:
            kda.kda_fused_replay_verify(heads=H, tokens=T, batch=B, q=new.q, k=new.k, v=new.v,
                                        raw_g=raw_g, raw_beta=new.raw_beta, a_log=a_log,
                                        dt_bias=dt_bias, lower_bound=lb, state=state,
                                        state_slot_stride=state_stride, state_indices=slots,
                                        corr=corr, kg=kg, record_tokens=RQ, record_rows=rows,
                                        pending=pending, out=out, gate=gate,
                                        norm_weight=norm_w, norm_eps=norm_eps)
        else:
            cs = conv["strides"]
            kda.kda_fused_conv_replay_verify(
                heads=H, tokens=T, batch=B, x=conv["x"], x_row_stride=conv["pitch"],
                conv_weight=conv["weight"], conv_bias=conv["bias"], conv_state=conv["pool"],
                conv_slot_stride=cs[0], conv_channel_stride=cs[1], conv_tap_stride=cs[2],
                q_scale=K ** -0.5, raw_g=raw_g, raw_beta=new.raw_beta, a_log=a_log,
                dt_bias=dt_bias, lower_bound=lb, state=state, state_slot_stride=state_stride,
                state_indices=slots, corr=corr, kg=kg, record_tokens=RQ, record_rows=rows,
                pending=pending, out=out, gate=gate, norm_weight=norm_w, norm_eps=norm_eps)
        if tf:
            e[1].record()
        kda.kda_defer_commit(batch=B, state_indices=slots, commit_lens=commit_lens,
                             record_rows=rows, pending=pending)
        kda.kda_flush_plan(batch=B, spec_query_len=T, state_indices=slots, record_rows=rows,
                           pending=pending, commit_lens=flush[0], final_indices=flush[1],
                           boundaries=flush[2], boundary_lens=flush[3])
        if tc:
            e[2].record()
        kda.kda_commit(**commit_args)
        if tc:
            e[3].record()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.warmup, total):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    if not bool(torch.isfinite(state[: 64 * page]).all()):
        sys.exit("non-finite state after the run")

    f_idx = [i for i in range(args.warmup, total) if times_fused(i)]
    c_idx = [i for i in range(args.warmup, total) if times_commit(i)]
    fused_ms = [ev[i][0].elapsed_time(ev[i][1]) for i in f_idx]
    commit_ms = [ev[i][2].elapsed_time(ev[i][3]) for i in c_idx]
    gp_ms = [ev[i][4].elapsed_time(ev[i][0]) for i in f_idx] if gp is not None else []

    # Algorithmic bytes from the plan of each step.
    sl_h, rr_h = slots.cpu().numpy(), rows.cpu().numpy()
    plan = simulate_plan(sl_h, rr_h, a["pending"].numpy(), a["accepted"].numpy(), total, T)
    fb = [fused_bytes(sl_h, rr_h, p, T, RQ, H, gated=args.gated_output, es=es,
                      conv=args.conv)
          for p, _ in plan[args.warmup:]]
    cb = [commit_bytes(sl_h, l, rr_h, H, RQ, es=es) for _, l in plan[args.warmup:]]
    state_bytes = sum(f[0] + c[0] for f, c in zip(fb, cb))
    ms_per_step = wall * 1e3 / args.steps
    value = state_bytes / wall / 1e9
    items = B * H
    fused_mean_ms = sum(fused_ms) / len(fused_ms)
    commit_mean_ms = sum(commit_ms) / len(commit_ms)
    # Per-launch bytes of the steps whose launches the events timed.
    fb_t = [fb[i - args.warmup] for i in f_idx]
    cb_t = [cb[i - args.warmup] for i in c_idx]
    fused_total = sum(f[1] for f in fb_t) / len(fb_t)
    fused_state = sum(f[0] for f in fb_t) / len(fb_t)
    commit_total = sum(c[1] for c in cb_t) / len(cb_t)
    commit_state = sum(c[0] for c in cb_t) / len(cb_t)
    achieved = fused_total / (fused_mean_ms * 1e-3) / 1e9
    tkey, tsrc = fused_variant(args)
    traffic = measured_traffic(tkey, source_digest(tsrc))

    result = {
        "metric": "state GB/s (% of HBM peak) + (req,head) items/s, KDA commit & fused verify",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "large_decode: L=1 H=64 K=V=128 B=512 q=8 FP32 state 512 slots "
                        "(2 GiB), ~5% no-op rows; step = fused replay+verify, defer, "
                        "flush plan, in-place FP32 commit" if not bf16 else
                        "large_decode with the pool rounded to BF16: L=1 H=64 K=V=128 B=512 "
                        "q=8 BF16 state 512 slots (1 GiB), ~5% no-op rows; step = fused "
                        "replay+verify, defer, flush plan, in-place BF16 commit",
            "global_batch": B, "seq_len": T, "heads": H, "parallelism": "none",
            "gated_output": bool(args.gated_output),
            "state_dtype": args.state_dtype,
            "conv_prologue": bool(args.conv),
            "conv_layout": args.conv_layout if args.conv else None,
            "gate_projection": bool(args.gate_proj),
        },
        "library": os.path.relpath(kda.library_path(), ROOT),
        "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "items_per_s": round(items / (wall / args.steps), 1),
        "kernels": {
            "fused_replay_verify": {
                "mean_ms": round(fused_mean_ms, 4), "min_ms": round(min(fused_ms), 4),
                **spread(fused_ms),
                "state_gbs": round(fused_state / (fused_mean_ms * 1e-3) / 1e9, 1),
                "total_gbs": round(achieved, 1),
                "items_per_s": round(items / (fused_mean_ms * 1e-3), 1)},
            ("commit_bf16_inplace" if bf16 else "commit_fp32_inplace"): {
                "mean_ms": round(commit_mean_ms, 4), "min_ms": round(min(commit_ms), 4),
                **spread(commit_ms),
                "state_gbs": round(commit_state / (commit_mean_ms * 1e-3) / 1e9, 1),
                "total_gbs": round(commit_total / (commit_mean_ms * 1e-3) / 1e9, 1),
                "items_per_s": round(items / (commit_mean_ms * 1e-3), 1)},
            **({"gate_projection": {
                "mean_ms": round(sum(gp_ms) / len(gp_ms), 4),
                "total_gbs": round((B * T * (256 + H * K * 2) + H * K * 256)
                                   / (sum(gp_ms) / len(gp_ms) * 1e-3) / 1e9, 1)}}
               if gp is not None else {}),
        },
        "roofline": {
            "kernel": "fused_replay_verify",
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": int(fused_total),
        },
    }
    # The in-place read+write ceiling of this pool in the fused kernel's access
    # pattern (every named page loaded and stored back unchanged; FP32 pools).
    pe = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    if bf16:
        pe = None
    if pe is not None:
        for _ in range(2):
            kda.kda_page_rw_probe(heads=H, batch=B, state=state,
                                  state_slot_stride=state_stride, state_indices=slots)
        pe[0].record()
        for _ in range(10):
            kda.kda_page_rw_probe(heads=H, batch=B, state=state,
                                  state_slot_stride=state_stride, state_indices=slots)
        pe[1].record()
        torch.cuda.synchronize()
        probe_ms = pe[0].elapsed_time(pe[1]) / 10
        probe_bytes = 2 * int((sl_h > 0).sum()) * H * V * K * 4
        ceiling = probe_bytes / (probe_ms * 1e-3) / 1e9
        result["rw_ceiling"] = {
            "kernel": "kda_page_rw_probe", "gbs": round(ceiling, 1),
            "pct_of_peak": round(100 * ceiling / HBM_PEAK_GBS, 2), "ms": round(probe_ms, 4),
            "fused_frac_of_ceiling": round(achieved / ceiling, 4),
            "commit_frac_of_ceiling": round(
                commit_total / (commit_mean_ms * 1e-3) / 1e9 / ceiling, 4),
        }
    if args.copy_probe:
        src = torch.empty(1 << 29, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / 5
        result["copy_probe"] = {"bytes": 2 * src.numel() * 4, "ms": round(ms, 4),
                                "gbs": round(2 * src.numel() * 4 / (ms * 1e-3) / 1e9, 1)}
        del src, dst
    if host is not None:
        result["cpu_baseline"] = cpu_baseline(host, H, T, RQ, args.cpu_requests, lb, bf16,
                                              args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
