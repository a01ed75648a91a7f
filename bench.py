"""Benchmark of the gated DeltaNet token mixer on one MI355X.

One step = one pass of the whole mixer over the prefill workload
(T = 4096 tokens, 16 K-heads, 48 V-heads, bf16 activations, one sequence),
inputs already resident in HBM, in two forms: the three calls
gdn_conv_gate_prep -> gdn_prefill_chunked -> gdn_gated_rmsnorm, and the one
call gdn_prefill_fused (q, k, v, beta, g computed inside the chunked
kernels). Each runs as plain launches and as the step captured in a HIP
graph and replayed; ``value`` is tokens per second over exactly ``--steps``
timed steps (after ``--warmup`` untimed ones) of the fastest of the four,
all reported under "prefill_modes" with the median and minimum of the
per-step times (an event pair around every step). "varlen_prefill" times the
varlen workload (8 packed sequences of 512 .. 8192 tokens, nonzero initial
states) the same way, fused forms only.

The same run also times the decode path on the batch-1 workload (32 V-heads,
1024 consecutive steps) and the batch-64 workload (256 steps), and reports
them under "decode": the three calls per token (gdn_conv_gate_prep ->
gdn_decode_step -> gdn_gated_rmsnorm) and the single gdn_decode_fused call,
each with plain launches and as the whole loop captured in one HIP graph.

Rooflines use the kernels' algorithmic work, timed with HIP events recorded
on the stream the kernels run on:
  * chunked delta rule (gdn_prefill_chunked): 9,000,277 flop per
    (chunk of 64, V-head) -- 5 CH^2 d + 6 CH d^2 + CH^3/3 with CH = 64,
    d = 128, triangles counted once -- against the bf16 dense MFMA peak;
  * decode step (gdn_decode_fused, graph replay): bytes of S read + written,
    the token's qkv row, conv state read + written, z read, y written, the
    logits and the parameters, against 8 TB/s HBM; and the delta-rule
    kernel alone (gdn_decode_step): S read + written, q, k, v, beta, g read,
    o written.
"roofline_fused" prices the same flops against the whole gdn_prefill_fused
call (events around each call), a lower bound on its chunked kernels' own
fraction. The CPU baseline is the fp64 oracle over the whole prefill workload
once, on one thread and with the V-heads split over threads, with the host's
CPU model and counts.

"block" times the projections around the mixer as well (gdn_in_proj ->
mixer -> gdn_out_proj) on the 27B prefill layer and the 35B-A3B batch-64
decode layer, with each projection's roofline: 2 M N K flop against the bf16
MFMA peak for prefill, and its weights plus activations in and out against
HBM for decode (the weights are streamed once per token batch).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

from gated_deltanet_layer_amd import binding as B  # noqa: E402
from gated_deltanet_layer_amd import layer as Lyr  # noqa: E402
from gated_deltanet_layer_amd import workloads as wl  # noqa: E402

PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "gated_deltanet_layer_amd", "csrc")
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
CHUNK = 64
FLOP_PER_CHUNK_HEAD = 5 * CHUNK ** 2 * 128 + 6 * CHUNK * 128 ** 2 + CHUNK ** 3 // 3   # 9,000,277


def dev(x: np.ndarray) -> torch.Tensor:
    if x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# Source files behind each traffic record (plus the shared headers): a record
# is only used while these are unchanged.
TRAFFIC_SOURCES = {
    "prefill_core": ("prefill.hip",), "prefill_fused_core": ("prefill.hip",),
    "prefill_prep": ("prep.hip",), "prefill_norm": ("norm.hip",),
    "decode_b64": ("decode.hip",), "decode_b1": ("decode.hip",),
    "decode_fused_b64": ("decode_fused.hip",), "decode_fused_b1": ("decode_fused.hip",),
}


def kernel_source_hash(key: str) -> str:
    """sha256 over the code (comments and whitespace removed) of the HIP
    source behind a traffic record and the shared device headers: the counters
    are only valid for that code."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in sorted(TRAFFIC_SOURCES[key]) + ["gdn_device.h", "gdn_internal.h"]:
        with open(os.path.join(CSRC, f)) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(f.encode())
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()


def measured_traffic(key: str):
    """HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, copy-calibrated) recorded in
    profiles/traffic.json for the current kernel sources, else None."""
    path = os.path.join(PROFILES, "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    k = rec.get("kernels", {}).get(key)
    if k is None or k.get("source_sha256") != kernel_source_hash(key):
        return None
    k = rec["kernels"][key]
    return int(k["fetch_bytes"] + k["write_bytes"])


def _kernel_key(name: str) -> str:
    """A kernel's name without namespace noise and argument list, with the
    precision enum spelled out (`chunk_state_kernel<BF16X3, gdn::bf16_t, true, false>`)."""
    name = name.replace("(anonymous namespace)::", "").replace("void ", "")
    name = name.replace("(gdn::Prec)1", "BF16X3").replace("(gdn::Prec)0", "F32")
    return name.split("(")[0]


def summarize_rocprof(db_path: str) -> str:
    """Per-kernel summary of a rocprofv3 database: durations from a kernel
    trace, or per-dispatch counter values from a --pmc run."""
    import collections
    import sqlite3
    db = sqlite3.connect(db_path)
    tables = {r[0] for r in db.execute("select name from sqlite_master")}
    lines = []

    def short(name):
        return _kernel_key(name)[:70]
    if "counters_collection" in tables and db.execute("select count(*) from counters_collection").fetchone()[0]:
        per = collections.defaultdict(float)
        for k, d, n, v in db.execute("select kernel_name, dispatch_id, counter_name, value from counters_collection"):
            per[(k, d, n)] += v
        agg = collections.defaultdict(list)
        for (k, d, n), v in per.items():
            agg[(short(k), n)].append(v)
        lines.append(f"{'kernel':70s} {'counter':12s} {'dispatches':>10s} {'mean':>14s}")
        for (k, n), v in sorted(agg.items()):
            lines.append(f"{k:70s} {n:12s} {len(v):10d} {sum(v) / len(v):14.1f}")
    else:
        agg = collections.defaultdict(list)
        for n, gx, gy, wx, dur in db.execute("select name, grid_x, grid_y, workgroup_x, duration from kernels"):
            agg[(short(n), gx, gy, wx)].append(dur)
        lines.append(f"{'kernel':70s} {'grid(threads)':>16s} {'wg':>5s} {'calls':>6s} {'avg_us':>9s} {'min_us':>9s}")
        for (k, gx, gy, wx), d in sorted(agg.items(), key=lambda kv: -sum(kv[1])):
            lines.append(f"{k:70s} {f'{gx}x{gy}':>16s} {wx:5d} {len(d):6d} {sum(d) / len(d) / 1e3:9.2f} "
                         f"{min(d) / 1e3:9.2f}")
    return "\n".join(lines)


def _pmc_means(db_path: str, counter: str, reduce=None) -> dict:
    """Mean (or `reduce`) over dispatches of one counter, by short kernel name."""
    import collections
    import sqlite3
    db = sqlite3.connect(db_path)
    per = collections.defaultdict(float)
    for k, d, n, v in db.execute("select kernel_name, dispatch_id, counter_name, value from counters_collection"):
        if n == counter:
            per[(k, d)] += v
    agg = collections.defaultdict(list)
    for (k, d), v in per.items():
        agg[_kernel_key(k)].append(v)
    return {k: (reduce(v) if reduce else sum(v) / len(v)) for k, v in agg.items()}


def write_traffic(dbs):
    """profiles/traffic.json: HBM bytes per launch of each kernel, from
    FETCH_SIZE / WRITE_SIZE (KiB per dispatch) scaled by what the same
    counters read for the plain 268,435,456-byte device copy (--calibrate-copy)
    in the same run."""
    copy_bytes = 256 << 20
    runs = {}
    for name, (fdb, wdb) in zip(("prefill", "decode_b64", "decode_b1"), zip(dbs[0::2], dbs[1::2])):
        f, wr = _pmc_means(fdb, "FETCH_SIZE"), _pmc_means(wdb, "WRITE_SIZE")
        # The calibration copy is the largest copyBuffer dispatch of the run.
        cf = max(v for k, v in _pmc_means(fdb, "FETCH_SIZE", max).items() if "copyBuffer" in k) * 1024.0
        cw = max(v for k, v in _pmc_means(wdb, "WRITE_SIZE", max).items() if "copyBuffer" in k) * 1024.0
        runs[name] = (f, wr, copy_bytes / cf, copy_bytes / cw)

    def pick(run, sub):
        f, wr, ff, fw = runs[run]
        keys = [k for k in f if sub in k]
        if not keys:
            return None
        return (sum(f[k] for k in keys) * 1024.0 * ff, sum(wr.get(k, 0.0) for k in keys) * 1024.0 * fw)

    kernels = {}
    for key, run, subs, what in (
            ("prefill_core", "prefill", ("chunk_local_kernel<BF16X3, gdn::bf16_t, false>",
                                         "chunk_state_kernel<BF16X3, gdn::bf16_t, false, false>"),
             "gdn_prefill_chunked on the T=4096, Hv=48 bf16 workload (chunk_local + chunk_state)"),
            ("prefill_fused_core", "prefill", ("chunk_local_kernel<BF16X3, gdn::bf16_t, true>",
                                               "chunk_state_kernel<BF16X3, gdn::bf16_t, true, false>"),
             "the kernels of gdn_prefill_fused, T=4096 Hv=48 bf16: chunk_local and chunk_state (q, k, v and the "
             "gates formed inside; y and the new conv state formed in chunk_state's launch)"),
            ("prefill_prep", "prefill", ("prep_kernel",), "gdn_conv_gate_prep, T=4096 Hv=48 bf16"),
            ("prefill_norm", "prefill", ("norm_kernel<gdn::bf16_t, false>",), "gdn_gated_rmsnorm, T=4096 Hv=48 bf16"),
            ("decode_b64", "decode_b64", ("decode_kernel",), "gdn_decode_step, batch 64, Hv=32"),
            ("decode_fused_b64", "decode_b64", ("decode_tokens_kernel<gdn::bf16_t, true>",), "gdn_decode_fused, batch 64, Hv=32"),
            ("decode_b1", "decode_b1", ("decode_kernel",), "gdn_decode_step, batch 1, Hv=32"),
            ("decode_fused_b1", "decode_b1", ("decode_tokens_kernel<gdn::bf16_t, true>",), "gdn_decode_fused, batch 1, Hv=32")):
        tot = [pick(run, sub) for sub in subs]
        if any(t is None for t in tot):
            continue
        kernels[key] = {"what": what, "fetch_bytes": int(sum(t[0] for t in tot)),
                        "write_bytes": int(sum(t[1] for t in tot)), "source_sha256": kernel_source_hash(key)}
    rec = {
           "note": "HBM bytes per launch from rocprofv3 FETCH_SIZE and WRITE_SIZE (KiB per dispatch, separate "
                   "runs), scaled by what the same counters read for a plain 256 MiB device copy in the same run.",
           "calibration": {k: {"fetch_factor": round(v[2], 4), "write_factor": round(v[3], 4)}
                           for k, v in runs.items()},
           "kernels": kernels,
           "commands": [f"rocprofv3 --pmc {c} -d <dir> -o run -- python3 bench.py {o} --calibrate-copy"
                        for o in ("--only prefill --steps 2 --warmup 1 --no-cpu-baseline",
                                  "--only decode-b64 --no-graph", "--only decode-b1 --no-graph")
                        for c in ("FETCH_SIZE", "WRITE_SIZE")]}
    with open(os.path.join(PROFILES, "traffic.json"), "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(kernels, indent=1))


def _timed_reps(fn, steps: int, warmup: int, stats_fn=None):
    """Run fn `warmup` times untimed, then exactly `steps` times between two
    events on the current stream (synchronised on both sides): the total.
    Then `steps` more runs of stats_fn (default fn), each between an event
    pair of its own, for the distribution per step: recording events between
    steps costs ~7 us per step on the 4,096-token prefill, so they stay out of
    the timed total. Returns (total ms, [ms per rep of the second pass])."""
    for _ in range(warmup):
        fn()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(steps):
        fn()
    end.record()
    torch.cuda.synchronize()
    total = start.elapsed_time(end)
    evs = _events(steps)
    for i in range(steps):
        evs[i][0].record()
        (stats_fn or fn)()
        evs[i][1].record()
    torch.cuda.synchronize()
    return total, [a.elapsed_time(b) for a, b in evs]


def _mode_stats(total_ms: float, per: list, steps: int, tokens: int) -> dict:
    return {"ms_per_step": round(total_ms / steps, 4), "tokens_per_s": round(tokens * steps / (total_ms * 1e-3), 1),
            "median_ms": round(float(np.median(per)), 4), "min_ms": round(float(np.min(per)), 4)}


def _core_roofline(flops: int, ms: float, what: str, traffic_key=None) -> dict:
    tf = flops / (ms * 1e-3) / 1e12
    return {"bound": "mfma", "achieved": round(tf, 2), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(tf / BF16_PEAK_TFLOPS, 4),
            "traffic": measured_traffic(traffic_key) if traffic_key else None,
            "kernel": what, "flop_per_launch": flops, "avg_launch_us": round(ms * 1e3, 2)}


def bench_prefill(steps: int, warmup: int, wid: int = 3, three_call: bool = True):
    """One prefill workload, whole mixer per step: the three calls (prep ->
    chunked -> norm) and the single gdn_prefill_fused call, each plain and as
    a captured graph (three_call=False: the fused forms only, plus the
    three-call step once per rep for the chunked call's events)."""
    w = wl.WORKLOADS[wid]
    x = wl.generate(w)
    t = {k: dev(v) for k, v in x.items()}
    del x
    cfg = B.make_config(w.n_qk_heads, w.n_v_heads, w.act)
    N = w.n_seqs
    lens = w.seq_lengths()
    T = int(sum(lens))
    run = Lyr.Prefill(cfg, N, T)
    conv_out = torch.empty_like(t["conv0"])
    S_out = torch.empty_like(t["S0"])
    args = (t["cu_seqlens"], t["qkv"], t["b"], t["a"], t["conv_w"], t["dt_bias"], t["A_log"], t["conv0"], conv_out)
    core_ev = []

    def step():
        run.prep(*args)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        run.core(t["cu_seqlens"], t["S0"], S_out)
        b.record()
        core_ev.append((a, b))
        run.norm(t["z"], t["norm_w"])

    def plain_step():
        run.prep(*args)
        run.core(t["cu_seqlens"], t["S0"], S_out)
        run.norm(t["z"], t["norm_w"])

    modes = {}
    # Timed without events; the chunked call's own duration comes from the
    # second pass, with an event pair around it in each step.
    total, per = _timed_reps(plain_step, steps, warmup, stats_fn=step)
    core_per = [a.elapsed_time(b) for a, b in core_ev]
    core_ms = float(np.mean(core_per))
    if three_call:
        modes["plain"] = _mode_stats(total, per, steps, T)

        # The same step captured once as a HIP graph (kernel nodes only, no
        # memset nodes) and replayed: what a caller that captures its layer gets.
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            plain_step()
        total, per = _timed_reps(g.replay, steps, warmup)
        modes["graph"] = _mode_stats(total, per, steps, T)
        del g
    # The same step as one gdn_prefill_fused call (q, k, v, beta, g computed
    # inside the chunked kernels), plain and as a graph.
    fused = Lyr.PrefillFused(cfg, N, T)
    conv_f = torch.empty_like(t["conv0"])
    S_f = torch.empty_like(t["S0"])

    def fstep():
        fused(t["cu_seqlens"], t["qkv"], t["z"], t["b"], t["a"], t["conv_w"], t["dt_bias"], t["A_log"],
              t["norm_w"], t["conv0"], conv_f, t["S0"], S_f)

    total, fper = _timed_reps(fstep, steps, warmup)
    modes["fused"] = _mode_stats(total, fper, steps, T)
    fused_call_ms = float(np.mean(fper))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fstep()
    total, per = _timed_reps(g.replay, steps, warmup)
    modes["fused_graph"] = _mode_stats(total, per, steps, T)
    del g
    best = min(modes, key=lambda m: modes[m]["ms_per_step"])
    n_chunk_heads = sum((L + CHUNK - 1) // CHUNK for L in lens) * w.n_v_heads
    # gdn_prefill_fused forms y inside chunk_state's launch when its 4 blocks
    # per (sequence, V-head), in whole rounds of the 8 XCDs, leave >= 32 CUs.
    folded = 256 - (len(lens) * w.n_v_heads + 7) // 8 * 8 * 4 >= 32
    flops = FLOP_PER_CHUNK_HEAD * n_chunk_heads
    out = dict(workload=w.name, tokens=T, best=best, ms_per_step=modes[best]["ms_per_step"],
               total_ms=modes[best]["ms_per_step"] * steps, core_ms=core_ms,
               tokens_per_s=modes[best]["tokens_per_s"], modes=modes,
               roofline=_core_roofline(flops, core_ms,
                                       "gdn_prefill_chunked (chunk_local + chunk_state), HIP events around each "
                                       "call in the three-call step", "prefill_core" if wid == 3 else None),
               roofline_fused=_core_roofline(
                   flops, fused_call_ms,
                   "gdn_prefill_fused, the whole call, HIP events around each call: chunk_local and chunk_state "
                   "with the conv, SiLU, L2 norm and gates folded in, and " +
                   ("the gated RMSNorm and new conv states formed in chunk_state's launch (on the CUs its "
                    "sequential blocks leave idle)" if folded else "a third launch for the norm and conv states"),
                   "prefill_fused_core" if wid == 3 and folded else None))
    out["roofline"]["median_launch_us"] = round(float(np.median(core_per)) * 1e3, 2)
    out["roofline"]["min_launch_us"] = round(float(np.min(core_per)) * 1e3, 2)
    out["roofline_fused"]["median_launch_us"] = round(float(np.median(fper)) * 1e3, 2)
    out["roofline_fused"]["min_launch_us"] = round(float(np.min(fper)) * 1e3, 2)
    return out


def _events(n):
    return [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]


def _mean_ms(evs):
    return float(np.mean([a.elapsed_time(b) for a, b in evs]))


def bench_block(steps: int, warmup: int):
    """The whole token-mixer block: gdn_in_proj -> the mixer -> gdn_out_proj.

    Prefill on the 27B layer (T = 4096, hidden 5120, 16 K-heads, 48 V-heads)
    with the mixer's three calls in between, plain launches and as one graph;
    decode on the 35B-A3B layer (64 sequences, hidden 2048, 32 V-heads) with
    gdn_decode_fused in between, 64 steps as one graph. The projections are
    also timed one by one (HIP events around each launch on its stream)."""
    out = {}
    # ---- prefill block
    w = wl.WORKLOADS[3]
    hidden = wl.HIDDEN[w.n_v_heads]
    x = wl.generate_block(w, hidden)
    t = {k: dev(v) for k, v in x.items() if k != "y"}
    cfg = B.make_config(w.n_qk_heads, w.n_v_heads, w.act)
    T = int(x["cu_seqlens"][-1])
    run = Lyr.Block(cfg, 1, T, hidden)
    conv_out = torch.empty_like(t["conv0"])
    S_out = torch.empty_like(t["S0"])
    P = run.proj
    wargs = (t["w_qkv"], t["w_gate"], t["w_beta"], t["w_alpha"])

    def step(evs=None):
        if evs is not None:
            evs[0][0].record()
        P.project_in(cfg, T, t["x"], *wargs, None)
        if evs is not None:
            evs[0][1].record()
        run.mixer(t["cu_seqlens"], P.qkv, P.z, P.b, P.a, t["conv_w"], t["dt_bias"], t["A_log"], t["norm_w"],
                  t["conv0"], conv_out, t["S0"], S_out)
        if evs is not None:
            evs[1][0].record()
        P.project_out(cfg, T, run.mixer.y, t["w_out"], None)
        if evs is not None:
            evs[1][1].record()

    for _ in range(warmup):
        step()
    ev_in, ev_out = _events(steps), _events(steps)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(steps):
        step((ev_in[i], ev_out[i]))
    end.record()
    torch.cuda.synchronize()
    plain_ms = start.elapsed_time(end)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    start.record()
    for _ in range(steps):
        g.replay()
    end.record()
    torch.cuda.synchronize()
    graph_ms = start.elapsed_time(end)
    del g
    C, Z, Hv = P.qkv.shape[1], P.z.shape[1] * P.z.shape[2], w.n_v_heads
    n_in = C + Z + 2 * Hv
    gemms = {}
    for name, evs, (M, N, K) in (("in_proj", ev_in, (T, n_in, hidden)), ("out_proj", ev_out, (T, hidden, Z))):
        ms = _mean_ms(evs)
        tf = 2.0 * M * N * K / (ms * 1e-3) / 1e12
        gemms[name] = {"M": M, "N": N, "K": K, "avg_launch_us": round(ms * 1e3, 2),
                       "roofline": {"bound": "mfma", "achieved": round(tf, 1), "peak": BF16_PEAK_TFLOPS,
                                    "unit": "TFLOP/s", "frac": round(tf / BF16_PEAK_TFLOPS, 4)}}
    best = min(plain_ms, graph_ms)
    out["prefill"] = {"workload": f"27B block prefill T={T} hidden={hidden} Hqk=16 Hv=48 bf16",
                      "tokens_per_s": round(T * steps / (best * 1e-3), 1),
                      "ms_per_step": round(best / steps, 4),
                      "modes": {"plain_ms_per_step": round(plain_ms / steps, 4),
                                "graph_ms_per_step": round(graph_ms / steps, 4)},
                      "gemms": gemms}
    del t, run, x
    torch.cuda.empty_cache()

    # ---- decode block (35B-A3B, 64 sequences)
    w = wl.WORKLOADS[4]
    hidden = wl.HIDDEN[w.n_v_heads]
    dsteps = 64
    x = wl.generate_block(w, hidden, max_steps=dsteps)
    t = {k: dev(v) for k, v in x.items() if k != "y"}
    cfg = B.make_config(w.n_qk_heads, w.n_v_heads, w.act)
    N = w.n_seqs
    run = Lyr.DecodeBlock(cfg, N, hidden, t["conv0"].clone())
    S = t["S0"].clone()
    P = run.proj
    wargs = (t["w_qkv"], t["w_gate"], t["w_beta"], t["w_alpha"])

    def dstep(s, evs=None):
        if evs is not None:
            evs[0][0].record()
        P.project_in(cfg, N, t["x"][s], *wargs, None)
        if evs is not None:
            evs[0][1].record()
        run.mixer(P.qkv, P.z, P.b, P.a, t["conv_w"], t["dt_bias"], t["A_log"], t["norm_w"], S, run.y)
        if evs is not None:
            evs[1][0].record()
        P.project_out(cfg, N, run.y, t["w_out"], None)
        if evs is not None:
            evs[1][1].record()

    for s in range(min(8, dsteps)):
        dstep(s)
    ev_in, ev_out = _events(dsteps), _events(dsteps)
    torch.cuda.synchronize()
    start.record()
    for s in range(dsteps):
        dstep(s, (ev_in[s], ev_out[s]))
    end.record()
    torch.cuda.synchronize()
    plain_ms = start.elapsed_time(end)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for s in range(dsteps):
            dstep(s)
    g.replay()
    torch.cuda.synchronize()
    start.record()
    g.replay()
    end.record()
    torch.cuda.synchronize()
    graph_ms = start.elapsed_time(end)
    del g
    C, Z = P.qkv.shape[1], P.z.shape[1] * P.z.shape[2]
    n_in = C + Z + 2 * w.n_v_heads
    gemms = {}
    for name, evs, (M, Nn, K) in (("in_proj", ev_in, (N, n_in, hidden)), ("out_proj", ev_out, (N, hidden, Z))):
        ms = _mean_ms(evs)
        byts = 2 * (Nn * K + M * K + M * Nn)        # weights once, activations in and out (bf16)
        gbs = byts / (ms * 1e-3) / 1e9
        gemms[name] = {"M": M, "N": Nn, "K": K, "avg_launch_us": round(ms * 1e3, 2),
                       "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                                    "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "bytes_per_launch": byts}}
    best = min(plain_ms, graph_ms)
    out["decode_b64"] = {"workload": f"35B-A3B block decode {N} seqs hidden={hidden} Hqk=16 Hv=32 bf16, "
                                     f"{dsteps} steps",
                         "tokens_per_s": round(N * dsteps / (best * 1e-3), 1),
                         "us_per_step": round(best * 1e3 / dsteps, 2),
                         "modes": {"plain_us_per_step": round(plain_ms * 1e3 / dsteps, 2),
                                   "graph_us_per_step": round(graph_ms * 1e3 / dsteps, 2)},
                         "gemms": gemms}
    return out


def decode_kernel_bytes(w: wl.Workload) -> int:
    """Algorithmic bytes of one gdn_decode_step launch: S read + written, q, k,
    v, beta, g read, o written."""
    N, Hqk, Hv, d = w.n_seqs, w.n_qk_heads, w.n_v_heads, w.head_dim
    act = 2 if w.act == "bf16" else 4
    return (2 * N * Hv * d * d * 4 + 2 * N * Hqk * d * 4 + N * Hv * d * 4 + 2 * N * Hv * 4
            + N * Hv * d * act)


def decode_step_bytes(w: wl.Workload) -> int:
    """Algorithmic bytes of one whole decode step (one gdn_decode_fused launch):
    S read + written, the token's qkv row, conv state read + written, z read,
    y written, the two logits, and the parameters (conv_w, dt_bias, A_log,
    norm_w)."""
    N, Hqk, Hv, d = w.n_seqs, w.n_qk_heads, w.n_v_heads, w.head_dim
    act = 2 if w.act == "bf16" else 4
    C = d * (2 * Hqk + Hv)
    return (2 * N * Hv * d * d * 4 + N * C * act + 2 * N * 3 * C * act + 2 * N * Hv * d * act
            + 2 * N * Hv * act + C * 4 * 4 + 2 * Hv * 4 + d * 4)


def bench_decode(wid: int, warmup_steps: int = 32, graphs: bool = True):
    """Time the workload's whole decode loop four ways: the three calls per
    step (prep, step, norm) and the single fused call, each with plain
    launches and as one captured HIP graph replayed once."""
    w = wl.WORKLOADS[wid]
    x = wl.generate(w)
    t = {k: dev(v) for k, v in x.items()}
    cfg = B.make_config(w.n_qk_heads, w.n_v_heads, w.act)
    N, steps = w.n_seqs, w.steps
    three = Lyr.Decode(cfg, N)
    conv = t["conv0"].clone()
    fused = Lyr.DecodeFused(cfg, N, t["conv0"].clone())
    S = t["S0"].clone()
    ys = torch.empty_like(t["z"])

    def three_step(s, evs=None):
        B.gdn_conv_gate_prep(cfg, N, N, three.cu, t["qkv"][s], t["b"][s], t["a"][s], t["conv_w"],
                             t["dt_bias"], t["A_log"], conv, conv, three.q, three.k, three.v, three.beta, three.g)
        if evs is not None:
            evs[0].record()
        B.gdn_decode_step(cfg, N, three.q, three.k, three.v, three.beta, three.g, S, S, three.o)
        if evs is not None:
            evs[1].record()
        B.gdn_gated_rmsnorm(cfg, N * w.n_v_heads, three.o, t["z"][s], t["norm_w"], ys[s])

    def fused_step(s, evs=None):
        fused(t["qkv"][s], t["z"][s], t["b"][s], t["a"][s], t["conv_w"], t["dt_bias"], t["A_log"], t["norm_w"],
              S, ys[s])

    def reset():
        S.copy_(t["S0"])
        conv.copy_(t["conv0"])
        fused.bufs[0].copy_(t["conv0"])
        fused.cur = 0
        torch.cuda.synchronize()

    def timed(fn):
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record()
        fn()
        end.record()
        torch.cuda.synchronize()
        return start.elapsed_time(end)

    for s in range(min(warmup_steps, steps)):
        three_step(s)
        fused_step(s)
    modes = {}
    # Plain launches; the three-call loop also times each gdn_decode_step launch.
    reset()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    ms = timed(lambda: [three_step(s, evs[s]) for s in range(steps)])
    k_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    modes["three_call"] = ms
    reset()
    modes["fused"] = timed(lambda: [fused_step(s) for s in range(steps)])
    # The whole loop captured as one graph, replayed once untimed, then timed.
    for name, fn in ((("three_call_graph", three_step), ("fused_graph", fused_step)) if graphs else ()):
        reset()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for s in range(steps):
                fn(s)
        reset()
        g.replay()
        reset()
        modes[name] = timed(g.replay)
        del g
    # A 16-token draft block verified in one gdn_decode_verify call per block
    # (the state and conv state after every token kept as snapshot planes).
    K = 16
    if steps % K == 0:
        cvt = lambda a: a[:steps].reshape((steps // K, K) + a.shape[1:]).transpose(1, 2).contiguous()
        vq, vz, vb, va = (cvt(t[k]) for k in ("qkv", "z", "b", "a"))           # [blocks][N][K]...
        conv_snap = torch.empty((N, K) + tuple(t["conv0"].shape[1:]), dtype=t["conv0"].dtype, device="cuda")
        S_snap = torch.empty((N, K) + tuple(t["S0"].shape[1:]), dtype=torch.float32, device="cuda")
        vy = torch.empty_like(vz)

        def verify_loop():
            for blk in range(steps // K):
                B.gdn_decode_verify(cfg, N, K, vq[blk], vb[blk], va[blk], vz[blk], t["conv_w"], t["dt_bias"],
                                    t["A_log"], t["norm_w"], t["conv0"], conv_snap, t["S0"], S_snap, vy[blk])
        verify_loop()
        torch.cuda.synchronize()
        modes["verify_k16"] = timed(verify_loop)
    best = min((m for m in modes if m != "verify_k16"), key=modes.get)
    per = {k: {"us_per_step": round(v * 1e3 / steps, 2), "tokens_per_s": round(N * steps / (v * 1e-3), 1)}
           for k, v in modes.items()}
    step_bytes = decode_step_bytes(w)
    f_us = modes["fused_graph" if graphs else "fused"] * 1e3 / steps
    gbs = step_bytes / (f_us * 1e-6) / 1e9
    kb = decode_kernel_bytes(w)
    kgbs = kb / (k_ms * 1e-3) / 1e9
    return {"workload": w.name, "best": best, "tokens_per_s": per[best]["tokens_per_s"],
            "us_per_step": per[best]["us_per_step"], "modes": per,
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4),
                         "traffic": measured_traffic("decode_fused_b64" if N > 1 else "decode_fused_b1"),
                         "kernel": "gdn_decode_fused (%s; launch duration = loop time / steps)"
                                   % ("graph replay" if graphs else "plain launches"),
                         "bytes_per_launch": step_bytes, "avg_launch_us": round(f_us, 2)},
            "roofline_decode_step": {"bound": "hbm", "achieved": round(kgbs, 1), "peak": HBM_PEAK_GBS,
                                     "unit": "GB/s", "frac": round(kgbs / HBM_PEAK_GBS, 4),
                                     "traffic": measured_traffic("decode_b64" if N > 1 else "decode_b1"),
                                     "kernel": "gdn_decode_step (plain launches, HIP events around each)",
                                     "bytes_per_launch": kb, "avg_launch_us": round(k_ms * 1e3, 2)}}


def cpu_baseline(max_threads: int = 16):
    """The fp64 oracle over the whole prefill workload, in two arms: one
    thread, and the V-heads split over up to `max_threads` threads (the
    heads are independent; each thread runs the oracle's delta rule on its
    share, and ctypes releases the GIL during the C call)."""
    import threading
    import oracle
    w = wl.WORKLOADS[3]
    x = wl.generate(w)
    xf = {}
    for k, v in x.items():
        if k in ("qkv", "z", "b", "a", "conv0"):
            xf[k] = wl.as_f32(v, w.act).astype(np.float64)
        elif v.dtype == np.int32:
            xf[k] = v
        else:
            xf[k] = v.astype(np.float64)
    orc = oracle.default()
    T = int(x["cu_seqlens"][-1])
    Hqk, Hv, d = w.n_qk_heads, w.n_v_heads, w.head_dim
    args = (xf["cu_seqlens"], Hqk, Hv, d, xf["qkv"], xf["z"], xf["b"], xf["a"], xf["conv_w"], xf["dt_bias"],
            xf["A_log"], xf["norm_w"], xf["conv0"], xf["S0"])

    t0 = time.perf_counter()
    orc.layer(*args)
    dt1 = time.perf_counter() - t0

    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    nt = max(1, min(max_threads, avail, Hv))
    groups = [list(range(i, Hv, nt)) for i in range(nt)]
    t0 = time.perf_counter()
    r = orc.conv_gate_prep(xf["cu_seqlens"], Hqk, Hv, d, xf["qkv"], xf["b"], xf["a"], xf["conv_w"], xf["dt_bias"],
                           xf["A_log"], xf["conv0"])
    outs = [None] * nt

    def work(i):
        outs[i] = orc.delta_rule(xf["cu_seqlens"], Hqk, Hv, d, r["q"], r["k"], r["v"], r["beta"], r["g"],
                                 xf["S0"], heads=groups[i])
    th = [threading.Thread(target=work, args=(i,)) for i in range(nt)]
    for t in th:
        t.start()
    for t in th:
        t.join()
    o = np.empty_like(outs[0][0])
    for i, hs in enumerate(groups):
        o[:, hs] = outs[i][0][:, hs]
    orc.gated_rmsnorm(o, xf["z"].reshape(T, Hv, d), xf["norm_w"])
    dtn = time.perf_counter() - t0
    return {"value": round(T / dtn, 2), "unit": "tokens/s", "cores": nt, "kind": "oracle",
            "sample": f"the whole prefill workload once ({T} tokens x {Hv} V-heads), fp64; V-heads split over "
                      f"{nt} threads, {dtn:.2f} s",
            "host": host_identity(), "threads_used": nt,
            "one_thread": {"value": round(T / dt1, 2), "unit": "tokens/s", "cores": 1, "seconds": round(dt1, 2)}}


def host_identity() -> dict:
    """The CPU the oracle ran on: its model name (/proc/cpuinfo), the logical
    CPUs the OS reports and those this process may run on."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.lower().startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = None
    return {"model_name": model, "nproc": os.cpu_count(), "affinity_cpus": avail}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-decode", action="store_true", help="skip the decode workloads")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip timing the oracle")
    ap.add_argument("--no-block", action="store_true", help="skip the block (projections + mixer)")
    ap.add_argument("--no-varlen", action="store_true", help="skip the varlen prefill workload")
    ap.add_argument("--only", choices=["prefill", "decode-b1", "decode-b64", "block"], default=None,
                    help="run one workload only (for counter collection)")
    ap.add_argument("--summarize-rocprof", metavar="DB", default=None,
                    help="print a per-kernel summary of a rocprofv3 results database and exit")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 256 MiB device copy 4 times (reference for HBM byte counters)")
    ap.add_argument("--no-graph", action="store_true", help="decode: plain launches only (for counter runs)")
    ap.add_argument("--write-traffic", nargs=6, metavar="DB", default=None,
                    help="write profiles/traffic.json from six rocprofv3 --pmc databases: FETCH_SIZE and "
                         "WRITE_SIZE runs of --only prefill, --only decode-b64, --only decode-b1 (in that order)")
    a = ap.parse_args()
    if a.summarize_rocprof:
        print(summarize_rocprof(a.summarize_rocprof))
        return
    if a.write_traffic:
        write_traffic(a.write_traffic)
        return
    if a.gpus != 1:
        print(f"bench.py measures one GPU only: the mixer's path here runs on a single MI355X; "
              f"--gpus {a.gpus} is not supported", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    B.load()
    if a.calibrate_copy:
        src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
        src.fill_(1)
        dst = torch.empty_like(src)
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("copy calibration: 4 x 268435456 bytes")
    if a.only in ("decode-b1", "decode-b64"):
        d = bench_decode(2 if a.only == "decode-b1" else 4, graphs=not a.no_graph)
        print(json.dumps(d), flush=True)
        return
    if a.only == "block":
        print(json.dumps(bench_block(a.steps, a.warmup)), flush=True)
        return
    log("prefill workload: T=4096 Hqk=16 Hv=48 bf16")
    pre = bench_prefill(a.steps, a.warmup)
    log(f"prefill: {pre['ms_per_step']:.3f} ms/step ({pre['best']}), core {pre['core_ms'] * 1e3:.1f} us; " + json.dumps(pre['modes']))
    varlen = None
    if not a.no_varlen and a.only is None:
        log("varlen prefill workload: 8 sequences, L ~ U[512, 8192], nonzero states")
        varlen = bench_prefill(a.steps, a.warmup, wid=5, three_call=False)
        log(json.dumps(varlen))
        torch.cuda.empty_cache()
    decode = None
    if not a.no_decode and a.only is None:
        decode = []
        for wid in (2, 4):
            log(f"decode workload {wid}")
            decode.append(bench_decode(wid, graphs=not a.no_graph))
            log(json.dumps(decode[-1]))
    block = None
    if not a.no_block and a.only is None:
        log("block: projections around the mixer")
        block = bench_block(a.steps, a.warmup)
        log(json.dumps(block))
    cpu = None
    if not a.no_cpu_baseline and a.only is None:
        log("cpu baseline (oracle)")
        cpu = cpu_baseline()
    line = {
        "metric": "GDN layer tokens/s: prefill T=4096 & decode step; % HBM/MFMA roofline",
        "value": round(pre["tokens"] * a.steps / (pre["total_ms"] * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
        "ms_per_step": round(pre["ms_per_step"], 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16 in/out, fp32 state and arithmetic", "data": "synthetic (seeded)",
        "config": {"workload": "prefill T=4096, 1 sequence, Hqk=16, Hv=48, d=128, chunk 64, bf16, zero states",
                   "global_batch": 1, "seq_len": pre["tokens"], "parallelism": "single GPU"},
        "prefill_modes": pre["modes"],
        "prefill_best_mode": pre["best"],
        "roofline": pre["roofline"],
        "roofline_fused": pre["roofline_fused"],
        "varlen_prefill": varlen,
        "decode": decode,
        "block": block,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
