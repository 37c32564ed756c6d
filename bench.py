#!/usr/bin/env python3
"""Benchmark of one full-width trie-constrained beam step on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config c3] [--gpus 1]

Workload (default): the LLM-vocabulary SID workload -- B = 32 requests,
K = 512 beams, rows of V = 151,936 bf16 logits, a 10M-SID depth-3 trie with
Zipf-skewed prefixes -- at step 1, where all 512 beams of every request are
live (step 0 reads one row per request).  Every timed step repeats gr_beam_step
from its own input state (gr_beam_rewind flips the double-buffered state back:
no copy, nothing enqueued) on logits already resident in HBM.

Prints one JSON line: logits scored per second (B*K*V per second), the row
kernel's achieved HBM bandwidth against the 8 TB/s peak (from HIP events the
library records around its kernels on the step's stream, in a second pass of
the same steps after the timed one; "frac"), the whole step's (every kernel,
wall time per step of the timed pass, which records no events; "step_frac"),
and the plain CPU oracle timed on a bounded sample of the same step.

    python bench.py --report profiles/step_report.md [--report-configs c1,c2,...]

instead runs every step of every workload (the search itself), timing each
step by repeating it from its own input state: 5 warm-ups, then 30 timed
repetitions (median), HIP events around gr_beam_step on the stream.  Steps
whose logits fit the 256 MB Infinity Cache read a rotating set of copies, so
that their bytes come from HBM.  Writes a markdown table.

    python bench.py --search-report profiles/search_report.md [--report-configs ...]

times whole searches (every step from reset) launched step by step (every step
as the two kernels, and the library's default with the fused step) and as one
gr_beam_search call (one kernel launch, or one graph launch), and writes a
markdown table.

    python bench.py --backward-report profiles/backward_report.md

times the surrogate backward (path extraction and one step's scatter) of each
workload's finished search.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0
METRIC = "beam-step logits scored/s (B·K·V per s) + achieved HBM GB/s vs peak"
# every source of the step's two kernels: a profile taken on other sources is stale
KERNEL_SOURCES = ("trie_constrained_beam_step_amd/csrc/row_kernel.hip",
                  "trie_constrained_beam_step_amd/csrc/select_kernel.hip",
                  "trie_constrained_beam_step_amd/csrc/fused_kernel.hip",
                  "trie_constrained_beam_step_amd/csrc/row_stream.h",
                  "trie_constrained_beam_step_amd/csrc/device_common.h",
                  "trie_constrained_beam_step_amd/csrc/internal.h")
TRAFFIC_FILE = "profiles/row_kernel_{cfg}_traffic.txt"

DESCR = {
    "c1": "tiny SID trie: V=48 fp32, 2,000 SIDs, depth 3",
    "c1x": "tiny SID trie, exhaustive width K=2,000: V=48 fp32, 2,000 SIDs, depth 3",
    "c2": "SID-only vocab: V=768 fp32, 1M SIDs (Zipf level 0), depth 3",
    "c3": "LLM-vocab rows: V=151,936 bf16, 10M SIDs (Zipf levels 0-1), depth 3",
    "c4": "deep wide trie: V=1,280 fp32, 50M SIDs by random branching, depth 5",
    "c5": "unconstrained with EOS: V=50,257 fp32, EOS id 0",
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def rows_kernel_name(stats, cfg):
    """The kernel that streams the rows in a timed step: the fused step's
    (one workgroup per request while its live rows fit one, else the split
    rows kernel) or the row kernel."""
    if not stats.get("fused_requests"):
        return "row_kernel"
    return "fused_step_kernel" if stats["rows_read"] <= 16 * cfg.batch else "fused_rows_kernel"


def read_traffic(cfg_name: str, per_launch_bytes_alg: float):
    """HBM bytes per row-kernel launch from the committed rocprofv3 counter
    summary, if it was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, TRAFFIC_FILE.format(cfg=cfg_name))
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256_16") != kernel_hash():
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def fill_step(X, cfg, t, rows, workers=None):
    """Copy the seeded logits of step t (first `rows` rows of every request)
    into the device tensor X [B, K, V]."""
    import numpy as np
    import torch
    import synth
    for b, blk in synth.iter_step_blocks(cfg, t, rows=rows, workers=workers):
        src = torch.from_numpy(blk.view(np.int16) if blk.dtype == np.uint16 else blk)
        X[b, :rows].copy_(src, non_blocking=False)


def _oracle_kwargs(cfg, trie, t, b, opts):
    lvl = (trie.offsets[t], trie.tokens[t], trie.children[t]) if trie is not None else None
    return dict(eos=cfg.eos, level=lvl, request=b, **opts)


def _oracle_inputs(cfg, trie, ts: int, b: int, opts: dict):
    """Request b's input to the oracle's step ts: its seeded logits and the
    state the oracle's own steps 0..ts-1 leave (untimed)."""
    import numpy as np
    import oracle
    import synth
    K, V, T = cfg.beam, cfg.vocab, cfg.steps
    score = np.full(K, -np.inf, np.float32)
    score[0] = 0
    node = np.full(K, -1, np.int32)
    if trie is not None:
        node[0] = 0
    fin = np.zeros(K, np.uint8)
    seq = np.full((K, T), -1, np.int32)
    for t in range(ts + 1):
        x = synth.step_logits(cfg, t, b, rows=K if t else 1)
        if x.shape[0] < K:
            pad = np.zeros((K, V), x.dtype)
            pad[:x.shape[0]] = x
            x = pad
        if t == ts:
            return x, score, node, fin, seq
        o = oracle.step(x, score, node, fin, seq, t, **_oracle_kwargs(cfg, trie, t, b, opts))
        score, node, fin, seq = o.score, o.node, o.fin, o.seq


def host_cpu() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown CPU"


def cpu_baseline(cfg, trie, ts: int, budget_s: float, max_requests: int, opts: dict):
    """The oracle, as it stands, on requests 0.. of the same step until the
    time budget is used: logits scored per second on one host core."""
    import numpy as np
    import oracle
    K, V = cfg.beam, cfg.vocab
    spent = 0.0
    done = 0
    for b in range(min(cfg.batch, max_requests)):
        x, score, node, fin, seq = _oracle_inputs(cfg, trie, ts, b, opts)
        live = int(np.sum(np.isfinite(score) & (fin == 0)))
        t0 = time.perf_counter()
        oracle.step(x, score, node, fin, seq, ts, **_oracle_kwargs(cfg, trie, ts, b, opts))
        dt = time.perf_counter() - t0
        spent += dt
        done += 1
        log(f"cpu oracle: request {b} step {ts}: {dt:.2f} s ({live} live rows)")
        if spent >= budget_s:
            break
    return dict(value=done * K * V / spent if spent else None, unit="logits/s", cores=1,
                kind="oracle",
                sample=f"{cfg.name} step {ts}, requests 0..{done - 1} of {cfg.batch} "
                       f"({done} x {K} x {V} logits, {spent:.1f} s on one host thread; "
                       f"{host_cpu()}, {os.cpu_count()} logical CPUs)")


def cpu_all_cores(cfg, trie, ts: int, threads: int, opts: dict):
    """The same oracle on every request of the step at once: the requests are
    shared among `threads` host threads (the oracle's C code runs outside
    Python's lock), each prepares its requests' inputs, then all start
    together; logits scored per second of the slowest thread's time."""
    import threading
    import oracle
    B, K, V = cfg.batch, cfg.beam, cfg.vocab
    threads = max(1, min(threads, B))
    shards = [list(range(w, B, threads)) for w in range(threads)]
    barrier = threading.Barrier(threads)
    times = [0.0] * threads
    errors = []

    def work(w):
        try:
            inputs = [(b, _oracle_inputs(cfg, trie, ts, b, opts)) for b in shards[w]]
            barrier.wait()
            t0 = time.perf_counter()
            for b, (x, score, node, fin, seq) in inputs:
                oracle.step(x, score, node, fin, seq, ts, **_oracle_kwargs(cfg, trie, ts, b, opts))
            times[w] = time.perf_counter() - t0
        except Exception as e:  # report it; release the others
            errors.append(e)
            barrier.abort()

    pool = [threading.Thread(target=work, args=(w,)) for w in range(threads)]
    for th in pool:
        th.start()
    for th in pool:
        th.join()
    if errors:
        raise errors[0]
    wall = max(times)
    log(f"cpu oracle, {threads} threads: {B} requests of step {ts} in {wall:.2f} s")
    return dict(value=B * K * V / wall, unit="logits/s", cores=threads,
                sample=f"{cfg.name} step {ts}, all {B} requests ({B} x {K} x {V} logits) on "
                       f"{threads} host threads started together, {wall:.2f} s")


MALL_BYTES = 256 << 20


def penalty_flags(args) -> str:
    f = ""
    if args.alpha:
        f += f" --alpha {args.alpha}"
    if args.min_length:
        f += f" --min-length {args.min_length}"
    if args.banned:
        f += f" --banned {args.banned}"
    if args.norm != "full":
        f += f" --norm {args.norm}"
        if args.norm_range:
            f += f" --norm-range {args.norm_range}"
    return f


def apply_dense(gtrie, cfg, args):
    """--dense-levels: give those trie levels ("all": every level) their dense
    child tables, skipping a level whose table would exceed --dense-max-bytes.
    Returns {level: table bytes} of the levels made dense."""
    if gtrie is None or not args.dense_levels:
        return {}
    import trie_constrained_beam_step_amd as gr
    levels = range(cfg.depth) if args.dense_levels == "all" else \
        [int(v) for v in args.dense_levels.split(",") if v.strip()]
    out = {}
    for level in levels:
        try:
            out[level] = gtrie.densify(level, args.dense_max_bytes)
        except gr.GrError as e:
            if e.status != 6:
                raise
            log(f"level {level} stays CSR: {e}")
    log(f"dense levels (table bytes): {out}")
    return out


def dense_flags(args) -> str:
    if not args.dense_levels:
        return ""
    return f" --dense-levels {args.dense_levels}" + \
        (f" --dense-max-bytes {args.dense_max_bytes}" if args.dense_max_bytes != DENSE_MAX_BYTES else "")


DENSE_MAX_BYTES = 4 << 30


def norm_range(cfg, args):
    """(lo, hi) of range normalisation: --norm-range, else the SID token
    block [sid_base, V) of a trie workload."""
    if args.norm != "range":
        return (0, cfg.vocab)
    if args.norm_range:
        lo, hi = (int(v) for v in args.norm_range.split(","))
        return (lo, hi)
    if not cfg.constrained:
        raise SystemExit("--norm range on an unconstrained workload needs --norm-range LO,HI")
    return (cfg.sid_base, cfg.vocab)


def apply_penalties(beam, args, cfg):
    banned = [int(v) for v in args.banned.split(",") if v.strip()]
    if args.alpha or args.min_length or banned:
        beam.set_penalties(args.alpha, args.min_length, banned)
    if args.norm != "full":
        beam.set_normalization(args.norm, *norm_range(cfg, args))


def row_bytes(cfg, stats, constrained, norm="full", nrange=(0, 0)):
    """What the row kernel must read: every live row once (its range
    [lo, hi) under range normalisation, only its children's logits under
    slice normalisation with a trie), the per-beam state (score, node, flag,
    CSR offset pair: 25 B) and each child token id (4 B).  With no normaliser
    only the candidates' logits are read."""
    isz = 2 if cfg.dtype == "bf16" else 4
    rows = stats["rows_read"]
    width = cfg.vocab if norm == "full" else (nrange[1] - nrange[0] if norm == "range" else None)
    if norm == "slice" and not constrained:
        width = cfg.vocab
    if norm == "none":
        width = None
    b = rows * 25
    if width is None:
        b += stats["candidates"] * isz
    else:
        b += rows * width * isz
    if constrained:
        b += stats["candidates"] * 4
    return b


def algorithmic_bytes(cfg, t, stats, constrained, norm="full", nrange=(0, 0)):
    """What one step must move: the row kernel's reads, each winner's child
    node (4 B, tries), the outputs (16 B per slot) and the sequence reorder
    (B*K*(2t+1)*4 B)."""
    B, K = cfg.batch, cfg.beam
    b = row_bytes(cfg, stats, constrained, norm, nrange) + B * K * 16 + B * K * (2 * t + 1) * 4
    if constrained:
        b += B * K * 4
    return b


def report(args):
    """Per-step table of every workload (see the module docstring)."""
    import numpy as np
    import torch
    import synth
    import trie_constrained_beam_step_amd as gr

    names = args.report_configs.split(",")
    samp = f" --temperature {args.temperature} --seed {args.seed}" if args.temperature > 0 else ""
    samp += penalty_flags(args) + dense_flags(args) + (f" --fused {args.fused}" if args.fused != 1 else "")
    lines = ["# Per-step timing of every workload (one MI355X)"
             + (f", Gumbel top-K sampling at temperature {args.temperature}" if args.temperature > 0 else "")
             + (f", {penalty_flags(args).strip()}" if penalty_flags(args) else "")
             + (f", trie levels read through dense tables ({dense_flags(args).strip()})"
                if args.dense_levels else ""), "",
             "command: `python bench.py --report " + args.report
             + (f" --report-configs {args.report_configs}" if args.report_configs != REPORT_CONFIGS else "")
             + samp + "`", "",
             f"kernel source sha256[:16] (the hash the committed profiles carry): {kernel_hash()}", "",
             "Each step is repeated from its own input state (gr_beam_rewind: no copy), 5 warm-ups then "
             f"{args.report_reps} repetitions, median of HIP events around `gr_beam_step` (both "
             "kernels); row / select kernel times are the library's own events (means). "
             "Logits that fit the 256 MB Infinity Cache rotate over copies so that they come from "
             "HBM. Algorithmic bytes: live rows x V x dtype + 25 B per live row + 4 B per child "
             "token and per winner (tries) + 16 B per output slot + the sequence reorder. "
             "Fraction = algorithmic GB/s / 8,000 GB/s.", "",
             "| workload | step | live rows | candidates | rescanned | step us | row us | select us "
             "| nominal logits/s | live logits/s | alg. GB/s | fraction | row-kernel fraction |",
             "|---|---|---|---|---|---|---|---|---|---|---|---|---|"]
    for name in names:
        cfg = synth.get(name)
        trie = synth.make_trie(cfg) if cfg.constrained else None
        gtrie = gr.Trie.from_csr(trie) if trie is not None else None
        apply_dense(gtrie, cfg, args)
        beam = gr.Beam(cfg.batch, cfg.beam, cfg.vocab, cfg.steps, eos=cfg.eos, dtype=cfg.dtype,
                       trie=gtrie)
        if args.temperature > 0:
            beam.set_sampling(args.temperature, args.seed)
        apply_penalties(beam, args, cfg)
        beam.set_fused(args.fused)
        tdt = torch.int16 if cfg.dtype == "bf16" else torch.float32
        B, K, V = cfg.batch, cfg.beam, cfg.vocab
        step_bytes = B * K * V * (2 if cfg.dtype == "bf16" else 4)
        ncopy = 1 if step_bytes > MALL_BYTES else int(min(64, max(2, (1536 << 20) // step_bytes)))
        Xs = [torch.zeros((B, K, V), dtype=tdt, device="cuda") for _ in range(ncopy)]
        for t in range(cfg.steps):
            fill_step(Xs[0], cfg, t, rows=1 if t == 0 else K)
            for X in Xs[1:]:
                X.copy_(Xs[0])
            torch.cuda.synchronize()

            def one(i):
                if i:  # repeat the step from its own input state (no copy)
                    beam.rewind()
                ev[2 * i].record()
                beam.step(Xs[i % ncopy])
                ev[2 * i + 1].record()

            n = 5 + args.report_reps
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * n)]
            for i in range(5):
                one(i)
            torch.cuda.synchronize()
            stats = beam.last_stats()
            beam.timing_reset()
            beam.timing_enable(True)
            for i in range(5, n):
                one(i)
            torch.cuda.synchronize()
            beam.timing_enable(False)
            tm = beam.timing()
            us = float(np.median([ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(5, n)])) * 1e3
            row_us = tm["row_ms"] / max(1, tm["steps"]) * 1e3
            sel_us = tm["select_ms"] / max(1, tm["steps"]) * 1e3
            nr = norm_range(cfg, args)
            alg = algorithmic_bytes(cfg, t, stats, trie is not None, args.norm, nr)
            row_alg = row_bytes(cfg, stats, trie is not None, args.norm, nr)
            gbs = alg / (us / 1e6) / 1e9
            lines.append(
                f"| {name} | {t} | {stats['rows_read']} | {stats['candidates']} | {stats['rescanned_rows']} "
                f"| {us:.1f} | {row_us:.1f} | {sel_us:.1f} | {B * K * V / (us / 1e6):.3g} "
                f"| {stats['rows_read'] * V / (us / 1e6):.3g} | {gbs:.0f} | {gbs / PEAK_HBM_GBPS:.3f} "
                f"| {row_alg / (row_us / 1e6) / 1e9 / PEAK_HBM_GBPS:.3f} |")
            log(lines[-1])
            # the last repetition has advanced the search (every copy of the
            # step's logits is the same)
        del Xs
        beam.close()
        if gtrie is not None:
            gtrie.close()
        torch.cuda.empty_cache()
    with open(args.report, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(json.dumps({"report": args.report, "rows": len(lines) - 9}), flush=True)


REPORT_CONFIGS = "c1,c1x,c2,c3,c4,c5"


def backward_report(args):
    """The surrogate backward of each workload's finished search: path
    extraction (gr_beam_backward) and one step's scatter, timed with HIP
    events; writes a markdown table."""
    import numpy as np
    import torch
    import synth
    import trie_constrained_beam_step_amd as gr

    names = args.report_configs.split(",")
    lines = ["# Surrogate backward timing of every workload (one MI355X)", "",
             "command: `python bench.py --backward-report " + args.backward_report
             + (f" --report-configs {args.report_configs}" if args.report_configs != REPORT_CONFIGS else "")
             + "`", "",
             f"kernel source sha256[:16] (the hash the committed profiles carry): {kernel_hash()}", "",
             "After the whole search (every step), gr_beam_backward writes every final beam's path "
             "(slot and token per step) and weight; gr_beam_backward_scatter adds the last step's "
             "log-probability gradient into a [B, K, V] fp32 buffer.  HIP events on the stream, 5 "
             f"warm-ups, then {args.report_reps} repetitions (median).  Bytes: the history read "
             "(8 B per step and slot), the paths written (8 B per step and slot), sequences and "
             "scores (4T + 8 B per slot).", "",
             "| workload | steps | B x K | backward us | scatter us (one step) | backward GB/s |",
             "|---|---|---|---|---|---|"]
    for name in names:
        cfg = synth.get(name)
        trie = synth.make_trie(cfg) if cfg.constrained else None
        gtrie = gr.Trie.from_csr(trie) if trie is not None else None
        beam = gr.Beam(cfg.batch, cfg.beam, cfg.vocab, cfg.steps, eos=cfg.eos, dtype=cfg.dtype,
                       trie=gtrie)
        tdt = torch.int16 if cfg.dtype == "bf16" else torch.float32
        B, K, V, T = cfg.batch, cfg.beam, cfg.vocab, cfg.steps
        X = torch.zeros((B, K, V), dtype=tdt, device="cuda")
        for t in range(T):
            fill_step(X, cfg, t, rows=1 if t == 0 else K)
            beam.step(X)
        del X
        torch.cuda.synchronize()
        g = torch.ones((B, K), dtype=torch.float32, device="cuda")
        grad = torch.zeros((B, K, V), dtype=torch.float32, device="cuda")
        res = {}
        for mode in ("backward", "scatter"):
            n = 5 + args.report_reps
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * n)]
            paths = beam.backward(g)
            for i in range(n):
                ev[2 * i].record()
                if mode == "backward":
                    paths = beam.backward(g)
                else:
                    beam.backward_scatter(T - 1, paths, grad)
                ev[2 * i + 1].record()
            torch.cuda.synchronize()
            res[mode] = float(np.median([ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(5, n)])) * 1e3
        nbytes = B * K * (16 * T + 4 * T + 8)
        lines.append(f"| {name} | {T} | {B * K} | {res['backward']:.1f} | {res['scatter']:.1f} "
                     f"| {nbytes / (res['backward'] / 1e6) / 1e9:.0f} |")
        log(lines[-1])
        del grad
        beam.close()
        if gtrie is not None:
            gtrie.close()
        torch.cuda.empty_cache()
    with open(args.backward_report, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(json.dumps({"backward_report": args.backward_report, "rows": len(names)}), flush=True)


def search_report(args):
    """Whole searches (every step from reset) of each workload, launched step
    by step and as one gr_beam_search call; writes a markdown table."""
    import numpy as np
    import torch
    import synth
    import trie_constrained_beam_step_amd as gr

    names = args.report_configs.split(",")
    lines = ["# Whole-search timing of every workload (one MI355X): step by step vs one gr_beam_search call", "",
             "command: `python bench.py --search-report " + args.search_report
             + (f" --report-configs {args.report_configs}" if args.report_configs != REPORT_CONFIGS else "")
             + "`", "",
             f"kernel source sha256[:16] (the hash the committed profiles carry): {kernel_hash()}", "",
             "Each search runs every step from reset (the reset kernel outside the timed region) on "
             "logits already resident in HBM; HIP events around the steps on the stream, 3 + "
             f"(number of logit sets) warm-ups, then {args.report_reps} timed searches (median).  "
             "Workloads whose logits fit the 256 MB Infinity Cache rotate over up to 8 copies of "
             "their logit sets (each copy is its own cached graph).  Eager: one gr_beam_step per "
             "step, the library's default choice (one fused launch for steps whose requests fit one "
             "workgroup, else the row and request kernels); two-kernel: the same with every step as "
             "the two kernels (gr_beam_set_fused 0), the launch pattern before the fused step; "
             "search: one gr_beam_search call for the whole loop (default choice per step): one kernel "
             "launch per eight steps when every step is a fused step of one workgroup per request "
             "(the tiny trie), else one graph launch.",
             "",
             "Host us: the caller's wall time to enqueue one search (Python binding included).", "",
             "| workload | steps | logit sets | two-kernel us / search | eager us / search | search-call us / search "
             "| two-kernel us / step | eager us / step | search-call us / step | eager vs two-kernel | search call vs eager "
             "| eager host us | search-call host us |",
             "|---|---|---|---|---|---|---|---|---|---|---|---|---|"]
    for name in names:
        cfg = synth.get(name)
        trie = synth.make_trie(cfg) if cfg.constrained else None
        gtrie = gr.Trie.from_csr(trie) if trie is not None else None
        beam = gr.Beam(cfg.batch, cfg.beam, cfg.vocab, cfg.steps, eos=cfg.eos, dtype=cfg.dtype,
                       trie=gtrie)
        tdt = torch.int16 if cfg.dtype == "bf16" else torch.float32
        B, K, V, T = cfg.batch, cfg.beam, cfg.vocab, cfg.steps
        total = T * B * K * V * (2 if cfg.dtype == "bf16" else 4)
        nsets = 1 if total > MALL_BYTES else int(min(8, max(2, -(-(1536 << 20) // total))))
        base = []
        for t in range(T):
            X = torch.zeros((B, K, V), dtype=tdt, device="cuda")
            fill_step(X, cfg, t, rows=1 if t == 0 else K)
            base.append(X)
        sets = [base] + [[X.clone() for X in base] for _ in range(nsets - 1)]
        torch.cuda.synchronize()
        res, host = {}, {}
        for mode in ("two_kernel", "eager", "graph"):
            beam.set_fused(0 if mode == "two_kernel" else 1)
            n = 3 + nsets + args.report_reps
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * n)]
            hs = []
            for i in range(n):
                xs = sets[i % nsets]
                beam.reset()
                ev[2 * i].record()
                h0 = time.perf_counter()
                if mode != "graph":
                    for X in xs:
                        beam.step(X)
                else:
                    beam.search(xs)
                hs.append(time.perf_counter() - h0)
                ev[2 * i + 1].record()
            torch.cuda.synchronize()
            w = 3 + nsets
            res[mode] = float(np.median([ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(w, n)])) * 1e3
            host[mode] = float(np.median(hs[w:])) * 1e6
        lines.append(f"| {name} | {T} | {nsets} | {res['two_kernel']:.1f} | {res['eager']:.1f} | {res['graph']:.1f} "
                     f"| {res['two_kernel'] / T:.1f} | {res['eager'] / T:.1f} | {res['graph'] / T:.1f} "
                     f"| {res['two_kernel'] / res['eager']:.2f} | {res['eager'] / res['graph']:.2f} "
                     f"| {host['eager']:.0f} | {host['graph']:.0f} |")
        log(lines[-1])
        del sets, base
        beam.close()
        if gtrie is not None:
            gtrie.close()
        torch.cuda.empty_cache()
    with open(args.search_report, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(json.dumps({"search_report": args.search_report, "rows": len(names)}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="c3", choices=sorted(DESCR))
    ap.add_argument("--step-index", type=int, default=None,
                    help="which beam step to time (default: 1, the first full-width step)")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle time")
    ap.add_argument("--cpu-max-requests", type=int, default=32)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-threads", type=int, default=min(16, os.cpu_count() or 1),
                    help="host threads of the all-cores oracle figure (1: skip it)")
    ap.add_argument("--no-probe", action="store_true")
    ap.add_argument("--gen-workers", type=int, default=None,
                    help="host processes generating logits (default 16, 1 under a profiler)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="only run the plain copy kernel 5 times over BYTES and exit "
                         "(a kernel of known traffic for scaling memory counters)")
    ap.add_argument("--report", default=None, metavar="PATH",
                    help="time every step of every workload and write a markdown table to PATH")
    ap.add_argument("--report-configs", default=REPORT_CONFIGS)
    ap.add_argument("--backward-report", default=None, metavar="PATH",
                    help="time the surrogate backward of every workload's search; write a table")
    ap.add_argument("--search-report", default=None, metavar="PATH",
                    help="time whole searches step by step and as one graph launch; write a table")
    ap.add_argument("--report-reps", type=int, default=30)
    ap.add_argument("--temperature", type=float, default=0.0,
                    help="> 0: time Gumbel top-K sampling at this temperature (default: deterministic)")
    ap.add_argument("--seed", type=int, default=1, help="Philox key of the sampled runs")
    ap.add_argument("--alpha", type=float, default=0.0, help="GNMT length penalty exponent")
    ap.add_argument("--min-length", type=int, default=0, help="minimum hypothesis length for EOS")
    ap.add_argument("--banned", default="", help="comma-separated token ids never emitted")
    ap.add_argument("--norm", default="full", choices=["full", "range", "slice", "none"],
                    help="row normaliser: the full row, a token range, a trie row's children, or "
                         "none (the values are log-probabilities)")
    ap.add_argument("--dense-levels", default="", metavar="all|L0,L1,...",
                    help="trie levels read through dense child tables (gr_trie_densify)")
    ap.add_argument("--dense-max-bytes", type=int, default=DENSE_MAX_BYTES,
                    help="largest dense table per level; wider levels stay CSR")
    ap.add_argument("--norm-range", default="", metavar="LO,HI",
                    help="token range of --norm range (default: the SID token block)")
    ap.add_argument("--fused", type=int, default=1, choices=[0, 1, 2],
                    help="gr_beam_set_fused mode: 0 row and request kernels always, 1 the library's "
                         "default, 2 the fused rows and merge kernel wherever they apply")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: --gpus {args.gpus} is not supported "
              "(the beam step is benchmarked on one GPU's share; see the design notes on sharding)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import synth
    import trie_constrained_beam_step_amd as gr

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.calibrate_copy:
        n = args.calibrate_copy - args.calibrate_copy % 16
        src = torch.ones(n // 4, dtype=torch.int32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            gr.probe_copy(dst, src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n, "launches": 5}), flush=True)
        return
    if args.report:
        report(args)
        return
    if args.search_report:
        search_report(args)
        return
    if args.backward_report:
        backward_report(args)
        return
    workers = args.gen_workers
    if workers is None:
        workers = 1 if "rocprof" in os.environ.get("LD_PRELOAD", "") else None
    cfg = synth.get(args.config)
    ts = 1 if args.step_index is None else args.step_index
    ts = min(ts, cfg.steps - 1)
    t0 = time.time()
    trie = synth.make_trie(cfg) if cfg.constrained else None
    log(f"workload {cfg.name}: trie ready in {time.time() - t0:.1f} s")
    gtrie = gr.Trie.from_csr(trie) if trie is not None else None
    dense = apply_dense(gtrie, cfg, args)
    beam = gr.Beam(cfg.batch, cfg.beam, cfg.vocab, cfg.steps, eos=cfg.eos, dtype=cfg.dtype, trie=gtrie)
    if args.temperature > 0:
        beam.set_sampling(args.temperature, args.seed)
    apply_penalties(beam, args, cfg)
    beam.set_fused(args.fused)
    tdt = torch.int16 if cfg.dtype == "bf16" else torch.float32
    X = torch.zeros((cfg.batch, cfg.beam, cfg.vocab), dtype=tdt, device="cuda")

    # steps before the timed one, on the GPU
    for t in range(ts):
        fill_step(X, cfg, t, rows=1 if t == 0 else cfg.beam, workers=workers)
        beam.step(X)
    torch.cuda.synchronize()
    t1 = time.time()
    fill_step(X, cfg, ts, rows=cfg.beam, workers=workers)
    torch.cuda.synchronize()
    log(f"logits of step {ts} resident ({X.numel() * X.element_size() / 1e9:.2f} GB) in "
        f"{time.time() - t1:.1f} s")

    stepped = [False]

    def one():  # the step, repeated from its own input state (gr_beam_rewind: no copy)
        if stepped[0]:
            beam.rewind()
        beam.step(X)
        stepped[0] = True

    for _ in range(args.warmup):
        one()
    torch.cuda.synchronize()
    stats = beam.last_stats()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        one()
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    # the kernels' split: the same steps again, with the library's timing events
    # (three event records per step: kept out of the timed loop above)
    beam.timing_reset()
    beam.timing_enable(True)
    for _ in range(args.steps):
        one()
    torch.cuda.synchronize()
    beam.timing_enable(False)
    tm = beam.timing()
    ms = el * 1e3 / args.steps
    B, K, V = cfg.batch, cfg.beam, cfg.vocab
    value = B * K * V / (ms / 1e3)
    row_ms = tm["row_ms"] / max(1, tm["steps"])
    sel_ms = tm["select_ms"] / max(1, tm["steps"])
    rows = stats["rows_read"]
    alg_row = row_bytes(cfg, stats, trie is not None, args.norm, norm_range(cfg, args))
    achieved = alg_row / (row_ms / 1e3) / 1e9
    alg_step = algorithmic_bytes(cfg, ts, stats, trie is not None, args.norm, norm_range(cfg, args))
    step_achieved = alg_step / (ms / 1e3) / 1e9
    # the committed counter summary covers the full-row normaliser only
    traffic = read_traffic(cfg.name, alg_row) if args.norm == "full" and not dense else None
    log(f"step {ts}: {ms:.4f} ms/step wall, row kernel {row_ms:.4f} ms, select kernel "
        f"{sel_ms:.4f} ms, stats {stats}")

    probe = None
    if not args.no_probe:
        sink = torch.zeros(65536, dtype=torch.int32, device="cuda")
        n = X.numel() * X.element_size()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        gr.probe_read(X, sink)
        ev0.record()
        for _ in range(5):
            gr.probe_read(X, sink)
        ev1.record()
        torch.cuda.synchronize()
        probe = dict(read_GBps=round(5 * n / (ev0.elapsed_time(ev1) / 1e3) / 1e9, 1), bytes=n)
        del sink

    del X
    beam.close()
    if gtrie is not None:
        gtrie.close()
    torch.cuda.synchronize()

    cpu = None
    if not args.no_cpu_baseline:
        opts = dict(temperature=args.temperature, seed=args.seed, alpha=args.alpha,
                    min_length=args.min_length,
                    banned=[int(v) for v in args.banned.split(",") if v.strip()] or None,
                    norm=args.norm, norm_range=norm_range(cfg, args))
        cpu = cpu_baseline(cfg, trie, ts, args.cpu_budget, args.cpu_max_requests, opts)
        if args.cpu_threads > 1:
            cpu["all_cores"] = cpu_all_cores(cfg, trie, ts, args.cpu_threads, opts)

    out = {
        "metric": METRIC,
        "value": value,
        "unit": "logits/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {
            "workload": f"{cfg.name}: {DESCR[cfg.name]}; B={B}, K={K}; step {ts} "
                        f"({rows} live rows)"
                        + (f"; Gumbel top-K sampling at temperature {args.temperature}"
                           if args.temperature > 0 else "")
                        + (f"; {args.norm} normalisation" if args.norm != "full" else "")
                        + (f"; dense trie levels {sorted(dense)}" if dense else ""),
            "batch": B, "beam": K, "vocab": V, "step": ts,
            "sids": cfg.n_sids if trie is not None else None,
        },
        # the dominant kernel (the row kernel, or the fused step's rows kernel:
        # its algorithmic bytes over its own time), then the whole step (every
        # kernel and the launches)
        "roofline": {
            "bound": "hbm", "kernel": rows_kernel_name(stats, cfg), "achieved": round(achieved, 1),
            "peak": PEAK_HBM_GBPS,
            "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBPS, 4),
            "traffic": traffic,
            "step_achieved": round(step_achieved, 1), "step_frac": round(step_achieved / PEAK_HBM_GBPS, 4),
            "step_bytes": alg_step,
        },
        "cpu_baseline": cpu,
        "kernels": {"row_kernel_ms": round(row_ms, 5), "select_kernel_ms": round(sel_ms, 5),
                    "row_kernel_alg_bytes": alg_row, "source_sha256_16": kernel_hash()},
        "step_stats": stats,
        "probe": probe,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
