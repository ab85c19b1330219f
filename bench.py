#!/usr/bin/env python3
"""Benchmark of the batched verify step on one MI355X.

    python bench.py [--gpus 1] [--steps 200] [--warmup 20]

One step = one specdec_verify call over one batch of the headline workload
(B=64 requests, k=5 drafts, V=128256, bf16 target and draft logits, T=0.8),
with inputs already resident in HBM.  The timed steps rotate over five
distinct seeded input sets (set_index 0..4, each with its own logits, drafts
and uniforms), so that the working set (>= 900 MB) exceeds the 256 MB
Infinity Cache and every step streams its logits from HBM.

Prints one JSON line: verified positions/s (sum over requests of k_b + 1 per
step), the algorithmic HBM bytes per step and their rate against the MI355X
peak (8 TB/s), the roofline of the dominant kernel (the row pass,
verify_rows, timed with events the library records around it inside each
call), the same for the whole call (call_roofline), and the fp64 CPU oracle
timed on the host cores on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0
NGRAM_N_MIN, NGRAM_N_MAX = 1, 4     # suffix lengths the n-gram workload's drafter tries
METRIC = "verified positions/s + HBM GB/s (% of peak), B=64 k=5 V=128256 bf16"
PROFILE_COUNTERS = {"headline": os.path.join(ROOT, "profiles", "verify_headline_counters.txt"),
                    "greedy": os.path.join(ROOT, "profiles", "verify_greedy_counters.txt")}
# Every source whose change can change a kernel or its launch geometry.
KERNEL_SOURCES = ["device_common.h", "internal.h", "slots.h", "verify.hip", "greedy.hip", "sampling.hip",
                  "api.cpp"]


def kernel_digest() -> str:
    """Hash of the kernel sources with comments and blank space removed, so
    that stored counter figures stay valid across comment-only edits."""
    import re
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "speculative_decoding_verification_10_amd", "csrc", f)) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def algorithmic_bytes(wl, num_accepted) -> int:
    """Bytes the step must move: every target row i <= k_b and draft row
    i < k_b once, the final row (pair) of every rejected request once more
    (stochastic path only), plus ids, uniforms and outputs."""
    import numpy as np
    s = 2 if wl.dtype == "bf16" else 4
    k = np.full(wl.B, wl.K) if wl.k_per_req is None else wl.k_per_req.astype(np.int64)
    rows = int(np.sum(k + 1)) + (int(np.sum(k)) if wl.draft is not None else 0)
    rejected = int(np.sum(num_accepted < k))
    reread = 0 if wl.greedy else rejected * (2 if wl.draft is not None else 1)
    small = int(np.sum(k)) * 4 + int(np.sum(k + 1)) * 4 + wl.B * (wl.K + 1) * 4 + wl.B * 4
    return (rows + reread) * wl.V * s + small


def row_pass_bytes(wl) -> int:
    """Bytes the pass over the rows (verify_rows, greedy_rows) must move:
    every target row i <= k_b and draft row i < k_b once (V elements each),
    plus the draft ids the stochastic pass gathers at."""
    import numpy as np
    s = 2 if wl.dtype == "bf16" else 4
    k = np.full(wl.B, wl.K) if wl.k_per_req is None else wl.k_per_req.astype(np.int64)
    rows = int(np.sum(k + 1)) + (int(np.sum(k)) if wl.draft is not None else 0)
    return rows * wl.V * s + (0 if wl.greedy else int(np.sum(k)) * 4)


def read_counters(workload, key):
    """Per-launch HBM bytes measured with rocprofv3 (FETCH_SIZE + WRITE_SIZE,
    scaled by a copy-kernel calibration) for the workloads whose counters are
    stored, if the stored summary was taken on the current kernel sources."""
    path = PROFILE_COUNTERS.get(workload)
    if path is None or not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_digest") != kernel_digest():
        return None
    try:
        return float(vals[key])
    except (KeyError, ValueError):
        return None


def cpu_baseline(wl, name: str, budget_s: float, ngram=None, parents=None, processing=None):
    """The fp64 oracle as it stands, on the host cores, over a bounded
    number of steps of the same workload (for the n-gram workload: the
    oracle drafter, then the oracle greedy verify; for the tree workload
    the oracle tree verify)."""
    import numpy as np
    import oracle
    oracle.default()
    cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    t0 = time.perf_counter()
    n = 0
    pos = 0
    while True:
        if ngram is not None:
            ctx, lens, n_min, n_max = ngram
            drafts, kp = oracle.ngram_propose(ctx, lens, n_min, n_max, wl.K)
            oracle.verify_greedy(wl.target, drafts, kp)
            pos += int(np.sum(kp.astype(np.int64) + 1))
        elif parents is not None:
            oracle.tree_verify_greedy(wl.target, wl.draft_tokens, parents)
            pos += wl.verified_positions()
        elif wl.greedy:
            oracle.verify_greedy(wl.target, wl.draft_tokens, wl.k_per_req)
            pos += wl.verified_positions()
        elif processing is not None:
            oracle.verify_processed(wl.target, wl.draft, wl.draft_tokens, wl.uniforms, wl.temperature,
                                    processing[0], processing[1], wl.k_per_req)
            pos += wl.verified_positions()
        else:
            oracle.verify(wl.target, wl.draft, wl.draft_tokens, wl.uniforms, wl.temperature,
                          wl.k_per_req)
            pos += wl.verified_positions()
        n += 1
        el = time.perf_counter() - t0
        if el >= budget_s or n >= 5000:
            break
    return {"value": pos / el, "unit": "verified positions/s", "cores": cores, "kind": "oracle",
            "sample": "%d full steps of the %s workload (%d verified positions) in %.1f s"
                      % (n, name, pos, el),
            "cpu_model": cpu_model()}


def cpu_model() -> str:
    """The host CPU's model name (first /proc/cpuinfo entry), and the core
    count the OS reports."""
    name = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    name = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return "%s (%d logical cores visible)" % (name, os.cpu_count() or 0)


def default_sets(workload: str) -> int:
    """Input sets to rotate over: enough distinct seeded sets that one
    rotation's logits (>= ~1 GB) exceed the 256 MB Infinity Cache, at most 5;
    one for the workloads whose single step is already larger."""
    per_set_mb = {"tiny": 0.04, "peaked": 4.6, "headline": 180.6, "greedy": 311.2, "ngram": 311.2,
                  "tree": 361.2, "ragged": 3110.0}
    mb = per_set_mb.get(workload, 200.0)
    if mb >= 1000.0:
        return 1
    return 5 if mb < 50.0 else max(2, min(5, int(-(-1000.0 // mb))))


def run_stream(args, torch, sd, dev):
    """The read-stream ceiling: the row pass's load pattern alone
    (specdec_read_stream) over the headline's row bytes (704 rows of
    V = 128256 bf16), rotating over distinct device buffers."""
    import ctypes
    import numpy as np
    lib = sd._lib.load()
    nbytes = 704 * 128256 * 2
    nsets = args.sets if args.sets is not None else 5
    bufs = [torch.randint(-2**15, 2**15, (nbytes // 2,), dtype=torch.int16, device=dev) for _ in range(nsets)]
    sink = torch.zeros(((nbytes // 16 + 1023) // 1024,), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for a, b in evs:
        a.record(stream)
        b.record(stream)
    handles = [(ctypes.c_void_p * 2)(a.cuda_event, b.cuda_event) for a, b in evs]
    for r in range(args.warmup):
        lib.specdec_read_stream(bufs[r % nsets].data_ptr(), nbytes, sink.data_ptr(), stream.cuda_stream, None)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for r in range(args.steps):
        rc = lib.specdec_read_stream(bufs[r % nsets].data_ptr(), nbytes, sink.data_ptr(), stream.cuda_stream,
                                     handles[r])
        if rc != 0:
            raise sd.SpecdecError(rc, "specdec_read_stream")
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = float(np.median([a.elapsed_time(b) for a, b in evs]))
    gbps = nbytes / (ms * 1e-3) / 1e9
    line = {"metric": "HBM read GB/s of the row pass's load pattern alone (read-stream ceiling)",
            "value": round(gbps, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(wall * 1e3 / args.steps, 5), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "u8", "data": "synthetic (random bits, %d distinct device buffers)" % nsets,
            "config": {"workload": "read stream over 180.6 MB (704 rows x 128256 bf16) in 16 KB tiles"},
            "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                         "frac": round(gbps / PEAK_HBM_GBPS, 4), "traffic": None, "kernel": "read_stream",
                         "algorithmic_bytes": nbytes, "launch_ms": round(ms, 5)},
            "cpu_baseline": None}
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--sets", type=int, default=None,
                    help="distinct seeded input sets (set_index 0..N-1), device-resident, rotated over "
                         "(default: enough for ~1 GB of logits per rotation, at most 5)")
    ap.add_argument("--phase-every", type=int, default=1,
                    help="take the kernels' own events on every N-th timed step only (the others run "
                         "the plain entry point, and the step before each sampled one records its "
                         "end-of-call event alone as a fence).  Default 1: every step, which matches "
                         "rocprofv3's kernel durations; sparser sampling leaves the events' cost "
                         "(~1.5 us per step) out of the step time but reads the row kernel ~1 us long. "
                         "Use a value coprime with the set count so that the samples visit every set.")
    ap.add_argument("--workload", default="headline",
                    help="headline (default), tiny, peaked, greedy, ragged, ngram (the n-gram "
                         "drafter over copy-heavy contexts, then the greedy verify of its drafts), "
                         "tree (greedy verification of 21-node draft trees), or stream (the row "
                         "pass's read pattern alone: the device's read-stream ceiling)")
    ap.add_argument("--top-k", type=int, default=None,
                    help="verify on top-k processed distributions (specdec_verify_processed)")
    ap.add_argument("--top-p", type=float, default=None,
                    help="verify on top-p processed distributions (specdec_verify_processed)")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle time")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--graph", action="store_true", help="replay each call from a captured HIP graph")
    ap.add_argument("--telemetry", action="store_true",
                    help="each step also adds the step's per-position acceptance counts "
                         "(specdec_acceptance_counts) to device counters")
    ap.add_argument("--no-phase-events", action="store_true",
                    help="time whole calls only (no events recorded inside specdec_verify)")
    ap.add_argument("--no-events", action="store_true",
                    help="no events at all: the wall clock alone (the roofline and call figures are "
                         "omitted); events cost the host ~15 us per call, which bounds small configs")
    ap.add_argument("--calibration-copy", type=int, default=0, metavar="MIB",
                    help="after the timed steps, copy a MIB-MiB device buffer 10 times (a plain copy "
                         "of known size, for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: this build runs on one GPU only; the verify step shards by request "
              "across GPUs with no exchange, so a multi-GPU figure is N times the 1-GPU one "
              "and is not measured here.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import speculative_decoding_verification_10_amd as sd
    from speculative_decoding_verification_10_amd import workloads
    from tests.gpu_util import dev_logits

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    sd.load(build_if_missing=True)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    if args.workload == "stream":
        run_stream(args, torch, sd, dev)
        return

    # The n-gram workload: the drafter over seeded copy-heavy contexts, then
    # the greedy verify of its drafts against the greedy workload's logits.
    ngram = args.workload == "ngram"
    tree = args.workload == "tree"
    nsets = args.sets if args.sets is not None else default_sets(args.workload)
    nsets = max(1, nsets)

    def make_set(r):
        if tree:
            # Node i's token is "draft position" i; row i + 1 follows node i.
            tw = workloads.tree(set_index=r)
            w = workloads.Workload("tree", tw.B, tw.N, tw.V, tw.dtype, 1.0, True, tw.target, None,
                                   tw.node_tokens, np.zeros((tw.B, tw.N + 1), np.float32),
                                   meta=dict(tw.meta))
            w.meta["parents"] = tw.parents
            return w
        return workloads.make("greedy" if ngram else args.workload, set_index=r)

    # Distinct seeded input sets (set_index 0..nsets-1), generated on the host
    # in parallel, then made device-resident.
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(max_workers=min(nsets, 5)) as pool:
        hosts = list(pool.map(make_set, range(nsets)))
    wl = hosts[0]
    parents_h = wl.meta.get("parents") if tree else None
    if tree:
        parents_d = torch.from_numpy(parents_h).to(dev)
    K = wl.K
    ngram_host = None
    if ngram:
        ctx_h, lens_h = workloads.ngram_contexts(B=wl.B, V=wl.V)
        ngram_host = (ctx_h, lens_h, NGRAM_N_MIN, NGRAM_N_MAX)
        ctx_d = torch.from_numpy(ctx_h).to(dev)
        lens_d = torch.from_numpy(lens_h).to(dev)
    greedy = wl.greedy
    code = 1 if wl.dtype == "bf16" else 0
    processed = (args.top_k is not None or args.top_p is not None) and not greedy
    top_k = int(args.top_k or 0)
    top_p = float(1.0 if args.top_p is None else args.top_p)
    sets = []
    for h in hosts:
        st = {"wl": h, "target": dev_logits(h.target, dev),
              "draft": None if h.draft is None else dev_logits(h.draft, dev)}
        if processed and h.draft is not None:
            # The drafts are drawn from the processed draft rows (the q that
            # drew them), the rows cut at the library's own floors.
            fl = sd.sampling_floors(st["draft"], h.temperature, top_k, top_p).cpu().numpy()
            dv = workloads.stored_as_f32(h.draft)
            rng = np.random.default_rng(2024 + h.meta.get("set_index", 0))
            for b in range(h.B):
                for i in range(h.k_of(b)):
                    row = np.where(dv[b, i] >= fl[b, i], dv[b, i], np.float32(-np.inf))
                    h.draft_tokens[b, i] = workloads.gumbel_draw(row[None], h.temperature, rng)[0]
        if ngram:                  # the drafter writes these every step (shared)
            st["tokens"] = torch.zeros((h.B, K), dtype=torch.int32, device=dev)
            st["kpr"] = torch.zeros((h.B,), dtype=torch.int32, device=dev)
        else:
            st["tokens"] = torch.from_numpy(h.draft_tokens).to(dev)
            st["kpr"] = None if h.k_per_req is None else torch.from_numpy(h.k_per_req).to(dev)
        st["unif"] = torch.from_numpy(h.uniforms).to(dev)
        sets.append(st)
    if ngram:
        for st in sets[1:]:
            st["tokens"], st["kpr"] = sets[0]["tokens"], sets[0]["kpr"]
    tokens, kpr = sets[0]["tokens"], sets[0]["kpr"]
    out = (torch.empty((wl.B, K + 1), dtype=torch.int32, device=dev),
           torch.empty((wl.B,), dtype=torch.int32, device=dev), None)
    if processed:
        nbytes = int(sd._lib.load().specdec_verify_processed_workspace_bytes(wl.B, K, wl.V, code,
                                                                             int(wl.draft is None)))
    elif tree:
        nbytes = int(sd._lib.load().specdec_tree_verify_greedy_workspace_bytes(wl.B, K, wl.V, code))
    elif greedy:
        nbytes = int(sd._lib.load().specdec_verify_greedy_workspace_bytes(wl.B, K, wl.V, code))
    else:
        nbytes = sd._lib.verify_workspace_bytes(wl.B, K, wl.V, code, wl.draft is None)
    ws = sd.Workspace(nbytes, dev)

    # The row pass is timed inside each stochastic call by events that its
    # kernel dispatches take themselves (specdec_verify_timed).
    phase = not args.graph and not args.no_phase_events and not args.no_events
    phase_ev = None
    handles = None

    # The timed steps call the C ABI directly with argument lists built once
    # (the binding's per-call checks cost more host time than the GPU work of
    # small calls); the first warm-up call goes through the checked binding.
    import ctypes
    lib = sd._lib.load()
    stream = torch.cuda.current_stream(dev)
    ptr = lambda t: None if t is None else t.data_ptr()
    cargs = []
    for st in sets:
        t_, u_, k_ = st["tokens"], st["unif"], st["kpr"]
        if tree:
            cargs.append((st["target"].data_ptr(), code, t_.data_ptr(), parents_d.data_ptr(), None,
                          wl.B, K, wl.V, out[0].data_ptr(), None, out[1].data_ptr(), ws.ptr(),
                          ws.nbytes, stream.cuda_stream))
        elif greedy:
            cargs.append((st["target"].data_ptr(), code, t_.data_ptr(), ptr(k_), wl.B, K, wl.V,
                          out[0].data_ptr(), out[1].data_ptr(), None, ws.ptr(), ws.nbytes,
                          stream.cuda_stream))
        elif processed:
            cargs.append((st["target"].data_ptr(), ptr(st["draft"]), code, t_.data_ptr(), ptr(k_),
                          u_.data_ptr(), float(wl.temperature), top_k, top_p, wl.B, K, wl.V,
                          out[0].data_ptr(), out[1].data_ptr(), None, ws.ptr(), ws.nbytes,
                          stream.cuda_stream))
        else:
            cargs.append((st["target"].data_ptr(), ptr(st["draft"]), code, t_.data_ptr(), ptr(k_),
                          u_.data_ptr(), float(wl.temperature), wl.B, K, wl.V, out[0].data_ptr(),
                          out[1].data_ptr(), None, ws.ptr(), ws.nbytes, stream.cuda_stream))

    counters = torch.zeros((3, max(K, 1)), dtype=torch.int64, device=dev) if args.telemetry else None

    def step(r, handle=None):
        a = cargs[r % len(cargs)]
        st = sets[r % len(sets)]
        if ngram:
            rc = lib.specdec_ngram_propose(ctx_d.data_ptr(), lens_d.data_ptr(), wl.B, ctx_d.shape[1],
                                           NGRAM_N_MIN, NGRAM_N_MAX, K, tokens.data_ptr(), kpr.data_ptr(),
                                           stream.cuda_stream)
            if rc != 0:
                raise sd.SpecdecError(rc, "bench drafter")
        if tree:
            fn, fn_timed = lib.specdec_tree_verify_greedy, lib.specdec_tree_verify_greedy_timed
        elif greedy:
            fn, fn_timed = lib.specdec_verify_greedy, lib.specdec_verify_greedy_timed
        elif processed:
            fn, fn_timed = lib.specdec_verify_processed, lib.specdec_verify_processed_timed
        else:
            fn, fn_timed = lib.specdec_verify, lib.specdec_verify_timed
        rc = fn_timed(*a, handle) if handle is not None else fn(*a)
        if rc == 0 and counters is not None:
            rc = lib.specdec_acceptance_counts(out[1].data_ptr(), ptr(st["kpr"]), wl.B, K,
                                               counters.data_ptr(), stream.cuda_stream)
        if rc != 0:
            raise sd.SpecdecError(rc, "bench step")

    def checked_step(r):
        st = sets[r % len(sets)]
        if ngram:
            sd.ngram_propose(ctx_d, lens_d, NGRAM_N_MIN, NGRAM_N_MAX, K, out=(tokens, kpr))
        if tree:
            sd.tree_verify_greedy(st["target"], st["tokens"], parents_d, workspace=ws, out=out)
        elif greedy:
            sd.verify_greedy(st["target"], st["tokens"], k_per_req=st["kpr"], workspace=ws, out=out)
        else:
            sd.verify(st["target"], st["draft"], st["tokens"], st["unif"], wl.temperature,
                      k_per_req=st["kpr"], workspace=ws, out=out, top_k=args.top_k if processed else None,
                      top_p=args.top_p if processed else None)

    # Each set once through the checked binding: its accepted counts give its
    # rejected requests and so its algorithmic bytes.
    set_nacc = []
    for r in range(len(sets)):
        checked_step(r)
        torch.cuda.synchronize()
        set_nacc.append(out[1].cpu().numpy().copy())
    if ngram:                      # the step's drafted positions come from the drafter
        for st in sets:
            st["wl"].k_per_req = kpr.cpu().numpy()
    graphs = None
    if args.graph:
        # Captured through the binding, which launches on the capture stream.
        graphs = []
        for r in range(len(sets)):
            checked_step(r)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                checked_step(r)
            graphs.append(g)
        torch.cuda.synchronize()

    def run(r, handle=None):
        if graphs is not None:
            graphs[r % len(graphs)].replay()
        else:
            step(r, handle)

    for r in range(args.warmup):
        run(r)
    torch.cuda.synchronize()
    nacc = set_nacc[0]

    # The kernels' own events (or, with --no-phase-events / --graph, stream
    # events around the call) are taken on every phase_every-th timed step
    # only: recording them costs the GPU several microseconds between kernels,
    # which the other steps -- and so the wall-clock figure -- do not pay.
    # A sampled step's start event is only exact when the step before it
    # also took an event at its end (otherwise it also counts the previous
    # kernel's tail), so that step records its end-of-call event alone.
    every = max(1, args.phase_every)
    sampled = [] if args.no_events else [r for r in range(args.steps) if r % every == every - 1]
    fences = [r - 1 for r in sampled if r >= 1 and (r - 1) not in sampled]
    if phase:
        nev = 3
        phase_ev = {r: [torch.cuda.Event(enable_timing=True) for _ in range(nev)] for r in sampled}
        fence_ev = {r: torch.cuda.Event(enable_timing=True) for r in fences}
        for e in list(fence_ev.values()) + [e for evs in phase_ev.values() for e in evs]:
            e.record(stream)              # torch creates an event at its first record
        handles = {r: (ctypes.c_void_p * nev)(*[e.cuda_event for e in evs]) for r, evs in phase_ev.items()}
        handles.update({r: (ctypes.c_void_p * nev)(None, None, e.cuda_event) for r, e in fence_ev.items()})
        starts = ends = None
    else:
        handles = {}
        starts = {r: torch.cuda.Event(enable_timing=True) for r in sampled}
        ends = {r: torch.cuda.Event(enable_timing=True) for r in sampled}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for r in range(args.steps):
        if starts is not None and r in starts:
            starts[r].record(stream)
        run(r, handles.get(r))
        if ends is not None and r in ends:
            ends[r].record(stream)
    host = time.perf_counter() - t0       # time to enqueue the steps
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    # The same number of steps again without any event (events cost the host
    # ~15 us per call, which bounds small configs): reported beside the
    # timed figures, which keep the events that the roofline is measured by.
    no_event_ms = None
    if sampled:
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for r in range(args.steps):
            run(r, None)
        torch.cuda.synchronize()
        no_event_ms = (time.perf_counter() - t1) * 1e3 / args.steps
    rows_ms = None
    if phase:
        rows_ms = float(np.median([e[0].elapsed_time(e[1]) for e in phase_ev.values()]))
        call_ms = float(np.median([e[0].elapsed_time(e[-1]) for e in phase_ev.values()]))
        per_launch_ms = call_ms
    elif sampled:
        per_launch_ms = float(np.median([starts[r].elapsed_time(ends[r]) for r in sampled]))
    else:
        per_launch_ms = None

    # Per set: verified positions and algorithmic bytes; the timed steps
    # visit set r % nsets.
    set_pos = [st["wl"].verified_positions() for st in sets]
    set_alg = [algorithmic_bytes(st["wl"], set_nacc[i]) for i, st in enumerate(sets)]
    set_rows = [row_pass_bytes(st["wl"]) for st in sets]
    if tree:
        set_alg = [a + wl.B * K * 4 for a in set_alg]      # the parent links
    drafter = None
    if ngram:
        # The drafter reads every context token once and writes the drafts.
        dbytes = int(np.sum(lens_h.astype(np.int64))) * 4 + wl.B * 4 + wl.B * (K + 1) * 4
        set_alg = [a + dbytes for a in set_alg]
    visits = [r % len(sets) for r in range(args.steps)]
    positions_total = sum(set_pos[i] for i in visits)
    alg_total = sum(set_alg[i] for i in visits)
    positions = positions_total / args.steps
    alg = alg_total / args.steps
    sampled_sets = [r % len(sets) for r in sampled] or list(range(len(sets)))
    alg_sampled = float(np.mean([set_alg[i] for i in sampled_sets]))
    rows_sampled = float(np.mean([set_rows[i] for i in sampled_sets]))
    # Stored counter figures belong to the unprocessed step's kernels.
    counters_key = args.workload + ("-processed" if processed else "")
    if ngram:
        n_dr = 200
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n_dr):
            lib.specdec_ngram_propose(ctx_d.data_ptr(), lens_d.data_ptr(), wl.B, ctx_d.shape[1],
                                      NGRAM_N_MIN, NGRAM_N_MAX, K, tokens.data_ptr(), kpr.data_ptr(),
                                      stream.cuda_stream)
        e1.record(stream)
        e1.synchronize()
        d_ms = e0.elapsed_time(e1) / n_dr
        drafter = {"kernel": "ngram_propose", "algorithmic_bytes": dbytes,
                   "us_per_call": round(d_ms * 1e3, 3),
                   "achieved_gbps": round(dbytes / (d_ms * 1e-3) / 1e9, 1),
                   "timing": "%d back-to-back calls between two stream events" % n_dr,
                   "drafted_requests": int(np.count_nonzero(wl.k_per_req)),
                   "n_min": NGRAM_N_MIN, "n_max": NGRAM_N_MAX}
    value = positions_total / wall
    gbps = alg_total / wall / 1e9
    achieved = None if per_launch_ms is None else alg_sampled / (per_launch_ms * 1e-3) / 1e9
    if phase:
        # The dominant kernel: the pass over the rows (all of the greedy
        # path's bytes, ~85% of the stochastic path's).
        rb = int(round(rows_sampled))
        rows_gbps = rb / (rows_ms * 1e-3) / 1e9
        roofline = {"bound": "hbm", "achieved": round(rows_gbps, 1), "peak": PEAK_HBM_GBPS,
                    "unit": "GB/s", "frac": round(rows_gbps / PEAK_HBM_GBPS, 4),
                    "traffic": read_counters(counters_key, "greedy_rows_hbm_bytes_per_launch" if greedy
                                             else "verify_rows_hbm_bytes_per_launch"),
                    "kernel": ("greedy_rows" if greedy else "floor_rows" if processed else "verify_rows"),
                    "algorithmic_bytes": rb,
                    "launch_ms": round(rows_ms, 5)}
        call = {"achieved": round(alg_sampled / (call_ms * 1e-3) / 1e9, 1),
                "frac": round(alg_sampled / (call_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
                "traffic": read_counters(counters_key, "hbm_bytes_per_launch"),
                "algorithmic_bytes": int(round(alg_sampled)),
                "launch_ms": round(call_ms, 5),
                "kernels": ("greedy_rows, tree_decisions" if tree else
                            "greedy_rows, greedy_decisions" if greedy else
                            "floor_rows, [verify_decide,] verify_final" if processed
                            else "verify_rows, [verify_decide,] verify_final")}
    elif per_launch_ms is None:
        roofline = None                   # --no-events: no per-launch figures
        call = None
    else:
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS,
                    "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBPS, 4),
                    "traffic": read_counters(counters_key, "greedy_rows_hbm_bytes_per_launch" if greedy
                                             else "hbm_bytes_per_launch"),
                    "kernel": ("greedy_rows" if greedy else
                               "specdec_verify call (verify_rows, [verify_decide,] verify_final)"),
                    "algorithmic_bytes": int(round(alg_sampled)), "launch_ms": round(per_launch_ms, 5)}
        call = None
    if processed:
        metric = ("verified positions/s + HBM GB/s (%% of peak), %s B=%d k=%d V=%d %s, top-k %d, top-p %g"
                  % (args.workload, wl.B, K, wl.V, wl.dtype, top_k, top_p))
    elif tree:
        metric = ("verified positions/s (tree nodes + 1 per request) + HBM GB/s (%% of peak), "
                  "tree B=%d nodes=%d V=%d %s" % (wl.B, K, wl.V, wl.dtype))
    else:
        metric = METRIC if args.workload == "headline" else (
            "verified positions/s + HBM GB/s (%% of peak), %s B=%d k=%d V=%d %s"
            % (args.workload, wl.B, K, wl.V, wl.dtype))
    line = {
        "metric": metric,
        "value": round(value, 1),
        "unit": "verified positions/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "host_enqueue_ms_per_step": round(host * 1e3 / args.steps, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": ("synthetic (seeded; inputs resident in HBM; %d distinct input sets, set_index 0..%d, "
                 "rotated)" % (len(sets), len(sets) - 1)),
        "config": {"workload": ("tree verify B=%d nodes=%d (branching %s) V=%d %s"
                                % (wl.B, K, ",".join(map(str, wl.meta["branching"])), wl.V, wl.dtype)
                                if tree else
                                "%s verify B=%d k=%d V=%d %s T=%g%s" % (
                                    args.workload, wl.B, K, wl.V, wl.dtype, wl.temperature,
                                    ", top-k %d, top-p %g" % (top_k, top_p) if processed else "")),
                   "B": wl.B, "k": K, "V": wl.V, "temperature": wl.temperature,
                   "top_k": top_k if processed else None, "top_p": top_p if processed else None,
                   "graph_replay": bool(args.graph)},
        "hbm_gbps": round(gbps, 1),
        "hbm_pct_peak": round(100.0 * gbps / PEAK_HBM_GBPS, 2),
        "algorithmic_bytes_per_step": int(round(alg)),
        "verified_positions_per_step": round(positions, 2),
        "bytes_per_verified_position": {
            "algorithmic": round(alg / positions, 1),
            "counters": (None if (call or roofline or {}).get("traffic") is None else
                         round((call or roofline)["traffic"] / set_pos[0], 1)),
            "note": "counters: rocprofv3 FETCH_SIZE + WRITE_SIZE per call (mean over the profiled calls), "
                    "scaled by the copy calibration, over the verified positions of one call"},
        "rejected_requests": (None if tree else
                              [int(np.sum(n_ < (st["wl"].K if st["wl"].k_per_req is None
                                                else st["wl"].k_per_req)))
                               for n_, st in zip(set_nacc, sets)]),
        "phase_events": {"every": every, "sampled_steps": len(sampled),
                         "fence_steps": len(fences) if phase else 0},
        "without_events": (None if no_event_ms is None else
                           {"ms_per_step": round(no_event_ms, 5),
                            "value": round(positions_total / args.steps / (no_event_ms * 1e-3), 1),
                            "note": "the same steps again right after the timed ones, with no event"}),
        "roofline": roofline,
        "cpu_baseline": None,
    }
    if call is not None:
        line["call_roofline"] = call
    if tree:
        nacc = set_nacc[0]
        line["tree"] = {"accepted_path_lengths": np.bincount(nacc, minlength=4).tolist(),
                        "mean_accepted": round(float(np.mean(nacc)), 4)}
    if drafter is not None:
        line["drafter"] = drafter
    if counters is not None:
        # The draft length the step's own acceptance counters suggest at the
        # worked example's draft cost ratio (c = 0.05).
        k_next, a_test, a_draft, sp = sd.choose_k(counters, 0.05, 1, max(K, 1))
        line["telemetry"] = {"kernel": "acceptance_counts", "alpha_test": round(a_test, 4),
                             "alpha_draft": round(a_draft, 4), "chosen_k_at_c_0.05": k_next,
                             "predicted_speedup": round(sp, 3)}
    if args.calibration_copy > 0:
        n = args.calibration_copy << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(10):
            dst.copy_(src)
        torch.cuda.synchronize()
        line["calibration_copy_bytes"] = n
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(wl, args.workload, args.cpu_budget, ngram_host, parents_h,
                                            (top_k, top_p) if processed else None)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
