"""Benchmark: blocks/s of the whole per-block path on one GPU.

One step = one block for every sequence of the batch: herald_select_merged
(merged-query full-cache scan + top-C), herald_refine_topk, herald_gather_kv,
then herald_block_attn for each of the T denoising steps. Inputs are seeded
synthetic tensors already resident in HBM. To keep the 256 MiB Infinity Cache
from serving the scan, the K/V cache is replicated until the replicas span at
least 512 MiB and consecutive steps rotate through them.

Prints one JSON line. The K timed steps run REPEATS times; `value` and
`ms_per_step` are the median run. `roofline` is for the kernel that takes the most
time per step, timed with HIP events recorded by the library around that kernel on
the stream it runs on. `fractions` puts the whole step against its roofline time
(`block`), the scan against HBM peak and attention against MFMA peak.
`cpu_baseline` times the CPU oracle on a bounded sample: on every core of the host
share (one worker process per core) and on one core, with the CPU model.

`--method offload` runs the speculative two-stream pipeline over consecutive blocks
with their own seeded inputs: block i's candidates come from block i-1's merged
queries (searched while block i-1 denoises), refined with block i's own queries, and
its subset is fetched by the GPU reading a pinned host pool (herald_gather_kv,
src_is_host = 2) into one of two sparse pools; `--method pipelined` runs the same
schedule with the cache in HBM as one captured graph. Both report the pipelined rate,
the same calls on one stream (checked bit for bit) and the fetch rate.
`--method compressed` runs the HERALD path with the selection over compressed keys
(herald_select_compressed; --ksize / --stride windows, the compressed cache built
once per replica before timing, as a serving system maintains it when the cache
grows). `--method dense` and `--method mage` time the two exact layer baselines instead,
through the same calls: dense attention over the whole cache for the T steps
(herald_block_attn with topk = L, the cache gathered once into the subset layout
before timing), and MAGE-exact selection (herald_refine_topk with every key a
candidate, then gather and the T steps over the top-K). Both need sequences of one
length. They print the same record with "method" set and `vs_herald` = their
blocks/s over the HERALD path's, measured in the same process.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "blocks/sec (select+refine+T-step sparse attn) at L=32K; % HBM/MFMA peak"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
FP32_PEAK_TFLOPS = 157.3
REPEATS = 5  # timed runs of K steps; value and per-launch figures are their medians


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_work(wl, lengths):
    """Algorithmic bytes / flops per launch of each kernel that gets a roofline."""
    esz = 2 if wl.dtype == "bf16" else 4
    total = int(sum(lengths))
    nk = wl.topk + wl.B
    return {
        # the merged-query scan streams the whole K cache once
        "scan": ("hbm", total * wl.Hkv * wl.d * esz),
        # refine: the two refine kernels each contract B*G query rows with C candidate rows
        "refine_stats": ("mfma", 2.0 * wl.nseq * wl.Hq * wl.B * wl.C * wl.d),
        "refine_scores": ("mfma", 2.0 * wl.nseq * wl.Hq * wl.B * wl.C * wl.d),
        # gather reads and writes topk rows of K and V
        "gather": ("hbm", 2 * 2 * wl.nseq * wl.Hkv * wl.topk * wl.d * esz),
        # attention (one call): 4*Hq*B*(topk+B)*d flop over the subset K/V, the step's
        # queries, in-block keys/values and outputs, i.e. ~114 flop/byte at G=4, below
        # MI355X's ridge (2.5 PFLOP/s / 8 TB/s = 312 flop/byte): bound by memory
        "attn": ("hbm", esz * wl.nseq * (2 * wl.Hkv * wl.topk * wl.d + 2 * wl.B * wl.Hq * wl.d
                                         + 2 * wl.B * wl.Hkv * wl.d)),
    }


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed counter runs, if the kernel is unchanged since."""
    from block_diffusion_sparse_herald_amd.profiling import KERNELS, sources_digest

    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}.json")
    if not os.path.exists(path) or kernel not in KERNELS:
        return None
    digest = sources_digest(KERNELS[kernel][1])
    for e in json.load(open(path)).get("entries", []):
        if e["kernel"] == kernel and e["sources_sha256"] == digest:
            return e["bytes_per_launch"]
    return None


# ---------------------------------------------------------------- CPU oracle baseline
#
# The oracle (numpy fp64, one BLAS thread per worker) on whole blocks of sequence 0.
# Worker processes are forked right after the inputs are drawn, before this process
# touches the GPU, and inherit sequence 0's arrays; they sit idle while the GPU runs.

_CPU_ARGS = None  # (args tuple for herald_block, C, topk, scale), set before the fork


def _cpu_init():
    from threadpoolctl import threadpool_limits

    threadpool_limits(limits=1)


def _cpu_blocks(budget_s: float):
    """Whole blocks until budget_s has passed: (blocks, seconds)."""
    import oracle.herald_oracle as orc

    args, C, topk, scale = _CPU_ARGS
    n, t0 = 0, time.perf_counter()
    while True:
        orc.herald_block(*args, C, topk, scale)
        n += 1
        if time.perf_counter() - t0 >= budget_s:
            return n, time.perf_counter() - t0


def host_cores() -> int:
    """Cores this process may use, capped at 16 (a one-GPU share of the host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_prepare(wl, batch):
    """Sets the oracle's inputs (sequence 0, widened to fp64) and forks the worker pool."""
    global _CPU_ARGS
    import multiprocessing as mp

    import numpy as np

    import oracle.herald_oracle as orc
    from block_diffusion_sparse_herald_amd.inputs import bf16_bits_to_f32

    def w(a):
        return (bf16_bits_to_f32(a) if a.dtype == np.uint16 else a).astype(np.float64)

    a, e = int(batch.seq_start[0]), int(batch.seq_start[1])
    _CPU_ARGS = ((w(batch.q0[0]), w(batch.k_cache[a:e]), w(batch.v_cache[a:e]), w(batch.q_steps[:, 0]),
                  w(batch.kb_steps[:, 0]), w(batch.vb_steps[:, 0])), wl.C, wl.topk, orc.default_scale(wl.d))
    cores = host_cores()
    return mp.get_context("fork").Pool(cores, initializer=_cpu_init), cores, e - a


def cpu_baseline(wl, pool, cores: int, L0: int, budget_s: float):
    """Oracle blocks/s on every core (one block stream per worker process) and on one core."""
    one_n, one_t = pool.apply(_cpu_blocks, (budget_s,))
    t0 = time.perf_counter()
    res = pool.map(_cpu_blocks, [budget_s] * cores, chunksize=1)
    wall = time.perf_counter() - t0
    n_all = sum(n for n, _ in res)
    what = f"whole blocks of sequence 0 (L={L0}, select+refine+gather+{wl.T} attention steps), numpy fp64"
    return {"value": n_all / wall, "unit": "blocks/s", "cores": cores, "kind": "oracle",
            "sample": f"{n_all} {what}, {cores} worker processes x 1 thread, {wall:.1f} s wall",
            "one_core": {"value": one_n / one_t, "unit": "blocks/s", "cores": 1,
                         "sample": f"{one_n} {what}, 1 thread, {one_t:.1f} s"},
            "nproc": os.cpu_count(), "cpu_model": cpu_model(),
            "note": "the oracle as written (plain fp64 numpy), not a tuned CPU implementation"}


def block_roofline(wl, lengths, esz: int, mfma_peak: float) -> dict:
    """Roofline time of one step (one block per sequence): the scan streams the K cache;
    refine contracts B*G query rows with C candidate rows; the gather reads and writes the
    subset; each of the T attention steps streams the subset and the step's tensors. Each
    term is the larger of its bytes / HBM peak and flops / MFMA peak."""
    bw = HBM_PEAK_GBS * 1e9
    fl = mfma_peak * 1e12
    n = wl.nseq
    scan_b = int(sum(lengths)) * wl.Hkv * wl.d * esz
    ref_b = n * (wl.Hkv * wl.C * wl.d * esz + wl.B * wl.Hq * wl.d * esz)
    ref_f = 2.0 * n * wl.B * wl.Hq * wl.C * wl.d
    gat_b = 4 * n * wl.Hkv * wl.topk * wl.d * esz
    att_b = esz * n * (2 * wl.Hkv * wl.topk * wl.d + 2 * wl.B * wl.Hq * wl.d + 2 * wl.B * wl.Hkv * wl.d)
    att_f = 4.0 * n * wl.B * wl.Hq * (wl.topk + wl.B) * wl.d
    t = scan_b / bw + max(ref_b / bw, ref_f / fl) + gat_b / bw + wl.T * max(att_b / bw, att_f / fl)
    return {"t_roof_us": round(t * 1e6, 3), "blocks_per_s": round(n / t, 1),
            "terms_us": {"scan": round(scan_b / bw * 1e6, 3), "refine": round(max(ref_b / bw, ref_f / fl) * 1e6, 3),
                         "gather": round(gat_b / bw * 1e6, 3),
                         "attention": round(wl.T * max(att_b / bw, att_f / fl) * 1e6, 3)}}


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="gqa32x8_L32768_b1")
    ap.add_argument("--cpu-budget", type=float, default=8.0,
                    help="seconds of oracle time per cpu_baseline leg (all cores, then one core)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--eager", action="store_true", help="launch every step directly instead of replaying graphs")
    ap.add_argument("--method", choices=["herald", "pipelined", "offload", "compressed", "dense", "mage"],
                    default="herald",
                    help="the HERALD path (default); the next block's selection overlapped with the current "
                         "block's steps (pipelined: cache in HBM, offload: subset from a pinned host pool); "
                         "compressed-key selection; or an exact layer baseline")
    ap.add_argument("--overlap-refine", action="store_true",
                    help="offload/pipelined: run a block's refine and fetch while the previous block denoises "
                         "(its queries taken as given) instead of after it")
    ap.add_argument("--ksize", type=int, default=32, help="compressed-key window (tokens), --method compressed")
    ap.add_argument("--stride", type=int, default=16, help="compressed-key block (tokens), --method compressed")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported (the per-block path needs no "
              f"cross-GPU exchange, so N GPUs would each run this same single-GPU workload)", file=sys.stderr)
        return 2

    import numpy as np

    from block_diffusion_sparse_herald_amd import herald as H
    from block_diffusion_sparse_herald_amd.hiprt import DevArray, Hip, HipError
    from block_diffusion_sparse_herald_amd.inputs import WORKLOADS, make_batch
    from block_diffusion_sparse_herald_amd.runner import BlockRunner

    wl = WORKLOADS[args.workload]
    log(f"[bench] workload {wl.name}: generating inputs")
    batch = make_batch(wl)
    # the CPU oracle's worker processes are forked now, before anything touches the GPU
    pool = None
    if args.method == "herald" and not args.no_cpu_baseline:
        pool, cores, L0 = cpu_prepare(wl, batch)
    # Device memory, streams, events and graphs come straight from the HIP runtime the
    # library links (no PyTorch in this process).
    hip = Hip()
    H.load()
    dev = {n: DevArray.from_host(hip, getattr(batch, n))
           for n in ["q0", "k_cache", "v_cache", "q_steps", "kb_steps", "vb_steps"]}
    cache_bytes = dev["k_cache"].nbytes + dev["v_cache"].nbytes
    replicas = max(1, math.ceil(512 * 2**20 / cache_bytes))
    kv = [(dev["k_cache"], dev["v_cache"])] + [(dev["k_cache"].clone(), dev["v_cache"].clone())
                                              for _ in range(replicas - 1)]
    seq_dev = DevArray.from_host(hip, batch.seq_start)
    r = BlockRunner(batch.seq_start, wl.B, wl.Hq, wl.Hkv, wl.d, wl.C, wl.topk, wl.dtype,
                    alloc=lambda shape, dt, zero=False, contiguous=False: DevArray(hip, shape, dt, zero, contiguous),
                    seq_start_dev=seq_dev)
    q0 = dev["q0"]
    qs, kbs, vbs = ([dev[n].offset(t) for t in range(wl.T)] for n in ("q_steps", "kb_steps", "vb_steps"))
    stream = hip.stream()
    placement = None
    if args.method == "herald":
        r.select(q0, kv[0][0], stream=stream)  # real subsets in the pools for the placement timing
        r.refine(q0, kv[0][0], stream=stream)
        r.gather(kv[0][0], kv[0][1], stream=stream)
        placement = place_attn_workspace(hip, r, stream, qs, kbs, vbs, wl.T)
    if placement:
        log(f"[bench] attention workspace at +{placement['offsets_mib']} MiB: {placement['us_per_call']} us per call; "
            f"using +{placement['chosen_mib']} MiB")
    if args.method in ("offload", "pipelined"):
        return offload_pipeline(args, hip, wl, batch, kv, seq_dev, r, q0, qs, kbs, vbs, stream)
    if args.method != "herald":
        return other_method(args, hip, wl, batch, kv, seq_dev, r, q0, qs, kbs, vbs, stream)

    call_of = {"scan": "select", "score_hist": "select", "radix": "select", "emit": "select",
               "refine_stats": "refine", "refine_scores": "refine", "refine_select": "refine",
               "gather": "gather", "attn": "attn", "attn_combine": "attn"}

    def step(i, timed=None, events=None, capturing=False):
        """One block per sequence. With `timed`, `events` bracket that kernel in one launch of
        the step; with timed == "attn_op" they bracket the whole T-step attention phase
        (T attention calls back to back)."""
        k, v = kv[i % replicas]

        def run(call, fn, last=True):
            on = timed is not None and timed != "attn_op" and call_of[timed] == call and last
            if on:
                H.herald_set_kernel_events(timed, *events)
            try:
                fn()
            finally:
                if on:
                    H.herald_set_kernel_events(timed, None, None)

        run("select", lambda: r.select(q0, k, stream=stream))
        run("refine", lambda: r.refine(q0, k, stream=stream))
        run("gather", lambda: r.gather(k, v, stream=stream))
        if timed == "attn_op":
            hip.record(events[0], stream, external=capturing)
        for t in range(wl.T):
            run("attn", lambda: r.attn(qs[t], kbs[t], vbs[t], stream=stream), last=t == wl.T - 1)
        if timed == "attn_op":
            hip.record(events[1], stream, external=capturing)

    log(f"[bench] {replicas} K/V replica(s); warm-up {args.warmup} steps")
    for i in range(args.warmup):
        step(i)
    hip.sync()
    launches = {"scan": 1, "score_hist": 1, "radix": 2, "emit": 1, "refine_stats": 1,
                "refine_scores": 1, "refine_select": 1, "gather": 1, "attn": wl.T,
                "attn_combine": wl.T if r.attn_splits > 1 else 0}
    per_launch_us = {}
    for name, n in launches.items():
        if n == 0:
            continue
        times = []
        for rep in range(3):
            st, sp = hip.event(), hip.event()
            step(rep, name, (st, sp))
            hip.sync()
            try:
                times.append(hip.elapsed_ms(st, sp) * 1e3)
            except HipError:  # this kernel is not launched for this shape
                break
        if times:
            per_launch_us[name] = float(np.median(times))
    per_step_us = {k: per_launch_us[k] * launches[k] for k in per_launch_us}
    per_step_us["attn"] += per_step_us.get("attn_combine", 0.0)  # one attention call: both kernels
    dominant = max((k for k in per_step_us if k in ("scan", "refine_stats", "refine_scores", "gather", "attn")),
                   key=lambda k: per_step_us[k])
    log(f"[bench] per-launch us: {json.dumps({k: round(v, 2) for k, v in per_launch_us.items()})}; "
        f"dominant: {dominant}")

    # Timed region: K steps, each replayed from a HIP graph captured from the same calls, which
    # takes the host out of the loop (--eager launches directly). Every step carries its own
    # event pair around the dominant operation: for attention, the whole phase of T calls
    # (attention kernel and, for split key ranges, their merge), divided by T (an event can
    # be recorded only once per graph); otherwise the one launch of the dominant kernel.
    timed = "attn_op" if dominant == "attn" else dominant
    nper = wl.T if timed == "attn_op" else 1
    evs = [(hip.event(light=True), hip.event(light=True)) for _ in range(args.steps)]
    graphs = []
    if not args.eager:
        log(f"[bench] capturing {args.steps} step graphs")
        for i in range(args.steps):
            graphs.append(hip.capture(stream, lambda: step(i, timed, evs[i], capturing=True)))
        # replays must reproduce the eager result bit for bit, with eager work in between
        outs = (r.cand, r.sel, r.k_sel, r.out)
        for i in sorted({0, 1 % args.steps, min(replicas, args.steps - 1)}):
            step(i)
            hip.sync()
            want = [o.numpy() for o in outs]
            for _ in range(2):
                hip.launch(graphs[i], stream)
                hip.sync()
                assert all(np.array_equal(w, o.numpy()) for w, o in zip(want, outs)), f"graph replay {i} differs"
                step(i + 1)
                hip.sync()
        log("[bench] graph replays match eager steps")
    # REPEATS timed runs of exactly K steps each; the reported figures are their medians
    reps_ms, reps_dom = [], []
    for rep in range(REPEATS):
        t_start, t_end = hip.event(), hip.event()
        hip.sync()
        w0 = time.perf_counter()
        hip.record(t_start, stream)
        for i in range(args.steps):
            if graphs:
                hip.launch(graphs[i], stream)
            else:
                step(i, timed, evs[i])
        hip.record(t_end, stream)
        hip.sync()
        wall = time.perf_counter() - w0
        reps_ms.append(hip.elapsed_ms(t_start, t_end))
        reps_dom.append(float(np.mean([hip.elapsed_ms(a, b) * 1e3 for a, b in evs])) / nper)
        log(f"[bench] run {rep}: {args.steps} steps in {reps_ms[-1]:.3f} ms (wall {wall * 1e3:.1f} ms); "
            f"{reps_ms[-1] / args.steps * 1e3:.1f} us/step; {timed}: {reps_dom[-1]:.2f} us per launch")
    ms = float(np.median(reps_ms))
    ms_per_step = ms / args.steps
    blocks_per_s = wl.nseq * args.steps / (ms / 1e3)
    dom_us = float(np.median(reps_dom))

    bound, work = kernel_work(wl, batch.lengths)[dominant]
    if bound == "hbm":
        achieved, peak, unit = work / (dom_us * 1e-6) / 1e9, HBM_PEAK_GBS, "GB/s"
    else:
        achieved = work / (dom_us * 1e-6) / 1e12
        peak = MFMA_BF16_PEAK_TFLOPS if wl.dtype == "bf16" else FP32_PEAK_TFLOPS
        unit = "TFLOP/s"
    if timed != "attn_op":
        rkernel = dominant
    elif wl.dtype == "f32":
        rkernel = "attn_f32_kernel"
    else:
        rkernel = "attn_kernel+attn_combine_kernel" if r.attn_splits > 1 else "attn_kernel"
    roofline = {"kernel": rkernel, "bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
                "frac": round(achieved / peak, 4), "traffic": measured_traffic(rkernel, wl.name),
                "avg_launch_us": round(dom_us, 3)}
    # the whole step against its roofline, and the two targeted kernels against their peaks
    esz = 2 if wl.dtype == "bf16" else 4
    mpeak = MFMA_BF16_PEAK_TFLOPS if wl.dtype == "bf16" else FP32_PEAK_TFLOPS
    broof = block_roofline(wl, batch.lengths, esz, mpeak)
    broof["frac"] = round(blocks_per_s / broof["blocks_per_s"], 4)
    work = kernel_work(wl, batch.lengths)
    scan_us = per_launch_us.get("scan")
    attn_us = dom_us if timed == "attn_op" else per_launch_us["attn"] + per_launch_us.get("attn_combine", 0.0)
    attn_flop = 4.0 * wl.nseq * wl.B * wl.Hq * (wl.topk + wl.B) * wl.d
    fractions = {
        "block": broof,
        "scan_hbm": None if scan_us is None else {
            "us": round(scan_us, 3), "GB_s": round(work["scan"][1] / scan_us / 1e3, 1),
            "frac": round(work["scan"][1] / scan_us / 1e3 / HBM_PEAK_GBS, 4)},
        "attn_mfma": {"us": round(attn_us, 3), "TFLOP_s": round(attn_flop / attn_us / 1e6, 2),
                      "frac": round(attn_flop / attn_us / 1e6 / mpeak, 4), "peak_TFLOP_s": mpeak},
    }

    result = {
        "metric": METRIC,
        "value": round(blocks_per_s, 2),
        "unit": "blocks/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": wl.name, "nseq": wl.nseq, "L": int(max(batch.lengths)), "Hq": wl.Hq, "Hkv": wl.Hkv,
                   "head_dim": wl.d, "B": wl.B, "C": wl.C, "topk": wl.topk, "T": wl.T, "kv_replicas": replicas,
                   "attn_splits": r.attn_splits},
        "tokens_per_s": round(blocks_per_s * wl.B, 1),
        "launch": "eager" if args.eager else "hip_graph_per_step",
        "per_launch_us": {k: round(v, 2) for k, v in per_launch_us.items()},
        "repeats": {"n": REPEATS, "ms_per_step": [round(x / args.steps, 4) for x in reps_ms], "value": "median"},
        "roofline": roofline,
        "fractions": fractions,
    }
    if placement:
        result["attn_ws_placement"] = placement
    if pool is not None:
        log(f"[bench] timing the CPU oracle ({cores} worker processes, then 1)")
        result["cpu_baseline"] = cpu_baseline(wl, pool, cores, L0, args.cpu_budget)
        pool.close()
        pool.join()
    print(json.dumps(result), flush=True)
    return 0


WS_PHASE = 2 << 20  # the two candidate positions of the attention workspace, 2 MiB apart


def place_attn_workspace(hip, r, stream, qs, kbs, vbs, T: int):
    """Where the split attention's workspace sits in physical memory sets how fast its partial
    results are written: measured on one block at 1 x 32K, a 3 MiB workspace costs ~1 us more per
    call for every MiB of it that falls in the wrong half of a 4 MiB period of 2 MiB units, and
    which half that is cannot be told from the address. So the workspace is taken from one
    contiguous allocation at one of two positions 2 MiB apart, whichever runs the T attention
    calls faster (timed here, before anything is measured). Returns the timings, or None when
    the attention does not split its keys (no workspace)."""
    import numpy as np

    from block_diffusion_sparse_herald_amd.hiprt import DevArray, DevView

    ws = r.ws.get("attn")
    if ws is None or r.attn_splits <= 1:
        return None
    n = int(ws.nbytes)
    block = DevArray(hip, (n + WS_PHASE,), np.uint8, zero=True, contiguous=True)
    offsets = (0, WS_PHASE)
    graphs = []
    for off in offsets:
        r.ws["attn"] = DevView(block, off, n)
        for t in range(T):
            r.attn(qs[t], kbs[t], vbs[t], stream=stream)
        hip.sync()
        graphs.append(hip.capture(stream, lambda: [r.attn(qs[t], kbs[t], vbs[t], stream=stream) for t in range(T)]))
    times = [[] for _ in offsets]
    for _ in range(3):  # few launches: a kernel trace of the run should hold mostly the timed steps
        for i, g in enumerate(graphs):
            a, b = hip.event(), hip.event()
            hip.record(a, stream)
            for _ in range(4):
                hip.launch(g, stream)
            hip.record(b, stream)
            hip.sync()
            times[i].append(hip.elapsed_ms(a, b) * 1e3 / (4 * T))
    med = [float(np.median(x)) for x in times]
    best = int(np.argmin(med))
    r.ws["attn"] = DevView(block, offsets[best], n)
    return {"offsets_mib": [o >> 20 for o in offsets], "us_per_call": [round(x, 2) for x in med],
            "chosen_mib": offsets[best] >> 20}


def time_steps(hip, stream, step, steps: int, warmup: int, eager: bool) -> float:
    """Milliseconds for `steps` steps (graph replays unless eager), after `warmup` eager steps."""
    for i in range(warmup):
        step(i)
    hip.sync()
    graphs = [] if eager else [hip.capture(stream, lambda: step(i)) for i in range(steps)]
    a, b = hip.event(), hip.event()
    hip.sync()
    hip.record(a, stream)
    for i in range(steps):
        if graphs:
            hip.launch(graphs[i], stream)
        else:
            step(i)
    hip.record(b, stream)
    hip.sync()
    return hip.elapsed_ms(a, b)


def offload_pipeline(args, hip, wl, batch, kv, seq_dev, r, q0, qs, kbs, vbs, stream):
    """The speculative two-stream pipeline (runner.SpeculativePipeline) over consecutive
    blocks, each with its own seeded queries and per-step inputs: block i's candidates come
    from block i-1's merged queries (the speculative search, overlapped with block i-1's
    steps), refined with block i's own queries. offload: the subset is fetched by the GPU
    reading a pinned host pool that holds the K/V cache (HBM keeps K for the search and
    refine), eager launches; pipelined: the cache stays in HBM and the run of blocks is one
    captured graph. `overlap_refine` selects whether a block's refine and fetch wait for
    the previous block's last step (default: they do, as in a decoder where the next
    block's queries exist only then) or overlap it. Compared with the same calls on one
    stream, bit for bit."""
    import numpy as np

    from block_diffusion_sparse_herald_amd import herald as H
    from block_diffusion_sparse_herald_amd.hiprt import DevArray, HostArray
    from block_diffusion_sparse_herald_amd.inputs import make_blocks
    from block_diffusion_sparse_herald_amd.runner import SpeculativePipeline, StreamOps

    device = args.method == "pipelined"
    el = np.uint16 if wl.dtype == "bf16" else np.float32
    nd = max(2, min(args.steps, 8))  # distinct blocks, cycled over the timed run
    log(f"[bench] {args.method}: drawing {nd} distinct blocks")
    bnp = make_blocks(wl, batch, nd)
    blk_dev = []
    for b in bnp:
        d = {"q0": DevArray.from_host(hip, b["q0"])}
        for k in ("q_steps", "kb_steps", "vb_steps"):
            arr = DevArray.from_host(hip, b[k])
            d[k] = [arr.offset(t) for t in range(wl.T)]
            d["_" + k] = arr
        blk_dev.append(d)
    if device:
        k_src, v_src = [k for k, _ in kv], [v for _, v in kv]
    else:
        pool_k = HostArray(hip, batch.k_cache.shape, el)
        pool_v = HostArray(hip, batch.v_cache.shape, el)
        pool_k.numpy()[...] = batch.k_cache
        pool_v.numpy()[...] = batch.v_cache
        k_src, v_src = pool_k, pool_v
    k_scan = [k for k, _ in kv]
    alloc = lambda shape, dt, zero=False, contiguous=False: DevArray(hip, shape, dt, zero, contiguous)  # noqa: E731
    pipe = SpeculativePipeline(r, alloc, StreamOps.hip(hip), src_is_host=0 if device else 2,
                               overlap_refine=args.overlap_refine)
    a_stream, b_stream = stream, hip.stream()
    fetch_bytes = 2 * wl.nseq * wl.Hkv * wl.topk * wl.d * np.dtype(el).itemsize
    n = args.steps
    blocks = [blk_dev[i % nd] for i in range(n)]
    outs = [[DevArray(hip, r.out.shape, el) for _ in range(wl.T)] for _ in range(2)]
    out_of = [outs[i % 2] for i in range(n)]  # the last two blocks' outputs stay for the check

    def pipelined():
        pipe.run(blocks, k_scan, k_src, v_src, a_stream, b_stream, outs=out_of)

    def serial():
        pipe.run_serial(blocks, k_scan, k_src, v_src, a_stream, outs=out_of)

    def timed(fn):
        if device:  # one graph: the search stream forks from the denoise stream and joins it at the end
            fork, join = hip.event(), hip.event()

            def body():
                hip.record(fork, a_stream)
                hip.wait(b_stream, fork)
                fn()
                hip.record(join, b_stream)
                hip.wait(a_stream, join)

            graph = hip.capture(a_stream, body)
            hip.launch(graph, a_stream)  # warm-up replay
            hip.sync()
            t = []
            for _ in range(3):
                a, b = hip.event(), hip.event()
                hip.record(a, a_stream)
                hip.launch(graph, a_stream)
                hip.record(b, a_stream)
                hip.sync()
                t.append(hip.elapsed_ms(a, b))
            return float(np.median(t))
        fn()  # warm-up
        hip.sync()
        t = []
        for _ in range(3):
            a, b = hip.event(), hip.event()
            hip.record(a, a_stream)
            hip.wait(b_stream, a)
            fn()
            hip.wait(a_stream, pipe.fetched[(n - 1) % 2])
            hip.record(b, a_stream)
            hip.sync()
            t.append(hip.elapsed_ms(a, b))
        return float(np.median(t))

    ms_pipe = timed(pipelined)
    last_pipe = [o.numpy() for o in out_of[-1]]
    ms_ser = timed(serial)
    last_ser = [o.numpy() for o in out_of[-1]]
    assert all(np.array_equal(x, y) for x, y in zip(last_pipe, last_ser)), \
        f"{args.method}: the pipelined schedule's last block differs from the one-stream schedule"
    # the fetch alone, on the search stream
    e0, e1 = hip.event(), hip.event()
    hip.sync()
    hip.record(e0, b_stream)
    for i in range(n):
        H.herald_gather_kv(r.problem, k_src[i % len(k_src)] if isinstance(k_src, list) else k_src,
                           v_src[i % len(v_src)] if isinstance(v_src, list) else v_src, 0 if device else 2, r.sel,
                           pipe.pools[0][0], pipe.pools[0][1], stream=b_stream)
    hip.record(e1, b_stream)
    hip.sync()
    fetch_us = hip.elapsed_ms(e0, e1) * 1e3 / n
    value = wl.nseq * n / (ms_pipe / 1e3)
    ser_value = wl.nseq * n / (ms_ser / 1e3)
    log(f"[bench] {args.method}: pipelined {ms_pipe / n * 1e3:.1f} us/block, one stream {ms_ser / n * 1e3:.1f}; "
        f"fetch {fetch_us:.1f} us for {fetch_bytes / 2**20:.2f} MiB; refine {'overlapped' if args.overlap_refine else 'after the previous block'}")
    result = {
        "metric": METRIC, "method": args.method, "value": round(value, 2), "unit": "blocks/s", "n_gpus": 1,
        "steps": n, "warmup": 1, "ms_per_step": round(ms_pipe / n, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": wl.dtype, "data": "synthetic",
        "config": {"workload": wl.name, "nseq": wl.nseq, "L": int(max(batch.lengths)), "Hq": wl.Hq, "Hkv": wl.Hkv,
                   "head_dim": wl.d, "B": wl.B, "C": wl.C, "topk": wl.topk, "T": wl.T, "distinct_blocks": nd,
                   "overlap_refine": bool(args.overlap_refine)},
        "tokens_per_s": round(value * wl.B, 1),
        "launch": f"one graph of {n} blocks, two streams" if device else "eager, two streams",
        "serialised_value": round(ser_value, 2), "pipeline_gain": round(ms_ser / ms_pipe, 4),
        "fetch": {"bytes": fetch_bytes, "us": round(fetch_us, 2), "GB_s": round(fetch_bytes / fetch_us / 1e3, 2),
                  "path": "device gather from HBM" if device else "GPU reads the pinned host pool over PCIe"},
    }
    print(json.dumps(result), flush=True)
    return 0


def other_method(args, hip, wl, batch, kv, seq_dev, r, q0, qs, kbs, vbs, stream):
    """Compressed-key selection, dense attention or MAGE-exact selection, timed like the
    HERALD path, with the HERALD path timed alongside in the same process for the ratio."""
    import numpy as np

    from block_diffusion_sparse_herald_amd import herald as H
    from block_diffusion_sparse_herald_amd.hiprt import DevArray
    from block_diffusion_sparse_herald_amd.runner import BlockRunner

    lengths = np.asarray(batch.lengths)
    if args.method != "compressed" and (lengths != lengths[0]).any():
        print(f"--method {args.method} needs sequences of one length (the subset size is one number per call); "
              f"workload {wl.name} is ragged", file=sys.stderr)
        return 2
    L = int(lengths.max())
    alloc = lambda shape, dt, zero=False, contiguous=False: DevArray(hip, shape, dt, zero, contiguous)  # noqa: E731
    iota = None if args.method == "compressed" else DevArray.from_host(hip, np.ascontiguousarray(
        np.broadcast_to(np.arange(L, dtype=np.int32), (wl.nseq, wl.Hkv, L))))
    if args.method == "compressed":
        b = r
        rows = H.herald_compressed_rows(b.problem, args.stride)
        ws_c = DevArray(hip, (H.herald_workspace_size(b.problem, H.HERALD_OP_SELECT_COMPRESSED),), np.uint8)
        comp_bytes = rows * wl.Hkv * wl.d * 4
        comps = []
        for _ in range(max(1, math.ceil(512 * 2**20 / comp_bytes))):
            kc = DevArray(hip, (rows, wl.Hkv, wl.d), np.float32)
            H.herald_compress_keys(b.problem, kv[len(comps) % len(kv)][0], args.ksize, args.stride, kc, stream=stream)
            comps.append(kc)
        hip.sync()

        def step(i):
            k, v = kv[i % len(kv)]
            H.herald_select_compressed(b.problem, q0, comps[i % len(comps)], args.stride, b.cand, b.cand_score, ws_c,
                                       stream=stream)
            b.refine(q0, k, stream=stream)
            b.gather(k, v, stream=stream)
            for t in range(wl.T):
                b.attn(qs[t], kbs[t], vbs[t], stream=stream)
        what = (f"selection over compressed keys (window {args.ksize}, block {args.stride}: {rows} rows, "
                f"{comp_bytes / 2**20:.1f} MiB fp32 per copy, {len(comps)} copies), refine, gather, {wl.T} steps")
    elif args.method == "dense":
        b = BlockRunner(batch.seq_start, wl.B, wl.Hq, wl.Hkv, wl.d, L, L, wl.dtype, alloc=alloc,
                        seq_start_dev=seq_dev)
        # the whole cache in the subset layout, once; copies rotate like the cache replicas
        pool_bytes = b.k_sel.nbytes + b.v_sel.nbytes
        pools = []
        for _ in range(max(1, math.ceil(512 * 2**20 / pool_bytes))):
            b.gather(kv[0][0], kv[0][1], sel=iota, stream=stream)
            hip.sync()
            pools.append((b.k_sel.clone(), b.v_sel.clone()))
        hip.sync()

        def step(i):
            ks, vs = pools[i % len(pools)]
            for t in range(wl.T):
                H.herald_block_attn(b.problem, qs[t], kbs[t], vbs[t], ks, vs, b.out, b.ws["attn"], stream=stream)
        what = f"dense attention over all {L} keys + {wl.B} in-block keys, {wl.T} steps; {len(pools)} pool copies"
    else:
        b = BlockRunner(batch.seq_start, wl.B, wl.Hq, wl.Hkv, wl.d, L, wl.topk, wl.dtype, alloc=alloc,
                        seq_start_dev=seq_dev)

        def step(i):
            k, v = kv[i % len(kv)]
            b.refine(q0, k, cand=iota, stream=stream)
            b.gather(k, v, stream=stream)
            for t in range(wl.T):
                b.attn(qs[t], kbs[t], vbs[t], stream=stream)
        what = f"exact top-{wl.topk} of the real queries over all {L} keys (refine with C = L), gather, {wl.T} steps"

    def herald_step(i):
        k, v = kv[i % len(kv)]
        r.select(q0, k, stream=stream)
        r.refine(q0, k, stream=stream)
        r.gather(k, v, stream=stream)
        for t in range(wl.T):
            r.attn(qs[t], kbs[t], vbs[t], stream=stream)

    log(f"[bench] {args.method}: {what}")
    ms = time_steps(hip, stream, step, args.steps, args.warmup, args.eager)
    ms_h = time_steps(hip, stream, herald_step, args.steps, args.warmup, args.eager)
    value = wl.nseq * args.steps / (ms / 1e3)
    herald_value = wl.nseq * args.steps / (ms_h / 1e3)
    log(f"[bench] {args.method}: {ms / args.steps * 1e3:.1f} us/step; HERALD path {ms_h / args.steps * 1e3:.1f} us/step")
    result = {
        "metric": METRIC, "method": args.method, "value": round(value, 2), "unit": "blocks/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms / args.steps, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": wl.dtype, "data": "synthetic",
        "config": {"workload": wl.name, "nseq": wl.nseq, "L": L, "Hq": wl.Hq, "Hkv": wl.Hkv, "head_dim": wl.d,
                   "B": wl.B, "topk": L if args.method == "dense" else wl.topk,
                   "C": wl.C if args.method == "compressed" else L, "T": wl.T,
                   **({"ksize": args.ksize, "stride": args.stride} if args.method == "compressed" else {})},
        "tokens_per_s": round(value * wl.B, 1), "launch": "eager" if args.eager else "hip_graph_per_step",
        "what": what, "herald_value": round(herald_value, 2), "vs_herald": round(value / herald_value, 4),
    }
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
