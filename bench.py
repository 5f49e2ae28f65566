"""Benchmark of the KDA decode op on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
    python bench.py --prefill [--matmul split_bf16|f32]

Compute-heavy launches (the chunked prefill, multi-token decode batches on a
bf16 pool) run back to back show a transient: the second launch is ~35%
slower than the first and the time settles over about 30 launches (the
pattern of the chip's clock and power management adjusting to the load;
the one-token batches, bound by HBM, do not show it).
So the default warmup is 40 launches for --prefill and for workloads with
more than one token per request, 5 otherwise (the one-token batches are
bound by HBM and show no transient).

A step is one kda_decode call over one batch of the workload (default: the
96-head layer, B=256 requests x 1 token, dk = dv = 128, bf16 q/k/v, fp32
state pool of 512 slots).  All inputs are resident in HBM before timing.
Prints one JSON line on stdout; progress goes to stderr.

Decode steps rotate state_indices over disjoint slot sets (as many as the
pool holds, --no-rotate keeps one), so that consecutive steps touch
different state tiles and the 256 MB Infinity Cache cannot serve a batch
whose touched state would fit in it.

--prefill times kda_prefill instead (the chunked whole-sequence form on the
matrix cores; default workload B=8 x 2048 tokens, 96 heads, value-first
fp32 state): value is tokens x heads per second.  Its roofline is the
binding one of two floors: HBM (algorithmic bytes / 8 TB/s) and the matrix
unit (algorithmic flops of the chunk form -- X, Y, the state update, U, O
and the P, R products; 16-token chunks, a ragged chunk counted whole --
times three for split-bf16, whose fp32 product is three bf16 products, over
the dense bf16 peak; or once over the fp32 matrix peak).

Fields beyond the common ones:
  roofline      roofline of the dominant kernel: achieved = algorithmic
                bytes per launch (state read + write of every active tile,
                plus every token tensor once) / mean launch duration (one
                pair of HIP events on the launch stream around the K timed
                launches, divided by K); peak 8000 GB/s;
                traffic = HBM bytes per launch from the committed rocprofv3
                FETCH_SIZE / WRITE_SIZE summary (null when the kernel source
                changed since the counters were taken).
  copy_ceiling  the fastest of the hand-written streaming copies of
                libkda_bench.so (and torch's copies) over the same byte
                count: the practical HBM ceiling on this machine.
  cpu_baseline  the fp64 oracle timed on every host core (one worker
                process per core, started before any GPU call, one BLAS
                thread each) on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "state GB/s (%HBM peak) + tokens·heads/s, KDA decode B=256 H=96 d=128"
PREFILL_METRIC = "tokens·heads/s, KDA chunked prefill B=8 T=2048 H=96 d=128"
HBM_PEAK_GBPS = 8000.0
MATRIX_PEAK_TFLOPS = {"split_bf16": 2500.0, "f32": 157.3}   # dense bf16 / fp32 matrix
CSRC = os.path.join(ROOT, "gated_delta_rule_82_amd", "csrc")
KERNEL_SOURCES = {
    "kda_decode": [os.path.join(CSRC, "kda_decode.hip"), os.path.join(CSRC, "kda_device.h")],
    "kda_prefill": [os.path.join(CSRC, "kda_prefill.hip"), os.path.join(CSRC, "kda_device.h")],
}
PROFILES = os.path.join(ROOT, "profiles")
CHUNK = 16


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash(op: str = "kda_decode") -> str:
    """Hash of the kernel's sources and of the compiler flags only that file
    gets (a counter summary is stale once either changes)."""
    from gated_delta_rule_82_amd.build import EXTRA_FLAGS
    h = hashlib.sha256()
    for path in KERNEL_SOURCES[op]:
        with open(path, "rb") as f:
            h.update(f.read())
    if op in EXTRA_FLAGS:
        h.update(repr(EXTRA_FLAGS[op]).encode())
    return h.hexdigest()[:16]


def committed_traffic(workload: str, op: str = "kda_decode"):
    """HBM bytes per launch from profiles/<op>_<workload>_counters.md, if
    that summary was taken on the current kernel source."""
    path = os.path.join(PROFILES, f"{op}_{workload}_counters.md")
    if not os.path.exists(path):
        return None, "no counter summary"
    text = open(path).read()
    m_hash = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    m_bytes = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not (m_hash and m_bytes):
        return None, "summary lacks traffic fields"
    if m_hash.group(1) != kernel_source_hash(op):
        return None, "kernel changed since counters were taken"
    return float(m_bytes.group(1)), path


# State a forked oracle worker inherits from the parent (copy-on-write): the
# drawn workload, set before the pool is created.
_CPU_INPUT = {}


def _cpu_worker_init():
    from threadpoolctl import threadpool_limits
    _CPU_INPUT["limits"] = threadpool_limits(limits=1)


def _cpu_steps(cfg, heads_per_step):
    """The baseline's units of work: (b0, b1, hv0, hv1) request and value-head
    ranges -- 8 requests with all their heads, or ``heads_per_step`` heads
    (a multiple of the GQA group) of one request."""
    if heads_per_step is None:
        return [(b, min(b + 8, cfg.B), 0, cfg.HV) for b in range(0, cfg.B, 8)]
    per = max(cfg.G, heads_per_step // cfg.G * cfg.G)
    return [(b, b + 1, hv, min(hv + per, cfg.HV)) for b in range(cfg.B) for hv in range(0, cfg.HV, per)]


def _cpu_worker_run(args):
    """One worker's share of the oracle baseline: the workload's units of
    work in order from its own starting point (wrapping around), each given
    to the oracle as the token rows and heads it covers, with initial states
    taken from a bank of tiles drawn from N(0, sigma) on the host (the
    distribution the device pool is filled with), until ``budget_s``
    seconds of oracle time are done."""
    import numpy as np
    from oracle import kda_oracle as ko
    wid, nworkers, budget_s, heads_per_step = args
    inp = _CPU_INPUT["inp"]
    cfg = inp.cfg
    lb = cfg.lower_bound if cfg.gate_mode == "lower_bound" else None
    steps = _cpu_steps(cfg, heads_per_step)
    rng = np.random.default_rng(1000 + wid)
    shape = (cfg.DV, cfg.DK) if cfg.state_layout == "v_first" else (cfg.DK, cfg.DV)
    bank = (rng.standard_normal((97,) + shape, dtype=np.float32) * np.float32(cfg.state_sigma))
    cu = np.asarray(inp.cu_seqlens, dtype=np.int64)
    i = wid * len(steps) // nworkers
    done_tiles = done_th = done_state = 0
    elapsed = 0.0
    while elapsed < budget_s:
        b0, b1, hv0, hv1 = steps[i % len(steps)]
        t0, t1 = int(cu[b0]), int(cu[b1])
        h0, h1 = hv0 // cfg.G, (hv1 - 1) // cfg.G + 1
        idx = inp.state_indices[b0:b1]
        tiles = [(bb, hv) for bb in range(b1 - b0) for hv in range(hv1 - hv0)]
        pool = {(int(idx[bb]), hv): bank[(done_tiles + n) % len(bank)]
                for n, (bb, hv) in enumerate(tiles) if idx[bb] >= 0}
        start = time.perf_counter()
        ko.kda_decode(inp.q[:, t0:t1, h0:h1], inp.k[:, t0:t1, h0:h1], inp.v[:, t0:t1, hv0:hv1],
                      inp.raw_gate[:, t0:t1, hv0:hv1], inp.beta_logits[:, t0:t1, hv0:hv1],
                      inp.a_log[hv0:hv1], inp.dt_bias[hv0:hv1], cu[b0:b1 + 1] - t0, pool, idx,
                      tiles=tiles, gate_mode=cfg.gate_mode, lower_bound=lb,
                      state_layout=cfg.state_layout, state_dtype=cfg.state_dtype)
        elapsed += time.perf_counter() - start
        for bb, hv in tiles:
            n = int(cu[b0 + bb + 1] - cu[b0 + bb])
            done_th += n
            if n > 0 and idx[bb] >= 0:
                done_state += 2 * cfg.DK * cfg.DV * cfg.state_elem_bytes
        done_tiles += len(tiles)
        i += 1
    return done_tiles, done_th, done_state, elapsed


def start_cpu_pool(inp):
    """Fork one oracle worker per host core.  Called before anything touches
    the GPU, so the children start from a process with no HIP state."""
    import multiprocessing
    _CPU_INPUT["inp"] = inp
    n = len(os.sched_getaffinity(0))
    pool = multiprocessing.get_context("fork").Pool(n, initializer=_cpu_worker_init)
    return pool, n


def cpu_baseline(cpu_pool, inp, budget_s: float, heads_per_step=None):
    """Time the fp64 oracle on every worker of ``cpu_pool`` at once: each
    takes the workload's (request, head) tiles in order from its own offset
    (wrapping around), a unit of work being up to 8 requests with all their
    heads or ``heads_per_step`` heads of one request, until ``budget_s``
    seconds of oracle time.  The rate is the sum of the workers' rates, each
    its work over its own oracle time (all workers run at once)."""
    pool, n = cpu_pool
    cfg = inp.cfg
    t0 = time.perf_counter()
    res = pool.map(_cpu_worker_run, [(w, n, budget_s, heads_per_step) for w in range(n)])
    wall = time.perf_counter() - t0
    tiles = sum(r[0] for r in res)
    th = sum(r[1] for r in res)
    state_rate = sum(r[2] / r[3] for r in res)
    th_rate = sum(r[1] / r[3] for r in res)
    total = cfg.B * cfg.HV
    return {
        "value": round(state_rate / 1e9, 6),
        "unit": "GB/s",
        "cores": n,
        "kind": "oracle",
        "sample": f"{tiles} (request, head) tiles ({tiles / total:.3f} passes over the batch's "
                  f"{total}), all their tokens: {th} token-heads, {n} worker processes at once "
                  f"(one BLAS thread each) for {budget_s:.0f} s of oracle time each "
                  f"({wall:.1f} s wall), fp64 numpy; initial states from the pool's "
                  f"N(0, {cfg.state_sigma}) distribution, drawn on the host",
        "tokens_heads_per_s": round(th_rate, 3),
        "host_cores_available": len(os.sched_getaffinity(0)),
    }


COPY_VARIANTS = {"nt_stream": 0, "nt_wave": 1, "wave": 2, "nt_kfirst_slabs": 3}


def bench_library():
    """libkda_bench.so: the hand-written streaming copies (built with the
    library by gated_delta_rule_82_amd.build; only this script loads it)."""
    import ctypes
    from gated_delta_rule_82_amd.build import BENCH_LIB
    if not os.path.exists(BENCH_LIB):
        raise RuntimeError(f"{BENCH_LIB} is not built; run `python -m gated_delta_rule_82_amd.build`")
    lib = ctypes.CDLL(BENCH_LIB)
    lib.kda_bench_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                                   ctypes.c_void_p]
    lib.kda_bench_copy.restype = ctypes.c_int
    return lib


def copy_ceiling(nbytes: int, reps: int = 10):
    """Streaming copies moving ``nbytes`` (half read, half written), each
    buffer pair rotated over enough copies that the 256 MB cache cannot
    serve them: the hand-written copies of libkda_bench.so and torch's
    device-to-device and elementwise copies.  Returns {name: GB/s of read +
    write bytes} (mean over ``reps`` launches, HIP events on the stream)."""
    import torch
    half = nbytes // 2 // 65536 * 65536
    sets = max(1, -(-(1 << 29) // half))      # >= 512 MB per rotation
    src = [torch.empty(half // 4, dtype=torch.float32, device="cuda").fill_(1.0) for _ in range(sets)]
    dst = [torch.empty_like(x) for x in src]
    stream = torch.cuda.current_stream()
    lib = bench_library()

    def hand(v):
        def run(i):
            rc = lib.kda_bench_copy(dst[i].data_ptr(), src[i].data_ptr(), half, v, stream.cuda_stream)
            if rc != 0:
                raise RuntimeError(f"kda_bench_copy failed ({rc})")
        return run

    variants = {name: hand(v) for name, v in COPY_VARIANTS.items()}
    variants["torch_d2d_copy"] = lambda i: dst[i].copy_(src[i])
    variants["torch_elementwise_copy"] = lambda i: torch.mul(src[i], 1.0, out=dst[i])
    res = {}
    for name, fn in variants.items():
        for i in range(sets):
            fn(i)
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record(stream)
        for r in range(reps):
            fn(r % sets)
        e.record(stream)
        torch.cuda.synchronize()
        ms = s.elapsed_time(e) / reps
        res[name] = round(2 * half / (ms * 1e-3) / 1e9, 1)
    del src, dst
    torch.cuda.empty_cache()
    return res


def rotation_sets(inp, k: int):
    """``k`` disjoint assignments of the batch's active requests to pool
    slots: the drawn state_indices first, then further permutations of the
    slots it leaves unused (negative indices stay negative)."""
    import numpy as np
    cfg = inp.cfg
    idx = np.asarray(inp.state_indices, dtype=np.int32)
    active = idx >= 0
    free = np.setdiff1d(np.arange(cfg.n_slots, dtype=np.int32), idx[active])
    free = np.random.default_rng(cfg.seed + 7).permutation(free)
    n = int(active.sum())
    sets = [idx]
    for j in range(1, k):
        if free.size < j * n:
            break
        nxt = idx.copy()
        nxt[active] = free[(j - 1) * n:j * n]
        sets.append(nxt)
    return sets


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed launches first (default 5; 40 for --prefill and for "
                         "workloads with more than one token per request, whose launches "
                         "show a slow-down transient that settles over about 30 of them)")
    ap.add_argument("--workload", default=None)
    ap.add_argument("--state-layout", choices=("k_first", "v_first"), default=None,
                    help="default: the workload's (key-first for the decode batches)")
    ap.add_argument("--state-dtype", choices=("f32", "bf16"), default=None)
    ap.add_argument("--prefill", action="store_true",
                    help="time kda_prefill (chunked, matrix cores) on the prefill workload")
    ap.add_argument("--matmul", choices=("split_bf16", "f32"), default="split_bf16",
                    help="matrix precision of --prefill")
    ap.add_argument("--gate", choices=("softplus", "lower_bound"), default=None,
                    help="override the workload's gate mode (lower_bound uses -5)")
    ap.add_argument("--conv", action="store_true",
                    help="time kda_decode_conv: the step with the short convolutions in front")
    ap.add_argument("--no-rotate", action="store_true",
                    help="reuse the same state slots every step (by default steps rotate over "
                         "disjoint slot sets so the 256 MB cache cannot hold the touched state)")
    ap.add_argument("--cpu-budget", type=float, default=12.0,
                    help="seconds of oracle work per host core for cpu_baseline (0 disables)")
    ap.add_argument("--no-copy-ceiling", action="store_true")
    args = ap.parse_args(argv)

    if args.prefill and args.conv:
        print("bench.py: --prefill and --conv are separate measurements", file=sys.stderr)
        return 2
    if args.gpus != 1:
        print(f"bench.py: this KDA decode build runs on one GPU; --gpus {args.gpus} is not "
              "supported (every (request, head) tile is independent, so more GPUs would each "
              "run their own share of requests or heads)", file=sys.stderr)
        return 2

    import numpy as np
    from gated_delta_rule_82_amd import workloads as wl

    name = args.workload or (wl.PREFILL_HEADLINE if args.prefill else wl.HEADLINE)
    over = {k: v for k, v in (("state_layout", args.state_layout), ("state_dtype", args.state_dtype))
            if v is not None}
    if args.gate is not None:
        over["gate_mode"] = args.gate
        over["lower_bound"] = -5.0 if args.gate == "lower_bound" else 0.0
    cfg = wl.preset(name, **over)
    log(f"[bench] workload {name}: {cfg.description}" + (f" (overrides {over})" if over else ""))
    if args.warmup is None:
        args.warmup = 40 if (args.prefill or cfg.tokens != "1") else 5
    inp = wl.draw(cfg)
    # the oracle workers fork here, before anything touches the GPU (the
    # conv step has no oracle baseline of its own here)
    cpu_pool = start_cpu_pool(inp) if args.cpu_budget > 0 and not args.conv else None

    import torch
    from gated_delta_rule_82_amd import kda

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    kda.library()     # fail loudly if the HIP library is not built

    dev = wl.to_device(inp)
    pool = wl.device_pool(inp)
    out = wl.empty_out(inp)
    state_b = wl.state_bytes(cfg, inp)
    token_b = wl.token_bytes(cfg, inp)
    alg_bytes = state_b + token_b
    tok_heads = inp.T * cfg.HV
    sets = rotation_sets(inp, 1 if args.no_rotate else max(1, cfg.n_slots // max(cfg.B, 1)))
    idx_sets = [torch.from_numpy(x.astype(np.int32)).to(pool.device) for x in sets]
    log(f"[bench] {len(sets)} disjoint slot set(s) of {int((sets[0] >= 0).sum())} requests, "
        f"{state_b / 2 / 1e6:.0f} MB of state each")
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    handle = stream.cuda_stream
    mode = dict(gate_mode=cfg.gate_mode, lower_bound=cfg.lower_bound, state_layout=cfg.state_layout)

    # The C ABI is called with descriptors built once per slot set, so that
    # the host enqueues a launch in a few microseconds and the GPU never
    # waits for the next one (the short batches' kernels take ~50 us).
    kmode = kda.make_mode(**mode)
    desc = lambda t, nm: kda._descriptor(t, nm)   # noqa: E731
    if args.conv:
        ci = wl.draw_conv(inp)
        cd = wl.conv_to_device(ci, cfg.qkv_dtype)
        conv_bytes = wl.conv_bytes(cfg, inp, ci.K)
        alg_bytes += conv_bytes
        torch.cuda.synchronize()
        conv = kda.KdaConv(*[desc(cd[n], n) for n in kda.CONV_FIELDS])
        out_d = desc(out, "out")
        tensors = dict(dev, state_pool=pool)
        rests = [[desc(ix, n) if n == "state_indices" else desc(tensors[n], n) for n in kda.CONV_REST]
                 for ix in idx_sets]

        def step(i):
            rc = kda.call_raw_conv(out_d, conv, rests[i % len(rests)], kmode, handle)
            if rc != kda.KDA_OK:
                raise kda.KdaError(rc, "kda_decode_conv")
    else:
        tensors = dict(dev, out=out, state_pool=pool)
        descs = [[desc(ix, n) if n == "state_indices" else desc(tensors[n], n) for n in kda.ARG_NAMES]
                 for ix in idx_sets]
        if args.prefill:
            mm = kda.MATMULS[args.matmul]

            def step(i):
                rc = kda.call_raw_prefill(descs[i % len(descs)], kmode, mm, handle)
                if rc != kda.KDA_OK:
                    raise kda.KdaError(rc, "kda_prefill")
        else:
            def step(i):
                rc = kda.call_raw(descs[i % len(descs)], kmode, handle)
                if rc != kda.KDA_OK:
                    raise kda.KdaError(rc)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    log(f"[bench] warmup {args.warmup} done; timing {args.steps} steps")

    # One pair of HIP events on the launch stream brackets the K back-to-back
    # launches: the mean launch duration is their span / K (events around
    # every launch would add their own latency to each, several us on the
    # short batches).
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for i in range(args.steps):
        step(args.warmup + i)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    mean_kernel_ms = start.elapsed_time(end) / args.steps
    log(f"[bench] wall {ms_per_step * 1e3:.1f} us/step, kernel mean {mean_kernel_ms * 1e3:.1f} us "
        f"(HIP events around all {args.steps} launches)")
    del dev, out
    torch.cuda.empty_cache()

    common = dict(args=args, cfg=cfg, name=name, inp=inp, cpu_pool=cpu_pool,
                  ms_per_step=ms_per_step, mean_kernel_ms=mean_kernel_ms, alg_bytes=alg_bytes,
                  tok_heads=tok_heads, rotation=len(sets))
    try:
        if args.prefill:
            del pool
            torch.cuda.empty_cache()
            return report_prefill(**common)
        del pool
        torch.cuda.empty_cache()
        return report_decode(state_b=state_b, **common)
    finally:
        if cpu_pool is not None:
            cpu_pool[0].terminate()


def measure_copies(nbytes):
    copies = copy_ceiling(nbytes)
    best = max(copies, key=copies.get)
    log(f"[bench] copy ceiling (read+write, {nbytes / 1e9:.2f} GB): {copies}")
    return copies, best


def report_decode(args, cfg, name, inp, cpu_pool, ms_per_step, mean_kernel_ms, alg_bytes,
                  tok_heads, rotation, state_b):
    import numpy as np
    value = state_b / (ms_per_step * 1e-3) / 1e9
    achieved = alg_bytes / (mean_kernel_ms * 1e-3) / 1e9
    variant = "" if (cfg.state_layout, cfg.state_dtype) == ("k_first", "f32") else \
        f"_{cfg.state_layout}_{cfg.state_dtype}"
    if args.conv:
        variant += "_conv"
    traffic, traffic_src = committed_traffic(name + variant)
    log(f"[bench] traffic: {traffic} ({traffic_src})")

    copies, best = (None, None) if args.no_copy_ceiling else measure_copies(state_b)
    cpu = None
    if cpu_pool is not None:
        log(f"[bench] cpu_baseline: oracle for ~{args.cpu_budget:.0f} s on {cpu_pool[1]} cores")
        cpu = cpu_baseline(cpu_pool, inp, args.cpu_budget)
        log(f"[bench] cpu_baseline {cpu['value']} GB/s, {cpu['tokens_heads_per_s']} token-heads/s")

    counts = np.diff(inp.cu_seqlens)
    line = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": name, "B": cfg.B, "H": cfg.H, "HV": cfg.HV, "dk": cfg.DK, "dv": cfg.DV,
            "tokens_per_request": cfg.tokens, "total_tokens": inp.T,
            "qkv_dtype": cfg.qkv_dtype, "state_dtype": cfg.state_dtype,
            "state_layout": cfg.state_layout, "gate": cfg.gate_mode,
            "short_conv": bool(args.conv), "slots": cfg.n_slots,
            "slot_sets_rotated": rotation, "parallelism": "single GPU",
        },
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBPS, 2),
        "tokens_heads_per_s": round(tok_heads / (ms_per_step * 1e-3), 1),
        "state_bytes_per_step": state_b,
        "algorithmic_bytes_per_step": alg_bytes,
        "kernel_us_mean": round(mean_kernel_ms * 1e3, 2),
        "copy_ceiling_GBps": None if copies is None else copies[best],
        "copy_ceiling_kernel": best,
        "copy_kernels_GBps": copies,
        "frac_of_copy_ceiling": None if copies is None else round(achieved / copies[best], 4),
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 3),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "kernel": "kda_decode_%s<%d,%d,%s q/k/v,%s state>" % (
                cfg.state_layout.replace("_", ""), cfg.DK, cfg.DV, cfg.qkv_dtype, cfg.state_dtype),
        },
        "cpu_baseline": cpu,
        "active_tiles": int(((counts > 0) & (inp.state_indices >= 0)).sum()) * cfg.HV,
    }
    print(json.dumps(line), flush=True)
    return 0


def chunk_flops(dk: int, dv: int) -> int:
    """Algorithmic flops of one 16-token chunk of one (request, head) tile:
    X = V - Kt S and Y = Qt S (2 C dk dv each), the state update Kup^T U
    (2 C dk dv), U = T X and R U (2 C^2 dv each), the P and R products
    (2 C^2 dk each)."""
    c = CHUNK
    return 2 * (3 * c * dk * dv + 2 * c * c * dv + 2 * c * c * dk)


# bf16 matrix products per fp32-equivalent product of each precision
PRODUCTS_PER_FLOP = {"split_bf16": 3, "f32": 1}


def report_prefill(args, cfg, name, inp, cpu_pool, ms_per_step, mean_kernel_ms, alg_bytes,
                   tok_heads, rotation):
    import numpy as np
    counts = np.diff(inp.cu_seqlens)
    active = (counts > 0) & (inp.state_indices >= 0)
    chunks = int((-(-counts[active] // CHUNK)).sum()) * cfg.HV
    flops = chunks * chunk_flops(cfg.DK, cfg.DV)
    t_kernel = mean_kernel_ms * 1e-3
    peak_tf = MATRIX_PEAK_TFLOPS[args.matmul]
    t_hbm = alg_bytes / (HBM_PEAK_GBPS * 1e9)
    t_mfma = PRODUCTS_PER_FLOP[args.matmul] * flops / (peak_tf * 1e12)
    matrix = {"achieved": round(flops / t_kernel / 1e12, 3), "peak": peak_tf, "unit": "TFLOP/s",
              "products_per_flop": PRODUCTS_PER_FLOP[args.matmul],
              "floor_us": round(t_mfma * 1e6, 2), "frac": round(t_mfma / t_kernel, 4)}
    hbm = {"achieved": round(alg_bytes / t_kernel / 1e9, 3), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
           "floor_us": round(t_hbm * 1e6, 2), "frac": round(t_hbm / t_kernel, 4)}
    variant = f"_{args.matmul}" + ("" if cfg.gate_mode == "lower_bound" else f"_{cfg.gate_mode}")
    traffic, traffic_src = committed_traffic(name + variant, "kda_prefill")
    log(f"[bench] traffic: {traffic} ({traffic_src})")
    if t_hbm >= t_mfma:
        roof = dict(bound="hbm", **{k: hbm[k] for k in ("achieved", "peak", "unit", "frac")})
    else:
        roof = dict(bound="mfma", **{k: matrix[k] for k in ("achieved", "peak", "unit", "frac")})
    roof["traffic"] = traffic
    # the launch form the library takes at dv = 128: the stage split, with
    # two workgroups per tile up to 128 (request, head) tiles
    tiles = cfg.B * cfg.HV
    form = ("" if cfg.DV != 128 else
            ",stage split, 2 workgroups per tile" if tiles <= 128 else ",stage split")
    roof["kernel"] = "kda_prefill_chunks<%d,%d,%s q/k/v,%s state,%s,%s%s>" % (
        cfg.DK, cfg.DV, cfg.qkv_dtype, cfg.state_dtype, cfg.state_layout.replace("_", ""),
        args.matmul, form)
    copies, best = (None, None) if args.no_copy_ceiling else measure_copies(alg_bytes)
    cpu = None
    if cpu_pool is not None:
        log(f"[bench] cpu_baseline: oracle for ~{args.cpu_budget:.0f} s on {cpu_pool[1]} cores")
        cpu = cpu_baseline(cpu_pool, inp, args.cpu_budget, heads_per_step=4)
        cpu["value"] = cpu["tokens_heads_per_s"]
        cpu["unit"] = "tokens·heads/s"
        log(f"[bench] cpu_baseline {cpu['value']} token-heads/s")
    line = {
        "metric": PREFILL_METRIC,
        "value": round(tok_heads / (ms_per_step * 1e-3), 1),
        "unit": "tokens·heads/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16x3" if args.matmul == "split_bf16" else "f32",
        "data": "synthetic",
        "config": {
            "workload": name, "B": cfg.B, "H": cfg.H, "HV": cfg.HV, "dk": cfg.DK, "dv": cfg.DV,
            "tokens_per_request": cfg.tokens, "total_tokens": inp.T,
            "qkv_dtype": cfg.qkv_dtype, "state_dtype": cfg.state_dtype,
            "state_layout": cfg.state_layout, "gate": cfg.gate_mode, "matmul": args.matmul,
            "chunk": CHUNK, "slots": cfg.n_slots, "slot_sets_rotated": rotation,
            "parallelism": "single GPU",
        },
        "kernel_us_mean": round(mean_kernel_ms * 1e3, 2),
        "algorithmic_flops_per_step": flops,
        "algorithmic_bytes_per_step": alg_bytes,
        "hbm": hbm,
        "matrix": matrix,
        "copy_ceiling_GBps": None if copies is None else copies[best],
        "copy_ceiling_kernel": best,
        "copy_kernels_GBps": copies,
        "pct_hbm_peak": round(100.0 * hbm["achieved"] / HBM_PEAK_GBPS, 2),
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
