"""Benchmark of the KDA decode op on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
    python bench.py --prefill [--matmul split_bf16|f32]

A step is one kda_decode call over one batch of the workload (default: the
96-head layer, B=256 requests x 1 token, dk = dv = 128, bf16 q/k/v, fp32
state pool of 512 slots).  All inputs are resident in HBM before timing.
Prints one JSON line on stdout; progress goes to stderr.

--prefill times kda_prefill instead (the chunked whole-sequence form on the
matrix cores; default workload B=8 x 2048 tokens, 96 heads, value-first
fp32 state): value is tokens x heads per second, and the roofline is the
matrix one -- algorithmic flops of the chunk form (X, Y, the state update,
U, O and the P, R products; 16-token chunks, a ragged chunk counted whole)
over the mean kernel time, against the dense bf16 peak (split-bf16
products) or the fp32 matrix peak.

Fields beyond the common ones:
  roofline      HBM roofline of the decode kernel: achieved = algorithmic
                bytes per launch (state read + write of every active tile,
                plus every token tensor once) / mean kernel time measured
                with HIP events on the launch stream; peak 8000 GB/s;
                traffic = HBM bytes per launch from the committed rocprofv3
                FETCH_SIZE / WRITE_SIZE summary (null when the kernel source
                changed since the counters were taken).
  cpu_baseline  the fp64 oracle timed on host cores on a bounded sample of
                the same workload (one BLAS thread).
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


def cpu_baseline(inp, pool_t, budget_s: float, heads_per_step=None):
    """Time the fp64 oracle on the workload's (request, head) tiles in order
    (wrapping around to further passes), one BLAS thread, until about
    ``budget_s`` seconds of work are done.  A step is up to 8 requests with
    all their heads, or ``heads_per_step`` heads of one request."""
    from threadpoolctl import threadpool_limits
    import torch
    from oracle import kda_oracle as ko

    def gather_tiles(slots, hvs):
        s = torch.as_tensor(slots, dtype=torch.int64, device=pool_t.device)
        h = torch.as_tensor(hvs, dtype=torch.int64, device=pool_t.device)
        return pool_t[s, h].float().cpu().numpy()

    cfg = inp.cfg
    lb = cfg.lower_bound if cfg.gate_mode == "lower_bound" else None
    order = [(bb, hv) for bb in range(cfg.B) for hv in range(cfg.HV)]
    per = heads_per_step or 8 * cfg.HV
    done_tiles, done_th, done_state, elapsed = 0, 0, 0, 0.0
    with threadpool_limits(limits=1):
        i = 0
        while elapsed < budget_s:
            if i >= len(order):     # whole batch done: start another pass
                i = 0
            tiles = order[i:i + per]
            valid = [(bb, hv) for bb, hv in tiles if inp.state_indices[bb] >= 0]
            init = gather_tiles([int(inp.state_indices[bb]) for bb, _ in valid],
                                [hv for _, hv in valid])
            pool = {(int(inp.state_indices[bb]), hv): S for (bb, hv), S in zip(valid, init)}
            t0 = time.perf_counter()
            ko.kda_decode(inp.q, inp.k, inp.v, inp.raw_gate, inp.beta_logits, inp.a_log,
                          inp.dt_bias, inp.cu_seqlens, pool, inp.state_indices, tiles=tiles,
                          gate_mode=cfg.gate_mode, lower_bound=lb, state_layout=cfg.state_layout,
                          state_dtype=cfg.state_dtype)
            elapsed += time.perf_counter() - t0
            for bb, hv in tiles:
                n = int(inp.cu_seqlens[bb + 1] - inp.cu_seqlens[bb])
                done_th += n
                if n > 0 and inp.state_indices[bb] >= 0:
                    done_state += 2 * cfg.DK * cfg.DV * cfg.state_elem_bytes
            done_tiles += len(tiles)
            i += per
    total = len(order)
    return {
        "value": round(done_state / elapsed / 1e9, 6),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"{done_tiles} (request, head) tiles ({done_tiles / total:.3f} passes over the "
                  f"batch's {total}), all their tokens: {done_th} token-heads in "
                  f"{elapsed:.1f} s, fp64 numpy, 1 BLAS thread",
        "tokens_heads_per_s": round(done_th / elapsed, 3),
        "host_cores_available": len(os.sched_getaffinity(0)),
    }


def copy_ceiling(nbytes: int, reps: int = 10):
    """Plain streaming copies moving ``nbytes`` (half read, half written):
    torch's device-to-device copy and an elementwise multiply-by-one kernel.
    Returns {name: GB/s of read + write bytes}; both also serve as the
    known-size reference kernels for the HBM byte counters."""
    import torch
    n = nbytes // 2 // 4
    src = torch.empty(n, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    variants = {"d2d_copy": lambda: dst.copy_(src),
                "elementwise_copy": lambda: torch.mul(src, 1.0, out=dst)}
    res = {}
    for name, fn in variants.items():
        fn()
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(reps):
            fn()
        e.record()
        torch.cuda.synchronize()
        ms = s.elapsed_time(e) / reps
        res[name] = round(2 * n * 4 / (ms * 1e-3) / 1e9, 1)
    del src, dst
    return res


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--state-layout", choices=("k_first", "v_first"), default=None,
                    help="default: the workload's (key-first for the decode batches)")
    ap.add_argument("--state-dtype", choices=("f32", "bf16"), default=None)
    ap.add_argument("--prefill", action="store_true",
                    help="time kda_prefill (chunked, matrix cores) on the prefill workload")
    ap.add_argument("--matmul", choices=("split_bf16", "f32"), default="split_bf16",
                    help="matrix precision of --prefill")
    ap.add_argument("--conv", action="store_true",
                    help="time kda_decode_conv: the step with the short convolutions in front")
    ap.add_argument("--cpu-budget", type=float, default=12.0,
                    help="seconds of oracle work for cpu_baseline (0 disables)")
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
    import torch
    from gated_delta_rule_82_amd import kda
    from gated_delta_rule_82_amd import workloads as wl

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    kda.library()     # fail loudly if the HIP library is not built

    name = args.workload or (wl.PREFILL_HEADLINE if args.prefill else wl.HEADLINE)
    over = {k: v for k, v in (("state_layout", args.state_layout), ("state_dtype", args.state_dtype))
            if v is not None}
    cfg = wl.preset(name, **over)
    log(f"[bench] workload {name}: {cfg.description}")
    inp = wl.draw(cfg)
    dev = wl.to_device(inp)
    pool = wl.device_pool(inp)
    out = wl.empty_out(inp)
    state_b = wl.state_bytes(cfg, inp)
    token_b = wl.token_bytes(cfg, inp)
    alg_bytes = state_b + token_b
    tok_heads = inp.T * cfg.HV
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    handle = stream.cuda_stream
    mode = dict(gate_mode=cfg.gate_mode, lower_bound=cfg.lower_bound, state_layout=cfg.state_layout)

    if args.conv:
        ci = wl.draw_conv(inp)
        cd = wl.conv_to_device(ci, cfg.qkv_dtype)
        conv_bytes = wl.conv_bytes(cfg, inp, ci.K)
        alg_bytes += conv_bytes
        torch.cuda.synchronize()

        def step():
            kda.decode_conv(out, cd["x_q"], cd["x_k"], cd["x_v"], cd["w_q"], cd["w_k"], cd["w_v"],
                            cd["win_q"], cd["win_k"], cd["win_v"], cd["q_conv"], cd["k_conv"],
                            dev["raw_gate"], dev["beta_logits"], dev["a_log"], dev["dt_bias"],
                            dev["cu_seqlens"], pool, dev["state_indices"], stream=handle, **mode)
    elif args.prefill:
        def step():
            kda.prefill(out, dev["q"], dev["k"], dev["v"], dev["raw_gate"], dev["beta_logits"],
                        dev["a_log"], dev["dt_bias"], dev["cu_seqlens"], pool, dev["state_indices"],
                        stream=handle, matmul=args.matmul, **mode)
    else:
        def step():
            kda.decode(out, dev["q"], dev["k"], dev["v"], dev["raw_gate"], dev["beta_logits"],
                       dev["a_log"], dev["dt_bias"], dev["cu_seqlens"], pool, dev["state_indices"],
                       stream=handle, **mode)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] warmup {args.warmup} done; timing {args.steps} steps")

    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kernel_ms = np.array([s.elapsed_time(e) for s, e in zip(starts, ends)])
    ms_per_step = wall * 1e3 / args.steps
    mean_kernel_ms = float(kernel_ms.mean())
    log(f"[bench] wall {ms_per_step * 1e3:.1f} us/step, kernel mean {mean_kernel_ms * 1e3:.1f} us "
        f"(min {kernel_ms.min() * 1e3:.1f}, max {kernel_ms.max() * 1e3:.1f})")

    if args.prefill:
        return report_prefill(args, cfg, name, inp, pool, ms_per_step, mean_kernel_ms, alg_bytes,
                              tok_heads)

    value = state_b / (ms_per_step * 1e-3) / 1e9
    achieved = alg_bytes / (mean_kernel_ms * 1e-3) / 1e9
    variant = "" if (cfg.state_layout, cfg.state_dtype) == ("k_first", "f32") else \
        f"_{cfg.state_layout}_{cfg.state_dtype}"
    if args.conv:
        variant += "_conv"
    traffic, traffic_src = committed_traffic(name + variant)
    log(f"[bench] traffic: {traffic} ({traffic_src})")

    copy_gbps = None
    if not args.no_copy_ceiling:
        copies = copy_ceiling(state_b)
        copy_gbps = max(copies.values())
        log(f"[bench] copy ceiling (read+write, {state_b / 1e9:.2f} GB): {copies}")

    cpu = None
    if args.cpu_budget > 0:
        log(f"[bench] cpu_baseline: oracle for ~{args.cpu_budget:.0f} s")
        cpu = cpu_baseline(inp, pool, args.cpu_budget) if not args.conv else None
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
            "short_conv": bool(args.conv),
            "slots": cfg.n_slots, "parallelism": "single GPU",
        },
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBPS, 2),
        "tokens_heads_per_s": round(tok_heads / (ms_per_step * 1e-3), 1),
        "state_bytes_per_step": state_b,
        "algorithmic_bytes_per_step": alg_bytes,
        "kernel_us_mean": round(mean_kernel_ms * 1e3, 2),
        "copy_ceiling_GBps": None if copy_gbps is None else round(copy_gbps, 1),
        "copy_kernels_GBps": None if copy_gbps is None else copies,
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


def report_prefill(args, cfg, name, inp, pool, ms_per_step, mean_kernel_ms, alg_bytes, tok_heads):
    import numpy as np
    counts = np.diff(inp.cu_seqlens)
    active = (counts > 0) & (inp.state_indices >= 0)
    chunks = int((-(-counts[active] // CHUNK)).sum()) * cfg.HV
    flops = chunks * chunk_flops(cfg.DK, cfg.DV)
    achieved = flops / (mean_kernel_ms * 1e-3) / 1e12
    peak = MATRIX_PEAK_TFLOPS[args.matmul]
    hbm = alg_bytes / (mean_kernel_ms * 1e-3) / 1e9
    variant = f"_{args.matmul}"
    traffic, traffic_src = committed_traffic(name + variant, "kda_prefill")
    log(f"[bench] traffic: {traffic} ({traffic_src})")
    copies = None
    if not args.no_copy_ceiling:
        copies = copy_ceiling(alg_bytes)
        log(f"[bench] copy ceiling (read+write, {alg_bytes / 1e9:.2f} GB): {copies}")
    cpu = None
    if args.cpu_budget > 0:
        log(f"[bench] cpu_baseline: oracle for ~{args.cpu_budget:.0f} s")
        cpu = cpu_baseline(inp, pool, args.cpu_budget, heads_per_step=4)
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
            "chunk": CHUNK, "slots": cfg.n_slots, "parallelism": "single GPU",
        },
        "kernel_us_mean": round(mean_kernel_ms * 1e3, 2),
        "algorithmic_flops_per_step": flops,
        "algorithmic_bytes_per_step": alg_bytes,
        "hbm_GBps": round(hbm, 1),
        "copy_kernels_GBps": copies,
        "pct_hbm_peak": round(100.0 * hbm / HBM_PEAK_GBPS, 2),
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 3),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4),
            "traffic": traffic,
            "kernel": "kda_prefill_chunks<%d,%d,%s q/k/v,%s state,%s,%s>" % (
                cfg.DK, cfg.DV, cfg.qkv_dtype, cfg.state_dtype, cfg.state_layout.replace("_", ""),
                args.matmul),
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
