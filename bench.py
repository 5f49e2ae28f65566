"""Benchmark of the KDA decode op on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one kda_decode call over one batch of the workload (default: the
96-head layer, B=256 requests x 1 token, dk = dv = 128, bf16 q/k/v, fp32
state pool of 512 slots).  All inputs are resident in HBM before timing.
Prints one JSON line on stdout; progress goes to stderr.

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
HBM_PEAK_GBPS = 8000.0
KERNEL_SOURCE = os.path.join(ROOT, "gated_delta_rule_82_amd", "csrc", "kda_decode.hip")
PROFILES = os.path.join(ROOT, "profiles")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    with open(KERNEL_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def committed_traffic(workload: str):
    """HBM bytes per launch from profiles/kda_decode_<workload>_counters.md, if
    that summary was taken on the current kernel source."""
    path = os.path.join(PROFILES, f"kda_decode_{workload}_counters.md")
    if not os.path.exists(path):
        return None, "no counter summary"
    text = open(path).read()
    m_hash = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    m_bytes = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not (m_hash and m_bytes):
        return None, "summary lacks traffic fields"
    if m_hash.group(1) != kernel_source_hash():
        return None, "kernel changed since counters were taken"
    return float(m_bytes.group(1)), path


def cpu_baseline(inp, pool_t, budget_s: float):
    """Time the fp64 oracle on the workload's requests in order (wrapping
    around to further passes), one BLAS thread, until about ``budget_s``
    seconds of work are done."""
    import numpy as np
    from threadpoolctl import threadpool_limits
    import torch
    from oracle import kda_oracle as ko

    def gather_tiles(slots, hvs):
        s = torch.as_tensor(slots, dtype=torch.int64, device=pool_t.device)
        h = torch.as_tensor(hvs, dtype=torch.int64, device=pool_t.device)
        return pool_t[s, h].float().cpu().numpy()

    cfg = inp.cfg
    lb = cfg.lower_bound if cfg.gate_mode == "lower_bound" else None
    done_req, done_th, done_state, elapsed = 0, 0, 0, 0.0
    with threadpool_limits(limits=1):
        b = 0
        while elapsed < budget_s:
            if b >= cfg.B:          # whole batch done: start another pass
                b = 0
            step = max(1, min(8, cfg.B - b))
            tiles = [(bb, hv) for bb in range(b, b + step) for hv in range(cfg.HV)]
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
            counts = np.diff(inp.cu_seqlens[b:b + step + 1])
            done_th += int(counts.sum()) * cfg.HV
            done_state += int(((counts > 0) & (inp.state_indices[b:b + step] >= 0)).sum()) \
                * cfg.HV * 2 * cfg.DK * cfg.DV * cfg.state_elem_bytes
            done_req += step
            b += step
    return {
        "value": round(done_state / elapsed / 1e9, 6),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"{done_req} requests x {cfg.HV} heads ({done_req / cfg.B:.2f} passes over the "
                  f"{cfg.B}-request batch), all their tokens: {done_th} token-heads in "
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
    ap.add_argument("--state-layout", choices=("k_first", "v_first"), default="k_first")
    ap.add_argument("--state-dtype", choices=("f32", "bf16"), default="f32")
    ap.add_argument("--conv", action="store_true",
                    help="time kda_decode_conv: the step with the short convolutions in front")
    ap.add_argument("--cpu-budget", type=float, default=12.0,
                    help="seconds of oracle work for cpu_baseline (0 disables)")
    ap.add_argument("--no-copy-ceiling", action="store_true")
    args = ap.parse_args(argv)

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

    name = args.workload or wl.HEADLINE
    cfg = wl.preset(name, state_layout=args.state_layout, state_dtype=args.state_dtype)
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


if __name__ == "__main__":
    sys.exit(main())
