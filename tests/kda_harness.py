"""Shared GPU-test plumbing: run the HIP path through the C ABI binding and
compare it with the fp64 oracle on the same seeded inputs.

Tolerances (fixed here, used by every GPU parity test):
  * fp32 state, per (request, head) tile: max|dS| / max|S_ref| <= 1e-4
    (required bound) and <= STATE_TIGHT (what fp32 arithmetic gives).
  * bf16 output: max|do| <= 2e-2 absolute (required bound) and, per element,
    |o_gpu - o_ref| <= 1 bf16 ulp of o_ref + 1e-5 * max|o_ref| (the rounding
    to bf16 costs half an ulp; fp32 arithmetic adds far less than the rest).
  * fp32 output: max|do| / max|o_ref| <= 1e-5.
  * bf16 state pool: both sides round the advanced state to bf16 once, so
    per element |S_gpu - S_ref| <= 1 bf16 ulp of S_ref (+ 1e-6 * max|S_ref|,
    the fp32 arithmetic's share; the prefill uses its tight state bound).
  * state_indices gathers: every slot not named in state_indices is
    bit-identical after the call.

The chunked prefill (kda_prefill) keeps the required bounds; its tight
bounds follow its matrix precision (PREFILL_TOL): the split-bf16 products
carry 16 significant bits per operand (relative error up to about 2^-16 =
1.5e-5 per product; observed state error up to 1.4e-5 of max|S|, bound
3e-5), the fp32 products fp32 rounding through the chunk's regrouping and
the triangular solve (observed up to 6e-6, bound 1e-5).
"""
from __future__ import annotations

import numpy as np

from gated_delta_rule_82_amd import workloads as wl
from oracle import kda_oracle as ko

STATE_REQUIRED = 1e-4
STATE_TIGHT = 2e-6
OUT_ABS_REQUIRED = 2e-2
OUT_ULP_FLOOR = 1e-5
OUT_F32_REL = 1e-5
STATE_BF16_FLOOR = 1e-6

DECODE_TOL = dict(state_tight=STATE_TIGHT, out_floor=OUT_ULP_FLOOR, out_f32_rel=OUT_F32_REL,
                  state_bf16_floor=STATE_BF16_FLOOR)
PREFILL_TOL = {
    "split_bf16": dict(state_tight=3e-5, out_floor=1e-4, out_f32_rel=1e-4, state_bf16_floor=3e-5),
    "f32": dict(state_tight=1e-5, out_floor=1e-5, out_f32_rel=1e-5, state_bf16_floor=1e-5),
}


def bf16_ulp(x):
    """Spacing of bfloat16 values at |x| (subnormal spacing below 2^-126)."""
    _, e = np.frexp(np.abs(np.asarray(x, dtype=np.float64)))
    return np.ldexp(1.0, np.maximum(e - 8, -133))


def out_to_f64(out_t):
    import torch
    return out_t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def gather_tiles(pool_t, slots, hvs):
    import torch
    s = torch.as_tensor(np.asarray(slots, dtype=np.int64), device=pool_t.device)
    h = torch.as_tensor(np.asarray(hvs, dtype=np.int64), device=pool_t.device)
    return pool_t[s, h].float().cpu().numpy()


def choose_tiles(inp, sample, seed=123):
    cfg = inp.cfg
    all_tiles = [(b, hv) for b in range(cfg.B) for hv in range(cfg.HV)]
    if sample is None or sample >= len(all_tiles):
        return all_tiles
    rng = np.random.default_rng(seed)
    pick = rng.choice(len(all_tiles), size=sample, replace=False)
    # always include the first and the last tile (grid edges)
    chosen = {all_tiles[0], all_tiles[-1]} | {all_tiles[i] for i in pick}
    return sorted(chosen)


def run_gpu(inp, dev, pool_t, out_t=None, mode_overrides=None, stream=None, entry="decode",
            matmul="split_bf16"):
    from gated_delta_rule_82_amd import kda
    cfg = inp.cfg
    if out_t is None:
        out_t = wl.empty_out(inp, pool_t.device)
    mode = dict(gate_mode=cfg.gate_mode, lower_bound=cfg.lower_bound, state_layout=cfg.state_layout)
    if mode_overrides:
        mode.update(mode_overrides)
    args = (out_t, dev["q"], dev["k"], dev["v"], dev["raw_gate"], dev["beta_logits"],
            dev["a_log"], dev["dt_bias"], dev["cu_seqlens"], pool_t, dev["state_indices"])
    if entry == "prefill":
        kda.prefill(*args, stream=stream, matmul=matmul, **mode)
    else:
        kda.decode(*args, stream=stream, **mode)
    return out_t


def oracle_tiles(inp, tiles, init_states, **mode):
    """Oracle over ``tiles``; ``init_states`` holds the initial state of each
    tile whose request has a valid slot, in the order of ``tiles``."""
    cfg = inp.cfg
    pool = {}
    valid = [(b, hv) for b, hv in tiles if inp.state_indices[b] >= 0]
    assert len(valid) == len(init_states)
    for (b, hv), S in zip(valid, init_states):
        pool[(int(inp.state_indices[b]), hv)] = S
    kw = dict(gate_mode=cfg.gate_mode,
              lower_bound=cfg.lower_bound if cfg.gate_mode == ko.GATE_LOWER_BOUND else None,
              state_layout=cfg.state_layout, state_dtype=cfg.state_dtype)
    kw.update(mode)
    return ko.kda_decode(inp.q, inp.k, inp.v, inp.raw_gate, inp.beta_logits, inp.a_log,
                         inp.dt_bias, inp.cu_seqlens, pool, inp.state_indices, tiles=tiles, **kw)


def compare_outputs(inp, tiles, out_gpu, out_ref, out_floor=OUT_ULP_FLOOR, out_f32_rel=OUT_F32_REL):
    """Element checks on the output rows of the chosen tiles; returns stats."""
    cfg = inp.cfg
    rows_g, rows_r = [], []
    for b, hv in tiles:
        t0, t1 = int(inp.cu_seqlens[b]), int(inp.cu_seqlens[b + 1])
        if t1 > t0:
            rows_g.append(out_gpu[0, t0:t1, hv])
            rows_r.append(out_ref[0, t0:t1, hv])
    if not rows_g:
        return {"out_max_abs": 0.0}
    g = np.concatenate(rows_g)
    r = np.concatenate(rows_r)
    assert np.isfinite(g).all(), "non-finite output"
    diff = np.abs(g - r)
    scale = float(np.max(np.abs(r))) if r.size else 0.0
    stats = {"out_max_abs": float(diff.max()), "out_ref_max": scale}
    if cfg.qkv_dtype == "bf16":
        assert diff.max() <= OUT_ABS_REQUIRED, f"bf16 out abs err {diff.max():.3e} > {OUT_ABS_REQUIRED}"
        bound = bf16_ulp(r) + out_floor * scale
        worst = float(np.max(diff / bound))
        stats["out_ulp_ratio"] = worst
        assert worst <= 1.0, f"bf16 out exceeds 1 ulp + floor (ratio {worst:.3f})"
    else:
        rel = float(diff.max() / max(scale, 1e-30))
        stats["out_rel"] = rel
        assert rel <= out_f32_rel, f"fp32 out rel err {rel:.3e} > {out_f32_rel}"
    return stats


def compare_states(states_gpu, states_ref, state_dtype="f32", state_tight=STATE_TIGHT,
                   bf16_floor=STATE_BF16_FLOOR):
    if state_dtype == "bf16":
        # both sides round once to bf16: equal, or one ulp apart where the
        # fp32 and fp64 results straddle a rounding boundary
        worst = 0.0
        for Sg, Sr in zip(states_gpu, states_ref):
            bound = bf16_ulp(Sr) + bf16_floor * float(np.max(np.abs(Sr)))
            worst = max(worst, float(np.max(np.abs(Sg.astype(np.float64) - Sr) / bound)))
        assert worst <= 1.0, f"bf16 state exceeds 1 ulp (ratio {worst:.3f})"
        return {"state_ulp_ratio": worst}
    worst = 0.0
    for Sg, Sr in zip(states_gpu, states_ref):
        denom = float(np.max(np.abs(Sr)))
        err = float(np.max(np.abs(Sg.astype(np.float64) - Sr)))
        rel = err / denom if denom > 0 else err
        worst = max(worst, rel)
    assert worst <= STATE_REQUIRED, f"state rel err {worst:.3e} > {STATE_REQUIRED}"
    assert worst <= state_tight, f"state rel err {worst:.3e} > tight bound {state_tight}"
    return {"state_rel": worst}


def parity_case(inp, device="cuda", sample=None, check_untouched=True, mode_overrides=None,
                oracle_mode=None, pool_t=None, entry="decode", matmul="split_bf16", tol=None):
    """Run one batch on the GPU (kda_decode, or kda_prefill with ``matmul``)
    and check it against the oracle.  Returns a dict with the observed errors.
    ``tol`` replaces the tight bounds (the required ones always apply)."""
    if tol is None:
        tol = PREFILL_TOL[matmul] if entry == "prefill" else DECODE_TOL
    import torch
    cfg = inp.cfg
    dev = wl.to_device(inp, device)
    if pool_t is None:
        pool_t = wl.device_pool(inp, device)
    tiles = choose_tiles(inp, sample)
    valid = [(b, hv) for b, hv in tiles if inp.state_indices[b] >= 0]
    slots = [int(inp.state_indices[b]) for b, hv in valid]
    hvs = [hv for b, hv in valid]
    init = gather_tiles(pool_t, slots, hvs) if valid else []
    before = pool_t.clone() if check_untouched else None
    out_t = wl.empty_out(inp, device)
    out_t.fill_(float("nan"))
    run_gpu(inp, dev, pool_t, out_t, mode_overrides, entry=entry, matmul=matmul)
    torch.cuda.synchronize()
    out_gpu = out_to_f64(out_t)
    after = gather_tiles(pool_t, slots, hvs) if valid else []

    out_ref, pool_ref = oracle_tiles(inp, tiles, init, **(oracle_mode or {}))
    stats = compare_outputs(inp, tiles, out_gpu, out_ref, tol["out_floor"], tol["out_f32_rel"])
    ref_states = [pool_ref[(s, hv)] for s, hv in zip(slots, hvs)]
    stats.update(compare_states(after, ref_states, cfg.state_dtype, tol["state_tight"],
                                tol["state_bf16_floor"]) if valid else {})
    # skipped requests: zero rows
    for b, hv in tiles:
        if inp.state_indices[b] < 0:
            t0, t1 = int(inp.cu_seqlens[b]), int(inp.cu_seqlens[b + 1])
            assert np.all(out_gpu[0, t0:t1, hv] == 0.0)
    if check_untouched:
        touched = sorted({int(s) for s, c in zip(inp.state_indices, np.diff(inp.cu_seqlens))
                          if s >= 0 and c > 0})
        mask = torch.ones(cfg.n_slots, dtype=torch.bool, device=pool_t.device)
        if touched:
            mask[torch.as_tensor(touched, device=pool_t.device)] = False
        assert torch.equal(pool_t[mask], before[mask]), "a slot outside state_indices changed"
        del before
    stats["tiles"] = len(tiles)
    return stats, out_t, pool_t


CONV_REL = 1e-5   # convolved q/k (fp32 SiLU of a K-term sum) against the oracle


def conv_parity_case(inp, ci, device="cuda", sample=None, in_place=False):
    """kda_decode_conv on the GPU against the oracle's decode step with the
    convolutions in front.  Checks outputs and states as parity_case does,
    the convolved q/k (relative CONV_REL), and every window bit-exact (they
    hold copies of pre-convolution inputs)."""
    import torch
    from gated_delta_rule_82_amd import kda
    cfg = inp.cfg
    dev = wl.to_device(inp, device)
    cd = wl.conv_to_device(ci, cfg.qkv_dtype, device)
    if in_place:          # fp32 activations convolved in place
        cd["q_conv"], cd["k_conv"] = cd["x_q"], cd["x_k"]
    pool_t = wl.device_pool(inp, device)
    tiles = choose_tiles(inp, sample)
    valid = [(b, hv) for b, hv in tiles if inp.state_indices[b] >= 0]
    slots = [int(inp.state_indices[b]) for b, hv in valid]
    hvs = [hv for b, hv in valid]
    init = gather_tiles(pool_t, slots, hvs) if valid else []
    out_t = wl.empty_out(inp, device)
    out_t.fill_(float("nan"))
    if not in_place:
        cd["q_conv"].fill_(float("nan"))
        cd["k_conv"].fill_(float("nan"))
    kda.decode_conv(out_t, cd["x_q"], cd["x_k"], cd["x_v"], cd["w_q"], cd["w_k"], cd["w_v"],
                    cd["win_q"], cd["win_k"], cd["win_v"], cd["q_conv"], cd["k_conv"],
                    dev["raw_gate"], dev["beta_logits"], dev["a_log"], dev["dt_bias"],
                    dev["cu_seqlens"], pool_t, dev["state_indices"], gate_mode=cfg.gate_mode,
                    lower_bound=cfg.lower_bound, state_layout=cfg.state_layout)
    torch.cuda.synchronize()
    out_gpu = out_to_f64(out_t)
    after = gather_tiles(pool_t, slots, hvs) if valid else []

    pool = {(s, hv): S for s, hv, S in zip(slots, hvs, init)}
    lb = cfg.lower_bound if cfg.gate_mode == ko.GATE_LOWER_BOUND else None
    out_ref, pool_ref, wq, wk, wv, qc, kc = ko.kda_decode_conv(
        ci.x["q"], ci.x["k"], ci.x["v"], ci.w["q"], ci.w["k"], ci.w["v"], ci.win["q"],
        ci.win["k"], ci.win["v"], inp.raw_gate, inp.beta_logits, inp.a_log, inp.dt_bias,
        inp.cu_seqlens, pool, inp.state_indices, tiles=tiles, gate_mode=cfg.gate_mode,
        lower_bound=lb, state_layout=cfg.state_layout, state_dtype=cfg.state_dtype)
    stats = compare_outputs(inp, tiles, out_gpu, out_ref)
    if valid:
        stats.update(compare_states(after, [pool_ref[(s, hv)] for s, hv in zip(slots, hvs)],
                                    cfg.state_dtype))
    for name, ref in (("win_q", wq), ("win_k", wk), ("win_v", wv)):
        got = cd[name].cpu().numpy().astype(np.float64)
        assert np.array_equal(got, ref), f"{name} differs"
    worst = 0.0
    for name, ref in (("q_conv", qc), ("k_conv", kc)):
        got = cd[name].float().cpu().numpy().astype(np.float64)
        assert np.isfinite(got).all(), f"{name} has non-finite values"
        bound = CONV_REL * np.abs(ref) + 1e-6 * max(float(np.abs(ref).max()), 1e-30)
        worst = max(worst, float(np.max(np.abs(got - ref) / bound)))
    assert worst <= 1.0, f"convolved q/k exceed tolerance (ratio {worst:.3f})"
    stats["conv_ratio"] = worst
    stats["tiles"] = len(tiles)
    return stats
