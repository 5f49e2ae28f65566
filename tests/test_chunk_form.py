"""The chunkwise form that the prefill kernel evaluates, written out in fp64
NumPy and checked against the oracle's token loop.

The pages give the recurrence token by token ("Delta-rule write", the
recurrent equations) and say that the whole-sequence chunk forward is not
pinned.  The prefill kernel regroups the same recurrence over chunks of C
tokens.  With Gamma_t the running sum of the log-decays since the chunk
start (inclusive of token t) and S0 the state before the chunk:

  X = V - Kt S0                    Kt[t] = k_t * exp(Gamma_t)
  Y = Qt S0                        Qt[t] = q_t * exp(Gamma_t)   (q scaled)
  (I + L) U = X                    L[t,s] = beta_s P[t,s], s < t
  O = Y + R' U                     R'[t,s] = beta_s R[t,s],  s <= t
  S = diag(exp(Gamma_last)) S0 + Kup^T U,  Kup[s] = beta_s k_s exp(Gamma_last - Gamma_s)

  P[t,s] = sum_d k_t[d] k_s[d] exp(Gamma_t[d] - Gamma_s[d])
  R[t,s] = sum_d q_t[d] k_s[d] exp(Gamma_t[d] - Gamma_s[d])

P and R are formed as products of Kt/Qt with Ks[s] = k_s exp(-Gamma_s) when
the chunk's decay span max_d(-Gamma_last[d]) is small enough for exp(-Gamma)
to stay finite in fp32.  Wider spans split the chunk's lower triangle
hierarchically (``tiered_pr``): the off-diagonal block between the two
halves of every aligned block of 2h tokens (h = 8, 4, 2, 1) factors through
the last token r of the lower half, exp(Gamma_t - Gamma_s) =
exp(Gamma_t - Gamma_r) exp(Gamma_r - Gamma_s), both factors at most 1 and
each a sum of the gates inside one half (segmented scans, so no large
prefix cancels); the diagonal blocks that remain, of the smallest size
whose decay spans are safe, use the midpoint factoring of their own
tokens, and at size 1 the diagonal is a plain sum.  A ragged last chunk is
padded with tokens whose k, q, v, beta and g are zero; such tokens change
nothing.  These tests pin that regrouping (and the padding) against the
token loop, so a mistake in the algebra the kernel follows shows up on the
CPU.
"""
import math

import numpy as np
import pytest

from gated_delta_rule_82_amd import workloads as wl
from oracle import kda_oracle as ko

SAFE_SPAN = 120.0   # the prefill kernel's one-product bound (natural log units)


def chunk_tile(S0, q, k, v, g, beta, C=16, force_pairwise=False):
    """One (request, head) tile over all its tokens in chunks of C.
    q, k are already normalised (q scaled), g the per-channel log-decays,
    beta the write strengths.  Returns (outputs [n, dv], final state)."""
    n, dk = k.shape
    dv = v.shape[1]
    S = S0.astype(np.float64).copy()
    out = np.zeros((n, dv))
    for c0 in range(0, n, C):
        m = min(C, n - c0)
        pad = lambda a, w: np.concatenate([a, np.zeros((C - m,) + a.shape[1:])]) if m < C else a
        qc, kc, vc, gc = pad(q[c0:c0 + m], 0), pad(k[c0:c0 + m], 0), pad(v[c0:c0 + m], 0), pad(g[c0:c0 + m], 0)
        bc = pad(beta[c0:c0 + m], 0)
        Gam = np.cumsum(gc, axis=0)
        last = Gam[-1]
        Kt = kc * np.exp(Gam)
        Qt = qc * np.exp(Gam)
        Kup = bc[:, None] * kc * np.exp(last[None, :] - Gam)
        if not force_pairwise and float(np.max(-last)) <= SAFE_SPAN:
            Ks = kc * np.exp(-Gam)
            P = Kt @ Ks.T
            R = Qt @ Ks.T
        else:
            E = np.exp(np.minimum(Gam[:, None, :] - Gam[None, :, :], 0.0))   # [t, s, d], s <= t used
            P = np.einsum("td,sd,tsd->ts", kc, kc, E)
            R = np.einsum("td,sd,tsd->ts", qc, kc, E)
        L = np.tril(P, -1) * bc[None, :]
        Rp = np.tril(R, 0) * bc[None, :]
        X = vc - Kt @ S
        U = np.linalg.solve(np.eye(C) + L, X)
        O = Qt @ S + Rp @ U
        S = np.exp(last)[:, None] * S + Kup.T @ U
        out[c0:c0 + m] = O[:m]
    return out, S


def seg_prefix(g, h):
    """Inclusive sums of g over its aligned blocks of h rows (axis 0)."""
    C = g.shape[0]
    out = np.zeros_like(g)
    for b0 in range(0, C, h):
        out[b0:b0 + h] = np.cumsum(g[b0:b0 + h], axis=0)
    return out


def seg_suffix_excl(g, h):
    """Sums of g over the rows after each row inside its aligned block of h."""
    C = g.shape[0]
    out = np.zeros_like(g)
    for b0 in range(0, C, h):
        blk = g[b0:b0 + h]
        rev = np.cumsum(blk[::-1], axis=0)[::-1]          # inclusive suffix
        out[b0:b0 + h] = np.concatenate([rev[1:], np.zeros((1,) + blk.shape[1:])])
    return out


def tiered_pr(q, k, g, tier, C=16):
    """P (s < t entries) and R (s <= t) of one chunk by the hierarchical
    factoring of tier 1..4: off-diagonal levels h = 8 .. 16 >> tier and
    diagonal blocks of 16 >> tier tokens (midpoint factoring; the plain
    diagonal when tier is 4).  Entries above the diagonal are zero."""
    P = np.zeros((C, C))
    R = np.zeros((C, C))
    t_idx, s_idx = np.meshgrid(np.arange(C), np.arange(C), indexing="ij")
    x = t_idx ^ s_idx
    b = C >> tier
    if tier < 4:
        fb = seg_prefix(g, b)
        c = np.repeat(fb[b - 1::b], b, axis=0) / 2.0     # half the block's total
        ep = np.exp(fb - c)
        kp, qp, ks = k * ep, q * ep, k / ep
        own = x < b
        P = np.where(own, kp @ ks.T, P)
        R = np.where(own, qp @ ks.T, R)
    else:
        R = np.where(x == 0, np.sum(q * k, axis=1)[:, None] * np.eye(C), R)
    for lvl in range(1, tier + 1):
        h = 8 >> (lvl - 1)
        upper = (np.arange(C) & h) != 0
        e = np.where(upper[:, None], seg_prefix(g, h), seg_suffix_excl(g, h))
        f = np.exp(e)                                        # every factor <= 1
        aP = np.where(upper[:, None], k * f, 0.0)
        aR = np.where(upper[:, None], q * f, 0.0)
        bK = np.where(upper[:, None], 0.0, k * f)
        own = (x >= h) & (x < 2 * h)
        P = np.where(own, aP @ bK.T, P)
        R = np.where(own, aR @ bK.T, R)
    return np.tril(P, -1), np.tril(R, 0)


def pairwise_pr(q, k, g):
    Gam = np.cumsum(g, axis=0)
    with np.errstate(invalid="ignore"):
        D = Gam[:, None, :] - Gam[None, :, :]
    E = np.exp(np.minimum(np.nan_to_num(D, nan=0.0), 0.0))
    return (np.tril(np.einsum("td,sd,tsd->ts", k, k, E), -1),
            np.tril(np.einsum("td,sd,tsd->ts", q, k, E), 0))


@pytest.mark.parametrize("tier", [1, 2, 3, 4])
@pytest.mark.parametrize("scale", [0.3, 3.0, 20.0])
def test_tiered_factoring_equals_pairwise(tier, scale):
    """Each tier reproduces the pair-by-pair P and R (every factor of the
    off-diagonal levels is at most 1, so this holds for any decay)."""
    rng = np.random.default_rng(40 + tier)
    C, dk = 16, 12
    q = rng.standard_normal((C, dk)); k = rng.standard_normal((C, dk))
    g = -scale * rng.uniform(0, 1, (C, dk))
    P, R = tiered_pr(q, k, g, tier)
    P0, R0 = pairwise_pr(q, k, g)
    tol = 1e-12 * max(1.0, np.abs(P0).max())
    np.testing.assert_allclose(P, P0, rtol=0, atol=tol)
    np.testing.assert_allclose(R, R0, rtol=0, atol=tol)


def test_tier4_handles_infinite_and_huge_decays():
    """Gates of -inf and -1e4 in the middle of a chunk: the level factors are
    exp of sums inside one half, so no infinity meets a zero and no large
    prefix cancels; tier 4 equals the pairwise sums (which see the same
    exact differences here)."""
    rng = np.random.default_rng(44)
    C, dk = 16, 8
    q = rng.standard_normal((C, dk)); k = rng.standard_normal((C, dk))
    g = -rng.uniform(0, 0.5, (C, dk))
    g[5, 0] = -np.inf
    g[9, 1:4] = -1e4
    P, R = tiered_pr(q, k, g, 4)
    assert np.isfinite(P).all() and np.isfinite(R).all()
    # reference: exp(Gamma_t - Gamma_s) as the product of the per-token factors
    E = np.zeros((C, C, dk))
    for t in range(C):
        for s in range(t + 1):
            E[t, s] = np.exp(np.sum(g[s + 1:t + 1], axis=0))
    P0 = np.tril(np.einsum("td,sd,tsd->ts", k, k, E), -1)
    R0 = np.tril(np.einsum("td,sd,tsd->ts", q, k, E), 0)
    np.testing.assert_allclose(P, P0, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(R, R0, rtol=1e-12, atol=1e-14)


def test_tier_choice_bounds_every_factor():
    """The kernel takes the smallest tier whose diagonal blocks each span at
    most the one-product bound; the midpoint factors of those blocks then
    lie within exp(+-bound/2), and every level factor within [0, 1]."""
    rng = np.random.default_rng(45)
    C, dk = 16, 32
    for scale in (2.0, 6.0, 12.0, 30.0, 80.0):
        g = -scale * rng.uniform(0, 1, (C, dk))
        tier = next((t for t in (1, 2, 3) if
                     np.max(-seg_prefix(g, C >> t)[(C >> t) - 1::C >> t]) <= SAFE_SPAN), 4)
        if tier < 4:
            b = C >> tier
            fb = seg_prefix(g, b)
            c = np.repeat(fb[b - 1::b], b, axis=0) / 2.0
            assert np.max(np.abs(fb - c)) <= SAFE_SPAN / 2 + 1e-9
        q = rng.standard_normal((C, dk)); k = rng.standard_normal((C, dk))
        P, R = tiered_pr(q, k, g, tier)
        P0, R0 = pairwise_pr(q, k, g)
        np.testing.assert_allclose(P, P0, rtol=1e-11, atol=1e-11 * np.abs(P0).max())
        np.testing.assert_allclose(R, R0, rtol=1e-11, atol=1e-11 * np.abs(R0).max())


def _per_token(inp, b, hv, gate_mode, lower_bound):
    cfg = inp.cfg
    t0, t1 = int(inp.cu_seqlens[b]), int(inp.cu_seqlens[b + 1])
    h = hv // cfg.G
    q = ko.l2_normalize(inp.q[0, t0:t1, h], 1e-6) * (cfg.DK ** -0.5)
    k = ko.l2_normalize(inp.k[0, t0:t1, h], 1e-6)
    v = inp.v[0, t0:t1, hv].astype(np.float64)
    g = ko.gate(inp.raw_gate[0, t0:t1, hv], inp.dt_bias[hv], float(inp.a_log[hv]), gate_mode, lower_bound)
    beta = ko.write_strength(inp.beta_logits[0, t0:t1, hv])
    return q, k, v, g, beta


@pytest.mark.parametrize("gate_mode,lb,C", [
    (ko.GATE_LOWER_BOUND, -5.0, 16), (ko.GATE_LOWER_BOUND, -5.0, 8),
    (ko.GATE_SOFTPLUS, None, 16), (ko.GATE_LOWER_BOUND, -0.5, 32)])
def test_chunk_form_equals_token_loop(gate_mode, lb, C):
    cfg = wl.Workload(name="chunk", B=3, H=2, HV=4, DK=16, DV=8, n_slots=4, qkv_dtype="f32",
                      cu_seqlens=(0, 37, 37 + 16, 37 + 16 + 5), state_indices=(1, 3, 0),
                      host_state=True, state_sigma=0.3,
                      gate_mode=wl.LOWER_BOUND if lb is not None else wl.SOFTPLUS,
                      lower_bound=lb if lb is not None else 0.0)
    inp = wl.draw(cfg)
    for b in range(cfg.B):
        for hv in range(cfg.HV):
            S0 = inp.touched_state[b, hv].astype(np.float64)
            t0, t1 = int(inp.cu_seqlens[b]), int(inp.cu_seqlens[b + 1])
            o_ref, S_ref = ko.decode_tile(
                S0, inp.q[0, t0:t1, hv // cfg.G], inp.k[0, t0:t1, hv // cfg.G], inp.v[0, t0:t1, hv],
                inp.raw_gate[0, t0:t1, hv], inp.beta_logits[0, t0:t1, hv], float(inp.a_log[hv]),
                inp.dt_bias[hv], gate_mode=gate_mode, lower_bound=lb)
            q, k, v, g, beta = _per_token(inp, b, hv, gate_mode, lb)
            o, S = chunk_tile(S0, q, k, v, g, beta, C=C)
            np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-11 * max(1.0, np.abs(o_ref).max()))
            np.testing.assert_allclose(S, S_ref, rtol=0, atol=1e-11 * np.abs(S_ref).max())


def test_pairwise_and_factored_agree_when_safe():
    rng = np.random.default_rng(5)
    n, dk, dv = 16, 12, 6
    q = rng.standard_normal((n, dk)); k = rng.standard_normal((n, dk))
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = rng.standard_normal((n, dv)); g = -rng.uniform(0, 4, (n, dk)); beta = rng.uniform(0, 1, n)
    S0 = rng.standard_normal((dk, dv))
    assert float(np.max(-g.sum(axis=0))) <= SAFE_SPAN
    a = chunk_tile(S0, q, k, v, g, beta)
    b = chunk_tile(S0, q, k, v, g, beta, force_pairwise=True)
    np.testing.assert_allclose(a[0], b[0], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(a[1], b[1], rtol=1e-12, atol=1e-12)


def test_strong_decay_needs_the_pairwise_form():
    """With a decay span far beyond fp64's exponent range the factored
    products overflow; the pair-by-pair form still matches the token loop."""
    rng = np.random.default_rng(6)
    n, dk, dv = 16, 8, 4
    q = rng.standard_normal((n, dk)); k = rng.standard_normal((n, dk))
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = rng.standard_normal((n, dv)); g = np.full((n, dk), -60.0); beta = rng.uniform(0, 1, n)
    S0 = rng.standard_normal((dk, dv))
    o, S = chunk_tile(S0, q, k, v, g, beta)           # span 960 > SAFE_SPAN: pairwise
    S_ref = S0.copy(); o_ref = np.zeros((n, dv))
    for t in range(n):
        S_ref = np.exp(g[t])[:, None] * S_ref
        S_ref = S_ref + np.outer(beta[t] * k[t], v[t] - k[t] @ S_ref)
        o_ref[t] = q[t] @ S_ref
    np.testing.assert_allclose(o, o_ref, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(S, S_ref, rtol=1e-10, atol=1e-300)
    assert math.isfinite(float(np.abs(o).max()))


def _chunk_group_tiers(inp, group=32, C=16):
    """The P, R form of every (request, value head, chunk, channel group) of
    a drawn workload, as the prefill picks it per wave's channel group from
    the oracle's gate: 0 for the one product, else the smallest tier 1..4
    whose diagonal blocks (8, 4, 2, 1 tokens) span at most SAFE_SPAN."""
    cfg = inp.cfg
    tiers = []
    for b in range(cfg.B):
        t0, t1 = int(inp.cu_seqlens[b]), int(inp.cu_seqlens[b + 1])
        if int(inp.state_indices[b]) < 0:
            continue
        for hv in range(cfg.HV):
            g = ko.gate(inp.raw_gate[0, t0:t1, hv], inp.dt_bias[hv], inp.a_log[hv],
                        gate_mode=cfg.gate_mode,
                        lower_bound=cfg.lower_bound if cfg.gate_mode == wl.LOWER_BOUND else None)
            for c0 in range(0, t1 - t0, C):
                gc = g[c0:c0 + C]
                gc = np.concatenate([gc, np.zeros((C - len(gc), gc.shape[1]))])
                for d0 in range(0, cfg.DK, group):
                    gg = gc[:, d0:d0 + group]
                    with np.errstate(invalid="ignore"):
                        span = lambda b: float(np.max(-seg_prefix(gg, b)))
                        tiers.append(next((t for t, b in enumerate((16, 8, 4, 2)) if span(b) <= SAFE_SPAN), 4))
    return np.array(tiers)


def test_prefill_gpu_cases_reach_every_p_r_form():
    """The GPU prefill cases must run every form of P and R: the lower-bound
    cases (span <= 16 * 5) only the one product, the softplus cases (with
    the strong-gate shifts of the degenerate tests) each of the wide tiers."""
    from tests.test_gpu_prefill import CASES
    seen = set()
    for name, cfg in CASES.items():
        tiers = _chunk_group_tiers(wl.draw(cfg), group=min(32, cfg.DK))
        if cfg.gate_mode == wl.SOFTPLUS:
            seen |= set(tiers.tolist())
        else:
            assert tiers.max() == 0, name
    from tests.test_gpu_degenerate import STRONG_SHIFTS, strong_softplus_inputs
    for shift in STRONG_SHIFTS:
        seen |= set(_chunk_group_tiers(strong_softplus_inputs(shift)).tolist())
    assert seen == {0, 1, 2, 3, 4}, seen
