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
to stay finite in fp32, and pair by pair otherwise.  A ragged last chunk is
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

SAFE_SPAN = 80.0


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


def _chunk_group_spans(inp, group=32, C=16):
    """max_d -Gamma_last[d] of every (request, value head, chunk, channel group)
    of a drawn workload, from the oracle's gate: the quantity the prefill
    compares with its one-product bound, per wave's channel group."""
    cfg = inp.cfg
    spans = []
    for b in range(cfg.B):
        t0, t1 = int(inp.cu_seqlens[b]), int(inp.cu_seqlens[b + 1])
        if int(inp.state_indices[b]) < 0:
            continue
        for hv in range(cfg.HV):
            g = ko.gate(inp.raw_gate[0, t0:t1, hv], inp.dt_bias[hv], inp.a_log[hv],
                        gate_mode=cfg.gate_mode,
                        lower_bound=cfg.lower_bound if cfg.gate_mode == wl.LOWER_BOUND else None)
            for c0 in range(0, t1 - t0, C):
                last = -g[c0:c0 + C].sum(axis=0)
                spans += [float(last[d0:d0 + group].max()) for d0 in range(0, cfg.DK, group)]
    return np.array(spans)


def test_prefill_gpu_cases_reach_both_p_r_forms():
    """The GPU prefill cases with a softplus gate must contain channel groups
    on both sides of the one-product bound (so both the factored and the
    pair-by-pair P, R run), and the lower-bound cases (span <= 16 * 5) only
    the factored side."""
    from tests.test_gpu_prefill import CASES
    wide = narrow = 0
    for name, cfg in CASES.items():
        spans = _chunk_group_spans(wl.draw(cfg), group=min(32, cfg.DK))
        if cfg.gate_mode == wl.SOFTPLUS:
            wide += int((spans > SAFE_SPAN).sum())
            narrow += int((spans <= SAFE_SPAN).sum())
        else:
            assert spans.max() <= 16 * abs(cfg.lower_bound) <= SAFE_SPAN, name
    assert wide > 0 and narrow > 0, (wide, narrow)
