"""Plain fp64 CPU oracle for the KDA (Kimi Delta Attention) decode recurrence.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the tests, the smoke check in
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` may import or
call this module.  It shares no code, header, table or helper with the HIP
library, and the HIP library never calls it.

Everything is computed in float64, one (request, value head) tile and one
token at a time, in the order the sources state the steps.  Sources, cited by
page title and section:

  [DRW] "Delta-rule write" (atlas explainer, Kimi-K3 > Kimi Delta Attention >
        Delta-rule memory): the one-line summary, the Explanation paragraph,
        and the ``naive_recurrent_kda`` code excerpt (fla/ops/kda/naive.py).
  [FWD] same page, the ``modeling_kimi_linear.py`` attention-forward excerpt:
        the flags the model passes to ``fused_recurrent_kda``.
  [TKG] "KDA Block TKG Kernel API Reference" (AWS Neuron NKI library): the
        function signature (``l2_eps`` default) and the parameters ``A_log``,
        ``dt_bias``, ``lower_bound``, ``scale`` and ``S``.
  [KDD] "KdaDecode" (Modular MAX Mojo builtin kernels): the default
        parameters (gate_mode, beta_mode, state_layout) and Tensor Shapes.
  [TKG] also, for the short convolution in front of the recurrence: the
        parameters conv_w (depthwise causal taps per q/k/v stream, tap 0 the
        oldest position, tap-major), conv_state (the last K-1 pre-convolution
        inputs per stream, read as the left part of the window and replaced by
        the window ending at the newest token), the Background's "short
        convolutions with SiLU", and Dimensions (K = 4 for Kimi K3).

Readings taken where the pages are silent or ambiguous (each also listed in
the design notes of the repository):
  * L2 normalisation is x / sqrt(sum(x^2) + eps); only eps = 1e-6 is given.
  * the softplus gate uses the exact stable form max(x,0) + log1p(exp(-|x|)).
  * lower-bound gate: g = lower_bound * sigmoid(exp(A_log) * (raw + dt_bias)).
  * the query scale multiplies the normalised query once; default dk**-0.5.
  * a negative state index means "skip": no state access, output rows zero.
  * an empty request (no tokens) leaves its state untouched.
  * state layout: key-first S[k, v] ([KDD] default state_layout); the
    value-first pool stores each tile transposed, S[v, k] (the layout [FWD]
    asks for with transpose_state_layout=True).  The recurrence is the same.
  * state dtype ([KDD] names state_dtype without its arithmetic): a bf16
    pool is read exactly, advanced in high precision through all of the
    request's tokens, and rounded to nearest-even when stored.
  * short convolution: y_t = SiLU(sum_j w[j] * x_{t-K+1+j}) per channel with
    no bias; windows are slotted like the state ([N, K-1, C], oldest first,
    channels head-outer as in the q/k/v tensors).  In the fused step the
    convolved q, k, v go to the recurrence unrounded ([TKG] Background: the
    block keeps every intermediate on chip), so only the output is rounded.

Parity status: every function below is pinned by the CPU tests
(``tests/test_oracle_pins.py``) against closed forms, hand-worked values,
brute-force matrix forms and invariants, except two choices the pages do
not fix: where the L2-norm epsilon goes, and the lower-bound gate reading.
For those two the result is parity unpinned beyond the stated readings (the
epsilon placements differ by about eps / |x|^2; the lower-bound form is
pinned only by the three statements it is read from).
"""
from __future__ import annotations

import numpy as np

GATE_SOFTPLUS = "softplus"
GATE_LOWER_BOUND = "lower_bound"
DEFAULT_L2_EPS = 1e-6
STATE_K_FIRST = "k_first"
STATE_V_FIRST = "v_first"


# ----------------------------------------------------------------------------
# per-channel activations
# ----------------------------------------------------------------------------

def l2_normalize(x, eps):
    """Unit-normalise ``x`` along its last axis.

    [TKG] signature: ``l2_eps = 1e-6``; [FWD] ``use_qk_l2norm_in_kernel``.
    Reading: x / sqrt(sum(x^2) + eps).
    """
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def softplus(x):
    """Numerically stable softplus, ln(1 + e^x) = max(x, 0) + ln(1 + e^-|x|).

    [KDD] default parameters: the "original" gate mode is a stable softplus.
    """
    x = np.asarray(x, dtype=np.float64)
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


def sigmoid(x):
    """Logistic function 1 / (1 + e^-x); exact 0 at -inf and 1 at +inf."""
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-x))


def gate(raw_gate, dt_bias, a_log, gate_mode=GATE_SOFTPLUS, lower_bound=None):
    """Per-key-channel log decay g (always <= 0).

    softplus ("original") mode, [KDD] default parameters and the problem
    statement:   g = -exp(A_log) * softplus(raw_gate + dt_bias)
    lower-bound mode, [TKG] parameters A_log (exp(A_log) scales the gate
    pre-activation), dt_bias (added before the sigmoid) and lower_bound (the
    activated gate is lower_bound times a sigmoid):
                 g = lower_bound * sigmoid(exp(A_log) * (raw_gate + dt_bias))
    ``a_log`` is the scalar for this value head, ``dt_bias`` its [dk] row.
    """
    x = np.asarray(raw_gate, dtype=np.float64) + np.asarray(dt_bias, dtype=np.float64)
    amp = np.exp(np.float64(a_log))
    if gate_mode == GATE_SOFTPLUS:
        return -amp * softplus(x)
    if gate_mode == GATE_LOWER_BOUND:
        if lower_bound is None:
            raise ValueError("lower-bound gate mode needs lower_bound")
        return np.float64(lower_bound) * sigmoid(amp * x)
    raise ValueError(f"unknown gate mode {gate_mode!r}")


def write_strength(beta_logits):
    """beta = sigmoid(beta_logits); [KDD] beta_mode "logits", [FWD]
    ``use_beta_sigmoid_in_kernel``."""
    return sigmoid(beta_logits)


# ----------------------------------------------------------------------------
# the recurrence on one state tile S[k, v]
# ----------------------------------------------------------------------------

def decay(S, g):
    """[DRW] code excerpt: S is multiplied by exp(g) broadcast over the value
    axis, i.e. row k of the key-first state is scaled by exp(g[k])."""
    return np.exp(g)[:, None] * S


def delta_write(S, k_hat, v, beta):
    """[DRW] code excerpt and Explanation: the write adds
    (beta * k) outer (v - k^T S), where k^T S = sum_k k[k] * S[k, :] is what
    the memory currently returns for the key."""
    recalled = k_hat @ S                      # [dv]: sum over the key axis
    return S + np.outer(beta * k_hat, v - recalled)


def read(S, q_hat):
    """[DRW] code excerpt: o = sum_k q[k] * S[k, :], taken from the state after
    this token's write."""
    return q_hat @ S


def decode_tile(S0, q, k, v, raw_gate, beta_logits, a_log, dt_bias, *,
                gate_mode=GATE_SOFTPLUS, lower_bound=None,
                l2_eps=DEFAULT_L2_EPS, scale=None):
    """Advance one (request, value head) state through its n tokens.

    S0 [dk, dv]; q, k, raw_gate [n, dk]; v [n, dv]; beta_logits [n];
    a_log scalar; dt_bias [dk].  Returns (o [n, dv], S_n [dk, dv]) in fp64.

    Order per token ([DRW] code excerpt): decay, correction read against the
    decayed state, write, then the output read from the updated state.  q is
    normalised and then scaled once ([TKG] ``scale``; default dk**-0.5 as in
    the [DRW] code excerpt).
    """
    S = np.array(S0, dtype=np.float64, copy=True)
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    raw_gate = np.asarray(raw_gate, dtype=np.float64)
    beta_logits = np.asarray(beta_logits, dtype=np.float64)
    dk = S.shape[0]
    if scale is None:
        scale = dk ** -0.5
    n = q.shape[0]
    o = np.zeros((n, S.shape[1]), dtype=np.float64)
    for t in range(n):
        q_hat = l2_normalize(q[t], l2_eps) * scale
        k_hat = l2_normalize(k[t], l2_eps)
        g = gate(raw_gate[t], dt_bias, a_log, gate_mode, lower_bound)
        beta = write_strength(beta_logits[t])
        S = decay(S, g)
        S = delta_write(S, k_hat, v[t], beta)
        o[t] = read(S, q_hat)
    return o, S


# ----------------------------------------------------------------------------
# the batched decode op: varlen packing, slotted pool, GQA
# ----------------------------------------------------------------------------

def _drop_batch_axis(x, name):
    x = np.asarray(x)
    if x.shape[0] != 1:
        raise ValueError(f"{name}: leading axis must be 1 (packed tokens), got {x.shape}")
    return x[0]


def kda_decode(q, k, v, raw_gate, beta_logits, a_log, dt_bias, cu_seqlens,
               state_pool, state_indices, *, gate_mode=GATE_SOFTPLUS,
               lower_bound=None, l2_eps=DEFAULT_L2_EPS, scale=None,
               tiles=None, state_layout=STATE_K_FIRST, state_dtype="f32"):
    """The decode op over a cu_seqlens-packed batch and a slotted state pool.

    Shapes follow [KDD] Tensor Shapes: q, k [1, T, H, dk]; v [1, T, HV, dv];
    raw_gate [1, T, HV, dk]; beta_logits [1, T, HV]; a_log [HV];
    dt_bias [HV, dk]; cu_seqlens [B+1]; state_pool [N, HV, dk, dv] (key-first
    layout, [KDD] default state_layout); state_indices [B].

    Request b owns tokens cu_seqlens[b] .. cu_seqlens[b+1]-1 and the state
    tile state_pool[state_indices[b], hv] for every value head hv.  Value head
    hv reads key head hv // G with G = HV // H ([DRW] code excerpt: q and k are
    repeated G times along the head axis).

    ``state_pool`` may be an array (returned updated as an fp64 copy) or a
    dict {(slot, hv): tile} holding only the tiles needed; in that case
    ``tiles`` lists the (b, hv) pairs to compute and the dict returned holds
    their advanced states.  Output rows not computed are NaN.  With
    ``state_layout="v_first"`` every tile is stored transposed ([dv, dk]);
    with ``state_dtype="bf16"`` each advanced tile is rounded to bfloat16
    (nearest-even) when stored.

    Returns (out [1, T, HV, dv] fp64, advanced pool).
    """
    q = _drop_batch_axis(q, "q").astype(np.float64)
    k = _drop_batch_axis(k, "k").astype(np.float64)
    v = _drop_batch_axis(v, "v").astype(np.float64)
    raw_gate = _drop_batch_axis(raw_gate, "raw_gate").astype(np.float64)
    beta_logits = _drop_batch_axis(beta_logits, "beta_logits").astype(np.float64)
    a_log = np.asarray(a_log, dtype=np.float64)
    dt_bias = np.asarray(dt_bias, dtype=np.float64)
    cu = [int(c) for c in np.asarray(cu_seqlens)]
    idx = [int(i) for i in np.asarray(state_indices)]
    T, H, dk = q.shape
    HV, dv = v.shape[1], v.shape[2]
    if HV % H != 0:
        raise ValueError(f"HV={HV} is not a multiple of H={H}")
    G = HV // H
    B = len(idx)
    if len(cu) != B + 1:
        raise ValueError("cu_seqlens must have B+1 entries")

    as_dict = isinstance(state_pool, dict)
    if as_dict:
        pool = {key: np.array(val, dtype=np.float64) for key, val in state_pool.items()}
    else:
        pool = np.array(state_pool, dtype=np.float64, copy=True)

    if tiles is None:
        tiles = [(b, hv) for b in range(B) for hv in range(HV)]
    out = np.full((T, HV, dv), np.nan, dtype=np.float64)

    for b, hv in tiles:
        t0, t1 = cu[b], cu[b + 1]
        slot = idx[b]
        if slot < 0:
            out[t0:t1, hv] = 0.0
            continue
        if t1 == t0:
            continue
        h = hv // G
        S0 = pool[(slot, hv)] if as_dict else pool[slot, hv]
        if state_layout == STATE_V_FIRST:
            S0 = S0.T
        elif state_layout != STATE_K_FIRST:
            raise ValueError(f"unknown state layout {state_layout!r}")
        o, S = decode_tile(S0, q[t0:t1, h], k[t0:t1, h], v[t0:t1, hv],
                           raw_gate[t0:t1, hv], beta_logits[t0:t1, hv],
                           a_log[hv], dt_bias[hv], gate_mode=gate_mode,
                           lower_bound=lower_bound, l2_eps=l2_eps, scale=scale)
        if state_dtype == "bf16":
            S = round_to_bf16(S)
        elif state_dtype != "f32":
            raise ValueError(f"unknown state dtype {state_dtype!r}")
        if state_layout == STATE_V_FIRST:
            S = S.T
        out[t0:t1, hv] = o
        if as_dict:
            pool[(slot, hv)] = S
        else:
            pool[slot, hv] = S
    return out[None], pool


# ----------------------------------------------------------------------------
# output rounding
# ----------------------------------------------------------------------------

BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127


def round_to_bf16(x):
    """Round float64 values to the nearest bfloat16 value, ties to even.

    bfloat16 keeps 8 significant bits with the exponent range of binary32:
    the rounding quantum of a value in [2^(e-1), 2^e) is 2^(e-8), and below
    the smallest normal 2^-126 it is the fixed subnormal quantum 2^-133.
    The output cast keeps v's dtype ([DRW] code excerpt: o is returned in
    v.dtype).
    """
    x = np.asarray(x, dtype=np.float64)
    finite = np.isfinite(x)
    xf = np.where(finite, x, 0.0)
    _, e = np.frexp(xf)
    quantum_exp = np.maximum(e - 8, -133)
    y = np.ldexp(np.rint(np.ldexp(xf, -quantum_exp)), quantum_exp)
    y = np.where(np.abs(y) > BF16_MAX, np.copysign(np.inf, y), y)
    return np.where(finite, y, x)


# ----------------------------------------------------------------------------
# the short causal convolution in front of the recurrence
# ----------------------------------------------------------------------------

def silu(x):
    """SiLU(x) = x * sigmoid(x); [TKG] Background: short convolutions with SiLU."""
    x = np.asarray(x, dtype=np.float64)
    return x * sigmoid(x)


def short_conv(x, window, w):
    """Depthwise causal convolution of one request's inputs, then SiLU.

    x [n, C] the request's new pre-convolution inputs in token order;
    window [K-1, C] the K-1 inputs before them, oldest first ([TKG]
    conv_state); w [K, C] the taps, tap 0 applied to the oldest position of
    the window ([TKG] conv_w).  With xx = window followed by x,
    y[t] = SiLU(sum_j w[j] * xx[t + j]) and the new window is the last K-1
    rows of xx.  Returns (y [n, C], new window [K-1, C]) in fp64.
    """
    x = np.asarray(x, dtype=np.float64)
    window = np.asarray(window, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    K = w.shape[0]
    xx = np.concatenate([window, x], axis=0)
    n = x.shape[0]
    y = np.zeros_like(x)
    for t in range(n):
        y[t] = silu(np.sum(w * xx[t:t + K], axis=0))
    return y, xx[xx.shape[0] - (K - 1):]


def kda_decode_conv(x_q, x_k, x_v, w_q, w_k, w_v, win_q, win_k, win_v, raw_gate,
                    beta_logits, a_log, dt_bias, cu_seqlens, state_pool, state_indices,
                    **decode_kw):
    """The decode step with the short convolutions in front of the recurrence.

    x_q, x_k [1, T, H, dk] and x_v [1, T, HV, dv] are the pre-convolution
    projections; w_* [K, C] the taps with C = H*dk (q, k) or HV*dv (v),
    channels head-outer; win_* [N, K-1, C] the slotted windows (slot
    state_indices[b], like the recurrent state).  Per request, each stream
    is convolved over its tokens (short_conv) and the recurrence (kda_decode)
    runs on the unrounded result.  A skipped
    request (negative index) leaves its windows alone and gets zero q/k
    rows; an empty request changes nothing.

    Returns (out, state pool, win_q, win_k, win_v, q_conv, k_conv), the
    windows as fp64 copies.
    """
    x = [np.asarray(a, dtype=np.float64)[0] for a in (x_q, x_k, x_v)]
    w = [np.asarray(a, dtype=np.float64) for a in (w_q, w_k, w_v)]
    win = [np.array(a, dtype=np.float64, copy=True) for a in (win_q, win_k, win_v)]
    T = x[0].shape[0]
    conv = [np.zeros_like(a) for a in x]
    cu = [int(c) for c in np.asarray(cu_seqlens)]
    idx = [int(i) for i in np.asarray(state_indices)]
    for b, slot in enumerate(idx):
        t0, t1 = cu[b], cu[b + 1]
        if slot < 0 or t1 == t0:
            continue
        for s in range(3):
            flat = x[s][t0:t1].reshape(t1 - t0, -1)
            y, new_win = short_conv(flat, win[s][slot], w[s])
            conv[s][t0:t1] = y.reshape(x[s][t0:t1].shape)
            win[s][slot] = new_win
    out, pool = kda_decode(conv[0][None], conv[1][None], conv[2][None], raw_gate, beta_logits,
                           a_log, dt_bias, cu_seqlens, state_pool, state_indices, **decode_kw)
    return out, pool, win[0], win[1], win[2], conv[0][None], conv[1][None]
