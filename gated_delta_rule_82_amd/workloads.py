"""Seeded synthetic inputs for the KDA decode op.

This module only draws random numbers and lays them out; it holds none of
the recurrence's arithmetic.  Both the HIP parity tests and the oracle take
their inputs from here, and the benchmark draws its workload from here too.

The presets mirror the decode workloads the pages describe: a 96-head layer
with dk = dv = 128 ("Delta-rule write" page, input/output shapes), the
Kimi-Linear 32-head shape, a GQA/varlen speculative-window batch and a tiny
dk = 16 case; plus one whole-sequence (prefill) batch of the 96-head layer
(the same page in prefill mode: [B, 96, T, 128] inputs).  Distributions: q, k, v, raw_gate, beta_logits ~ N(0, 1);
A_log ~ U(0, ln 16); dt_bias ~ N(0, 0.1); state ~ N(0, sigma).

Draw order from ``numpy.random.default_rng(seed)`` (fixed, so every consumer
sees identical values): token counts, q, k, v, raw_gate, beta_logits, A_log,
dt_bias, state indices, and last the touched state tiles (host-state
workloads only).  bf16 tensors are fp32 draws rounded to nearest-even.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Optional, Tuple

import numpy as np

SOFTPLUS = "softplus"
LOWER_BOUND = "lower_bound"


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    HV: int
    DK: int
    DV: int
    n_slots: int
    tokens: str = "1"                 # "n" fixed per request, or "u:lo..hi"
    qkv_dtype: str = "bf16"           # "bf16" or "f32"
    gate_mode: str = SOFTPLUS
    lower_bound: float = 0.0
    state_sigma: float = 0.05
    seed: int = 0
    cu_seqlens: Optional[Tuple[int, ...]] = None
    state_indices: Optional[Tuple[int, ...]] = None
    host_state: bool = False          # draw touched tiles on the host
    state_layout: str = "k_first"     # "k_first" [N,HV,DK,DV] or "v_first" [N,HV,DV,DK]
    state_dtype: str = "f32"          # "f32" or "bf16"
    description: str = field(default="", compare=False)

    @property
    def G(self) -> int:
        return self.HV // self.H

    @property
    def pool_shape(self):
        if self.state_layout == "v_first":
            return (self.n_slots, self.HV, self.DV, self.DK)
        return (self.n_slots, self.HV, self.DK, self.DV)

    @property
    def state_elem_bytes(self) -> int:
        return 2 if self.state_dtype == "bf16" else 4


PRESETS = {
    "tiny": Workload(
        name="tiny", B=2, H=4, HV=4, DK=16, DV=16, n_slots=4,
        qkv_dtype="f32", state_sigma=0.1, cu_seqlens=(0, 3, 5),
        state_indices=(2, 0), host_state=True,
        description="B=2 (3 and 2 tokens), 4 heads, dk=dv=16, fp32, softplus"),
    "kimi_b64_h32": Workload(
        name="kimi_b64_h32", B=64, H=32, HV=32, DK=128, DV=128, n_slots=256,
        description="B=64, 1 token, 32 heads, dk=dv=128, bf16, softplus"),
    "varlen_gqa_b128": Workload(
        name="varlen_gqa_b128", B=128, H=16, HV=32, DK=128, DV=128,
        n_slots=512, tokens="u:1..8", gate_mode=LOWER_BOUND, lower_bound=-5.0,
        description="B=128, 1..8 tokens, 16 key / 32 value heads, lower-bound gate"),
    "wide_b256_h96": Workload(
        name="wide_b256_h96", B=256, H=96, HV=96, DK=128, DV=128, n_slots=512,
        description="B=256, 1 token, 96 heads, dk=dv=128, bf16, softplus"),
    "stress_b1024_n4": Workload(
        name="stress_b1024_n4", B=1024, H=96, HV=96, DK=128, DV=128,
        n_slots=2048, tokens="4", gate_mode=LOWER_BOUND, lower_bound=-5.0,
        description="B=1024, 4 tokens, 96 heads, lower-bound gate"),
    # whole-sequence (prefill) workload of the 96-head layer, as the model
    # runs it: value-first state, lower-bound gate
    "prefill_b8_t2048_h96": Workload(
        name="prefill_b8_t2048_h96", B=8, H=96, HV=96, DK=128, DV=128, n_slots=16,
        tokens="2048", gate_mode=LOWER_BOUND, lower_bound=-5.0, state_layout="v_first",
        description="prefill: B=8 x 2048 tokens, 96 heads, dk=dv=128, bf16, lower-bound gate, "
                    "value-first fp32 state"),
    # one long prompt: only 96 (request, head) tiles, fewer than the chip's
    # 256 compute units
    "prefill_b1_t16384_h96": Workload(
        name="prefill_b1_t16384_h96", B=1, H=96, HV=96, DK=128, DV=128, n_slots=2,
        tokens="16384", gate_mode=LOWER_BOUND, lower_bound=-5.0, state_layout="v_first",
        description="prefill: B=1 x 16384 tokens, 96 heads, dk=dv=128, bf16, lower-bound gate, "
                    "value-first fp32 state"),
}

PREFILL_HEADLINE = "prefill_b8_t2048_h96"

HEADLINE = "wide_b256_h96"


def preset(name: str, **overrides) -> Workload:
    return replace(PRESETS[name], **overrides)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bfloat16 (nearest, ties to even); return the bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    nan = np.isnan(np.asarray(x, dtype=np.float32))
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    bits = rounded.astype(np.uint16)
    bits[nan] = 0x7FC0
    return bits


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclass
class Inputs:
    """One drawn batch.  Float tensors are fp32 arrays holding the exact values
    the device sees; for bf16 tensors ``bits`` holds the stored bit patterns."""
    cfg: Workload
    cu_seqlens: np.ndarray            # int32 [B+1]
    state_indices: np.ndarray         # int32 [B]
    q: np.ndarray                     # [1, T, H, DK]
    k: np.ndarray
    v: np.ndarray                     # [1, T, HV, DV]
    raw_gate: np.ndarray              # fp32 [1, T, HV, DK]
    beta_logits: np.ndarray           # fp32 [1, T, HV]
    a_log: np.ndarray                 # fp32 [HV]
    dt_bias: np.ndarray               # fp32 [HV, DK]
    bits: dict                        # name -> uint16 bf16 bits
    touched_state: Optional[np.ndarray] = None   # fp32 [B, HV, DK, DV] (host_state)

    @property
    def T(self) -> int:
        return int(self.cu_seqlens[-1])


def _token_counts(cfg: Workload, rng: np.random.Generator) -> np.ndarray:
    if cfg.cu_seqlens is not None:
        return np.diff(np.asarray(cfg.cu_seqlens, dtype=np.int64))
    if cfg.tokens.startswith("u:"):
        lo, hi = (int(s) for s in cfg.tokens[2:].split(".."))
        return rng.integers(lo, hi + 1, size=cfg.B)
    return np.full(cfg.B, int(cfg.tokens), dtype=np.int64)


def draw(cfg: Workload) -> Inputs:
    rng = np.random.default_rng(cfg.seed)
    counts = _token_counts(cfg, rng)
    cu = np.zeros(cfg.B + 1, dtype=np.int32)
    cu[1:] = np.cumsum(counts)
    T = int(cu[-1])

    def normal(shape, sigma=1.0):
        return (rng.standard_normal(size=shape, dtype=np.float32) * np.float32(sigma)).astype(np.float32)

    q = normal((1, T, cfg.H, cfg.DK))
    k = normal((1, T, cfg.H, cfg.DK))
    v = normal((1, T, cfg.HV, cfg.DV))
    raw_gate = normal((1, T, cfg.HV, cfg.DK))
    beta_logits = normal((1, T, cfg.HV))
    a_log = rng.uniform(0.0, math.log(16.0), size=cfg.HV).astype(np.float32)
    dt_bias = normal((cfg.HV, cfg.DK), 0.1)
    if cfg.state_indices is not None:
        idx = np.asarray(cfg.state_indices, dtype=np.int32)
    else:
        idx = rng.permutation(cfg.n_slots)[: cfg.B].astype(np.int32)

    bits = {}
    if cfg.qkv_dtype == "bf16":
        for name, arr in (("q", q), ("k", k), ("v", v)):
            bits[name] = f32_to_bf16_bits(arr)
        q, k, v = (bf16_bits_to_f32(bits[n]) for n in ("q", "k", "v"))
    elif cfg.qkv_dtype != "f32":
        raise ValueError(cfg.qkv_dtype)

    touched = None
    if cfg.host_state:
        touched = normal((cfg.B, cfg.HV, cfg.DK, cfg.DV), cfg.state_sigma)
    return Inputs(cfg, cu, idx, q, k, v, raw_gate, beta_logits, a_log, dt_bias,
                  bits, touched)


def host_pool(inp: Inputs, fill_sigma: Optional[float] = None, seed_offset: int = 1) -> np.ndarray:
    """Full pool on the host as fp32 values, in the workload's layout: the
    touched tiles from ``inp`` and every other slot drawn from its own
    generator (seed + seed_offset).  For a bf16 pool the values are rounded
    to bf16 (nearest-even), i.e. they are exactly what the device holds."""
    cfg = inp.cfg
    rng = np.random.default_rng(cfg.seed + seed_offset)
    sigma = cfg.state_sigma if fill_sigma is None else fill_sigma
    pool = (rng.standard_normal((cfg.n_slots, cfg.HV, cfg.DK, cfg.DV), dtype=np.float32)
            * np.float32(sigma)).astype(np.float32)
    if inp.touched_state is not None:
        for b, slot in enumerate(inp.state_indices):
            if slot >= 0:
                pool[slot] = inp.touched_state[b]
    if cfg.state_layout == "v_first":
        pool = np.ascontiguousarray(np.swapaxes(pool, 2, 3))
    if cfg.state_dtype == "bf16":
        pool = bf16_bits_to_f32(f32_to_bf16_bits(pool))
    return pool


# ----------------------------------------------------------------------------
# device copies (torch is used only for device memory)
# ----------------------------------------------------------------------------

def to_device(inp: Inputs, device="cuda"):
    """Upload the token tensors and metadata; returns a dict of torch tensors
    keyed like the kda_decode arguments (no state pool, no output)."""
    import torch

    def f32(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)

    def qkv(name, arr):
        if inp.cfg.qkv_dtype == "bf16":
            bits = np.ascontiguousarray(inp.bits[name]).view(np.int16)
            return torch.from_numpy(bits).view(torch.bfloat16).to(device)
        return f32(arr)

    return {
        "q": qkv("q", inp.q), "k": qkv("k", inp.k), "v": qkv("v", inp.v),
        "raw_gate": f32(inp.raw_gate), "beta_logits": f32(inp.beta_logits),
        "a_log": f32(inp.a_log), "dt_bias": f32(inp.dt_bias),
        "cu_seqlens": torch.from_numpy(inp.cu_seqlens.astype(np.int32)).to(device),
        "state_indices": torch.from_numpy(inp.state_indices.astype(np.int32)).to(device),
    }


def empty_out(inp: Inputs, device="cuda"):
    import torch
    dt = torch.bfloat16 if inp.cfg.qkv_dtype == "bf16" else torch.float32
    return torch.empty((1, inp.T, inp.cfg.HV, inp.cfg.DV), dtype=dt, device=device)


def device_pool(inp: Inputs, device="cuda", seed_offset: int = 1):
    """The fp32 state pool on the device.  Host-state workloads upload
    ``host_pool``; the others are filled on the device from torch's seeded
    generator (N(0, sigma)), which keeps multi-GB pools off the host."""
    import torch
    cfg = inp.cfg
    dt = torch.bfloat16 if cfg.state_dtype == "bf16" else torch.float32
    if cfg.host_state:
        return torch.from_numpy(host_pool(inp, seed_offset=seed_offset)).to(device).to(dt)
    gen = torch.Generator(device=device)
    gen.manual_seed(cfg.seed + seed_offset)
    pool = torch.empty(cfg.pool_shape, dtype=dt, device=device)
    pool.normal_(0.0, cfg.state_sigma, generator=gen)
    return pool


def state_bytes(cfg: Workload, inp: Inputs) -> int:
    """Algorithmic state traffic of one call: every (request, value head) tile
    with at least one token and a valid slot is read once and written once."""
    counts = np.diff(inp.cu_seqlens)
    active = int(np.sum((counts > 0) & (inp.state_indices >= 0)))
    return active * cfg.HV * 2 * cfg.DK * cfg.DV * cfg.state_elem_bytes


def token_bytes(cfg: Workload, inp: Inputs) -> int:
    """Algorithmic bytes of everything but the state, counted once each:
    q, k (per key head), v, raw_gate, beta_logits, out, a_log, dt_bias and
    the two metadata arrays."""
    T = inp.T
    e = 2 if cfg.qkv_dtype == "bf16" else 4
    return (2 * T * cfg.H * cfg.DK * e + T * cfg.HV * cfg.DV * e + T * cfg.HV * cfg.DK * 4
            + T * cfg.HV * 4 + T * cfg.HV * cfg.DV * e + cfg.HV * 4 + cfg.HV * cfg.DK * 4
            + (cfg.B + 1) * 4 + cfg.B * 4)



# ----------------------------------------------------------------------------
# inputs of the decode step with the short convolutions in front
# ----------------------------------------------------------------------------

@dataclass
class ConvInputs:
    """Pre-convolution q/k/v (fp32 values, bf16-exact for bf16 workloads),
    taps [K, C] and windows [N, K-1, C] for the three streams."""
    K: int
    x: dict            # "q", "k" [1, T, H, DK]; "v" [1, T, HV, DV]
    w: dict            # "q", "k" [K, H*DK]; "v" [K, HV*DV]
    win: dict          # "q", "k" [N, K-1, H*DK]; "v" [N, K-1, HV*DV]
    taps_dtype: str = "f32"


def draw_conv(inp: Inputs, K: int = 4, taps_dtype: str = "f32", seed_offset: int = 2) -> ConvInputs:
    """Seeded conv inputs from their own generator (seed + seed_offset), so
    the recurrence inputs of ``inp`` are unchanged.  Draw order: x_q, x_k,
    x_v ~ N(0, 1); taps ~ N(0, 0.5) per stream; windows ~ N(0, 1).  Window
    values hold earlier pre-convolution inputs, so they are bf16-exact when
    the activations are bf16."""
    cfg = inp.cfg
    rng = np.random.default_rng(cfg.seed + seed_offset)
    T = inp.T
    shapes = {"q": (1, T, cfg.H, cfg.DK), "k": (1, T, cfg.H, cfg.DK), "v": (1, T, cfg.HV, cfg.DV)}
    chans = {"q": cfg.H * cfg.DK, "k": cfg.H * cfg.DK, "v": cfg.HV * cfg.DV}

    def act(a):
        a = a.astype(np.float32)
        return bf16_bits_to_f32(f32_to_bf16_bits(a)) if cfg.qkv_dtype == "bf16" else a

    x = {s: act(rng.standard_normal(shapes[s], dtype=np.float32)) for s in "qkv"}
    w = {}
    for s in "qkv":
        taps = (rng.standard_normal((K, chans[s]), dtype=np.float32) * np.float32(0.5)).astype(np.float32)
        w[s] = bf16_bits_to_f32(f32_to_bf16_bits(taps)) if taps_dtype == "bf16" else taps
    win = {s: act(rng.standard_normal((cfg.n_slots, K - 1, chans[s]), dtype=np.float32)) for s in "qkv"}
    return ConvInputs(K, x, w, win, taps_dtype)


def conv_to_device(ci: ConvInputs, qkv_dtype: str, device="cuda"):
    """Device tensors keyed like the kda_decode_conv arguments, plus empty
    fp32 q_conv / k_conv outputs."""
    import torch
    act = torch.bfloat16 if qkv_dtype == "bf16" else torch.float32
    tap = torch.bfloat16 if ci.taps_dtype == "bf16" else torch.float32
    d = {}
    for s in "qkv":
        d["x_" + s] = torch.from_numpy(ci.x[s]).to(device).to(act)
        d["w_" + s] = torch.from_numpy(ci.w[s]).to(device).to(tap)
        d["win_" + s] = torch.from_numpy(ci.win[s]).to(device)
    d["q_conv"] = torch.empty(d["x_q"].shape, dtype=torch.float32, device=device)
    d["k_conv"] = torch.empty(d["x_k"].shape, dtype=torch.float32, device=device)
    return d


def conv_bytes(cfg: Workload, inp: Inputs, K: int) -> int:
    """Algorithmic bytes the convolutions add to a step: the pre-convolution
    inputs, the fp32 convolved q/k written and read back, the taps, and the
    fp32 windows of every active request read and written."""
    e = 2 if cfg.qkv_dtype == "bf16" else 4
    T = inp.T
    cqk, cv = cfg.H * cfg.DK, cfg.HV * cfg.DV
    counts = np.diff(inp.cu_seqlens)
    active = int(np.sum((counts > 0) & (inp.state_indices >= 0)))
    return (T * (2 * cqk + cv) * e + 2 * (T * 2 * cqk * 4) + K * (2 * cqk + cv) * 4
            + 2 * active * (K - 1) * (2 * cqk + cv) * 4)
