"""Thin ctypes binding of libkda (argument marshalling only).

Every step of the decode and of the chunked prefill runs in the HIP library; this module turns torch
device tensors into ``kda_tensor`` descriptors, passes the current HIP stream
and raises :class:`KdaError` on a nonzero status.  There is no fallback: if
the library is missing or a tensor is not on a GPU, the call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "lib", "libkda.so")

# enum values of include/kda.h
KDA_OK = 0
KDA_ERR_NULL = -1
KDA_ERR_DTYPE = -2
KDA_ERR_SHAPE = -3
KDA_ERR_UNSUPPORTED = -4
KDA_ERR_MODE = -5
KDA_ERR_LAUNCH = -6
KDA_ERR_PRECONDITION = -7

KDA_F32 = 0
KDA_BF16 = 1
KDA_I32 = 2

KDA_GATE_SOFTPLUS = 0
KDA_GATE_LOWER_BOUND = 1
GATE_MODES = {"softplus": KDA_GATE_SOFTPLUS, "lower_bound": KDA_GATE_LOWER_BOUND}

KDA_STATE_K_FIRST = 0
KDA_STATE_V_FIRST = 1
STATE_LAYOUTS = {"k_first": KDA_STATE_K_FIRST, "v_first": KDA_STATE_V_FIRST}

KDA_MATMUL_SPLIT_BF16 = 0
KDA_MATMUL_F32 = 1
MATMULS = {"split_bf16": KDA_MATMUL_SPLIT_BF16, "f32": KDA_MATMUL_F32}

EXPORTED_SYMBOLS = ("kda_decode", "kda_decode_conv", "kda_prefill", "kda_check_host",
                    "kda_status_string", "kda_abi_version")
CONV_FIELDS = ("x_q", "x_k", "x_v", "w_q", "w_k", "w_v", "win_q", "win_k", "win_v", "q_conv",
               "k_conv")


class KdaTensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32),
                ("ndim", ctypes.c_int32), ("shape", ctypes.c_int64 * 4)]


class KdaConv(ctypes.Structure):
    _fields_ = [(n, KdaTensor) for n in CONV_FIELDS]


class KdaMode(ctypes.Structure):
    _fields_ = [("gate_mode", ctypes.c_int32), ("lower_bound", ctypes.c_float),
                ("l2_eps", ctypes.c_float), ("scale", ctypes.c_float),
                ("state_layout", ctypes.c_int32)]


class KdaError(RuntimeError):
    def __init__(self, code: int, where: str = "kda_decode"):
        self.code = code
        super().__init__(f"{where} failed with status {code}: {status_string(code)}")


class KdaLibraryMissing(RuntimeError):
    pass


_lib: Optional[ctypes.CDLL] = None


def library() -> ctypes.CDLL:
    """Load libkda.so (built in-tree by ``gated_delta_rule_82_amd.build``).

    torch is imported first so that the library binds to the HIP runtime torch
    already loaded (both carry the soname libamdhip64.so.7): one runtime, one
    set of streams."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise KdaLibraryMissing(
            f"{LIB_PATH} is not built; run `python -m gated_delta_rule_82_amd.build`")
    import torch  # noqa: F401  (binds the process to torch's HIP runtime first)
    lib = ctypes.CDLL(LIB_PATH, mode=ctypes.RTLD_LOCAL)
    P = ctypes.POINTER(KdaTensor)
    lib.kda_decode.argtypes = [P] * 11 + [ctypes.POINTER(KdaMode), ctypes.c_void_p]
    lib.kda_decode.restype = ctypes.c_int
    lib.kda_decode_conv.argtypes = [P, ctypes.POINTER(KdaConv)] + [P] * 7 + [ctypes.POINTER(KdaMode),
                                                                        ctypes.c_void_p]
    lib.kda_decode_conv.restype = ctypes.c_int
    lib.kda_prefill.argtypes = [P] * 11 + [ctypes.POINTER(KdaMode), ctypes.c_int32,
                                            ctypes.c_void_p]
    lib.kda_prefill.restype = ctypes.c_int
    lib.kda_check_host.argtypes = [ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32),
                                   ctypes.c_int64, ctypes.c_int64, ctypes.c_int64]
    lib.kda_check_host.restype = ctypes.c_int
    lib.kda_status_string.argtypes = [ctypes.c_int]
    lib.kda_status_string.restype = ctypes.c_char_p
    lib.kda_abi_version.argtypes = []
    lib.kda_abi_version.restype = ctypes.c_int
    _lib = lib
    return lib


def status_string(code: int) -> str:
    try:
        return library().kda_status_string(int(code)).decode()
    except KdaLibraryMissing:
        return "libkda not built"


def make_mode(gate_mode="softplus", lower_bound=0.0, l2_eps=0.0, scale=0.0,
              state_layout="k_first") -> KdaMode:
    gm = GATE_MODES[gate_mode] if isinstance(gate_mode, str) else int(gate_mode)
    sl = STATE_LAYOUTS[state_layout] if isinstance(state_layout, str) else int(state_layout)
    return KdaMode(gm, float(lower_bound), float(l2_eps), float(scale), sl)


def raw_tensor(data_ptr: int, dtype: int, shape) -> KdaTensor:
    t = KdaTensor()
    t.data = data_ptr
    t.dtype = dtype
    t.ndim = len(shape)
    for i, s in enumerate(shape):
        t.shape[i] = int(s)
    return t


def call_raw(tensors, mode: KdaMode, stream: int = 0) -> int:
    """Call kda_decode on 11 prepared descriptors (None passes NULL); returns
    the status code without raising."""
    lib = library()
    ptrs = [ctypes.byref(t) if t is not None else None for t in tensors]
    return lib.kda_decode(*ptrs, ctypes.byref(mode) if mode is not None else None,
                          ctypes.c_void_p(stream))


def call_raw_prefill(tensors, mode: KdaMode, matmul: int = KDA_MATMUL_SPLIT_BF16,
                     stream: int = 0) -> int:
    """Call kda_prefill on 11 prepared descriptors (None passes NULL); returns
    the status code without raising."""
    lib = library()
    ptrs = [ctypes.byref(t) if t is not None else None for t in tensors]
    return lib.kda_prefill(*ptrs, ctypes.byref(mode) if mode is not None else None,
                           ctypes.c_int32(matmul), ctypes.c_void_p(stream))


def call_raw_conv(out, conv, rest, mode: KdaMode, stream: int = 0) -> int:
    """Call kda_decode_conv on prepared descriptors: ``out``, a KdaConv (or
    None), and the 7 remaining tensors (raw_gate .. state_indices)."""
    lib = library()
    ref = lambda t: ctypes.byref(t) if t is not None else None  # noqa: E731
    return lib.kda_decode_conv(ref(out), ref(conv), *[ref(t) for t in rest], ref(mode),
                               ctypes.c_void_p(stream))


def _descriptor(t, name):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name}: must be a GPU tensor, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if t.dim() > 4:
        raise ValueError(f"{name}: at most 4 dimensions")
    dt = {torch.float32: KDA_F32, torch.bfloat16: KDA_BF16, torch.int32: KDA_I32}.get(t.dtype)
    if dt is None:
        raise ValueError(f"{name}: unsupported dtype {t.dtype}")
    return raw_tensor(t.data_ptr(), dt, t.shape)


ARG_NAMES = ("out", "q", "k", "v", "raw_gate", "beta_logits", "a_log", "dt_bias",
             "cu_seqlens", "state_pool", "state_indices")


def decode(out, q, k, v, raw_gate, beta_logits, a_log, dt_bias, cu_seqlens, state_pool,
           state_indices, *, gate_mode="softplus", lower_bound=0.0, l2_eps=0.0, scale=0.0,
           state_layout="k_first", stream: Optional[int] = None) -> None:
    """Advance the KDA decode recurrence in place (see include/kda.h).

    Tensors are torch GPU tensors with the shapes of kda.h; ``out`` and
    ``state_pool`` are written.  ``state_pool`` is float32 or bfloat16, laid
    out [N, HV, dk, dv] ("k_first") or [N, HV, dv, dk] ("v_first").  The work
    is enqueued on ``stream`` (a raw hipStream_t handle; default: torch's
    current stream of q's device)."""
    import torch
    tensors = (out, q, k, v, raw_gate, beta_logits, a_log, dt_bias, cu_seqlens, state_pool,
               state_indices)
    descs = [_descriptor(t, n) for t, n in zip(tensors, ARG_NAMES)]
    dev = q.device
    for t, n in zip(tensors, ARG_NAMES):
        if t.device != dev:
            raise ValueError(f"{n}: on {t.device}, expected {dev}")
    mode = make_mode(gate_mode, lower_bound, l2_eps, scale, state_layout)
    with torch.cuda.device(dev):
        if stream is None:
            stream = torch.cuda.current_stream(dev).cuda_stream
        rc = call_raw(descs, mode, stream)
    if rc != KDA_OK:
        raise KdaError(rc)


def prefill(out, q, k, v, raw_gate, beta_logits, a_log, dt_bias, cu_seqlens, state_pool,
            state_indices, *, gate_mode="softplus", lower_bound=0.0, l2_eps=0.0, scale=0.0,
            state_layout="k_first", matmul="split_bf16", stream: Optional[int] = None) -> None:
    """The recurrence over long requests in chunks of 16 tokens on the matrix
    cores (kda_prefill in include/kda.h): same tensors and result as
    :func:`decode`; ``matmul`` is "split_bf16" (default) or "f32"."""
    import torch
    tensors = (out, q, k, v, raw_gate, beta_logits, a_log, dt_bias, cu_seqlens, state_pool,
               state_indices)
    descs = [_descriptor(t, n) for t, n in zip(tensors, ARG_NAMES)]
    dev = q.device
    for t, n in zip(tensors, ARG_NAMES):
        if t.device != dev:
            raise ValueError(f"{n}: on {t.device}, expected {dev}")
    mode = make_mode(gate_mode, lower_bound, l2_eps, scale, state_layout)
    mm = MATMULS[matmul] if isinstance(matmul, str) else int(matmul)
    with torch.cuda.device(dev):
        if stream is None:
            stream = torch.cuda.current_stream(dev).cuda_stream
        rc = call_raw_prefill(descs, mode, mm, stream)
    if rc != KDA_OK:
        raise KdaError(rc, "kda_prefill")


def check_host(cu_seqlens, state_indices, T: int, n_slots: int) -> int:
    """Run kda_check_host on host int32 arrays; returns the status code."""
    import numpy as np
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    idx = np.ascontiguousarray(state_indices, dtype=np.int32)
    if cu.ndim != 1 or idx.ndim != 1 or len(cu) != len(idx) + 1:
        # kda_check_host reads B + 1 entries of cu_seqlens
        raise ValueError(f"cu_seqlens needs len(state_indices) + 1 = {len(idx) + 1} entries, "
                         f"got shape {cu.shape}")
    P = ctypes.POINTER(ctypes.c_int32)
    return library().kda_check_host(cu.ctypes.data_as(P), idx.ctypes.data_as(P),
                                    len(idx), int(T), int(n_slots))


CONV_REST = ("raw_gate", "beta_logits", "a_log", "dt_bias", "cu_seqlens", "state_pool",
             "state_indices")


def decode_conv(out, x_q, x_k, x_v, w_q, w_k, w_v, win_q, win_k, win_v, q_conv, k_conv, raw_gate,
                beta_logits, a_log, dt_bias, cu_seqlens, state_pool, state_indices, *,
                gate_mode="softplus", lower_bound=0.0, l2_eps=0.0, scale=0.0,
                state_layout="k_first", stream: Optional[int] = None) -> None:
    """The decode step with the short convolutions in front (see
    kda_decode_conv in include/kda.h): x_q, x_k [1, T, H, dk] and x_v
    [1, T, HV, dv] pre-convolution inputs; taps w_* [K, C]; windows win_*
    [N, K-1, C] (updated in place); q_conv, k_conv [1, T, H, dk] receive the
    convolved q and k (they may be x_q and x_k themselves)."""
    import torch
    conv_t = (x_q, x_k, x_v, w_q, w_k, w_v, win_q, win_k, win_v, q_conv, k_conv)
    rest_t = (raw_gate, beta_logits, a_log, dt_bias, cu_seqlens, state_pool, state_indices)
    conv = KdaConv(*[_descriptor(t, n) for t, n in zip(conv_t, CONV_FIELDS)])
    rest = [_descriptor(t, n) for t, n in zip(rest_t, CONV_REST)]
    out_d = _descriptor(out, "out")
    dev = out.device
    for t, n in zip(conv_t + rest_t, CONV_FIELDS + CONV_REST):
        if t.device != dev:
            raise ValueError(f"{n}: on {t.device}, expected {dev}")
    mode = make_mode(gate_mode, lower_bound, l2_eps, scale, state_layout)
    with torch.cuda.device(dev):
        if stream is None:
            stream = torch.cuda.current_stream(dev).cuda_stream
        rc = call_raw_conv(out_d, conv, rest, mode, stream)
    if rc != KDA_OK:
        raise KdaError(rc, "kda_decode_conv")
