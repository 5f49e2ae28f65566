"""CPU tests of the C ABI: the library loads, exports what include/kda.h
declares, and rejects every malformed call before any device work.

No test here launches a kernel: each kda_decode call below is either
invalid (the checker returns before any HIP call) or has nothing to do
(B = 0 or T = 0, which return before the launch).  The data pointers are
fake aligned addresses that are never dereferenced.
"""
import os
import re
import subprocess

import numpy as np
import pytest

from gated_delta_rule_82_amd import kda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")

pytestmark = pytest.mark.skipif(not os.path.exists(kda.LIB_PATH),
                                reason="libkda.so not built (run the build first)")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int|const char\*)\s+(kda_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_expected_api():
    assert header_functions() == sorted(kda.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol():
    lib = kda.library()
    for name in header_functions():
        assert hasattr(lib, name), name
    nm = subprocess.run(["nm", "-D", "--defined-only", kda.LIB_PATH], capture_output=True,
                        text=True, check=True).stdout
    exported = {line.split()[-1] for line in nm.splitlines() if " T " in line}
    assert exported == set(header_functions())


def test_abi_version_and_status_strings():
    lib = kda.library()
    assert lib.kda_abi_version() == 4
    codes = [kda.KDA_OK, kda.KDA_ERR_NULL, kda.KDA_ERR_DTYPE, kda.KDA_ERR_SHAPE,
             kda.KDA_ERR_UNSUPPORTED, kda.KDA_ERR_MODE, kda.KDA_ERR_LAUNCH,
             kda.KDA_ERR_PRECONDITION]
    strings = [kda.status_string(c) for c in codes]
    assert len(set(strings)) == len(codes)
    assert kda.status_string(12345) == "unknown status"


# ---------------------------------------------------------------------------
# kda_check_host
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("cu,idx,T,N,expect", [
    ([0, 3, 5], [2, 0], 5, 4, kda.KDA_OK),
    ([0, 3, 5], [2, -1], 5, 4, kda.KDA_OK),
    ([0, 0, 0], [1, 2], 0, 4, kda.KDA_OK),
    ([0], [], 0, 0, kda.KDA_OK),
    ([1, 3, 5], [2, 0], 5, 4, kda.KDA_ERR_PRECONDITION),     # cu[0] != 0
    ([0, 3, 4], [2, 0], 5, 4, kda.KDA_ERR_PRECONDITION),     # cu[B] != T
    ([0, 3, 2, 5], [1, 2, 3], 5, 4, kda.KDA_ERR_PRECONDITION),  # decreasing
    ([0, 3, 5], [2, 2], 5, 4, kda.KDA_ERR_PRECONDITION),     # duplicate slot
    ([0, 3, 5], [2, 4], 5, 4, kda.KDA_ERR_PRECONDITION),     # slot >= N
    ([0, 3, 5], [-1, -1], 5, 4, kda.KDA_OK),                 # negatives may repeat
])
def test_check_host(cu, idx, T, N, expect):
    assert kda.check_host(cu, idx, T, N) == expect


def test_check_host_binding_rejects_short_cu_seqlens():
    # the C function reads B + 1 entries; the binding refuses a shorter array
    with pytest.raises(ValueError):
        kda.check_host([0, 3], [2, 0], 5, 4)
    with pytest.raises(ValueError):
        kda.check_host([0, 3, 5, 6], [2, 0], 5, 4)


def test_check_host_bad_sizes_and_nulls():
    lib = kda.library()
    assert lib.kda_check_host(None, None, 0, 0, 0) == kda.KDA_ERR_NULL
    cu = np.array([0, 1], dtype=np.int32)
    P = __import__("ctypes").POINTER(__import__("ctypes").c_int32)
    assert lib.kda_check_host(cu.ctypes.data_as(P), None, 1, 1, 4) == kda.KDA_ERR_NULL
    assert lib.kda_check_host(cu.ctypes.data_as(P), None, -1, 1, 4) == kda.KDA_ERR_SHAPE
    assert lib.kda_check_host(cu.ctypes.data_as(P), None, 1, -1, 4) == kda.KDA_ERR_SHAPE


# ---------------------------------------------------------------------------
# kda_decode argument checking (never reaches a launch)
# ---------------------------------------------------------------------------

_FAKE = [0x100000 * (i + 1) for i in range(11)]


def descriptors(B=2, T=3, H=2, HV=4, DK=128, DV=128, N=8, qkv=kda.KDA_BF16):
    shapes = {
        "out": (qkv, (1, T, HV, DV)), "q": (qkv, (1, T, H, DK)), "k": (qkv, (1, T, H, DK)),
        "v": (qkv, (1, T, HV, DV)), "raw_gate": (kda.KDA_F32, (1, T, HV, DK)),
        "beta_logits": (kda.KDA_F32, (1, T, HV)), "a_log": (kda.KDA_F32, (HV,)),
        "dt_bias": (kda.KDA_F32, (HV, DK)), "cu_seqlens": (kda.KDA_I32, (B + 1,)),
        "state_pool": (kda.KDA_F32, (N, HV, DK, DV)), "state_indices": (kda.KDA_I32, (B,)),
    }
    return {n: kda.raw_tensor(_FAKE[i], *shapes[n]) for i, n in enumerate(kda.ARG_NAMES)}


def call(descs, mode=None, **mode_kw):
    if mode is None:
        mode = kda.make_mode(**mode_kw)
    return kda.call_raw([descs[n] for n in kda.ARG_NAMES], mode, 0)


def reshape(desc, shape):
    return kda.raw_tensor(desc.data, desc.dtype, shape)


def test_nothing_to_do_returns_ok_without_launch():
    d = descriptors(B=0, T=0)
    assert call(d) == kda.KDA_OK
    d = descriptors(B=3, T=0)
    assert call(d) == kda.KDA_OK


def test_null_arguments():
    d = descriptors(B=0, T=0)
    assert kda.call_raw([d[n] for n in kda.ARG_NAMES], None, 0) == kda.KDA_ERR_NULL
    for n in kda.ARG_NAMES:
        e = dict(d)
        e[n] = None
        assert call(e) == kda.KDA_ERR_NULL, n
    d = descriptors()
    for n in kda.ARG_NAMES:
        e = dict(d)
        e[n] = kda.raw_tensor(0, d[n].dtype, tuple(d[n].shape[:d[n].ndim]))
        assert call(e) == kda.KDA_ERR_NULL, n


@pytest.mark.parametrize("name,dtype", [
    ("q", kda.KDA_F32), ("k", kda.KDA_F32), ("out", kda.KDA_F32), ("v", kda.KDA_I32),
    ("raw_gate", kda.KDA_BF16), ("beta_logits", kda.KDA_BF16), ("a_log", kda.KDA_I32),
    ("dt_bias", kda.KDA_BF16), ("state_pool", kda.KDA_I32), ("cu_seqlens", kda.KDA_F32),
    ("state_indices", kda.KDA_F32),
])
def test_dtype_errors(name, dtype):
    d = descriptors()
    d[name] = kda.raw_tensor(d[name].data, dtype, tuple(d[name].shape[:d[name].ndim]))
    assert call(d) == kda.KDA_ERR_DTYPE


def test_shape_errors():
    base = descriptors()
    cases = {
        "q": (2, 3, 2, 128), "k": (1, 3, 2, 64), "v": (1, 4, 4, 128), "out": (1, 3, 4, 64),
        "raw_gate": (1, 3, 2, 128), "beta_logits": (1, 3, 3), "a_log": (3,),
        "dt_bias": (4, 64), "cu_seqlens": (4,), "state_pool": (8, 4, 128, 64),
        "state_indices": (3,),
    }
    for name, shape in cases.items():
        d = dict(base)
        d[name] = reshape(base[name], shape)
        assert call(d) == kda.KDA_ERR_SHAPE, name
    d = dict(base)
    d["a_log"] = reshape(base["a_log"], (4, 1))           # wrong rank
    assert call(d) == kda.KDA_ERR_SHAPE
    d = descriptors(H=3, HV=4)                             # HV % H != 0
    assert call(d) == kda.KDA_ERR_SHAPE
    d = dict(base)
    d["q"] = kda.raw_tensor(base["q"].data, base["q"].dtype, (1, 3, 2, -128))
    assert call(d) == kda.KDA_ERR_SHAPE


@pytest.mark.parametrize("dk,dv", [(48, 128), (128, 96), (256, 128), (128, 8)])
def test_unsupported_head_dims(dk, dv):
    assert call(descriptors(DK=dk, DV=dv)) == kda.KDA_ERR_UNSUPPORTED


def test_misaligned_pointer_is_unsupported():
    d = descriptors()
    d["state_pool"] = kda.raw_tensor(d["state_pool"].data + 4, kda.KDA_F32, (8, 4, 128, 128))
    assert call(d) == kda.KDA_ERR_UNSUPPORTED


@pytest.mark.parametrize("kw", [
    dict(gate_mode=7),
    dict(gate_mode="lower_bound", lower_bound=0.5),
    dict(gate_mode="lower_bound", lower_bound=float("nan")),
    dict(gate_mode="lower_bound", lower_bound=float("-inf")),
    dict(l2_eps=-1e-6), dict(l2_eps=float("inf")), dict(l2_eps=float("nan")),
    dict(scale=-1.0), dict(scale=float("nan")), dict(scale=float("inf")),
])
def test_mode_errors(kw):
    assert call(descriptors(), **kw) == kda.KDA_ERR_MODE


def test_python_binding_rejects_cpu_tensors():
    torch = pytest.importorskip("torch")
    t = torch.zeros(4)
    with pytest.raises(ValueError):
        kda.decode(*([t] * 11))


def test_state_layout_and_dtype_checks():
    # an invalid layout value is a mode error
    assert call(descriptors(), state_layout=2) == kda.KDA_ERR_MODE
    # value-first pools are [N, HV, dv, dk]: with dk != dv the key-first shape
    # is rejected and the transposed one gets as far as the (invalid) gate mode
    d = descriptors(DK=128, DV=64)
    assert call(d, state_layout="v_first") == kda.KDA_ERR_SHAPE
    d["state_pool"] = reshape(d["state_pool"], (8, 4, 64, 128))
    assert call(d, state_layout="v_first", gate_mode=9) == kda.KDA_ERR_MODE
    assert call(d, state_layout="k_first", gate_mode=9) == kda.KDA_ERR_SHAPE
    # a bf16 pool passes the dtype check (stopped later by the invalid gate mode)
    d = descriptors()
    d["state_pool"] = kda.raw_tensor(d["state_pool"].data, kda.KDA_BF16, (8, 4, 128, 128))
    assert call(d, gate_mode=9) == kda.KDA_ERR_MODE



# ---------------------------------------------------------------------------
# kda_decode_conv argument checking (never reaches a launch)
# ---------------------------------------------------------------------------

_FAKE_CONV = [0x4000000 + 0x100000 * i for i in range(11)]


def conv_descriptors(B=2, T=3, H=2, HV=4, DK=128, DV=128, N=8, K=4, act=kda.KDA_BF16,
                     taps=kda.KDA_F32):
    d = descriptors(B=B, T=T, H=H, HV=HV, DK=DK, DV=DV, N=N, qkv=act)
    shapes = {
        "x_q": (act, (1, T, H, DK)), "x_k": (act, (1, T, H, DK)), "x_v": (act, (1, T, HV, DV)),
        "w_q": (taps, (K, H * DK)), "w_k": (taps, (K, H * DK)), "w_v": (taps, (K, HV * DV)),
        "win_q": (kda.KDA_F32, (N, K - 1, H * DK)), "win_k": (kda.KDA_F32, (N, K - 1, H * DK)),
        "win_v": (kda.KDA_F32, (N, K - 1, HV * DV)),
        "q_conv": (kda.KDA_F32, (1, T, H, DK)), "k_conv": (kda.KDA_F32, (1, T, H, DK)),
    }
    conv = {n: kda.raw_tensor(_FAKE_CONV[i], *shapes[n]) for i, n in enumerate(kda.CONV_FIELDS)}
    return d, conv


def call_conv(d, conv, **mode_kw):
    c = None if conv is None else kda.KdaConv(*[conv[n] for n in kda.CONV_FIELDS])
    return kda.call_raw_conv(d["out"], c, [d[n] for n in kda.CONV_REST], kda.make_mode(**mode_kw), 0)


def test_conv_nothing_to_do_and_null():
    d, conv = conv_descriptors(B=0, T=0)
    assert call_conv(d, conv) == kda.KDA_OK
    assert call_conv(d, None) == kda.KDA_ERR_NULL
    d, conv = conv_descriptors()
    conv["win_k"] = kda.raw_tensor(0, kda.KDA_F32, (8, 3, 256))
    assert call_conv(d, conv) == kda.KDA_ERR_NULL


@pytest.mark.parametrize("K", [1, 5, 8])
def test_conv_width_outside_2_to_4_is_unsupported(K):
    d, conv = conv_descriptors(K=K)
    assert call_conv(d, conv) == kda.KDA_ERR_UNSUPPORTED


def test_conv_dtype_and_shape_errors():
    d, conv = conv_descriptors()
    conv["x_q"] = kda.raw_tensor(conv["x_q"].data, kda.KDA_F32, (1, 3, 2, 128))
    assert call_conv(d, conv) == kda.KDA_ERR_DTYPE
    d, conv = conv_descriptors()
    conv["w_v"] = kda.raw_tensor(conv["w_v"].data, kda.KDA_BF16, (4, 512))
    assert call_conv(d, conv) == kda.KDA_ERR_DTYPE
    d, conv = conv_descriptors()
    conv["win_q"] = kda.raw_tensor(conv["win_q"].data, kda.KDA_BF16, (8, 3, 256))
    assert call_conv(d, conv) == kda.KDA_ERR_DTYPE
    d, conv = conv_descriptors()      # the convolved q/k are fp32
    conv["k_conv"] = kda.raw_tensor(conv["k_conv"].data, kda.KDA_BF16, (1, 3, 2, 128))
    assert call_conv(d, conv) == kda.KDA_ERR_DTYPE
    for name, shape in (("win_v", (8, 3, 256)), ("win_q", (8, 2, 256)), ("w_k", (4, 512)),
                        ("w_k", (3, 256)), ("x_k", (1, 3, 2, 64)), ("q_conv", (1, 3, 4, 128))):
        d, conv = conv_descriptors()
        conv[name] = kda.raw_tensor(conv[name].data, conv[name].dtype, shape)
        assert call_conv(d, conv) == kda.KDA_ERR_SHAPE, name
    # the recurrence arguments are checked as in kda_decode
    d, conv = conv_descriptors()
    assert call_conv(d, conv, gate_mode="lower_bound", lower_bound=1.0) == kda.KDA_ERR_MODE


# ---------------------------------------------------------------------------
# kda_prefill: the decode checks, plus the matmul selector and head sizes
# ---------------------------------------------------------------------------

def call_prefill(descs, matmul=kda.KDA_MATMUL_SPLIT_BF16, mode=None, **mode_kw):
    if mode is None:
        mode = kda.make_mode(**mode_kw)
    return kda.call_raw_prefill([descs[n] for n in kda.ARG_NAMES], mode, matmul, 0)


def test_prefill_nothing_to_do_and_nulls():
    assert call_prefill(descriptors(B=0, T=0)) == kda.KDA_OK
    assert call_prefill(descriptors(B=3, T=0), matmul=kda.KDA_MATMUL_F32) == kda.KDA_OK
    d = descriptors(B=0, T=0)
    assert kda.call_raw_prefill([d[n] for n in kda.ARG_NAMES], None, 0, 0) == kda.KDA_ERR_NULL
    for n in kda.ARG_NAMES:
        e = dict(d)
        e[n] = None
        assert call_prefill(e) == kda.KDA_ERR_NULL, n


@pytest.mark.parametrize("matmul", [-1, 2, 7])
def test_prefill_rejects_unknown_matmul(matmul):
    assert call_prefill(descriptors(B=0, T=0), matmul=matmul) == kda.KDA_ERR_MODE


@pytest.mark.parametrize("dk,dv", [(16, 128), (128, 16), (16, 16)])
def test_prefill_rejects_head_size_16(dk, dv):
    # decode takes 16; the chunked kernel needs whole 32-wide operand slices
    assert call(descriptors(B=0, T=0, DK=dk, DV=dv)) == kda.KDA_OK
    assert call_prefill(descriptors(B=0, T=0, DK=dk, DV=dv)) == kda.KDA_ERR_UNSUPPORTED


def test_prefill_shares_the_decode_checks():
    d = descriptors()
    e = dict(d)
    e["v"] = reshape(d["v"], (1, 4, 4, 128))              # T disagrees with q
    assert call_prefill(e) == kda.KDA_ERR_SHAPE
    assert call_prefill(d, gate_mode=7) == kda.KDA_ERR_MODE
    assert call_prefill(d, gate_mode="lower_bound", lower_bound=0.5) == kda.KDA_ERR_MODE


# ---------------------------------------------------------------------------
# sizes one launch cannot take (rejected by the checker, nothing launched)
# ---------------------------------------------------------------------------

def test_grids_beyond_one_dispatch_are_unsupported():
    # a dispatch covers at most 2^32 - 1 work-items; decode and prefill run
    # 64 per (request, value head, 32-column slab): 2^22 x 4 x 4 x 64 = 2^32
    d = descriptors(B=2 ** 22, HV=4, DV=128)
    assert call(d) == kda.KDA_ERR_UNSUPPORTED
    assert call_prefill(d) == kda.KDA_ERR_UNSUPPORTED
    d = descriptors(B=2 ** 24, H=2, HV=4, DV=16)          # one slab: 2^24 x 4 x 64
    assert call(d) == kda.KDA_ERR_UNSUPPORTED
    # the q/k convolution runs 128 per (request, key head): 2^24 x 2 x 128
    d, conv = conv_descriptors(B=2 ** 24, H=2, HV=2, DV=16)
    assert call_conv(d, conv) == kda.KDA_ERR_UNSUPPORTED


@pytest.mark.parametrize("B,T", [(2 ** 31, 3), (2 ** 62, 3), (2 ** 63 - 2, 3), (2, 2 ** 31),
                                 (2, 2 ** 62)])
def test_huge_extents_are_rejected_without_overflow(B, T):
    d = descriptors(B=B, T=T)
    assert call(d) == kda.KDA_ERR_UNSUPPORTED
    assert call_prefill(d) == kda.KDA_ERR_UNSUPPORTED
    d, conv = conv_descriptors(B=B, T=T)
    assert call_conv(d, conv) == kda.KDA_ERR_UNSUPPORTED
