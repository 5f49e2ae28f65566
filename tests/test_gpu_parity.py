"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Tolerances are the ones fixed in tests/kda_harness.py.  Every case prints
its name and shape before it touches the GPU.
"""
import itertools
import math

import numpy as np
import pytest

from gated_delta_rule_82_amd import workloads as wl
from oracle import kda_oracle as ko
from tests import kda_harness as H

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gated_delta_rule_82_amd import kda
    kda.library()
    return torch


def _say(*a):
    print("[case]", *a, flush=True)


def small(name="small", B=5, H_=2, HV=4, DK=128, DV=128, tokens="u:0..5", qkv="bf16",
          gate=wl.SOFTPLUS, lb=0.0, slots=None, seed=0, **kw):
    return wl.Workload(name=name, B=B, H=H_, HV=HV, DK=DK, DV=DV,
                       n_slots=slots if slots is not None else 2 * B + 3, tokens=tokens,
                       qkv_dtype=qkv, gate_mode=gate, lower_bound=lb, seed=seed,
                       host_state=True, **kw)


# ---------------------------------------------------------------------------
# the configured workloads
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["tiny", "kimi_b64_h32", "varlen_gqa_b128"])
def test_preset_all_tiles(torch_cuda, name):
    cfg = wl.PRESETS[name]
    _say(name, cfg.description)
    stats, _, _ = H.parity_case(wl.draw(cfg))
    print(name, stats, flush=True)


@pytest.mark.parametrize("name,sample", [("wide_b256_h96", 384), ("stress_b1024_n4", 192)])
def test_preset_full_size_sampled(torch_cuda, name, sample):
    cfg = wl.PRESETS[name]
    _say(name, cfg.description, "sampled tiles", sample)
    stats, _, _ = H.parity_case(wl.draw(cfg), sample=sample)
    print(name, stats, flush=True)
    torch_cuda.cuda.empty_cache()


# ---------------------------------------------------------------------------
# every specialization, ragged batches
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dk,dv", list(itertools.product([16, 32, 64, 128], repeat=2)))
@pytest.mark.parametrize("qkv", ["bf16", "f32"])
@pytest.mark.parametrize("gate", [wl.SOFTPLUS, wl.LOWER_BOUND])
def test_head_dims_and_modes(torch_cuda, dk, dv, qkv, gate):
    cfg = small(DK=dk, DV=dv, qkv=qkv, gate=gate, lb=-5.0 if gate == wl.LOWER_BOUND else 0.0,
                seed=dk * 3 + dv)
    _say("dims", dk, dv, qkv, gate)
    H.parity_case(wl.draw(cfg))


@pytest.mark.parametrize("dk,dv", list(itertools.product([16, 32, 64, 128], repeat=2)))
@pytest.mark.parametrize("layout,sdt", [("v_first", "f32"), ("k_first", "bf16"), ("v_first", "bf16")])
def test_state_layouts_and_dtypes(torch_cuda, dk, dv, layout, sdt):
    gate = wl.LOWER_BOUND if (dk + dv) % 64 else wl.SOFTPLUS
    qkv = "f32" if dk == dv == 16 else "bf16"
    cfg = small(DK=dk, DV=dv, qkv=qkv, gate=gate, lb=-5.0 if gate == wl.LOWER_BOUND else 0.0,
                seed=dk * 5 + dv, state_layout=layout, state_dtype=sdt)
    _say("layout", layout, sdt, dk, dv, qkv, gate)
    H.parity_case(wl.draw(cfg))


@pytest.mark.parametrize("name,sample,layout,sdt", [
    ("wide_b256_h96", 256, "v_first", "f32"),
    ("wide_b256_h96", 256, "k_first", "bf16"),
    ("varlen_gqa_b128", 512, "v_first", "f32"),
    ("stress_b1024_n4", 128, "v_first", "bf16"),
])
def test_full_size_other_layouts(torch_cuda, name, sample, layout, sdt):
    cfg = wl.preset(name, state_layout=layout, state_dtype=sdt)
    _say(name, layout, sdt, "sampled tiles", sample)
    stats, _, _ = H.parity_case(wl.draw(cfg), sample=sample)
    print(name, layout, sdt, stats, flush=True)
    torch_cuda.cuda.empty_cache()


@pytest.mark.parametrize("tokens,slabs", [("1", 16384), ("u:1..4", 32768)])
@pytest.mark.parametrize("dk,dv", [(16, 64), (32, 64), (64, 64), (128, 64), (16, 128), (64, 128)])
def test_kfirst_bf16_wide_slabs_every_tile(torch_cuda, dk, dv, tokens, slabs):
    """Batches of at least 16384 32-column slabs (one token per request) or
    32768 (longer requests) on a key-first bf16 pool run on 64-column slabs
    (two sums per lane after the reduction); every tile of such a batch
    against the oracle, GQA, both gate modes across the shapes, every other
    slot bit-identical."""
    B = slabs // (4 * dv // 32)
    gate = wl.LOWER_BOUND if dk % 32 else wl.SOFTPLUS
    cfg = wl.Workload(name="wide_slabs", B=B, H=2, HV=4, DK=dk, DV=dv, n_slots=B + 7, tokens=tokens,
                      gate_mode=gate, lower_bound=-5.0 if gate == wl.LOWER_BOUND else 0.0,
                      seed=31 + dk + dv, state_dtype="bf16")
    _say("k-first bf16 wide slabs", dk, dv, B, tokens, gate)
    stats, _, _ = H.parity_case(wl.draw(cfg))
    print("wide slabs", dk, dv, stats, flush=True)


@pytest.mark.parametrize("layout,sdt", [("k_first", "f32"), ("v_first", "f32"),
                                        ("k_first", "bf16"), ("v_first", "bf16")])
@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 32)])
def test_custom_scale_and_eps(torch_cuda, layout, sdt, dk, dv):
    """kda_mode.scale and kda_mode.l2_eps replace the defaults dk^-0.5 and
    1e-6 ("KDA Block TKG" scale parameter and l2_eps default); the oracle
    runs with the same values.  eps = 16 is large against sum(x^2) ~ dk, so
    it moves every normalised q and k by several percent."""
    cfg = small(B=6, H_=2, HV=4, DK=dk, DV=dv, tokens="u:1..6", gate=wl.LOWER_BOUND, lb=-5.0,
                seed=21 + dk, state_layout=layout, state_dtype=sdt)
    over = {"scale": 0.3, "l2_eps": 16.0}
    _say("scale/eps", layout, sdt, dk, dv, over)
    stats, out_t, _ = H.parity_case(wl.draw(cfg), mode_overrides=over, oracle_mode=over)
    print("scale/eps", layout, sdt, stats, flush=True)
    # each override must matter: the oracle with either one left at its
    # default is far from this output
    inp = wl.draw(cfg)
    tiles = [(b, hv) for b in range(cfg.B) for hv in range(cfg.HV)]
    pool = wl.host_pool(inp)    # in the workload's layout and dtype, as uploaded
    init = [pool[int(inp.state_indices[b]), hv] for b, hv in tiles if inp.state_indices[b] >= 0]
    og = H.out_to_f64(out_t)
    floor = max(stats["out_max_abs"], 1e-6)
    for partial in ({"scale": 0.3}, {"l2_eps": 16.0}):
        o_part, _ = H.oracle_tiles(inp, tiles, init, **partial)
        assert np.max(np.abs(og - o_part)) > 10 * floor, partial


def test_ragged_grid_not_multiple_of_8(torch_cuda):
    cfg = small(B=37, H_=5, HV=5, tokens="u:0..3", slots=50, seed=5)
    _say("ragged", cfg)
    stats, _, _ = H.parity_case(wl.draw(cfg))
    print(stats)


@pytest.mark.parametrize("gate", [wl.LOWER_BOUND, wl.SOFTPLUS])
@pytest.mark.parametrize("layout,sdt", [("k_first", "f32"), ("v_first", "f32"),
                                        ("k_first", "bf16"), ("v_first", "bf16")])
def test_long_requests(torch_cuda, gate, layout, sdt):
    """Requests of 40 to 64 tokens: the kernels' deferred decay folds each
    key's pending factor into the slab several times within a request (a
    lower-bound gate of -5 takes it below 2^-64 in about nine tokens, the
    drawn softplus gates in fewer)."""
    cfg = small(B=3, H_=2, HV=4, tokens="u:40..64", gate=gate,
                lb=-5.0 if gate == wl.LOWER_BOUND else 0.0, seed=9, state_layout=layout,
                state_dtype=sdt)
    _say("long", gate, layout, sdt)
    stats, _, _ = H.parity_case(wl.draw(cfg))
    print(stats)


def test_gqa_g4(torch_cuda):
    cfg = small(B=6, H_=2, HV=8, tokens="u:1..4", seed=11)
    _say("gqa4", cfg)
    H.parity_case(wl.draw(cfg))


# ---------------------------------------------------------------------------
# special cases the method has
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("gate,layout,sdt", [(wl.SOFTPLUS, "k_first", "f32"),
                                              (wl.LOWER_BOUND, "k_first", "f32"),
                                              (wl.SOFTPLUS, "v_first", "f32"),
                                              (wl.LOWER_BOUND, "v_first", "bf16"),
                                              (wl.SOFTPLUS, "k_first", "bf16")])
def test_pass_through_is_bit_exact(torch_cuda, gate, layout, sdt):
    """beta = 0 and g = 0 leave the state bit-identical."""
    torch = torch_cuda
    cfg = small(B=4, tokens="u:1..3", gate=gate, lb=0.0, seed=21, state_layout=layout,
                state_dtype=sdt)
    inp = wl.draw(cfg)
    inp.beta_logits[:] = -np.inf
    if gate == wl.SOFTPLUS:
        inp.a_log[:] = -np.inf
    _say("pass-through", gate)
    dev = wl.to_device(inp)
    pool = wl.device_pool(inp)
    before = pool.clone()
    out = H.run_gpu(inp, dev, pool)
    torch.cuda.synchronize()
    assert torch.equal(pool, before)
    tiles = H.choose_tiles(inp, None)
    init = [before[int(inp.state_indices[b]), hv].float().cpu().numpy() for b, hv in tiles
            if inp.state_indices[b] >= 0]
    ref, _ = H.oracle_tiles(inp, tiles, init)
    H.compare_outputs(inp, tiles, H.out_to_f64(out), ref)


def test_skip_index_and_empty_request(torch_cuda):
    torch = torch_cuda
    cfg = small(B=4, cu_seqlens=(0, 2, 2, 5, 6), state_indices=(3, 5, -1, 0), slots=8, seed=22)
    inp = wl.draw(cfg)
    _say("skip/empty", cfg)
    stats, out, pool = H.parity_case(inp)
    o = H.out_to_f64(out)
    assert np.all(o[0, 2:5] == 0.0)              # request 2 skipped
    assert np.isfinite(o).all()


@pytest.mark.parametrize("layout", ["k_first", "v_first"])
def test_deterministic_bitwise(torch_cuda, layout):
    torch = torch_cuda
    cfg = small(B=16, HV=8, H_=4, tokens="u:1..6", seed=23, state_layout=layout)
    inp = wl.draw(cfg)
    _say("determinism", cfg)
    dev = wl.to_device(inp)
    p1 = wl.device_pool(inp)
    p2 = p1.clone()
    o1 = H.run_gpu(inp, dev, p1)
    o2 = H.run_gpu(inp, dev, p2)
    torch.cuda.synchronize()
    assert torch.equal(p1, p2)
    assert torch.equal(o1.view(torch.int16) if o1.dtype == torch.bfloat16 else o1,
                       o2.view(torch.int16) if o2.dtype == torch.bfloat16 else o2)


@pytest.mark.parametrize("layout", ["k_first", "v_first"])
def test_split_invariance(torch_cuda, layout):
    """One call over n tokens equals n calls of one token each (fp32 state)."""
    torch = torch_cuda
    n = 5
    cfg = small(B=3, tokens=str(n), seed=24, state_layout=layout)
    inp = wl.draw(cfg)
    _say("split", cfg)
    dev = wl.to_device(inp)
    pool_a = wl.device_pool(inp)
    pool_b = pool_a.clone()
    out_a = H.run_gpu(inp, dev, pool_a)
    outs = []
    for t in range(n):
        rows = np.array([b * n + t for b in range(cfg.B)])
        one = dict(dev)
        for key in ("q", "k", "v", "raw_gate", "beta_logits"):
            one[key] = dev[key][:, torch.as_tensor(rows, device=dev[key].device)].contiguous()
        one["cu_seqlens"] = torch.arange(cfg.B + 1, dtype=torch.int32, device=pool_b.device)
        o = torch.empty((1, cfg.B, cfg.HV, cfg.DV), dtype=out_a.dtype, device=pool_b.device)
        from gated_delta_rule_82_amd import kda
        kda.decode(o, one["q"], one["k"], one["v"], one["raw_gate"], one["beta_logits"],
                   one["a_log"], one["dt_bias"], one["cu_seqlens"], pool_b, one["state_indices"],
                   state_layout=layout)
        outs.append(o)
    torch.cuda.synchronize()
    assert torch.allclose(pool_a, pool_b, rtol=0, atol=1e-6 * float(pool_a.abs().max()))
    for t in range(n):
        rows = [b * n + t for b in range(cfg.B)]
        assert torch.equal(out_a[0, rows].float(), outs[t][0].float())


def test_gqa_equals_repeated_heads(torch_cuda):
    torch = torch_cuda
    cfg = small(B=4, H_=2, HV=6, tokens="u:1..3", seed=25)
    inp = wl.draw(cfg)
    _say("gqa-equivalence", cfg)
    dev = wl.to_device(inp)
    p1 = wl.device_pool(inp)
    p2 = p1.clone()
    o1 = H.run_gpu(inp, dev, p1)
    rep = dict(dev)
    rep["q"] = dev["q"].repeat_interleave(3, dim=2).contiguous()
    rep["k"] = dev["k"].repeat_interleave(3, dim=2).contiguous()
    o2 = H.run_gpu(inp, rep, p2)
    torch.cuda.synchronize()
    assert torch.equal(p1, p2)
    assert torch.equal(o1.float(), o2.float())


def test_delta_property_unit_key(torch_cuda):
    """g = 0, beta = 1, unit key e_j: after the write the key reads back v."""
    torch = torch_cuda
    cfg = small(B=2, H_=1, HV=1, tokens="1", qkv="f32", seed=26)
    inp = wl.draw(cfg)
    inp.k[:] = 0.0
    inp.k[0, 0, 0, 7] = 1.0
    inp.k[0, 1, 0, 100] = 2.0
    inp.beta_logits[:] = np.inf
    inp.a_log[:] = -np.inf
    _say("delta property", cfg)
    dev = wl.to_device(inp)
    pool = wl.device_pool(inp)
    # a negligible l2_eps makes the normalised key exactly e_j in fp32
    H.run_gpu(inp, dev, pool, mode_overrides={"l2_eps": 1e-30})
    torch.cuda.synchronize()
    for b, j in ((0, 7), (1, 100)):
        row = pool[int(inp.state_indices[b]), 0, j].cpu().numpy()
        np.testing.assert_allclose(row, inp.v[0, b, 0], rtol=2e-7, atol=1e-30)


def test_runs_on_a_side_stream(torch_cuda):
    torch = torch_cuda
    cfg = small(B=8, tokens="u:1..3", seed=27)
    inp = wl.draw(cfg)
    _say("side stream", cfg)
    s = torch.cuda.Stream()
    dev = wl.to_device(inp)
    pool = wl.device_pool(inp)
    ref_pool = pool.clone()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        out = H.run_gpu(inp, dev, pool)
    s.synchronize()
    out2 = H.run_gpu(inp, dev, ref_pool)
    torch.cuda.synchronize()
    assert torch.equal(pool, ref_pool) and torch.equal(out.float(), out2.float())


def test_argument_errors_raise_before_launch(torch_cuda):
    torch = torch_cuda
    from gated_delta_rule_82_amd import kda
    cfg = small(B=2, tokens="1", seed=28)
    inp = wl.draw(cfg)
    dev = wl.to_device(inp)
    pool = wl.device_pool(inp)
    before = pool.clone()
    out = wl.empty_out(inp)
    with pytest.raises(kda.KdaError) as e:      # out must take v's dtype
        kda.decode(out.float(), dev["q"], dev["k"], dev["v"], dev["raw_gate"], dev["beta_logits"],
                   dev["a_log"], dev["dt_bias"], dev["cu_seqlens"], pool, dev["state_indices"])
    assert e.value.code == kda.KDA_ERR_DTYPE
    with pytest.raises(kda.KdaError) as e:
        kda.decode(out, dev["q"], dev["k"], dev["v"], dev["raw_gate"], dev["beta_logits"],
                   dev["a_log"], dev["dt_bias"], dev["cu_seqlens"], pool, dev["state_indices"],
                   gate_mode="lower_bound", lower_bound=1.0)
    assert e.value.code == kda.KDA_ERR_MODE
    with pytest.raises(ValueError):
        kda.decode(out, dev["q"].cpu(), dev["k"], dev["v"], dev["raw_gate"], dev["beta_logits"],
                   dev["a_log"], dev["dt_bias"], dev["cu_seqlens"], pool, dev["state_indices"])
    torch.cuda.synchronize()
    assert torch.equal(pool, before)


def test_one_hip_runtime_in_process(torch_cuda):
    cfg = small(B=2, tokens="1", seed=29)
    H.parity_case(wl.draw(cfg))
    with open("/proc/self/maps") as f:
        libs = {line.split()[-1] for line in f if "libamdhip64" in line}
    assert len(libs) == 1, libs
    assert any("libkda.so" in line for line in open("/proc/self/maps"))
