"""The decode and prefill calls captured in a HIP graph (torch.cuda.graph)
and replayed: a serving loop replays one captured decode step per token.

Each call advances the pool in place, so every replay is compared with the
same number of eager calls on a copy of the pool; replays are separated by
eager work and synchronisations.  Same kernel, same inputs: the results
must be bit-identical.
"""
import pytest

from gated_delta_rule_82_amd import workloads as wl
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


def _bits(t, torch):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t


@pytest.mark.parametrize("entry", ["decode", "prefill"])
def test_graph_replays_match_eager_calls(torch_cuda, entry):
    torch = torch_cuda
    tokens = "1" if entry == "decode" else "u:10..40"
    cfg = wl.Workload(name="graph", B=8, H=4, HV=8, DK=128, DV=128, n_slots=12, tokens=tokens,
                      gate_mode=wl.LOWER_BOUND, lower_bound=-5.0, seed=31, state_layout="v_first")
    print("[case] graph", entry, cfg, flush=True)
    inp = wl.draw(cfg)
    dev = wl.to_device(inp)
    pool_graph = wl.device_pool(inp)
    pool_eager = pool_graph.clone()
    out_graph = wl.empty_out(inp)
    out_eager = wl.empty_out(inp)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):           # warm-up outside the capture
        warm = pool_graph.clone()
        H.run_gpu(inp, dev, warm, wl.empty_out(inp), entry=entry)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    del warm

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        H.run_gpu(inp, dev, pool_graph, out_graph, entry=entry)
    torch.cuda.synchronize()

    for step in range(4):
        graph.replay()
        H.run_gpu(inp, dev, pool_eager, out_eager, entry=entry)
        torch.cuda.synchronize()
        assert torch.equal(_bits(out_graph, torch), _bits(out_eager, torch)), f"replay {step}: out"
        assert torch.equal(pool_graph, pool_eager), f"replay {step}: state"
        # unrelated eager work between replays
        (pool_eager.sum() + 1.0).item()
