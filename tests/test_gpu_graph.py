"""The pipeline captured into a HIP graph (torch.cuda.graph) and replayed.

The library only enqueues kernels on the caller's stream (no allocation, no
memset, no synchronisation), so a whole step can be captured once and
replayed.  Each replay runs on new inputs copied into the captured input
buffers, with eager work of the program between replays, and every replay is
checked against the oracle element by element.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import GpuRun, host_bits, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible MI355X")


def _check(run: GpuRun, w, quant: bool, what: str):
    got = run.host()
    ref = oracle.pipeline(w.x, w.x_dtype, w.topk_idx, w.topk_w, w.expert_num_per_rank, w.rank_size,
                          quant, w.x_dtype)
    assert np.array_equal(got["send_token_idx"], ref["layout"]["send_token_idx"]), what
    assert np.array_equal(got["token_per_expert"], ref["layout"]["token_per_expert"]), what
    assert np.array_equal(got["put_offset"], ref["notify"]["put_offset"]), what
    assert np.array_equal(got["out"], ref["out"]), f"{what}: combine output"


@pytest.mark.parametrize("name,quant,fused", [
    ("tiny", False, True), ("small", True, True), ("small", True, False), ("mid", True, True),
])
def test_graph_replays_match_oracle(name, quant, fused):
    base = W.make_workload(name)
    run = GpuRun(base, quant=quant)
    log(f"graph {name} quant={quant} fused={fused}: eager warm-up")
    run.run_all(fused=fused)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    log(f"graph {name}: capture")
    with torch.cuda.graph(graph):
        run.run_all(fused=fused)
    torch.cuda.synchronize()

    other = GpuRun(W.random_case(900, 64, base.hidden, base.topk, base.num_experts, base.rank_size),
                   quant=quant)
    for r in range(3):
        w = W.random_case(910 + r, base.bs, base.hidden, base.topk, base.num_experts, base.rank_size,
                          routing="dup" if r == 1 else "uniform")
        run.w = w
        run.x.copy_(torch.from_numpy(w.x.view(np.int16)).view(run.x.dtype))
        run.idx.copy_(torch.from_numpy(w.topk_idx))
        run.wts.copy_(torch.from_numpy(w.topk_w))
        torch.cuda.synchronize()
        log(f"graph {name}: replay {r}")
        graph.replay()
        torch.cuda.synchronize()
        _check(run, w, quant, f"{name} replay {r}")
        # eager work of the program between replays, on other buffers
        other.run_all(fused=fused)
        torch.cuda.synchronize()
    got_other = host_bits(other.buf.out) if other.out_kind != "fp32" else other.buf.out.cpu().numpy()
    ref_other = oracle.pipeline(other.w.x, other.w.x_dtype, other.w.topk_idx, other.w.topk_w,
                                other.w.expert_num_per_rank, other.w.rank_size, quant, other.w.x_dtype)
    assert np.array_equal(got_other, ref_other["out"]), "eager run between replays"
