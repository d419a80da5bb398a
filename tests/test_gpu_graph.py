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


def test_graph_expert_side_replays_match_oracle():
    """The first expert matmul and its epilogue captured together and
    replayed on new rows and new per-expert counts, with eager matmuls
    between replays; every replay against the oracle."""
    import combine_moe_layout_03_amd as M

    rows, k, n_out, groups, stride = 300, 96, 64, 4, 128
    wts = W.gemm_case(920, 1, k, 2 * n_out, groups).w
    ws = (0.5 + W.uniform01(920, 5, 2 * n_out)).astype(np.float32) * np.float32(2.0 ** -10)
    ts = (0.005 + 0.015 * W.uniform01(920, 6, rows)).astype(np.float32)
    a = torch.zeros(rows * stride, dtype=torch.uint8, device="cuda")
    gc = torch.zeros(groups, dtype=torch.int32, device="cuda")
    w_d = torch.from_numpy(wts.view(np.uint8)).cuda()
    ws_d, ts_d = torch.from_numpy(ws).cuda(), torch.from_numpy(ts).cuda()
    acc = torch.zeros((rows, 2 * n_out), dtype=torch.int32, device="cuda")
    rb = M.moe_recv_row_bytes(n_out, M.MOE_INT8_ROWSCALE)
    out = torch.zeros(rows * rb, dtype=torch.uint8, device="cuda")

    def step():
        M.moe_grouped_gemm_i8(a, stride, rows, k, gc, w_d, acc)
        M.moe_deq_swiglu_quant(acc, ws_d, ts_d, out)

    log("graph expert side: eager warm-up")
    step()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    log("graph expert side: capture")
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    other = W.gemm_case(930, 200, k, 2 * n_out, groups, stride=stride, counts=[50, 50, 50, 50])
    other_a = torch.from_numpy(other.a.reshape(-1).view(np.uint8)).cuda()
    other_out = torch.zeros((200, 2 * n_out), dtype=torch.int32, device="cuda")
    for r, counts in enumerate(([100, 0, 150, 50], [300, 0, 0, 0], [10, 20, 30, 40])):
        c = W.gemm_case(940 + r, rows, k, 2 * n_out, groups, stride=stride, counts=counts)
        a.copy_(torch.from_numpy(c.a.reshape(-1).view(np.uint8)))
        gc.copy_(torch.from_numpy(c.group_count))
        acc.fill_(0)
        torch.cuda.synchronize()
        log(f"graph expert side: replay {r}")
        graph.replay()
        torch.cuda.synchronize()
        exp_acc, grp = oracle.grouped_gemm_i8(c.a, k, c.group_count, wts)
        exp_acc[grp < 0] = 0   # rows of no expert keep the zeros set before the replay
        assert np.array_equal(acc.cpu().numpy(), exp_acc), f"replay {r}: matmul"
        exp = oracle.swiglu_quant(exp_acc, ws, ts)
        raw = out.cpu().numpy().reshape(rows, rb)
        assert np.array_equal(np.ascontiguousarray(raw[:, :n_out]).view(np.int8), exp["codes"]), f"replay {r}"
        off = (n_out + 31) // 32 * 32
        inv = np.ascontiguousarray(raw[:, off:off + 4]).view(np.float32).reshape(-1)
        assert np.array_equal(inv.view(np.uint32), exp["inv"].view(np.uint32)), f"replay {r}: scales"
        M.moe_grouped_gemm_i8(other_a, stride, 200, k, torch.from_numpy(other.group_count).cuda(), w_d,
                              other_out)
        torch.cuda.synchronize()
    exp_o, _ = oracle.grouped_gemm_i8(other.a, k, other.group_count, wts)
    assert np.array_equal(other_out.cpu().numpy(), exp_o), "eager matmul between replays"


def test_graph_fused_expert_side_replays_match_oracle():
    """The matmul with its epilogue fused (three kernels: the row maxima
    cleared by a fill kernel, the matmul with the activation, the
    quantisation) captured once and replayed on new rows and new per-expert
    counts, with eager fused calls on other buffers between replays; every
    replay against the oracle, rows of no expert untouched."""
    import combine_moe_layout_03_amd as M

    rows, k, n, groups, stride = 300, 160, 40, 4, 192
    base = W.gemm_case(950, 1, k, 2 * n, groups)
    ws, ts = W.gemm_swiglu_scales(950, rows, k, n, groups)
    a = torch.zeros(rows * stride, dtype=torch.uint8, device="cuda")
    gc = torch.zeros(groups, dtype=torch.int32, device="cuda")
    w_d = torch.from_numpy(base.w.view(np.uint8)).cuda()
    ws_d, ts_d = torch.from_numpy(ws).cuda(), torch.from_numpy(ts).cuda()
    rb = M.moe_recv_row_bytes(n, M.MOE_INT8_ROWSCALE)
    out = torch.full((rows * rb,), 0xA5, dtype=torch.uint8, device="cuda")
    wsp = torch.empty(M.moe_gemm_swiglu_quant_workspace_bytes(rows, n), dtype=torch.uint8, device="cuda")

    def step():
        M.moe_grouped_gemm_swiglu_quant_i8(a, stride, rows, k, gc, w_d, ws_d, ts_d, out, wsp)

    log("graph fused expert side: eager warm-up")
    step()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    log("graph fused expert side: capture")
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    other = W.gemm_case(951, 120, k, 2 * n, groups, stride=stride, counts=[30, 30, 30, 30])
    other_a = torch.from_numpy(other.a.reshape(-1).view(np.uint8)).cuda()
    other_out = torch.zeros(120 * rb, dtype=torch.uint8, device="cuda")
    other_ws = torch.empty(M.moe_gemm_swiglu_quant_workspace_bytes(120, n), dtype=torch.uint8, device="cuda")
    off = (n + 31) // 32 * 32
    for r, counts in enumerate(([100, 0, 150, 20], [300, 0, 0, 0], [10, 20, 30, 40])):
        c = W.gemm_case(960 + r, rows, k, 2 * n, groups, stride=stride, counts=counts)
        a.copy_(torch.from_numpy(c.a.reshape(-1).view(np.uint8)))
        gc.copy_(torch.from_numpy(c.group_count))
        out.fill_(0xA5)
        torch.cuda.synchronize()
        log(f"graph fused expert side: replay {r}")
        graph.replay()
        torch.cuda.synchronize()
        acc, grp = oracle.grouped_gemm_i8(c.a, k, c.group_count, base.w)
        raw = out.cpu().numpy().reshape(rows, rb)
        for m in range(rows):
            if grp[m] < 0:
                assert (raw[m] == 0xA5).all(), f"replay {r}: row {m} of no expert was written"
                continue
            codes, inv, _ = oracle.swiglu_quant_row(acc[m], ws[grp[m]], ts[m])
            assert np.array_equal(raw[m, :n].view(np.int8), codes), f"replay {r}: row {m} codes"
            assert raw[m, off:off + 4].view(np.uint32)[0] == np.float32(inv).view(np.uint32), \
                f"replay {r}: row {m} scale"
        M.moe_grouped_gemm_swiglu_quant_i8(other_a, stride, 120, k, torch.from_numpy(other.group_count).cuda(),
                                           w_d, ws_d, ts_d, other_out, other_ws)
        torch.cuda.synchronize()
    acc_o, grp_o = oracle.grouped_gemm_i8(other.a, k, other.group_count, base.w)
    raw_o = other_out.cpu().numpy().reshape(120, rb)
    for m in range(120):
        codes, inv, _ = oracle.swiglu_quant_row(acc_o[m], ws[grp_o[m]], ts[m])
        assert np.array_equal(raw_o[m, :n].view(np.int8), codes), f"eager fused call between replays, row {m}"
