"""Expert-side epilogue (dequantise, SwiGLU, requantise) on the GPU against
the CPU oracle, through the C ABI.

Bar: int8 codes and inverse scales bit-exact (both sides compute e^x by the
same written-out binary32 method, divide with correctly rounded binary32
division and round every operation on its own), on every row of every case,
including the shape the benchmark times.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import GpuRun, align32, dev_f32, dev_i32, int8_row_bytes, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible MI355X")


def M():
    import combine_moe_layout_03_amd as mod

    return mod


def unpack_rows(out: torch.Tensor, rows: int, n: int):
    rb = int8_row_bytes(n)
    raw = out.cpu().numpy()[: rows * rb].reshape(rows, rb)
    codes = np.ascontiguousarray(raw[:, :n]).view(np.int8)
    inv = np.ascontiguousarray(raw[:, align32(n):align32(n) + 4]).view(np.float32).reshape(-1)
    return codes, inv


def run_gpu(case, guard_rows: int = 0):
    mod = M()
    rb = mod.moe_recv_row_bytes(case.n, mod.MOE_INT8_ROWSCALE)
    out = torch.full(((case.rows + guard_rows) * rb,), 0xA5, dtype=torch.uint8, device="cuda")
    mod.moe_deq_swiglu_quant(dev_i32(case.acc), dev_f32(case.weight_scale), dev_f32(case.token_scale), out)
    torch.cuda.synchronize()
    return out


def assert_same(case, out, what):
    exp = oracle.swiglu_quant(case.acc, case.weight_scale, case.token_scale)
    codes, inv = unpack_rows(out, case.rows, case.n)
    bad_rows = np.nonzero(np.any(codes != exp["codes"], axis=1))[0]
    assert bad_rows.size == 0, f"{what}: codes differ in rows {bad_rows[:10].tolist()}"
    assert np.array_equal(inv.view(np.uint32), exp["inv"].view(np.uint32)), f"{what}: inverse scales differ"


# n covers one wave per row with 1, 2 and 4 chunks per lane, two and four
# waves per row, and chunk counts that leave lanes and waves partly idle.
@pytest.mark.parametrize("rows,n,seed", [
    (6, 4, 1), (37, 12, 2), (9, 256, 3), (130, 1020, 4), (257, 1024, 5), (100, 1028, 6),
    (64, 2048, 7), (33, 2052, 8), (19, 4096, 9), (1, 8, 10), (5, 3000, 11),
])
def test_epilogue_matches_oracle(rows, n, seed):
    case = W.epilogue_case(seed, rows, n)
    log(f"epilogue rows={rows} n={n} seed={seed}")
    out = run_gpu(case, guard_rows=2)
    assert_same(case, out, f"rows={rows} n={n}")
    rb = int8_row_bytes(n)
    tail = out.cpu().numpy()[rows * rb:]
    assert np.all(tail == 0xA5), "bytes past the last row were written"


def test_epilogue_full_size():
    c = W.EPILOGUE_CONFIG
    case = W.epilogue_case(c["seed"], c["rows"], c["n"])
    log(f"epilogue full size rows={case.rows} n={case.n}")
    out = run_gpu(case)
    assert_same(case, out, "full size")


def test_epilogue_extreme_gate_values():
    """Gates spread over the whole binary32 range of e^-g: overflow to +inf,
    subnormal and zero results, and exactly representable huge products."""
    rows, n = 8, 256
    rng = np.random.default_rng(3)
    acc = rng.integers(-(2 ** 31), 2 ** 31 - 1, (rows, 2 * n)).astype(np.int32)
    ws = np.float32(2.0) ** rng.integers(-40, -20, 2 * n).astype(np.float32)
    ts = np.float32(2.0) ** rng.integers(-4, 4, rows).astype(np.float32)
    case = W.EpilogueCase(rows=rows, n=n, acc=acc, weight_scale=ws.astype(np.float32),
                          token_scale=ts.astype(np.float32), seed=3)
    log("epilogue extreme gates")
    assert_same(case, run_gpu(case), "extreme gates")


def test_epilogue_token_scales_in_place_from_receive_buffer():
    """The int8 receive buffer's inverse scales used in place as the token
    scales (stride = receive row bytes), after a GPU dispatch."""
    w = W.make_workload("small")
    run = GpuRun(w, quant=True).layout().notify().dispatch()
    torch.cuda.synchronize()
    rows = w.bs * w.topk
    n = 512
    case = W.epilogue_case(21, rows, n)
    mod = M()
    base, stride = mod.token_scales_of(run.buf.recv_x, w.hidden)
    rb = mod.moe_recv_row_bytes(n, mod.MOE_INT8_ROWSCALE)
    out = torch.zeros(rows * rb, dtype=torch.uint8, device="cuda")
    log("epilogue with token scales read from the receive buffer")
    mod.moe_deq_swiglu_quant(dev_i32(case.acc), dev_f32(case.weight_scale), base, out,
                             token_scale_stride=stride)
    torch.cuda.synchronize()
    # the oracle's own dispatch gives the token scales it uses; the GPU's
    # receive buffer must hold the same inverse scales bit for bit
    ref = oracle.pipeline(w.x, w.x_dtype, w.topk_idx, w.topk_w, w.expert_num_per_rank, w.rank_size,
                          True, w.x_dtype)["dispatch"]
    recv = run.host()["recv"]
    assert np.array_equal(recv["inv"].view(np.uint32), ref["inv"].view(np.uint32))
    case_ts = W.EpilogueCase(rows=rows, n=n, acc=case.acc, weight_scale=case.weight_scale,
                             token_scale=np.ascontiguousarray(ref["inv"]), seed=21)
    assert_same(case_ts, out, "in-place token scales")


def test_epilogue_zero_rows_and_repeat():
    mod = M()
    case = W.epilogue_case(31, 40, 64)
    out = torch.full((8,), 7, dtype=torch.uint8, device="cuda")
    log("epilogue rows=0")
    mod.moe_deq_swiglu_quant(dev_i32(case.acc[:0]), dev_f32(case.weight_scale),
                             dev_f32(case.token_scale[:0]), out)
    torch.cuda.synchronize()
    assert out.cpu().tolist() == [7] * 8
    log("epilogue repeated calls")
    a = run_gpu(case).cpu().numpy()
    b = run_gpu(case).cpu().numpy()
    assert np.array_equal(a, b)


def test_epilogue_errors_raise():
    mod = M()
    case = W.epilogue_case(41, 4, 8)
    out = torch.zeros(4 * 64, dtype=torch.uint8, device="cuda")
    with pytest.raises(mod.MoeEpError):
        mod.moe_deq_swiglu_quant(dev_i32(case.acc), dev_f32(case.weight_scale), dev_f32(case.token_scale),
                                 out[:100])
    with pytest.raises(mod.MoeEpError):
        mod.moe_deq_swiglu_quant(dev_i32(case.acc), dev_f32(case.weight_scale), dev_f32(case.token_scale),
                                 out, token_scale_stride=2)
