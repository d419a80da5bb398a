"""The fused layout + notify + dispatch entry point against the oracle,
through the C ABI: every output bit-identical to the three stages."""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import GpuRun, log
from test_gpu_parity import compare, oracle_run, workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible MI355X")


@pytest.mark.parametrize("name,kind,quant", [("tiny", "bf16", False), ("small", "bf16", True),
                                             ("mid", "fp16", True), ("mid", "bf16", False),
                                             ("large", "bf16", True), ("large", "bf16", False),
                                             ("stress", "bf16", True)])
def test_fused_configs(name, kind, quant):
    """The workloads through the fused entry point, whole outputs compared; at
    large these are the launches the benchmark times (fused_kernel at 14
    chunks per lane, int8 and passthrough, then combine)."""
    w = workload(name, kind)
    log(f"fused {name} {kind} quant={quant}")
    g = GpuRun(w, quant).run_all(fused=True).host()
    compare(w, quant, kind, g, oracle_run(w, quant, kind))


FUSED_RANDOM = [
    # seed, bs, h, k, E, R, routing, bad, kind, quant
    (301, 1, 8, 1, 1, 1, "uniform", 0.0, "bf16", True),
    (302, 3, 136, 2, 4, 2, "dup", 0.0, "bf16", False),
    (303, 37, 1000, 3, 12, 3, "dup", 0.1, "bf16", True),
    (304, 256, 64, 8, 1, 1, "hot", 0.0, "bf16", True),
    (305, 300, 256, 8, 512, 16, "uniform", 0.0, "fp16", True),
    (306, 64, 128, 32, 64, 4, "dup", 0.05, "bf16", True),
    (307, 5, 8192, 3, 8, 2, "uniform", 0.0, "bf16", True),
    (308, 4100, 24, 8, 64, 8, "dup", 0.2, "bf16", True),
    (309, 9000, 16, 8, 32, 4, "zipf1.2", 0.01, "bf16", False),
    (310, 40000, 16, 8, 64, 8, "dup", 0.0, "bf16", True),
    (311, 700, 64, 4, 2048, 16, "uniform", 0.01, "bf16", True),
    (312, 100, 32, 8, 1024, 8, "dup", 0.0, "fp16", False),
    (313, 255, 40, 5, 3, 3, "hot", 0.3, "bf16", True),
    (314, 257, 7168, 8, 256, 16, "zipf1.2", 0.0, "bf16", True),
    (315, 4096, 512, 8, 256, 16, "hot", 0.0, "bf16", True),
    (316, 8192, 64, 8, 256, 16, "hot", 0.01, "bf16", True),
    (317, 2000, 24, 8, 2048, 64, "hot", 0.0, "fp16", True),
    # three scanning waves (E = 130), and eight with two experts per lane (E = 576)
    (318, 700, 96, 6, 130, 10, "uniform", 0.02, "bf16", True),
    (319, 1500, 40, 4, 576, 12, "zipf1.2", 0.0, "bf16", True),
    # 8 tokens per workgroup at h = 7168: every row loaded during the count
    (320, 2048, 7168, 8, 256, 16, "dup", 0.0, "bf16", True),
]


@pytest.mark.parametrize("case", FUSED_RANDOM, ids=[str(c[0]) for c in FUSED_RANDOM])
def test_fused_random(case):
    seed, bs, h, k, e, r, routing, bad, kind, quant = case
    w = W.random_case(seed, bs, h, k, e, r, x_dtype=kind, routing=routing, bad_frac=bad,
                      zero_rows=1 if bs > 1 else 0)
    log(f"fused random {case}")
    g = GpuRun(w, quant).run_all(fused=True).host()
    compare(w, quant, kind, g, oracle_run(w, quant, kind))


def test_fused_repeated_calls():
    """Several calls in a row on the same buffers, with different routings:
    nothing of one call leaks into the next."""
    import combine_moe_layout_03_amd as M

    bs, h, k, e, r = 2048, 256, 8, 64, 8
    buf = M.EpBuffers(bs, h, k, e // r, r, quant_int8=True)
    for rep in range(5):
        w = W.random_case(320 + rep, bs, h, k, e, r, routing="dup" if rep % 2 else "uniform")
        log(f"fused repeat {rep}")
        x = torch.from_numpy(w.x.view(np.int16)).cuda().view(torch.bfloat16)
        idx = torch.from_numpy(w.topk_idx).cuda()
        buf.layout_notify_dispatch(x, idx)
        torch.cuda.synchronize()
        ref = oracle.pipeline(w.x, "bf16", w.topk_idx, w.topk_w, e // r, r, True, "bf16")
        np.testing.assert_array_equal(buf.send_token_idx.cpu().numpy(), ref["layout"]["send_token_idx"])
        np.testing.assert_array_equal(buf.put_offset.cpu().numpy(), ref["notify"]["put_offset"])
        raw = buf.recv_x.cpu().numpy().reshape(-1, buf.row_bytes)
        total = bs * k
        np.testing.assert_array_equal(raw[:total, :h].view(np.int8), ref["dispatch"]["codes"][:total])


@pytest.mark.parametrize("seed,bs,h,k,e,r", [(330, 200, 8704, 4, 64, 8), (331, 8193, 16, 8, 32, 4)],
                         ids=["hidden_above_8192", "entries_above_2^16"])
def test_fused_fallback_shape_matches(seed, bs, h, k, e, r):
    """Shapes the one kernel does not take run the three stages through the
    same entry point."""
    import combine_moe_layout_03_amd as M

    assert not M.moe_fused_supported(bs, h, k, e // r, r, torch.bfloat16, True)
    w = W.random_case(seed, bs, h, k, e, r, routing="uniform")
    log(f"fused entry point, fallback shape {bs}x{h} k={k} E={e}")
    g = GpuRun(w, True).run_all(fused=True).host()
    compare(w, True, "bf16", g, oracle_run(w, True, "bf16"))


@pytest.mark.parametrize("seed,bs,h,k,e,r", [(340, 4096, 256, 8, 256, 16), (341, 37, 64, 3, 12, 3),
                                             (342, 1000, 128, 6, 64, 8)],
                         ids=["one_whole_round", "few_ids", "partial_round"])
def test_fused_ids_not_16_byte_aligned(seed, bs, h, k, e, r):
    """topk_idx at an address that is 4- but not 16-byte aligned: the
    counting waves read the ids four at a time with 4-byte loads."""
    w = W.random_case(seed, bs, h, k, e, r, routing="dup", bad_frac=0.01)
    run = GpuRun(w, True)
    store = torch.empty(bs * k + 1, dtype=torch.int32, device="cuda")
    store[1:] = run.idx.reshape(-1)
    run.idx = store[1:].view(bs, k)
    assert run.idx.data_ptr() % 16 != 0
    log(f"fused with unaligned ids {bs}x{h} k={k} E={e}")
    g = run.run_all(fused=True).host()
    compare(w, True, "bf16", g, oracle_run(w, True, "bf16"))
