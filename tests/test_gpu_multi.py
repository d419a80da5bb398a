"""Several source ranks sharing one receive buffer (the multi-source notify,
dispatch and combine entry points) against the oracle, through the C ABI:
counts, offsets, every written receive row and every output bit-identical."""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import dev_f32, dev_half, dev_i32, host_bits, log, unpack_recv

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible MI355X")


def _sources(seed, sizes, h, k, e, r, routing, bad, kind):
    return [W.random_case(seed + i, bs, h, k, e, r, x_dtype=kind, routing=routing, bad_frac=bad,
                          zero_rows=1 if bs > 1 else 0)
            for i, bs in enumerate(sizes)]


def _run_gpu(cases, h, k, e, r, kind, quant, streams=None):
    import combine_moe_layout_03_amd as M

    x_dtype = torch.bfloat16 if kind == "bf16" else torch.float16
    buf = M.EpMultiBuffers([c.bs for c in cases], h, k, e // r, r, x_dtype=x_dtype, quant_int8=quant)
    xs = [dev_half(c.x, kind) for c in cases]
    idxs = [dev_i32(c.topk_idx) for c in cases]
    ws = [dev_f32(c.topk_w) for c in cases]
    if streams is None:
        buf.run(xs, idxs, ws)
    else:
        # each source's layout, dispatch and combine on its own stream (each
        # source has its own layout workspace and outputs, and sources write
        # disjoint receive rows); the notify over all sources' counts on the
        # current stream after the layouts have joined
        ev0 = torch.cuda.Event()
        ev0.record()
        for s in range(len(cases)):
            st = streams[s % len(streams)]
            st.wait_event(ev0)
            with torch.cuda.stream(st):
                buf.layout(s, idxs[s])
        for st in streams:
            torch.cuda.current_stream().wait_stream(st)
        buf.notify()
        ev = torch.cuda.Event()
        ev.record()
        for s in range(len(cases)):
            st = streams[s % len(streams)]
            st.wait_event(ev)
            with torch.cuda.stream(st):
                buf.dispatch(s, xs[s], idxs[s])
        for st in streams:
            torch.cuda.current_stream().wait_stream(st)
        ev2 = torch.cuda.Event()
        ev2.record()
        for s in range(len(cases)):
            st = streams[s % len(streams)]
            st.wait_event(ev2)
            with torch.cuda.stream(st):
                buf.combine(s, idxs[s], ws[s])
        for st in streams:
            torch.cuda.current_stream().wait_stream(st)
    torch.cuda.synchronize()
    return buf


def _compare(buf, cases, h, e, r, kind, quant):
    ref = oracle.pipeline_multi([c.x for c in cases], kind, [c.topk_idx for c in cases],
                                [c.topk_w for c in cases], e // r, r, quant)
    for s, lay in enumerate(ref["layouts"]):
        np.testing.assert_array_equal(buf.token_per_expert[s].cpu().numpy(), lay["token_per_expert"])
        np.testing.assert_array_equal(buf.token_per_rank[s].cpu().numpy(), lay["token_per_rank"])
        np.testing.assert_array_equal(buf.send_token_idx[s].cpu().numpy(), lay["send_token_idx"])
        assert int(buf.bad_id_count[s].item()) == lay["bad"]
    no = ref["notify"]
    np.testing.assert_array_equal(buf.put_offset.cpu().numpy(), no["put_offset"])
    np.testing.assert_array_equal(buf.recv_count.cpu().numpy(), no["recv_count"])
    np.testing.assert_array_equal(buf.recv_base.cpu().numpy(), no["recv_base"])
    np.testing.assert_array_equal(buf.recv_token_per_expert.cpu().numpy(), no["recv_token_per_expert"])
    written = int(no["recv_base"][-1] + no["recv_count"][-1])
    got = unpack_recv(buf.recv_x, h, "int8" if quant else kind)
    if quant:
        np.testing.assert_array_equal(got["codes"][:written], ref["dispatch"]["codes"][:written])
        np.testing.assert_array_equal(got["inv"][:written].view(np.uint32),
                                      ref["dispatch"]["inv"][:written].view(np.uint32))
    else:
        np.testing.assert_array_equal(got["rows"][:written], ref["dispatch"]["rows"][:written])
    for s, out in enumerate(ref["outs"]):
        np.testing.assert_array_equal(host_bits(buf.out[s]), out)


MULTI_CASES = [
    # seed, sizes, h, k, E, R, routing, bad, kind, quant
    (501, (5, 3), 8, 2, 4, 2, "dup", 0.0, "bf16", True),
    (502, (40, 0, 17, 33), 136, 4, 12, 3, "dup", 0.1, "bf16", False),
    (503, (64,) * 8, 256, 8, 64, 8, "uniform", 0.0, "bf16", True),
    (504, (100, 1, 250), 1024, 8, 256, 16, "zipf1.2", 0.02, "fp16", True),
    (505, (30, 30), 64, 3, 2, 1, "hot", 0.0, "bf16", True),
    (506, (300, 200, 100), 520, 6, 2048, 64, "uniform", 0.0, "bf16", True),
    (507, (1,) * 16, 8192, 8, 256, 16, "uniform", 0.0, "bf16", True),
]


@pytest.mark.parametrize("case", MULTI_CASES, ids=[str(c[0]) for c in MULTI_CASES])
def test_multi_source_pipeline(case):
    seed, sizes, h, k, e, r, routing, bad, kind, quant = case
    cases = _sources(seed, sizes, h, k, e, r, routing, bad, kind)
    log(f"multi-source {case}")
    buf = _run_gpu(cases, h, k, e, r, kind, quant)
    _compare(buf, cases, h, e, r, kind, quant)


def test_multi_source_large_shape_split_over_16_sources():
    """The large workload's shape (4096 tokens, h 7168, top-8, 256 experts
    over 16 ranks) as 16 sources of 256 tokens each, int8."""
    cases = _sources(520, (256,) * 16, 7168, 8, 256, 16, "uniform", 0.0, "bf16")
    log("multi-source 16 x 256 tokens, h 7168")
    buf = _run_gpu(cases, 7168, 8, 256, 16, "bf16", True)
    _compare(buf, cases, 7168, 256, 16, "bf16", True)


def test_multi_source_on_separate_streams():
    cases = _sources(530, (200, 150, 90, 40), 512, 8, 64, 8, "dup", 0.01, "bf16")
    log("multi-source, layout, dispatch and combine on three streams")
    streams = [torch.cuda.Stream(), torch.cuda.Stream(), torch.cuda.Stream()]
    buf = _run_gpu(cases, 512, 8, 64, 8, "bf16", True, streams=streams)
    _compare(buf, cases, 512, 64, 8, "bf16", True)


def test_notify_multi_at_the_limits():
    """384 sources x 2048 experts: the count matrix the kernel scans is at
    its maximum size."""
    import combine_moe_layout_03_amd as M

    s_num, e, r = M.MOE_MAX_SOURCES, M.MOE_MAX_EXPERTS, 64
    counts = (W.u64(540, 0, s_num * e) % np.uint64(3)).astype(np.int32).reshape(s_num, e)
    log("notify_multi 384 x 2048")
    dev = dev_i32(counts)
    put = torch.zeros((e, s_num), dtype=torch.int32, device="cuda")
    cnt = torch.zeros(r, dtype=torch.int32, device="cuda")
    base = torch.zeros(r, dtype=torch.int32, device="cuda")
    rtpe = torch.zeros(e, dtype=torch.int32, device="cuda")
    M.moe_notify_multi(dev, e // r, r, put, cnt, base, rtpe)
    torch.cuda.synchronize()
    ref = oracle.notify_multi(counts, e // r, r)
    np.testing.assert_array_equal(put.cpu().numpy(), ref["put_offset"])
    np.testing.assert_array_equal(cnt.cpu().numpy(), ref["recv_count"])
    np.testing.assert_array_equal(base.cpu().numpy(), ref["recv_base"])
    np.testing.assert_array_equal(rtpe.cpu().numpy(), ref["recv_token_per_expert"])


def test_single_source_multi_entry_points_match_the_plain_ones():
    """numSrc = 1 through the multi-source entry points gives the
    single-source results."""
    import combine_moe_layout_03_amd as M

    c = W.random_case(550, 300, 256, 4, 32, 4, routing="dup", bad_frac=0.02)
    log("multi-source entry points with one source")
    buf = _run_gpu([c], 256, 4, 32, 4, "bf16", True)
    one = M.EpBuffers(300, 256, 4, 8, 4, quant_int8=True)
    one.run(dev_half(c.x, "bf16"), dev_i32(c.topk_idx), dev_f32(c.topk_w))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(buf.put_offset[:, 0].cpu().numpy(), one.put_offset.cpu().numpy())
    np.testing.assert_array_equal(buf.recv_x.cpu().numpy(), one.recv_x.cpu().numpy())
    np.testing.assert_array_equal(host_bits(buf.out[0]), host_bits(one.out))
