"""moe_layout_no_alloc (the layout with the library's static workspace)
against moe_layout (the same stage with a caller-allocated workspace),
through the C ABI: two calls in a row, the second with a smaller input, every
output bit for bit; both also against the oracle."""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible MI355X")


def _outputs(e, r, bs, k):
    dev = "cuda"
    return dict(token_per_expert=torch.full((e,), -7, dtype=torch.int32, device=dev),
                token_per_rank=torch.full((r,), -7, dtype=torch.int32, device=dev),
                send_token_idx=torch.full((bs, k), -7, dtype=torch.int32, device=dev),
                bad_id_count=torch.full((1,), -7, dtype=torch.int32, device=dev))


# the first call covers many tiles (its table fills most of a 1 MiB scratch
# at E = 256: 1000 tiles); the second is smaller and leaves the first call's
# table in the scratch beyond its own tiles
CALLS = [(611, 256000, 8, 256, 16, "dup", 0.01), (612, 3000, 6, 64, 8, "zipf1.2", 0.02)]


def test_no_alloc_layout_matches_moe_layout_on_two_calls_in_a_row():
    import combine_moe_layout_03_amd as M

    for seed, bs, k, e, r, routing, bad in CALLS:
        w = W.random_case(seed, bs, 8, k, e, r, routing=routing, bad_frac=bad)
        idx = torch.from_numpy(w.topk_idx).cuda()
        epr = e // r
        need = M.moe_layout_workspace_bytes(bs, k, e)
        assert 0 < need <= M.MOE_NO_ALLOC_SCRATCH_BYTES
        ref = _outputs(e, r, bs, k)
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        log(f"moe_layout bs={bs} k={k} E={e}")
        M.moe_layout(idx, epr, r, ref["token_per_expert"], ref["token_per_rank"], ref["send_token_idx"],
                     ref["bad_id_count"], ws)
        got = _outputs(e, r, bs, k)
        log(f"moe_layout_no_alloc bs={bs} k={k} E={e}")
        M.moe_layout_no_alloc(idx, epr, r, got["token_per_expert"], got["token_per_rank"], got["send_token_idx"],
                              got["bad_id_count"])
        torch.cuda.synchronize()
        for name in ref:
            np.testing.assert_array_equal(got[name].cpu().numpy(), ref[name].cpu().numpy(), err_msg=name)
        o = oracle.layout(w.topk_idx, epr, r)
        np.testing.assert_array_equal(got["send_token_idx"].cpu().numpy(), o["send_token_idx"])
        np.testing.assert_array_equal(got["token_per_expert"].cpu().numpy(), o["token_per_expert"])
        assert int(got["bad_id_count"].item()) == o["bad"]


def test_no_alloc_layout_rejects_shapes_beyond_its_scratch():
    import combine_moe_layout_03_amd as M

    bs, k, e, r = 300000, 8, 256, 16   # 1172 tiles x 257 counts x 4 B > 1 MiB
    assert M.moe_layout_workspace_bytes(bs, k, e) > M.MOE_NO_ALLOC_SCRATCH_BYTES
    idx = torch.zeros((bs, k), dtype=torch.int32, device="cuda")
    out = _outputs(e, r, bs, k)
    log("moe_layout_no_alloc above the scratch limit")
    with pytest.raises(M.MoeEpError) as ei:
        M.moe_layout_no_alloc(idx, e // r, r, out["token_per_expert"], out["token_per_rank"],
                              out["send_token_idx"], out["bad_id_count"])
    assert ei.value.status == 9
    torch.cuda.synchronize()
    assert (out["token_per_expert"] == -7).all().item()


def test_no_alloc_layout_in_a_replayed_hip_graph():
    """The callers the no-allocation entry point exists for: the whole step
    (no-alloc layout, notify, dispatch, combine) captured once in a HIP
    graph and replayed on new routings written into the captured inputs,
    with eager work of the program (including the workspace form of the
    layout on other buffers) between replays; every replay against the
    oracle."""
    import combine_moe_layout_03_amd as M

    bs, h, k, e, r = 3000, 256, 8, 64, 8   # 24000 entries: 12 layout tiles
    epr = e // r
    w0 = W.random_case(620, bs, h, k, e, r, routing="dup", bad_frac=0.01)
    buf = M.EpBuffers(bs, h, k, epr, r, quant_int8=True)
    x = torch.from_numpy(w0.x.view(np.int16)).cuda().view(torch.bfloat16)
    idx = torch.from_numpy(w0.topk_idx).cuda()
    wts = torch.from_numpy(w0.topk_w).cuda()

    def step():
        M.moe_layout_no_alloc(idx, epr, r, buf.token_per_expert, buf.token_per_rank, buf.send_token_idx,
                              buf.bad_id_count)
        buf.notify()
        buf.dispatch(x, idx)
        buf.combine(idx, wts)

    def check(w, what):
        torch.cuda.synchronize()
        ref = oracle.pipeline(w.x, "bf16", w.topk_idx, w.topk_w, epr, r, True, "bf16")
        np.testing.assert_array_equal(buf.send_token_idx.cpu().numpy(), ref["layout"]["send_token_idx"], err_msg=what)
        np.testing.assert_array_equal(buf.token_per_expert.cpu().numpy(), ref["layout"]["token_per_expert"],
                                      err_msg=what)
        np.testing.assert_array_equal(buf.out.view(torch.int16).cpu().numpy().view(np.uint16), ref["out"],
                                      err_msg=what)

    log("no-alloc step eager (first call on the device looks up the scratch)")
    step()
    check(w0, "eager")
    graph = torch.cuda.CUDAGraph()
    log("no-alloc step: capture")
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    other = M.EpBuffers(500, h, k, epr, r)
    other_idx = torch.from_numpy(W.random_case(630, 500, h, k, e, r).topk_idx).cuda()
    for rep in range(3):
        w = W.random_case(621 + rep, bs, h, k, e, r, routing="uniform" if rep % 2 else "dup", bad_frac=0.02)
        x.copy_(torch.from_numpy(w.x.view(np.int16)).view(torch.bfloat16))
        idx.copy_(torch.from_numpy(w.topk_idx))
        wts.copy_(torch.from_numpy(w.topk_w))
        other.layout(other_idx)   # eager work between replays
        torch.cuda.synchronize()
        log(f"no-alloc step: replay {rep}")
        graph.replay()
        check(w, f"replay {rep}")
