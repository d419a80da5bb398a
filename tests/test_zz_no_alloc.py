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
