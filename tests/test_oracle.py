"""The CPU oracle against its pins (no GPU).  See tests/pins.py."""

import numpy as np
import pytest

import pins
import workloads as W


def test_conversions(orc):
    pins.check_conversions(orc)


def test_layout_bruteforce_all_tiny_inputs(orc):
    pins.check_layout_bruteforce(orc)


@pytest.mark.parametrize("name", ["tiny", "small", "mid"])
def test_layout_stable_sort_configs(orc, name):
    w = W.make_workload(name)
    pins.check_layout_sort(orc, w.topk_idx, w.expert_num_per_rank, w.rank_size)
    pins.check_layout_invariants(orc, w.topk_idx, w.expert_num_per_rank, w.rank_size)


@pytest.mark.parametrize("seed,bs,k,e,r,routing,bad", [
    (11, 300, 6, 16, 4, "dup", 0.0),
    (12, 777, 8, 12, 3, "dup", 0.05),
    (13, 64, 3, 5, 5, "hot", 0.0),
    (14, 1000, 4, 64, 8, "zipf1.2", 0.02),
    (15, 1, 1, 1, 1, "uniform", 0.0),
])
def test_layout_stable_sort_random(orc, seed, bs, k, e, r, routing, bad):
    w = W.random_case(seed, bs, 8, k, e, r, routing=routing, bad_frac=bad)
    pins.check_layout_sort(orc, w.topk_idx, e // r, r)
    pins.check_layout_invariants(orc, w.topk_idx, e // r, r)


def test_layout_empty_batch(orc):
    got = orc.layout(np.zeros((0, 4), np.int32), 2, 3)
    assert got["token_per_expert"].tolist() == [0] * 6
    assert got["token_per_rank"].tolist() == [0] * 3 and got["bad"] == 0


@pytest.mark.parametrize("epr,ranks,seed", [(1, 1, 1), (4, 2, 2), (16, 16, 3), (4, 64, 4), (7, 3, 5)])
def test_notify_cumsum(orc, epr, ranks, seed):
    rng = np.random.default_rng(seed)
    tpe = rng.integers(0, 50, size=epr * ranks)
    tpe[rng.random(tpe.size) < 0.3] = 0
    pins.check_notify(orc, tpe, epr, ranks)


def test_notify_from_layout(orc):
    w = W.make_workload("mid")
    lay = orc.layout(w.topk_idx, w.expert_num_per_rank, w.rank_size)
    pins.check_notify(orc, lay["token_per_expert"], w.expert_num_per_rank, w.rank_size)


@pytest.mark.parametrize("name,kind", [("tiny", "bf16"), ("small", "bf16"), ("mid", "fp16")])
def test_dispatch_passthrough_closed_form(orc, name, kind):
    w = W.make_workload(name, x_dtype=kind)
    pins.check_dispatch_passthrough(orc, w.x, kind, w.topk_idx, w.expert_num_per_rank, w.rank_size)


def test_dispatch_passthrough_with_bad_ids_and_duplicates(orc):
    w = W.random_case(21, 200, 16, 6, 8, 2, routing="dup", bad_frac=0.1)
    pins.check_dispatch_passthrough(orc, w.x, "bf16", w.topk_idx, 4, 2)


def test_dispatch_int8_rows(orc):
    w = W.random_case(22, 40, 64, 4, 8, 4, routing="dup", bad_frac=0.05, zero_rows=2)
    pins.check_dispatch_int8_rows(orc, w.x, "bf16", w.topk_idx, 2, 4)
    w = W.random_case(23, 24, 32, 3, 6, 3, x_dtype="fp16", routing="uniform")
    pins.check_dispatch_int8_rows(orc, w.x, "fp16", w.topk_idx, 2, 3)


def test_quant_golden_rows(orc):
    pins.check_quant_golden(orc)


def test_quant_power_of_two_scales(orc):
    pins.check_quant_power_of_two(orc)


@pytest.mark.parametrize("kind,std", [("bf16", 1.0), ("bf16", 100.0), ("fp16", 2.0), ("bf16", 1e-20),
                                      ("fp16", 1e-5)])
def test_quant_exact_rational(orc, kind, std):
    w = W.random_case(31, 12, 96, 1, 1, 1, x_dtype=kind, x_std=std, zero_rows=1)
    pins.check_quant_exact(orc, w.x, kind)


def test_quant_large_outlier_rows(orc):
    w = W.make_workload("large")
    big = np.flatnonzero(np.abs(pins.widen16(w.x[:, :64], "bf16")).max(axis=1) > 20)[:3]
    rows = np.concatenate([w.x[big][:, :512], w.x[:3, :512]])
    pins.check_quant_exact(orc, np.ascontiguousarray(rows), "bf16")


def test_combine_golden_order(orc):
    pins.check_combine_golden(orc)


@pytest.mark.parametrize("quant", [False, True])
@pytest.mark.parametrize("seed,bs,h,k,e,r,routing,bad", [
    (41, 16, 32, 4, 8, 2, "uniform", 0.0),
    (42, 33, 40, 8, 16, 4, "dup", 0.1),
    (43, 9, 24, 2, 2, 1, "hot", 0.0),
])
def test_combine_float64_bound(orc, quant, seed, bs, h, k, e, r, routing, bad):
    w = W.random_case(seed, bs, h, k, e, r, routing=routing, bad_frac=bad)
    epr = e // r
    lay = orc.layout(w.topk_idx, epr, r)
    no = orc.notify(lay["token_per_expert"], epr, r)
    d = orc.dispatch(w.x, "bf16", w.topk_idx, lay["send_token_idx"], no["put_offset"],
                     no["recv_base"], epr, r, quant)
    pins.check_combine_bound(orc, d, "int8" if quant else "bf16", w.topk_idx, w.topk_w,
                             lay["send_token_idx"], no["put_offset"], no["recv_base"], epr, r)


def test_combine_random_receive_rows(orc):
    pins.check_combine_random_rows(orc)


def test_combine_identity_k1(orc):
    w = W.random_case(51, 20, 48, 1, 4, 2, zero_rows=1)
    pins.check_combine_identity(orc, w.x, "bf16", 2, 2)
    w = W.random_case(52, 10, 16, 1, 3, 1, x_dtype="fp16")
    pins.check_combine_identity(orc, w.x, "fp16", 3, 1)


def test_combine_bad_ids_add_nothing(orc):
    """An entry with a bad id contributes exactly nothing: the output equals
    that of the same routing with the entry's weight set to zero."""
    w = W.random_case(61, 30, 16, 4, 8, 2, routing="uniform")
    idx_bad = w.topk_idx.copy()
    idx_bad[::3, 1] = -1
    idx_bad[1::5, 3] = 99
    w0 = w.topk_w.copy()
    w0[idx_bad != w.topk_idx] = 0.0
    for quant in (False, True):
        a = orc.pipeline(w.x, "bf16", idx_bad, w.topk_w, 4, 2, quant, "fp32")["out"]
        b = orc.pipeline(w.x, "bf16", w.topk_idx, w0, 4, 2, quant, "fp32")["out"]
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_passthrough_round_trip_unit_weights(orc):
    """dispatch then combine with weights summing to 1 returns x within the
    combine bound (k roundings)."""
    w = W.make_workload("small")
    res = orc.pipeline(w.x, "bf16", w.topk_idx, w.topk_w, w.expert_num_per_rank, w.rank_size,
                       False, "fp32")
    x = pins.widen16(w.x, "bf16").astype(np.float64)
    wsum = w.topk_w.astype(np.float64).sum(axis=1, keepdims=True)
    err = np.abs(res["out"] - x * wsum)
    assert np.all(err <= 2 * w.topk * 2.0 ** -24 * np.abs(x) * wsum + 1e-38)


# --------------------------------------------------------------------------
# several source ranks sharing one receive buffer
# --------------------------------------------------------------------------

def _sources(seed, sizes, h, k, e, r, routing="dup", bad=0.0, kind="bf16"):
    cases = [W.random_case(seed + i, bs, h, k, e, r, x_dtype=kind, routing=routing, bad_frac=bad)
             for i, bs in enumerate(sizes)]
    return ([c.x for c in cases], [c.topk_idx for c in cases], [c.topk_w for c in cases])


def test_notify_multi_golden(orc):
    pins.check_notify_multi_golden(orc)


@pytest.mark.parametrize("epr,ranks,seed", [(1, 1, 11), (4, 2, 12), (16, 16, 13), (7, 3, 14)])
def test_notify_multi_single_source(orc, epr, ranks, seed):
    tpe = (W.u64(seed, 0, epr * ranks) % np.uint64(50)).astype(np.int32)
    pins.check_notify_multi_single_source(orc, tpe, epr, ranks)


@pytest.mark.parametrize("seed,sizes,k,e,r,routing,bad", [
    (401, (5, 3), 2, 4, 2, "dup", 0.0),
    (402, (40, 0, 17, 33), 4, 12, 3, "dup", 0.1),
    (403, (64,) * 8, 8, 64, 8, "uniform", 0.0),
    (404, (100, 1, 250), 8, 256, 16, "zipf1.2", 0.02),
    (405, (30, 30), 3, 2, 1, "hot", 0.0),
])
def test_multi_receive_order_lexsort(orc, seed, sizes, k, e, r, routing, bad):
    _, idxs, _ = _sources(seed, sizes, 8, k, e, r, routing, bad)
    pins.check_multi_receive_order(orc, idxs, e // r, r)


@pytest.mark.parametrize("quant,kind", [(False, "bf16"), (True, "bf16"), (True, "fp16")])
def test_pipeline_multi_equals_each_single_source(orc, quant, kind):
    xs, idxs, ws = _sources(410, (24, 0, 9, 31), 40, 4, 16, 4, "dup", 0.05, kind)
    pins.check_pipeline_multi_vs_single(orc, xs, kind, idxs, ws, 4, 4, quant)


# ---- expert-side epilogue (dequantise, SwiGLU, requantise) ----------------

def test_exp_against_float64(orc):
    pins.check_exp(orc)


def test_swiglu_golden_rows(orc):
    pins.check_swiglu_golden(orc)


def test_swiglu_bound_and_exact_quantiser(orc):
    pins.check_swiglu_bound(orc, seeds=(1, 2, 3, 4, 5), n=300)


def test_swiglu_dequant_rounding_exact(orc):
    pins.check_swiglu_dequant_exact(orc)


def test_swiglu_rows_equal_row_by_row(orc):
    rng = np.random.default_rng(77)
    rows, n = 9, 40
    acc = rng.integers(-(2 ** 31), 2 ** 31 - 1, (rows, 2 * n)).astype(np.int32)
    ws = rng.uniform(0.5, 2, 2 * n).astype(np.float32) * np.float32(2 ** -26)
    ts = rng.uniform(0.01, 0.1, rows).astype(np.float32)
    got = orc.swiglu_quant(acc, ws, ts)
    for m in range(rows):
        codes, inv, _ = orc.swiglu_quant_row(acc[m], ws, ts[m])
        assert np.array_equal(got["codes"][m], codes)
        assert pins.f32_bits(got["inv"][m]) == pins.f32_bits(inv)
    empty = orc.swiglu_quant(np.zeros((0, 2 * n), np.int32), ws, np.zeros(0, np.float32))
    assert empty["codes"].shape == (0, n)


def test_gemm_per_expert_matmul(orc):
    pins.check_gemm_per_expert_matmul(orc)


def test_gemm_closed_forms(orc):
    pins.check_gemm_closed_forms(orc)


def test_gemm_column_picking_weights(orc):
    pins.check_gemm_permutation(orc)


def test_gemm_row_ownership(orc):
    pins.check_gemm_ownership(orc)
