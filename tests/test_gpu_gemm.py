"""First expert matmul (int8 receive rows x int8 expert weights -> int32) on
the GPU against the CPU oracle, through the C ABI.

Bar: bit-exact int32 outputs (integer sums, exact on both sides), rows owned
by no expert left as they were, on every row of the small cases; at the
shape the benchmark times and at the layer's second matmul, on every row of
each expert's first whole row tile and of its last (partial) tile -- so
every row on both sides of every expert boundary, and the output's last
rows -- plus rows drawn at random, all columns of each.  The cases cover
several row and column tiles with ragged ends; k a whole number of 128-byte
stages and k ending inside one, each with every remainder of the stage
count modulo 6 (the period of the kernel's LDS slot rotation); empty and
negative counts, counts past the row capacity, more experts than one wave
scans at once, and the int8 receive buffer used in place.
"""

import concurrent.futures

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import GpuRun, align32, dev_i32, int8_row_bytes, log

pytestmark = pytest.mark.gpu

SENTINEL = -0x5A5A5A5B


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible MI355X")


def M():
    import combine_moe_layout_03_amd as mod

    return mod


def run_gpu(case, rows=None):
    rows = case.rows if rows is None else rows
    a = torch.from_numpy(case.a.reshape(-1).view(np.uint8)).cuda()
    w = torch.from_numpy(case.w.view(np.uint8)).cuda()
    out = torch.full((rows, case.n), SENTINEL, dtype=torch.int32, device="cuda")
    M().moe_grouped_gemm_i8(a, case.stride, rows, case.k, dev_i32(case.group_count), w, out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def oracle_rows(case, rows):
    """The oracle on the listed rows, split over host threads (the oracle is
    plain C called through ctypes, which releases the interpreter lock, and
    keeps no state between calls)."""
    rows = np.asarray(rows, dtype=np.int64)
    parts = [p for p in np.array_split(rows, 16) if p.size]
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(parts)) as ex:
        res = list(ex.map(lambda p: oracle.grouped_gemm_i8(case.a, case.k, case.group_count, case.w, rows=p),
                          parts))
    return np.concatenate([r[0] for r in res]), np.concatenate([r[1] for r in res])


def assert_same(case, got, what, rows=None):
    if rows is None:
        exp, grp = oracle.grouped_gemm_i8(case.a, case.k, case.group_count, case.w)
    else:
        exp, grp = oracle_rows(case, rows)
    sel = np.arange(case.rows) if rows is None else np.asarray(rows)
    got = got[sel]
    owned = grp >= 0
    bad = np.nonzero(np.any(got[owned] != exp[owned], axis=1))[0]
    assert bad.size == 0, f"{what}: rows {sel[owned][bad[:10]].tolist()} differ"
    assert (got[~owned] == SENTINEL).all(), f"{what}: a row of no expert was written"


def _tile_m() -> int:
    """Rows of one output tile, as the library's header sets it."""
    import os
    import re

    hdr = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "combine_moe_layout_03_amd",
                       "csrc", "gemm.h")
    return int(re.search(r"kGemmTileM = (\d+)", open(hdr).read()).group(1))


TILE_M = _tile_m()


def boundary_tile_rows(case, seed, n_random=32):
    """Every row of each expert's first whole tile and of its last tile (the
    partial one when the count is not a multiple of the tile), the rows of
    the buffer's last tile, and `n_random` random rows."""
    counts = np.maximum(case.group_count.astype(np.int64), 0)
    starts = np.cumsum(counts) - counts
    sel = []
    for s0, c in zip(starts, counts):
        s0, c = int(min(s0, case.rows)), int(min(c, case.rows - min(s0, case.rows)))
        if c == 0:
            continue
        sel.append(np.arange(s0, s0 + min(c, TILE_M)))
        last = s0 + (c - 1) // TILE_M * TILE_M
        sel.append(np.arange(last, s0 + c))
    sel.append(np.arange(max(case.rows - TILE_M, 0), case.rows))
    sel.append((W.u64(seed, 0, n_random) % np.uint64(case.rows)).astype(np.int64))
    return np.unique(np.concatenate(sel))


@pytest.mark.parametrize("rows,k,n,groups,counts,seed", [
    # 4 row tiles and 2 column tiles, both ragged; k ends inside the 3rd stage
    (1000, 320, 300, 5, "owned:900", 501),
    # empty and negative counts; one expert spans three row tiles
    (830, 128, 128, 6, [0, 300, -5, 1, 0, 517], 502),
    # one 16-byte piece of k, one row
    (3, 16, 16, 3, [0, 1, 0], 503),
    # 130 experts (the slot search walks three chunks of 64)
    (2000, 64, 128, 130, "owned:2000", 504),
    # counts past the capacity: the last expert is cut at `rows`
    (1000, 96, 48, 3, [400, 400, 400], 505),
    # counts whose sum passes 2^31: the first expert owns every row
    (300, 128, 96, 3, [2 ** 31 - 1, 2 ** 31 - 1, 5], 515),
    # n = 1 and a single expert
    (257, 48, 1, 1, [257], 506),
    # 4 and 8 column tiles (the XCD-aware tile order), empty and negative counts,
    # k 5 whole stages
    (1000, 640, 1024, 6, [0, 300, -5, 1, 0, 517], 507),
    # k ending inside the 9th stage
    (1500, 1088, 2048, 9, "owned:1490", 508),
    # k ending inside the 8th stage; 3 ragged column tiles
    (900, 1008, 520, 4, "owned:880", 509),
    # k 3, 12 whole stages; k ending inside the 6th, 10th, 11th stage
    (700, 384, 600, 3, "owned:690", 510),
    (600, 1536, 260, 2, [300, 290], 511),
    (500, 656, 256, 3, "owned:500", 512),
    (400, 1264, 384, 2, [150, 250], 513),
    (300, 1392, 256, 1, [300], 514),
])
def test_gemm_matches_oracle(rows, k, n, groups, counts, seed):
    if isinstance(counts, str):
        case = W.gemm_case(seed, rows, k, n, groups, stride=align32(k) + 32,
                           owned=int(counts.split(":")[1]))
    else:
        case = W.gemm_case(seed, rows, k, n, groups, stride=align32(k) + 32, counts=counts)
    log(f"grouped gemm rows={rows} k={k} n={n} groups={groups} seed={seed}")
    got = run_gpu(case)
    assert_same(case, got, f"rows={rows} k={k} n={n}")


def test_gemm_full_size_tile_rows():
    """The benchmark's shape (32768 receive rows of 7296 bytes, k = 7168, n = 4096,
    16 experts) in the same launch: every row of each expert's first and last
    row tiles, the last rows of the buffer and 32 random rows, all 4096
    columns (every column tile) of each."""
    cfg = W.GEMM_CONFIG
    case = W.gemm_case(cfg["seed"], cfg["rows"], cfg["k"], cfg["n"], cfg["groups"],
                       stride=int8_row_bytes(cfg["k"]))
    log("grouped gemm full size")
    got = run_gpu(case)
    rows = boundary_tile_rows(case, 7)
    assert rows.size >= 16 * TILE_M
    log(f"grouped gemm full size: oracle on {rows.size} rows")
    assert_same(case, got, "full size", rows=rows)


def test_gemm_second_matmul_shape_tile_rows():
    """The shape of the layer's second expert matmul on the same share: the
    epilogue's int8 rows (k = 2048 codes in 2176-byte rows) times weights
    [16][7168][2048]; the same row tiles as above, all 7168 columns."""
    rows, k, n, groups = 32768, 2048, 7168, 16
    case = W.gemm_case(3002, rows, k, n, groups, stride=int8_row_bytes(k))
    log("grouped gemm second-matmul shape")
    got = run_gpu(case)
    sel = boundary_tile_rows(case, 8)
    log(f"grouped gemm second-matmul shape: oracle on {sel.size} rows")
    assert_same(case, got, "second-matmul shape", rows=sel)


def test_gemm_on_receive_buffer_then_epilogue():
    """Dispatch (int8) on the GPU, then the matmul reads the receive buffer
    in place (row stride of an int8 receive row) with the experts' received
    counts, then the epilogue takes its int32 output and the receive buffer's
    inverse scales; each stage against the oracle's own chain."""
    w = W.make_workload("small")
    run = GpuRun(w, quant=True).layout().notify().dispatch()
    torch.cuda.synchronize()
    mod = M()
    rows, h, e = w.bs * w.topk, w.hidden, w.expert_num_per_rank * w.rank_size
    n_out = 128
    wts = W.gemm_case(601, 1, h, 2 * n_out, e).w
    acc = torch.full((rows, 2 * n_out), SENTINEL, dtype=torch.int32, device="cuda")
    log("grouped gemm on the receive buffer")
    mod.moe_grouped_gemm_i8(run.buf.recv_x, run.buf.row_bytes, rows, h, run.buf.recv_token_per_expert,
                            torch.from_numpy(wts.view(np.uint8)).cuda(), acc)
    ws = (0.5 + W.uniform01(601, 5, 2 * n_out)).astype(np.float32) * np.float32(2.0 ** -12)
    base, stride = mod.token_scales_of(run.buf.recv_x, h)
    rb = mod.moe_recv_row_bytes(n_out, mod.MOE_INT8_ROWSCALE)
    out = torch.zeros(rows * rb, dtype=torch.uint8, device="cuda")
    log("epilogue after the grouped gemm")
    mod.moe_deq_swiglu_quant(acc, torch.from_numpy(ws).cuda(), base, out, token_scale_stride=stride)
    torch.cuda.synchronize()

    ref = oracle.pipeline(w.x, w.x_dtype, w.topk_idx, w.topk_w, w.expert_num_per_rank, w.rank_size,
                          True, w.x_dtype)
    codes, inv = ref["dispatch"]["codes"], ref["dispatch"]["inv"]
    counts = ref["notify"]["recv_token_per_expert"]
    exp_acc, grp = oracle.grouped_gemm_i8(codes, h, counts, wts)
    got_acc = acc.cpu().numpy()
    owned = grp >= 0
    assert np.array_equal(got_acc[owned], exp_acc[owned])
    assert (got_acc[~owned] == SENTINEL).all()
    # rows that no expert owns hold the sentinel on both sides of the epilogue
    exp_acc[~owned] = SENTINEL
    exp = oracle.swiglu_quant(exp_acc, ws, inv)
    raw = out.cpu().numpy().reshape(rows, rb)
    got_codes = np.ascontiguousarray(raw[:, :n_out]).view(np.int8)
    got_inv = np.ascontiguousarray(raw[:, align32(n_out):align32(n_out) + 4]).view(np.float32).reshape(-1)
    assert np.array_equal(got_codes, exp["codes"])
    assert np.array_equal(got_inv.view(np.uint32), exp["inv"].view(np.uint32))


def test_gemm_extremes_at_max_k():
    """k = MOE_GEMM_MAX_K with the int8 extremes: (-128)(-128) summed 65536
    times is 2^30 and 127(-128) summed is -1065353216, both exact in int32;
    the same values from the oracle and from the closed form."""
    mod = M()
    k, n, rows = mod.MOE_GEMM_MAX_K, 32, 6
    a = np.full((rows, k), -128, np.int8)
    a[1::2] = 127
    wts = np.full((2, n, k), -128, np.int8)
    wts[1, ::2] = 127
    counts = np.array([3, 3], np.int32)
    case = W.GemmCase(rows=rows, k=k, n=n, stride=k, a=a, group_count=counts, w=wts, seed=0)
    log("grouped gemm extremes at k = 65536")
    got = run_gpu(case)
    assert_same(case, got, "extremes")
    assert got[0, 0] == 2 ** 30 and got[1, 0] == -1065353216
    assert got[3, 0] == 127 * 127 * k and got[4, 1] == 2 ** 30 and got[4, 0] == -1065353216


def test_gemm_zero_rows_and_repeat():
    """rows = 0 enqueues nothing; two calls in a row give the same bits, the
    second on fewer rows with other counts."""
    case = W.gemm_case(701, 600, 256, 144, 4, stride=288, counts=[100, 250, 0, 250])
    mod = M()
    a = torch.from_numpy(case.a.reshape(-1).view(np.uint8)).cuda()
    wt = torch.from_numpy(case.w.view(np.uint8)).cuda()
    out = torch.full((600, 144), SENTINEL, dtype=torch.int32, device="cuda")
    log("grouped gemm rows=0")
    mod.moe_grouped_gemm_i8(a, 288, 0, 256, dev_i32(case.group_count), wt, out)
    torch.cuda.synchronize()
    assert (out == SENTINEL).all()
    log("grouped gemm twice")
    mod.moe_grouped_gemm_i8(a, 288, 600, 256, dev_i32(case.group_count), wt, out)
    first = out.cpu().numpy().copy()
    assert_same(case, first, "first call")
    small = W.GemmCase(rows=300, k=256, n=144, stride=288, a=case.a[:300], w=case.w,
                       group_count=np.array([50, 0, 200, 7], np.int32), seed=701)
    out2 = torch.full((300, 144), SENTINEL, dtype=torch.int32, device="cuda")
    mod.moe_grouped_gemm_i8(a, 288, 300, 256, dev_i32(small.group_count), wt, out2)
    torch.cuda.synchronize()
    assert_same(small, out2.cpu().numpy(), "second call")


def test_gemm_errors_raise():
    mod = M()
    a = torch.zeros(1024, dtype=torch.uint8, device="cuda")
    wt = torch.zeros((1, 16, 32), dtype=torch.int8, device="cuda")
    gc = torch.ones(1, dtype=torch.int32, device="cuda")
    out = torch.zeros((4, 16), dtype=torch.int32, device="cuda")
    with pytest.raises(mod.MoeEpError):
        mod.moe_grouped_gemm_i8(a, 40, 4, 32, gc, wt, out)      # row stride % 16
    with pytest.raises(mod.MoeEpError):
        mod.moe_grouped_gemm_i8(a, 48, 5, 32, gc, wt, out)      # out too small
    wt2 = torch.zeros((1, 16, 24), dtype=torch.int8, device="cuda")
    with pytest.raises(mod.MoeEpError):
        mod.moe_grouped_gemm_i8(a, 48, 4, 24, gc, wt2, out)     # k % 16
    assert (out == 0).all()
