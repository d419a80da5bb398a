"""The first expert matmul with its epilogue fused, on the GPU against the
CPU oracle, through the C ABI.

Bar: for every row an expert owns, int8 codes and inverse scale bit-exact
against the oracle's matmul followed by the oracle's epilogue with that
expert's column scales (integer sums exact on both sides, then the same
binary32 arithmetic); rows of no expert left as they were.  Small cases on
every row; the benchmarked shape on every row against the library's own two
calls (the matmul, then the epilogue expert by expert), and on the rows
around every expert boundary against the oracle.
"""

import concurrent.futures

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import align32, dev_f32, dev_i32, int8_row_bytes, log

pytestmark = pytest.mark.gpu

GUARD = 0xA5


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible MI355X")


def M():
    import combine_moe_layout_03_amd as mod

    return mod


def make_case(seed, rows, k, n, groups, counts):
    stride = align32(k) + 32
    if isinstance(counts, str):
        case = W.gemm_case(seed, rows, k, 2 * n, groups, stride=stride, owned=int(counts.split(":")[1]))
    else:
        case = W.gemm_case(seed, rows, k, 2 * n, groups, stride=stride, counts=counts)
    ws, ts = W.gemm_swiglu_scales(seed, rows, k, n, groups)
    return case, ws, ts


def run_fused(case, ws, ts):
    mod = M()
    n = case.n // 2
    rb = int8_row_bytes(n)
    a = torch.from_numpy(case.a.reshape(-1).view(np.uint8)).cuda()
    w = torch.from_numpy(case.w.view(np.uint8)).cuda()
    out = torch.full((case.rows * rb,), GUARD, dtype=torch.uint8, device="cuda")
    wsp = torch.empty(mod.moe_gemm_swiglu_quant_workspace_bytes(case.rows, n), dtype=torch.uint8, device="cuda")
    mod.moe_grouped_gemm_swiglu_quant_i8(a, case.stride, case.rows, case.k, dev_i32(case.group_count), w,
                                         dev_f32(ws), dev_f32(ts), out, wsp)
    torch.cuda.synchronize()
    return out.cpu().numpy().reshape(case.rows, rb)


def owner_of_rows(case):
    counts = np.maximum(case.group_count.astype(np.int64), 0)
    owner = np.full(case.rows, -1, np.int64)
    start = 0
    for g, c in enumerate(counts):
        owner[start:min(start + c, case.rows)] = g
        start += c
    return owner


def expected_rows(case, ws, ts, rows):
    """Codes and inverse scales of the listed rows: the oracle's matmul, then
    its epilogue row by row with the row's expert's scales."""
    rows = np.asarray(rows, dtype=np.int64)
    parts = [p for p in np.array_split(rows, 16) if p.size]
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(parts)) as ex:
        res = list(ex.map(lambda p: oracle.grouped_gemm_i8(case.a, case.k, case.group_count, case.w, rows=p),
                          parts))
    acc = np.concatenate([r[0] for r in res])
    grp = np.concatenate([r[1] for r in res])
    n = case.n // 2
    codes = np.zeros((rows.size, n), np.int8)
    inv = np.zeros(rows.size, np.float32)
    for i, (m, g) in enumerate(zip(rows, grp)):
        if g >= 0:
            codes[i], inv[i], _ = oracle.swiglu_quant_row(acc[i], ws[g], ts[m])
    return codes, inv, grp


def assert_rows(case, ws, ts, got, rows, what):
    n = case.n // 2
    codes, inv, grp = expected_rows(case, ws, ts, rows)
    raw = got[np.asarray(rows)]
    owned = grp >= 0
    gc = np.ascontiguousarray(raw[:, :n]).view(np.int8)
    gi = np.ascontiguousarray(raw[:, align32(n):align32(n) + 4]).view(np.float32).reshape(-1)
    bad = np.nonzero(np.any(gc[owned] != codes[owned], axis=1))[0]
    assert bad.size == 0, f"{what}: codes differ in rows {np.asarray(rows)[owned][bad[:10]].tolist()}"
    assert np.array_equal(gi[owned].view(np.uint32), inv[owned].view(np.uint32)), f"{what}: inverse scales differ"
    assert (raw[~owned] == GUARD).all(), f"{what}: a row of no expert was written"


@pytest.mark.parametrize("rows,k,n,groups,counts,seed", [
    # 2 column tiles, the second ragged; k ends inside the 3rd stage
    (1000, 320, 152, 5, "owned:900", 701),
    # one stage; empty and negative counts
    (830, 128, 64, 6, [0, 300, -5, 1, 0, 517], 702),
    # 4 column tiles (the XCD-aware order)
    (700, 1024, 512, 4, [100, 0, 350, 240], 703),
    # 3 column tiles, the last 4 columns wide; k ends inside a stage
    (650, 336, 260, 3, [300, -2, 340], 704),
    # 130 experts
    (2000, 64, 128, 130, "owned:2000", 705),
    # the narrowest rows; one expert
    (257, 48, 4, 1, [257], 706),
    # counts past the capacity
    (1000, 96, 48, 3, [400, 400, 400], 707),
    # 8 column tiles, 9 experts, k 8.5 stages
    (1500, 1088, 1024, 9, "owned:1490", 708),
    # counts whose sum passes 2^31 (the first expert owns every row)
    (300, 128, 64, 3, [2 ** 31 - 1, 2 ** 31 - 1, 5], 709),
])
def test_fused_matches_oracle(rows, k, n, groups, counts, seed):
    case, ws, ts = make_case(seed, rows, k, n, groups, counts)
    log(f"gemm+swiglu rows={rows} k={k} n={n} groups={groups} seed={seed}")
    got = run_fused(case, ws, ts)
    assert_rows(case, ws, ts, got, np.arange(rows), f"rows={rows} k={k} n={n}")


def test_fused_full_size_equals_the_two_calls_and_the_oracle_at_boundaries():
    """The benchmarked shape (32768 rows, k 7168, n 2048, 16 experts): every
    row against the library's matmul followed by its epilogue expert by
    expert, and the rows around each expert boundary against the oracle."""
    mod = M()
    cfg = W.GEMM_CONFIG
    n = cfg["n"] // 2
    case = W.gemm_case(cfg["seed"], cfg["rows"], cfg["k"], cfg["n"], cfg["groups"],
                       stride=int8_row_bytes(cfg["k"]))
    ws, ts = W.gemm_swiglu_scales(cfg["seed"], cfg["rows"], cfg["k"], n, cfg["groups"])
    log("gemm+swiglu full size: fused")
    got = run_fused(case, ws, ts)
    log("gemm+swiglu full size: matmul, then the epilogue per expert")
    a = torch.from_numpy(case.a.reshape(-1).view(np.uint8)).cuda()
    w = torch.from_numpy(case.w.view(np.uint8)).cuda()
    acc = torch.zeros((case.rows, cfg["n"]), dtype=torch.int32, device="cuda")
    mod.moe_grouped_gemm_i8(a, case.stride, case.rows, case.k, dev_i32(case.group_count), w, acc)
    rb = int8_row_bytes(n)
    ref = torch.full((case.rows * rb,), GUARD, dtype=torch.uint8, device="cuda")
    ts_d = dev_f32(ts)
    ws_d = dev_f32(ws)
    start = 0
    for g, c in enumerate(np.maximum(case.group_count.astype(np.int64), 0)):
        c = int(min(c, case.rows - start))
        if c > 0:
            mod.moe_deq_swiglu_quant(acc[start:start + c], ws_d[g], ts_d[start:start + c],
                                     ref[start * rb:(start + c) * rb])
        start += c
    torch.cuda.synchronize()
    ref = ref.cpu().numpy().reshape(case.rows, rb)
    bad = np.nonzero(np.any(got != ref, axis=1))[0]
    assert bad.size == 0, f"fused and two-call outputs differ in rows {bad[:10].tolist()}"
    codes = np.ascontiguousarray(got[:, :n]).view(np.int8)
    assert np.unique(codes).size > 200, "the activations should spread over the int8 codes"
    owner = owner_of_rows(case)
    starts = [int(np.argmax(owner == g)) for g in range(cfg["groups"]) if (owner == g).any()]
    sel = np.unique(np.concatenate([np.arange(max(s - 16, 0), min(s + 16, case.rows)) for s in starts]
                                   + [np.arange(case.rows - 16, case.rows)]))
    log(f"gemm+swiglu full size: oracle on {sel.size} rows")
    assert_rows(case, ws, ts, got, sel, "full size")


def test_fused_on_the_receive_buffer_with_its_scales_in_place():
    """Dispatch's int8 receive buffer as the matmul's rows and its inverse
    scales as the token scales, in place; against the two calls."""
    mod = M()
    w0 = W.random_case(711, 300, 256, 4, 16, 4, routing="uniform")
    buf = mod.EpBuffers(300, 256, 4, 4, 4, quant_int8=True)
    x = torch.from_numpy(w0.x.view(np.int16)).cuda().view(torch.bfloat16)
    idx = torch.from_numpy(w0.topk_idx).cuda()
    buf.layout(idx)
    buf.notify()
    buf.dispatch(x, idx)
    rows, k, n, groups = 1200, 256, 96, 16
    gcase = W.gemm_case(712, 1, k, 2 * n, groups)
    ws, _ = W.gemm_swiglu_scales(712, 1, k, n, groups)
    w = torch.from_numpy(gcase.w.view(np.uint8)).cuda()
    ts_base, ts_stride = mod.token_scales_of(buf.recv_x, 256)
    rb = int8_row_bytes(n)
    out = torch.full((rows * rb,), GUARD, dtype=torch.uint8, device="cuda")
    wsp = torch.empty(mod.moe_gemm_swiglu_quant_workspace_bytes(rows, n), dtype=torch.uint8, device="cuda")
    log("gemm+swiglu on the receive buffer")
    mod.moe_grouped_gemm_swiglu_quant_i8(buf.recv_x, buf.row_bytes, rows, k, buf.recv_token_per_expert, w,
                                         dev_f32(ws), ts_base, out, wsp, token_scale_stride=ts_stride)
    acc = torch.zeros((rows, 2 * n), dtype=torch.int32, device="cuda")
    mod.moe_grouped_gemm_i8(buf.recv_x, buf.row_bytes, rows, k, buf.recv_token_per_expert, w, acc)
    ref = torch.full((rows * rb,), GUARD, dtype=torch.uint8, device="cuda")
    counts = buf.recv_token_per_expert.cpu().numpy()
    ws_d = dev_f32(ws)
    start = 0
    for g, c in enumerate(counts):
        if c > 0:
            mod.moe_deq_swiglu_quant(acc[start:start + c], ws_d[g], ts_base[start * ts_stride:],
                                     ref[start * rb:(start + c) * rb], token_scale_stride=ts_stride, rows=int(c))
        start += int(c)
    torch.cuda.synchronize()
    assert start == rows
    assert torch.equal(out, ref)


def test_fused_errors_raise():
    mod = M()
    case, ws, ts = make_case(720, 64, 64, 8, 2, [30, 34])
    a = torch.from_numpy(case.a.reshape(-1).view(np.uint8)).cuda()
    w = torch.from_numpy(case.w.view(np.uint8)).cuda()
    out = torch.zeros(64 * int8_row_bytes(8), dtype=torch.uint8, device="cuda")
    small = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(mod.MoeEpError) as ei:
        mod.moe_grouped_gemm_swiglu_quant_i8(a, case.stride, 64, 64, dev_i32(case.group_count), w, dev_f32(ws),
                                             dev_f32(ts), out, small)
    assert ei.value.status == 5   # workspace too small
    assert mod.moe_gemm_swiglu_quant_workspace_bytes(0, 8) == 0
