"""The C ABI without a GPU: the library loads, exports every function that
include/moe_ep.h declares, and rejects bad arguments on the host (these
paths return before any HIP call, so they run anywhere)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_ep.h")


@pytest.fixture(scope="module")
def M():
    import combine_moe_layout_03_amd as mod

    return mod


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def test_header_symbols_exported(M):
    names = declared_functions()
    assert {"moe_layout", "moe_notify", "moe_dispatch", "moe_combine"} <= set(names)
    lib = ctypes.CDLL(M.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in moe_ep.h but not exported"


def declarations():
    """{name: (preceding comment, parameter count)} for every function the
    header declares."""
    text = open(HEADER).read()
    out = {}
    for m in re.finditer(r"(/\*(?:(?!\*/).)*\*/)\s*(?:const char\*|int)\s+(moe_[a-z0-9_]+)\s*\(([^)]*)\)\s*;",
                         text, flags=re.S):
        params = [p for p in m.group(3).split(",") if p.strip() and p.strip() != "void"]
        out[m.group(2)] = (m.group(1), len(params))
    return out


def test_every_declaration_cites_its_passage_or_says_it_has_none():
    """Each entry point's comment cites the passage that defines it, says it
    has none on the pages, or (the no-allocation variant) names the callers
    it exists for."""
    decls = declarations()
    assert set(decls) == set(declared_functions()), "a declaration without its own comment block"
    for name, (comment, _) in decls.items():
        assert re.search(r"section \d|page \d|\bpage's\b|[Nn]o counterpart on the pages|callers that cannot allocate",
                         comment), f"{name}: its comment cites no passage of the pages"


def test_binding_signatures_match_header(M):
    for name, (_, nparams) in declarations().items():
        assert name in M._SIGS, f"{name} has no binding"
        assert len(M._SIGS[name][0]) == nparams, f"{name}: binding takes {len(M._SIGS[name][0])} arguments"


def test_design_boundary_table_lists_every_entry_point():
    text = open(os.path.join(ROOT, "DESIGN.md")).read()
    section = text[text.index("## 2. The boundary"):text.index("## 3. ")]
    for name in declared_functions():
        assert f"`{name}`" in section, f"{name} missing from the boundary table"


def test_header_constants_match_binding(M):
    text = open(HEADER).read()
    for name in ("MOE_MAX_EXPERTS", "MOE_MAX_HIDDEN", "MOE_MAX_TOPK", "MOE_MAX_SOURCES",
                 "MOE_EPILOGUE_MAX_N", "MOE_GEMM_MAX_K", "MOE_GEMM_MAX_N", "MOE_GEMM_MAX_GROUPS"):
        val = int(re.search(rf"#define {name} (\d+)", text).group(1))
        assert getattr(M, name) == val


@pytest.mark.parametrize("hidden,dtype,expect", [(7168, 3, 7296), (1000, 3, 1152), (8, 3, 128),
                                                 (2048, 3, 2176), (4064, 3, 4096),
                                                 (8, 0, 16), (7168, 1, 14336)])
def test_recv_row_bytes(M, hidden, dtype, expect):
    assert M.moe_recv_row_bytes(hidden, dtype) == expect


def test_recv_row_bytes_errors(M):
    out = ctypes.c_size_t(0)
    assert M._lib.moe_recv_row_bytes(0, 0, ctypes.byref(out)) == 2
    assert M._lib.moe_recv_row_bytes(8, 2, ctypes.byref(out)) == 4   # fp32 is not a receive type
    assert M._lib.moe_recv_row_bytes(8, 0, None) == 1


# Tiles hold 2048 entries; the workspace holds (tiles - 1) rows of E + 1
# counts.
@pytest.mark.parametrize("bs,k,e,expect", [(4096, 8, 256, 15 * 257 * 4), (0, 1, 1, 0), (256, 8, 16, 0),
                                           (257, 8, 16, 1 * 17 * 4), (16384, 8, 256, 63 * 257 * 4),
                                           (5000, 8, 1024, 19 * 1025 * 4)])
def test_layout_workspace_bytes(M, bs, k, e, expect):
    assert M.moe_layout_workspace_bytes(bs, k, e) == expect


def test_status_strings(M):
    for s in range(9):
        assert M.moe_status_str(s) and M.moe_status_str(s) != "unknown status"
    assert M.moe_status_str(99) == "unknown status"


P = 0x100000  # a non-NULL, 256-byte aligned stand-in pointer (never dereferenced: every call below fails validation)


def test_layout_rejects_on_host(M):
    # every call below has an invalid argument, so it returns before any HIP call
    L = M._lib
    assert L.moe_layout(P, -1, 8, 16, 16, P, P, P, None, None, 0, None) == 2
    assert L.moe_layout(P, 16, 0, 16, 16, P, P, P, None, None, 0, None) == 2
    assert L.moe_layout(P, 16, 33, 16, 16, P, P, P, None, None, 0, None) == 7
    assert L.moe_layout(P, 16, 8, 0, 16, P, P, P, None, None, 0, None) == 2
    assert L.moe_layout(P, 16, 8, 2049, 1, P, P, P, None, None, 0, None) == 7
    assert L.moe_layout(P, 16, 8, 16, 16, None, P, P, None, None, 0, None) == 1
    assert L.moe_layout(P, 16, 8, 16, 16, P, None, P, None, None, 0, None) == 1
    assert L.moe_layout(None, 16, 8, 16, 16, P, P, P, None, None, 0, None) == 1
    assert L.moe_layout(P, 16, 8, 16, 16, P, P, None, None, None, 0, None) == 1
    assert L.moe_layout(P + 2, 16, 8, 16, 16, P, P, P, None, None, 0, None) == 3
    assert L.moe_layout(P, 16, 8, 16, 16, P, P, P, P + 1, None, 0, None) == 3


def test_layout_no_alloc_rejects_on_host(M):
    # the same argument errors as moe_layout, and shapes beyond the static
    # scratch, all before any HIP call
    L = M._lib
    assert L.moe_layout_no_alloc(P, -1, 8, 16, 16, P, P, P, None, None) == 2
    assert L.moe_layout_no_alloc(P, 16, 33, 16, 16, P, P, P, None, None) == 7
    assert L.moe_layout_no_alloc(P, 16, 8, 2049, 1, P, P, P, None, None) == 7
    assert L.moe_layout_no_alloc(P, 16, 8, 16, 16, None, P, P, None, None) == 1
    assert L.moe_layout_no_alloc(None, 16, 8, 16, 16, P, P, P, None, None) == 1
    assert L.moe_layout_no_alloc(P + 2, 16, 8, 16, 16, P, P, P, None, None) == 3
    assert L.moe_layout_no_alloc(P, 16, 8, 16, 16, P, P, P, P + 1, None) == 3
    # the per-tile count table of 300000 x 8 entries at 256 experts exceeds the 1 MiB scratch
    assert M.moe_layout_workspace_bytes(300000, 8, 256) > M.MOE_NO_ALLOC_SCRATCH_BYTES
    assert L.moe_layout_no_alloc(P, 300000, 8, 16, 16, P, P, P, None, None) == 9


def test_notify_rejects_on_host(M):
    L = M._lib
    assert L.moe_notify(P, 0, 4, P, P, P, P, None) == 2
    assert L.moe_notify(P, 4, 1024, P, P, P, P, None) == 7
    assert L.moe_notify(None, 4, 4, P, P, P, P, None) == 1
    assert L.moe_notify(P, 4, 4, P, P, None, P, None) == 1
    assert L.moe_notify(P, 4, 4, P + 2, P, P, P, None) == 3


def test_dispatch_rejects_on_host(M):
    L = M._lib
    rb = M.moe_recv_row_bytes(7168, 3)
    cap = 4096 * 8 * rb
    args = lambda **kw: [kw.get("x", P), kw.get("xt", 0), kw.get("bs", 4096), kw.get("h", 7168),
                         kw.get("k", 8), kw.get("idx", P), P, P, P, 16, 16, kw.get("q", 1),
                         kw.get("recv", P), kw.get("cap", cap), None]
    assert L.moe_dispatch(*args(xt=2)) == 4        # fp32 input
    assert L.moe_dispatch(*args(q=2)) == 4         # quant flag not 0/1
    assert L.moe_dispatch(*args(h=7164)) == 7      # hidden % 8
    assert L.moe_dispatch(*args(h=16392)) == 7     # hidden > max
    assert L.moe_dispatch(*args(h=0)) == 2
    assert L.moe_dispatch(*args(k=0)) == 2
    assert L.moe_dispatch(*args(cap=cap - 1)) == 6
    assert L.moe_dispatch(*args(x=None)) == 1
    assert L.moe_dispatch(*args(idx=None)) == 1
    assert L.moe_dispatch(*args(x=P + 8)) == 3
    assert L.moe_dispatch(*args(recv=P + 4)) == 3
    # passthrough needs 2*h bytes per row
    assert L.moe_dispatch(*args(q=0, cap=cap)) == 6
    # an empty batch is accepted with NULL pointers and enqueues nothing
    assert L.moe_dispatch(*args(bs=0, x=None, idx=None, recv=None, cap=0)) == 0


def test_combine_rejects_on_host(M):
    L = M._lib
    rb = M.moe_recv_row_bytes(7168, 3)
    cap = 4096 * 8 * rb
    args = lambda **kw: [kw.get("recv", P), kw.get("rt", 3), kw.get("cap", cap), kw.get("bs", 4096),
                         kw.get("h", 7168), 8, P, kw.get("w", P), P, P, P, 16, 16, kw.get("out", P),
                         kw.get("ot", 0), None]
    assert L.moe_combine(*args(rt=2)) == 4
    assert L.moe_combine(*args(ot=3)) == 4
    assert L.moe_combine(*args(cap=cap - 32)) == 6
    assert L.moe_combine(*args(w=None)) == 1
    assert L.moe_combine(*args(out=P + 2)) == 3
    assert L.moe_combine(*args(h=12)) == 7
    assert L.moe_combine(*args(bs=0, recv=None, out=None, w=None, cap=0)) == 0


def test_multi_source_rejects_on_host(M):
    # every call below has an invalid argument, so it returns before any HIP call
    L = M._lib
    assert L.moe_notify_multi(P, 0, 4, 4, P, P, P, P, None) == 2          # no source
    assert L.moe_notify_multi(P, 385, 4, 4, P, P, P, P, None) == 7        # above MOE_MAX_SOURCES
    assert L.moe_notify_multi(P, 4, 0, 4, P, P, P, P, None) == 2
    assert L.moe_notify_multi(P, 4, 4, 1024, P, P, P, P, None) == 7       # E above the maximum
    assert L.moe_notify_multi(None, 4, 4, 4, P, P, P, P, None) == 1
    assert L.moe_notify_multi(P, 4, 4, 4, P, P, P, None, None) == 1
    assert L.moe_notify_multi(P, 4, 4, 4, P + 2, P, P, P, None) == 3
    rb = M.moe_recv_row_bytes(7168, 3)
    cap = 4096 * 8 * rb

    def dis(**kw):
        return L.moe_dispatch_src(kw.get("x", P), 0, kw.get("bs", 4096), 7168, 8, P, P, P, P, 16, 16,
                                  kw.get("ns", 4), kw.get("src", 0), 1, P, kw.get("cap", cap), None)

    def com(**kw):
        return L.moe_combine_src(P, 3, kw.get("cap", cap), kw.get("bs", 4096), 7168, 8, P,
                                 kw.get("w", P), P, P, P, 16, 16, kw.get("ns", 4), kw.get("src", 0),
                                 kw.get("out", P), 0, None)
    for f in (dis, com):
        assert f(src=-1) == 2
        assert f(src=4) == 2
        assert f(ns=0) == 2
        assert f(ns=385, src=1) == 7
        assert f(src=3, cap=cap - 1) == 6
    assert dis(src=2, x=None) == 1
    assert com(src=2, w=None) == 1
    assert com(src=1, out=P + 2) == 3


def test_fused_supported_is_host_logic(M):
    # one kernel unless bs == 0, hidden > 8192 or bs * topk > 2^16; any expert count up to the maximum
    import torch

    bf16 = torch.bfloat16
    assert M.moe_fused_supported(4096, 7168, 8, 16, 16, bf16, True)
    assert not M.moe_fused_supported(16384, 7168, 8, 4, 64, bf16, True)
    assert M.moe_fused_supported(64, 128, 4, 1024, 2, bf16, True)
    assert M.moe_fused_supported(1, 8192, 1, 1, 1, torch.float16, False)
    assert not M.moe_fused_supported(0, 128, 4, 8, 2, bf16, True)
    assert not M.moe_fused_supported(16, 8200, 4, 8, 2, bf16, True)
    assert M.moe_fused_supported(8192, 16, 8, 8, 2, bf16, True)         # 2^16 entries
    assert not M.moe_fused_supported(8193, 16, 8, 8, 2, bf16, True)


def test_fused_rejects_on_host(M):
    # every call below has an invalid argument, so it returns before any HIP call
    L = M._lib
    rb = M.moe_recv_row_bytes(7168, 3)
    cap = 4096 * 8 * rb
    big = 70000  # bs * 8 above 2^16: the three-stage form, which needs moe_layout's workspace
    ws_big = M.moe_layout_workspace_bytes(big, 8, 256)
    cap_big = big * 8 * rb

    def call(**kw):
        a = dict(x=P, xt=0, bs=4096, h=7168, k=8, idx=P, epr=16, r=16, q=1, tpe=P, tpr=P, slot=P, bad=None,
                 put=P, cnt=P, base=P, rtpe=P, recv=P, cap=cap, ws=P, wsb=0)
        a.update(kw)
        return L.moe_layout_notify_dispatch(a["x"], a["xt"], a["bs"], a["h"], a["k"], a["idx"], a["epr"], a["r"],
                                            a["q"], a["tpe"], a["tpr"], a["slot"], a["bad"], a["put"], a["cnt"],
                                            a["base"], a["rtpe"], a["recv"], a["cap"], a["ws"], a["wsb"], None)
    assert ws_big > 0
    assert call(xt=2) == 4
    assert call(q=3) == 4
    assert call(h=7160 + 4) == 7
    assert call(k=0) == 2
    assert call(epr=4096, r=1) == 7
    assert call(bs=big, cap=cap_big, ws=None, wsb=ws_big) == 1
    assert call(bs=big, cap=cap_big, wsb=ws_big - 4) == 5
    assert call(cap=cap - 1) == 6
    assert call(x=None) == 1
    assert call(tpe=None) == 1
    assert call(recv=P + 8) == 3
    assert call(ws=P + 2) == 3
    assert call(put=P + 2) == 3
    out = ctypes.c_int(5)
    assert L.moe_fused_supported(16, 8, 2, 4, 2, 2, 1, ctypes.byref(out)) == 4   # fp32 input
    assert L.moe_fused_supported(16, 12, 2, 4, 2, 0, 1, ctypes.byref(out)) == 7  # hidden % 8
    assert L.moe_fused_supported(16, 8, 2, 4, 2, 0, 2, ctypes.byref(out)) == 4   # quant flag


def test_grouped_gemm_swiglu_rejects_on_host(M):
    """The fused matmul + epilogue call: every shape, limit, alignment, NULL,
    buffer and workspace error returns before anything is enqueued."""
    L = M._lib
    rb = M.moe_recv_row_bytes(2048, M.MOE_INT8_ROWSCALE)
    ws_need = M.moe_gemm_swiglu_quant_workspace_bytes(64, 2048)
    assert ws_need == 64 * 2048 * 4 + 256
    ok = dict(a_row_bytes=7296, rows=64, k=7168, groups=16, n=2048, ts_stride=7296, out_bytes=64 * rb,
              ws_bytes=ws_need)

    def call(a=P, a_row_bytes=ok["a_row_bytes"], rows=ok["rows"], k=ok["k"], gc=P, groups=ok["groups"], w=P,
             n=ok["n"], wsc=P, ts=P, ts_stride=ok["ts_stride"], out=P, out_bytes=ok["out_bytes"], wsp=P,
             ws_bytes=ok["ws_bytes"]):
        return L.moe_grouped_gemm_swiglu_quant_i8(a, a_row_bytes, rows, k, gc, groups, w, n, wsc, ts, ts_stride,
                                                  out, out_bytes, wsp, ws_bytes, None)

    assert call(rows=-1) == 2 and call(k=0) == 2 and call(n=0) == 2 and call(groups=0) == 2
    assert call(a_row_bytes=7152) == 2                       # shorter than k
    assert call(ts_stride=2) == 2 and call(ts_stride=6) == 2  # token-scale stride below 4 or not a multiple
    assert call(k=7160, a_row_bytes=7168) == 7               # k % 16
    assert call(n=2046) == 7 and call(n=32772) == 7          # n % 4; 2n above MOE_GEMM_MAX_N
    assert call(k=65552, a_row_bytes=65552) == 7 and call(groups=65537) == 7
    assert call(a_row_bytes=7304) == 3                       # row stride not a multiple of 16
    assert call(rows=0, a=None, gc=None, w=None, wsc=None, ts=None, out=None, wsp=None) == 0
    for name in ("a", "gc", "w", "wsc", "ts", "out", "wsp"):
        assert call(**{name: None}) == 1, name
    assert call(a=P + 8) == 3 and call(w=P + 8) == 3 and call(out=P + 8) == 3 and call(wsp=P + 8) == 3
    assert call(gc=P + 2) == 3 and call(wsc=P + 2) == 3 and call(ts=P + 2) == 3
    assert call(out_bytes=64 * rb - 1) == 6
    assert call(ws_bytes=ws_need - 1) == 5
    # more workgroups than one launch takes: (rows / 256 + groups) row slots x n / 128 column tiles
    big_rows, big_n = 2 ** 31 - 1, 32768
    big_rb = M.moe_recv_row_bytes(big_n, M.MOE_INT8_ROWSCALE)
    assert call(rows=big_rows, a_row_bytes=16, k=16, n=big_n, out_bytes=big_rows * big_rb,
                ws_bytes=M.moe_gemm_swiglu_quant_workspace_bytes(big_rows, big_n)) == 7
    # the size query
    out = ctypes.c_size_t(0)
    assert L.moe_gemm_swiglu_quant_workspace_bytes(64, 2048, None) == 1
    assert L.moe_gemm_swiglu_quant_workspace_bytes(-1, 2048, ctypes.byref(out)) == 2
    assert L.moe_gemm_swiglu_quant_workspace_bytes(64, 0, ctypes.byref(out)) == 2
    assert L.moe_gemm_swiglu_quant_workspace_bytes(0, 8, ctypes.byref(out)) == 0 and out.value == 0


def test_binding_rejects_host_tensors(M):
    import torch

    idx = torch.zeros((4, 2), dtype=torch.int32)
    with pytest.raises(ValueError):
        M.moe_layout(idx, 2, 2, torch.zeros(4, dtype=torch.int32), torch.zeros(2, dtype=torch.int32),
                     torch.zeros((4, 2), dtype=torch.int32))


def test_binding_rejects_undersized_arrays(M):
    """The C calls take bare pointers, so the binding checks each array's
    length against the shape arguments before anything reaches the library
    (host tensors suffice: the length check comes first)."""
    import torch

    i32 = dict(dtype=torch.int32)
    bs, k, epr, r = 4, 2, 2, 2
    idx = torch.zeros((bs, k), **i32)

    def raises(name, fn, *args, **kw):
        with pytest.raises(ValueError, match=name):
            fn(*args, **kw)

    raises("token_per_expert", M.moe_layout, idx, epr, r, torch.zeros(3, **i32), torch.zeros(2, **i32),
           torch.zeros((bs, k), **i32))
    raises("token_per_rank", M.moe_layout, idx, epr, r, torch.zeros(4, **i32), torch.zeros(1, **i32),
           torch.zeros((bs, k), **i32))
    raises("send_token_idx", M.moe_layout_no_alloc, idx, epr, r, torch.zeros(4, **i32), torch.zeros(2, **i32),
           torch.zeros(7, **i32))
    raises("recv_base", M.moe_notify, torch.zeros(4, **i32), epr, r, torch.zeros(4, **i32),
           torch.zeros(2, **i32), torch.zeros(1, **i32), torch.zeros(4, **i32))
    raises("put_offset", M.moe_dispatch, torch.zeros((bs, 64), dtype=torch.bfloat16), idx,
           torch.zeros((bs, k), **i32), torch.zeros(3, **i32), torch.zeros(2, **i32), epr, r, True,
           torch.zeros(1 << 12, dtype=torch.uint8))
    raises("topk_weights", M.moe_combine, torch.zeros(1 << 12, dtype=torch.uint8), M.MOE_INT8_ROWSCALE, 64,
           idx, torch.zeros(bs * k - 1), torch.zeros((bs, k), **i32), torch.zeros(4, **i32),
           torch.zeros(2, **i32), epr, r, torch.zeros((bs, 64), dtype=torch.bfloat16))
    raises("put_offset", M.moe_dispatch_src, torch.zeros((bs, 64), dtype=torch.bfloat16), idx,
           torch.zeros((bs, k), **i32), torch.zeros((3, 2), **i32), torch.zeros(2, **i32), epr, r, 1, True,
           torch.zeros(1 << 12, dtype=torch.uint8))
    raises("token_scale", M.moe_deq_swiglu_quant, torch.zeros((3, 16), **i32), torch.zeros(16),
           torch.zeros(2), torch.zeros(1 << 10, dtype=torch.uint8))
    # a pair the library rejects (E above MOE_MAX_EXPERTS) is left to its status code: no length check
    with pytest.raises(ValueError, match="device tensor"):
        M.moe_layout(idx, 4096, 1, torch.zeros(4, **i32), torch.zeros(1, **i32), torch.zeros((bs, k), **i32))


def test_product_path_never_touches_the_oracle():
    """Nothing in the package or the header refers to the CPU oracle."""
    pkg = os.path.join(ROOT, "combine_moe_layout_03_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in text.lower(), f"{f} mentions the oracle"
    assert "oracle" not in open(HEADER).read().lower()


def test_rank_division_by_multiply_high_is_exact():
    """The kernels find an expert's rank as (e * ceil(2^32 / EPR)) >> 32; this
    equals e // EPR for every expert id and every EPR the library accepts."""
    import numpy as np

    e = np.arange(2048, dtype=np.uint64)
    for d in range(1, 2049):
        m = np.uint64(((1 << 32) + d - 1) // d)
        assert np.array_equal((e * m) >> np.uint64(32), e // np.uint64(d)), d


def test_epilogue_rejects_on_host(M):
    L = M._lib
    rb = 2176  # moe_recv_row_bytes(2048, int8)
    ok = dict(rows=16, n=2048, stride=4, out_bytes=16 * rb)

    def call(acc=P, rows=ok["rows"], n=ok["n"], ws=P, ts=P, stride=ok["stride"], out=P,
             out_bytes=ok["out_bytes"]):
        return L.moe_deq_swiglu_quant(acc, rows, n, ws, ts, stride, out, out_bytes, None)

    assert call(rows=-1) == 2
    assert call(n=0) == 2
    assert call(stride=2) == 2 and call(stride=6) == 2 and call(stride=0) == 2
    assert call(n=6) == 7                       # n % 4
    assert call(n=4100) == 7                    # above MOE_EPILOGUE_MAX_N
    assert call(rows=0, acc=None, ws=None, ts=None, out=None) == 0  # nothing to do
    assert call(acc=None) == 1 and call(ws=None) == 1 and call(ts=None) == 1 and call(out=None) == 1
    assert call(acc=P + 4) == 3 and call(ws=P + 8) == 3 and call(out=P + 4) == 3 and call(ts=P + 2) == 3
    assert call(out_bytes=16 * rb - 1) == 6


def test_grouped_gemm_rejects_on_host(M):
    L = M._lib
    ok = dict(a_row_bytes=7200, rows=64, k=7168, groups=16, n=4096, out_bytes=64 * 4096 * 4)

    def call(a=P, a_row_bytes=ok["a_row_bytes"], rows=ok["rows"], k=ok["k"], gc=P,
             groups=ok["groups"], w=P, n=ok["n"], out=P, out_bytes=ok["out_bytes"]):
        return L.moe_grouped_gemm_i8(a, a_row_bytes, rows, k, gc, groups, w, n, out, out_bytes, None)

    assert call(rows=-1) == 2 and call(k=0) == 2 and call(n=0) == 2 and call(groups=0) == 2
    assert call(a_row_bytes=7152) == 2          # shorter than k
    assert call(k=7160, a_row_bytes=7168) == 7  # k % 16
    assert call(k=65552, a_row_bytes=65552) == 7 and call(n=65537) == 7 and call(groups=65537) == 7
    assert call(a_row_bytes=7208) == 3          # row stride not a multiple of 16
    assert call(rows=0, a=None, gc=None, w=None, out=None) == 0  # nothing to do
    assert call(a=None) == 1 and call(gc=None) == 1 and call(w=None) == 1 and call(out=None) == 1
    assert call(a=P + 8) == 3 and call(w=P + 4) == 3 and call(gc=P + 2) == 3 and call(out=P + 2) == 3
    assert call(out_bytes=64 * 4096 * 4 - 1) == 6
    # more workgroups than one launch takes: rows / 256 + groups row slots x n / 128 column tiles
    assert call(rows=2 ** 31 - 1, a_row_bytes=16, k=16, n=65536,
                out_bytes=(2 ** 31 - 1) * 65536 * 4) == 7
