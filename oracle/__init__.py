"""numpy front end of the CPU oracle (``oracle/moe_oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke check and by the
benchmark's CPU-baseline leg, never by the product library.  Every function
forwards host arrays to the single-threaded C oracle, which computes the
method's plain definition (the header of moe_oracle.c names the passages of
"UMDK/CAM communication acceleration library deep analysis v2", sections 2 and
4, it follows and the readings it takes).

Receive buffers are returned in canonical form: passthrough rows as uint16
patterns ``[rows, h]``; quantised rows as int8 codes ``[rows, h]`` plus the
float32 inverse scales ``[rows]``.  ``rows = bs * k`` is the capacity; rows past
the dispatched total stay zero.

``Oracle(path)`` wraps one build of the library; the module-level functions use
the default build ``oracle/liboracle.so`` (compiled on first use if missing).
The mutation tests load deliberately broken builds through ``Oracle(path)``.
"""

from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional

import numpy as np

from . import build as _build

KIND_BF16, KIND_FP16, KIND_FP32, KIND_INT8 = 0, 1, 2, 3
_KIND = {"bf16": KIND_BF16, "fp16": KIND_FP16, "fp32": KIND_FP32, "int8": KIND_INT8}

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_INT = ctypes.c_int

_SIGS = {
    "oracle_bf16_to_f32": [_P, _P, _I64],
    "oracle_f16_to_f32": [_P, _P, _I64],
    "oracle_f32_to_bf16": [_P, _P, _I64],
    "oracle_f32_to_f16": [_P, _P, _I64],
    "oracle_layout": [_P, _I64, _I64, _I64, _I64, _P, _P, _P, _P],
    "oracle_notify": [_P, _I64, _I64, _P, _P, _P, _P],
    "oracle_notify_multi": [_P, _I64, _I64, _I64, _P, _P, _P, _P],
    "oracle_quant_row": [_P, _INT, _I64, _P, _P, _P],
    "oracle_dispatch": [_P, _INT, _I64, _I64, _I64, _P, _P, _P, _P, _I64, _I64, _INT, _I64,
                        _P, _P, _P],
    "oracle_combine": [_P, _P, _P, _INT, _I64, _I64, _I64, _P, _P, _P, _P, _P, _I64, _I64,
                       _I64, _P, _INT, _P],
    "oracle_exp_f32": [_P, _P, _I64],
    "oracle_swiglu_quant_row": [_P, _I64, _P, ctypes.c_float, _P, _P, _P],
    "oracle_swiglu_quant": [_P, _I64, _I64, _P, _P, _I64, _P, _P],
    "oracle_grouped_gemm_i8": [_P, _I64, _I64, _I64, _P, _I64, _P, _I64, _P, _I64, _P, _P],
}


class OracleError(RuntimeError):
    pass


def _ptr(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise OracleError(f"{what} returned {rc}")


class Oracle:
    """One loaded build of the C oracle."""

    def __init__(self, path: str):
        self.path = path
        L = ctypes.CDLL(path)
        for name, argtypes in _SIGS.items():
            fn = getattr(L, name)
            fn.argtypes = argtypes
            fn.restype = ctypes.c_int
        self.L = L

    # -- conversions (exported for the exhaustive pins) --------------------

    def bf16_to_f32(self, bits: np.ndarray) -> np.ndarray:
        bits = np.ascontiguousarray(bits, dtype=np.uint16)
        out = np.empty(bits.shape, np.float32)
        _check(self.L.oracle_bf16_to_f32(_ptr(bits), _ptr(out), bits.size), "bf16_to_f32")
        return out

    def f16_to_f32(self, bits: np.ndarray) -> np.ndarray:
        bits = np.ascontiguousarray(bits, dtype=np.uint16)
        out = np.empty(bits.shape, np.float32)
        _check(self.L.oracle_f16_to_f32(_ptr(bits), _ptr(out), bits.size), "f16_to_f32")
        return out

    def f32_to_bf16(self, x: np.ndarray) -> np.ndarray:
        x = np.ascontiguousarray(x, dtype=np.float32)
        out = np.empty(x.shape, np.uint16)
        _check(self.L.oracle_f32_to_bf16(_ptr(x), _ptr(out), x.size), "f32_to_bf16")
        return out

    def f32_to_f16(self, x: np.ndarray) -> np.ndarray:
        x = np.ascontiguousarray(x, dtype=np.float32)
        out = np.empty(x.shape, np.uint16)
        _check(self.L.oracle_f32_to_f16(_ptr(x), _ptr(out), x.size), "f32_to_f16")
        return out

    # -- the four stages ---------------------------------------------------

    def layout(self, topk_idx: np.ndarray, expert_num_per_rank: int,
               rank_size: int) -> Dict[str, object]:
        """Stage 1: tokenPerExpert [E], tokenPerRank [R], sendTokenIdx [bs, k], bad."""
        idx = np.ascontiguousarray(topk_idx, dtype=np.int32)
        if idx.ndim != 2:
            raise ValueError("topk_idx must be [bs, k]")
        bs, k = idx.shape
        e = expert_num_per_rank * rank_size
        tpe = np.zeros(e, np.int32)
        tpr = np.zeros(rank_size, np.int32)
        slot = np.zeros((bs, k), np.int32)
        bad = ctypes.c_int64(0)
        _check(self.L.oracle_layout(_ptr(idx), bs, k, expert_num_per_rank, rank_size, _ptr(tpe),
                                    _ptr(tpr), _ptr(slot), ctypes.addressof(bad)), "layout")
        return dict(token_per_expert=tpe, token_per_rank=tpr, send_token_idx=slot,
                    bad=int(bad.value))

    def notify(self, token_per_expert: np.ndarray, expert_num_per_rank: int,
               rank_size: int) -> Dict[str, np.ndarray]:
        """Stage 2: putOffset [E], recvCount [R], recvBase [R], recvTokenPerExpert [E]."""
        tpe = np.ascontiguousarray(token_per_expert, dtype=np.int32)
        e = expert_num_per_rank * rank_size
        if tpe.shape != (e,):
            raise ValueError("token_per_expert must be [E]")
        put = np.zeros(e, np.int32)
        cnt = np.zeros(rank_size, np.int32)
        base = np.zeros(rank_size, np.int32)
        rtpe = np.zeros(e, np.int32)
        _check(self.L.oracle_notify(_ptr(tpe), expert_num_per_rank, rank_size, _ptr(put),
                                    _ptr(cnt), _ptr(base), _ptr(rtpe)), "notify")
        return dict(put_offset=put, recv_count=cnt, recv_base=base, recv_token_per_expert=rtpe)

    def notify_multi(self, token_per_expert: np.ndarray, expert_num_per_rank: int,
                     rank_size: int) -> Dict[str, np.ndarray]:
        """Stage 2 over the count matrix of several sources: token_per_expert
        [S, E] -> putOffset [E, S], recvCount [R], recvBase [R],
        recvTokenPerExpert [E]."""
        tpe = np.ascontiguousarray(token_per_expert, dtype=np.int32)
        e = expert_num_per_rank * rank_size
        if tpe.ndim != 2 or tpe.shape[1] != e:
            raise ValueError("token_per_expert must be [S, E]")
        num_src = tpe.shape[0]
        put = np.zeros((e, num_src), np.int32)
        cnt = np.zeros(rank_size, np.int32)
        base = np.zeros(rank_size, np.int32)
        rtpe = np.zeros(e, np.int32)
        _check(self.L.oracle_notify_multi(_ptr(tpe), num_src, expert_num_per_rank, rank_size,
                                          _ptr(put), _ptr(cnt), _ptr(base), _ptr(rtpe)),
               "notify_multi")
        return dict(put_offset=put, recv_count=cnt, recv_base=base, recv_token_per_expert=rtpe)

    def quant_row(self, x_bits: np.ndarray, x_kind: str = "bf16"):
        """QuantProcess on one row: (codes int8 [h], inv float32, scale float32)."""
        x = np.ascontiguousarray(x_bits, dtype=np.uint16).reshape(-1)
        codes = np.zeros(x.size, np.int8)
        inv = ctypes.c_float(0.0)
        s = ctypes.c_float(0.0)
        _check(self.L.oracle_quant_row(_ptr(x), _KIND[x_kind], x.size, _ptr(codes),
                                       ctypes.addressof(inv), ctypes.addressof(s)), "quant_row")
        return codes, np.float32(inv.value), np.float32(s.value)

    def exp_f32(self, x: np.ndarray) -> np.ndarray:
        """The oracle's binary32 e^x (Cody-Waite reduction, degree-7 Taylor)."""
        xs = np.ascontiguousarray(x, dtype=np.float32)
        out = np.zeros_like(xs)
        _check(self.L.oracle_exp_f32(_ptr(xs), _ptr(out), xs.size), "exp_f32")
        return out

    def swiglu_quant_row(self, acc: np.ndarray, weight_scale: np.ndarray, token_scale: float):
        """Epilogue of one row (acc int32 [2n]): (codes int8 [n], inv float32,
        activations float32 [n] before quantisation)."""
        a = np.ascontiguousarray(acc, dtype=np.int32).reshape(-1)
        ws = np.ascontiguousarray(weight_scale, dtype=np.float32).reshape(-1)
        if a.size % 2 or ws.size != a.size:
            raise ValueError("acc and weight_scale: 2n values each")
        n = a.size // 2
        codes = np.zeros(n, np.int8)
        act = np.zeros(n, np.float32)
        inv = ctypes.c_float(0.0)
        _check(self.L.oracle_swiglu_quant_row(_ptr(a), n, _ptr(ws), float(np.float32(token_scale)),
                                              _ptr(codes), ctypes.addressof(inv), _ptr(act)),
               "swiglu_quant_row")
        return codes, np.float32(inv.value), act

    def swiglu_quant(self, acc: np.ndarray, weight_scale: np.ndarray,
                     token_scale: np.ndarray) -> Dict[str, np.ndarray]:
        """Epilogue of every row: acc int32 [rows, 2n], weight_scale float32
        [2n], token_scale float32 [rows] -> codes int8 [rows, n], inv [rows]."""
        a = np.ascontiguousarray(acc, dtype=np.int32)
        rows, n2 = a.shape
        if n2 % 2:
            raise ValueError("acc: [rows, 2n]")
        n = n2 // 2
        ws = np.ascontiguousarray(weight_scale, dtype=np.float32).reshape(-1)
        ts = np.ascontiguousarray(token_scale, dtype=np.float32).reshape(-1)
        if ws.size != n2 or ts.size != rows:
            raise ValueError("weight_scale [2n], token_scale [rows]")
        codes = np.zeros((rows, n), np.int8)
        inv = np.zeros(rows, np.float32)
        _check(self.L.oracle_swiglu_quant(_ptr(a), rows, n, _ptr(ws), _ptr(ts), 1, _ptr(codes),
                                          _ptr(inv)), "swiglu_quant")
        return dict(codes=codes, inv=inv)

    def grouped_gemm_i8(self, a: np.ndarray, k: int, group_count: np.ndarray, w: np.ndarray,
                        rows: Optional[np.ndarray] = None):
        """First expert matmul: a int8 [R, stride] receive rows (codes in the
        first k bytes of each row), group_count int32 [G], w int8 [G, n, k].
        Returns (out int32 [len(rows), n], row_group int32 [len(rows)]) for
        the listed rows (all R rows when ``rows`` is None); a row that no
        expert owns gets group -1 and an all-zero out row."""
        a8 = np.ascontiguousarray(a).view(np.int8)
        if a8.ndim != 2 or a8.shape[1] < k:
            raise ValueError("a: [rows, stride >= k]")
        gc = np.ascontiguousarray(group_count, dtype=np.int32).reshape(-1)
        w8 = np.ascontiguousarray(w).view(np.int8)
        if w8.ndim != 3 or w8.shape[0] != gc.size or w8.shape[2] != k:
            raise ValueError("w: [groups, n, k]")
        n = w8.shape[1]
        lst = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64).reshape(-1)
        nl = a8.shape[0] if lst is None else lst.size
        out = np.zeros((nl, n), np.int32)
        grp = np.zeros(nl, np.int32)
        _check(self.L.oracle_grouped_gemm_i8(_ptr(a8), a8.shape[1], a8.shape[0], k, _ptr(gc), gc.size,
                                             _ptr(w8), n, _ptr(lst), nl, _ptr(out), _ptr(grp)),
               "grouped_gemm_i8")
        return out, grp

    def dispatch(self, x_bits: np.ndarray, x_kind: str, topk_idx: np.ndarray,
                 send_token_idx: np.ndarray, put_offset: np.ndarray, recv_base: np.ndarray,
                 expert_num_per_rank: int, rank_size: int, quant: bool,
                 into: Optional[Dict[str, np.ndarray]] = None) -> Dict[str, np.ndarray]:
        """Stage 3: scatter rows (optionally quantised) into a [bs*k]-row
        buffer, or into the rows of ``into`` (a buffer shared by several
        sources, as returned by an earlier call)."""
        x = np.ascontiguousarray(x_bits, dtype=np.uint16)
        bs, h = x.shape
        idx = np.ascontiguousarray(topk_idx, dtype=np.int32)
        k = idx.shape[1]
        slot = np.ascontiguousarray(send_token_idx, dtype=np.int32)
        put = np.ascontiguousarray(put_offset, dtype=np.int32)
        base = np.ascontiguousarray(recv_base, dtype=np.int32)
        recv = codes = inv = None
        if into is not None:
            if quant:
                codes, inv = into["codes"], into["inv"]
                rows = codes.shape[0]
                if codes.dtype != np.int8 or inv.dtype != np.float32 or not codes.flags.c_contiguous:
                    raise ValueError("into: int8 codes [rows, h] and float32 inv [rows]")
            else:
                recv = into["rows"]
                rows = recv.shape[0]
                if recv.dtype != np.uint16 or not recv.flags.c_contiguous:
                    raise ValueError("into: uint16 rows [rows, h]")
        else:
            rows = bs * k
            if quant:
                codes = np.zeros((rows, h), np.int8)
                inv = np.zeros(rows, np.float32)
            else:
                recv = np.zeros((rows, h), np.uint16)
        _check(self.L.oracle_dispatch(_ptr(x), _KIND[x_kind], bs, h, k, _ptr(idx), _ptr(slot),
                                      _ptr(put), _ptr(base), expert_num_per_rank, rank_size,
                                      1 if quant else 0, rows, _ptr(recv), _ptr(codes),
                                      _ptr(inv)), "dispatch")
        if quant:
            return dict(codes=codes, inv=inv)
        return dict(rows=recv)

    def combine(self, recv: Dict[str, np.ndarray], recv_kind: str, topk_idx: np.ndarray,
                topk_w: np.ndarray, send_token_idx: np.ndarray, put_offset: np.ndarray,
                recv_base: np.ndarray, expert_num_per_rank: int, rank_size: int,
                out_kind: str) -> np.ndarray:
        """Stage 4: weighted gather.  Returns uint16 patterns (bf16/fp16) or float32."""
        idx = np.ascontiguousarray(topk_idx, dtype=np.int32)
        bs, k = idx.shape
        w = np.ascontiguousarray(topk_w, dtype=np.float32)
        slot = np.ascontiguousarray(send_token_idx, dtype=np.int32)
        put = np.ascontiguousarray(put_offset, dtype=np.int32)
        base = np.ascontiguousarray(recv_base, dtype=np.int32)
        if recv_kind == "int8":
            codes = np.ascontiguousarray(recv["codes"], dtype=np.int8)
            inv = np.ascontiguousarray(recv["inv"], dtype=np.float32)
            rows_arr = None
            rows, h = codes.shape
        else:
            rows_arr = np.ascontiguousarray(recv["rows"], dtype=np.uint16)
            codes = inv = None
            rows, h = rows_arr.shape
        out = np.zeros((bs, h), np.float32 if out_kind == "fp32" else np.uint16)
        scratch = np.zeros(h, np.float32)
        _check(self.L.oracle_combine(_ptr(rows_arr), _ptr(codes), _ptr(inv), _KIND[recv_kind], bs,
                                     h, k, _ptr(idx), _ptr(w), _ptr(slot), _ptr(put), _ptr(base),
                                     expert_num_per_rank, rank_size, rows, _ptr(out),
                                     _KIND[out_kind], _ptr(scratch)), "combine")
        return out

    def pipeline(self, x_bits: np.ndarray, x_kind: str, topk_idx: np.ndarray,
                 topk_w: np.ndarray, expert_num_per_rank: int, rank_size: int, quant: bool,
                 out_kind: Optional[str] = None) -> Dict[str, object]:
        """All four stages in order; returns every intermediate."""
        lay = self.layout(topk_idx, expert_num_per_rank, rank_size)
        no = self.notify(lay["token_per_expert"], expert_num_per_rank, rank_size)
        dis = self.dispatch(x_bits, x_kind, topk_idx, lay["send_token_idx"], no["put_offset"],
                            no["recv_base"], expert_num_per_rank, rank_size, quant)
        out_kind = out_kind or x_kind
        out = self.combine(dis, "int8" if quant else x_kind, topk_idx, topk_w,
                           lay["send_token_idx"], no["put_offset"], no["recv_base"],
                           expert_num_per_rank, rank_size, out_kind)
        return dict(layout=lay, notify=no, dispatch=dis, out=out)

    def pipeline_multi(self, xs, x_kind: str, idxs, ws, expert_num_per_rank: int,
                       rank_size: int, quant: bool, out_kind: Optional[str] = None
                       ) -> Dict[str, object]:
        """All four stages with several source ranks sharing one receive
        buffer: a layout per source, notify over the [S, E] count matrix,
        each source's dispatch with its column of putOffset, then each
        source's combine.  Returns every intermediate; ``outs`` per source."""
        lays = [self.layout(idx, expert_num_per_rank, rank_size) for idx in idxs]
        counts = np.stack([l["token_per_expert"] for l in lays]) if lays else None
        no = self.notify_multi(counts, expert_num_per_rank, rank_size)
        h = xs[0].shape[1]
        rows = sum(int(np.asarray(i).shape[0]) * int(np.asarray(i).shape[1]) for i in idxs)
        if quant:
            buf = dict(codes=np.zeros((rows, h), np.int8), inv=np.zeros(rows, np.float32))
        else:
            buf = dict(rows=np.zeros((rows, h), np.uint16))
        for src, (x, idx, lay) in enumerate(zip(xs, idxs, lays)):
            self.dispatch(x, x_kind, idx, lay["send_token_idx"], no["put_offset"][:, src],
                          no["recv_base"], expert_num_per_rank, rank_size, quant, into=buf)
        out_kind = out_kind or x_kind
        outs = [self.combine(buf, "int8" if quant else x_kind, idx, w, lay["send_token_idx"],
                             no["put_offset"][:, src], no["recv_base"], expert_num_per_rank,
                             rank_size, out_kind)
                for src, (idx, w, lay) in enumerate(zip(idxs, ws, lays))]
        return dict(layouts=lays, counts=counts, notify=no, dispatch=buf, outs=outs)


_default: Optional[Oracle] = None


def default() -> Oracle:
    """The oracle built from oracle/moe_oracle.c (compiled here if missing)."""
    global _default
    if _default is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        _default = Oracle(_build.LIB)
    return _default


def bf16_to_f32(bits):
    return default().bf16_to_f32(bits)


def f16_to_f32(bits):
    return default().f16_to_f32(bits)


def f32_to_bf16(x):
    return default().f32_to_bf16(x)


def f32_to_f16(x):
    return default().f32_to_f16(x)


def layout(*a, **kw):
    return default().layout(*a, **kw)


def notify(*a, **kw):
    return default().notify(*a, **kw)


def notify_multi(*a, **kw):
    return default().notify_multi(*a, **kw)


def pipeline_multi(*a, **kw):
    return default().pipeline_multi(*a, **kw)


def quant_row(*a, **kw):
    return default().quant_row(*a, **kw)


def dispatch(*a, **kw):
    return default().dispatch(*a, **kw)


def combine(*a, **kw):
    return default().combine(*a, **kw)


def pipeline(*a, **kw):
    return default().pipeline(*a, **kw)


def exp_f32(*a, **kw):
    return default().exp_f32(*a, **kw)


def swiglu_quant_row(*a, **kw):
    return default().swiglu_quant_row(*a, **kw)


def swiglu_quant(*a, **kw):
    return default().swiglu_quant(*a, **kw)


def grouped_gemm_i8(*a, **kw):
    return default().grouped_gemm_i8(*a, **kw)
