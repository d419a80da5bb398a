"""Python binding of libmoe_ep.so, the MI355X (gfx950) MoE expert-parallel
dispatch/combine library.

The functions below carry the names of the C entry points declared in
include/moe_ep.h and only marshal arguments: they check that tensors are
CUDA (HIP) tensors of the right dtype and contiguity, pass their device
pointers and torch's current stream to the C call, and raise ``MoeEpError``
on a non-zero status.  Every step of the path runs in the library's HIP
kernels; there is no fallback.  Importing this module fails loudly if the
library has not been built (``python combine_moe_layout_03_amd/build.py`` or
``__graft_entry__.build()``).

``EpBuffers`` allocates (through torch) every device buffer the four stages
need for one shape, so a caller can run the pipeline without allocating.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

__all__ = [
    "MOE_BF16", "MOE_FP16", "MOE_FP32", "MOE_INT8_ROWSCALE", "MoeEpError", "LIB_PATH",
    "moe_recv_row_bytes", "moe_layout_workspace_bytes", "moe_layout", "moe_notify",
    "moe_dispatch", "moe_combine", "moe_status_str", "moe_last_hip_error", "EpBuffers",
    "dtype_code", "moe_fused_supported", "moe_layout_notify_dispatch", "moe_notify_multi",
    "moe_dispatch_src", "moe_combine_src", "EpMultiBuffers", "MOE_MAX_SOURCES",
    "moe_deq_swiglu_quant", "token_scales_of", "MOE_EPILOGUE_MAX_N", "moe_grouped_gemm_i8",
    "MOE_GEMM_MAX_K", "MOE_GEMM_MAX_N", "MOE_GEMM_MAX_GROUPS", "moe_layout_no_alloc",
    "moe_gemm_swiglu_quant_workspace_bytes", "moe_grouped_gemm_swiglu_quant_i8",
    "MOE_NO_ALLOC_SCRATCH_BYTES",
]

MOE_BF16, MOE_FP16, MOE_FP32, MOE_INT8_ROWSCALE = 0, 1, 2, 3
MOE_MAX_EXPERTS, MOE_MAX_HIDDEN, MOE_MAX_TOPK, MOE_MAX_SOURCES = 2048, 16384, 32, 384
MOE_EPILOGUE_MAX_N = 4096
MOE_GEMM_MAX_K = MOE_GEMM_MAX_N = MOE_GEMM_MAX_GROUPS = 65536
MOE_NO_ALLOC_SCRATCH_BYTES = 1 << 20

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe_ep.so")

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_INT = ctypes.c_int
_SZ = ctypes.c_size_t

# name -> (argtypes, restype); mirrors include/moe_ep.h
_SIGS = {
    "moe_recv_row_bytes": ([_I32, _INT, ctypes.POINTER(_SZ)], _INT),
    "moe_layout_workspace_bytes": ([_I32, _I32, _I32, ctypes.POINTER(_SZ)], _INT),
    "moe_layout": ([_P, _I32, _I32, _I32, _I32, _P, _P, _P, _P, _P, _SZ, _P], _INT),
    "moe_layout_no_alloc": ([_P, _I32, _I32, _I32, _I32, _P, _P, _P, _P, _P], _INT),
    "moe_notify": ([_P, _I32, _I32, _P, _P, _P, _P, _P], _INT),
    "moe_dispatch": ([_P, _INT, _I32, _I32, _I32, _P, _P, _P, _P, _I32, _I32, _INT, _P, _SZ, _P],
                     _INT),
    "moe_combine": ([_P, _INT, _SZ, _I32, _I32, _I32, _P, _P, _P, _P, _P, _I32, _I32, _P, _INT, _P],
                    _INT),
    "moe_notify_multi": ([_P, _I32, _I32, _I32, _P, _P, _P, _P, _P], _INT),
    "moe_dispatch_src": ([_P, _INT, _I32, _I32, _I32, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _INT, _P,
                          _SZ, _P], _INT),
    "moe_combine_src": ([_P, _INT, _SZ, _I32, _I32, _I32, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _P,
                         _INT, _P], _INT),
    "moe_fused_supported": ([_I32, _I32, _I32, _I32, _I32, _INT, _INT, ctypes.POINTER(_INT)], _INT),
    "moe_layout_notify_dispatch": ([_P, _INT, _I32, _I32, _I32, _P, _I32, _I32, _INT, _P, _P, _P, _P, _P, _P,
                                    _P, _P, _P, _SZ, _P, _SZ, _P], _INT),
    "moe_deq_swiglu_quant": ([_P, _I32, _I32, _P, _P, ctypes.c_int64, _P, _SZ, _P], _INT),
    "moe_grouped_gemm_i8": ([_P, ctypes.c_int64, _I32, _I32, _P, _I32, _P, _I32, _P, _SZ, _P], _INT),
    "moe_gemm_swiglu_quant_workspace_bytes": ([_I32, _I32, ctypes.POINTER(_SZ)], _INT),
    "moe_grouped_gemm_swiglu_quant_i8": ([_P, ctypes.c_int64, _I32, _I32, _P, _I32, _P, _I32, _P, _P,
                                          ctypes.c_int64, _P, _SZ, _P, _SZ, _P], _INT),
    "moe_status_str": ([_INT], ctypes.c_char_p),
    "moe_last_hip_error": ([], _INT),
}


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; build it with `python combine_moe_layout_03_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (argtypes, restype) in _SIGS.items():
        fn = getattr(lib, name)
        fn.argtypes = argtypes
        fn.restype = restype
    return lib


_lib = _load()


class MoeEpError(RuntimeError):
    def __init__(self, fn: str, status: int):
        msg = _lib.moe_status_str(status).decode()
        if status == 8:
            msg += f" (hipError {_lib.moe_last_hip_error()})"
        super().__init__(f"{fn}: status {status}: {msg}")
        self.status = status


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise MoeEpError(fn, status)


def moe_status_str(status: int) -> str:
    return _lib.moe_status_str(status).decode()


def moe_last_hip_error() -> int:
    return _lib.moe_last_hip_error()


_DTYPE = {torch.bfloat16: MOE_BF16, torch.float16: MOE_FP16, torch.float32: MOE_FP32}


def dtype_code(dtype: torch.dtype) -> int:
    try:
        return _DTYPE[dtype]
    except KeyError:
        raise ValueError(f"unsupported dtype {dtype}") from None


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _dev(t: Optional[torch.Tensor], name: str, dtype=None, optional: bool = False):
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _need(t: Optional[torch.Tensor], name: str, count: int) -> None:
    """Raise unless ``t`` (if given) holds at least ``count`` elements: the
    library takes bare pointers, so an undersized tensor would be written or
    read past its end."""
    if isinstance(t, torch.Tensor) and t.numel() < count:
        raise ValueError(f"{name} holds {t.numel()} elements, the call needs {count}")


def _experts(expert_num_per_rank: int, rank_size: int) -> Optional[int]:
    """E = EPR * R when the library accepts the pair (else None: the call's
    own status reports it, and there is no size to check against)."""
    if expert_num_per_rank >= 1 and rank_size >= 1 and expert_num_per_rank * rank_size <= MOE_MAX_EXPERTS:
        return expert_num_per_rank * rank_size
    return None


def _need_routes(expert_num_per_rank: int, rank_size: int, put_offset: Optional[torch.Tensor],
                 recv_base: Optional[torch.Tensor], num_src: int = 1) -> None:
    e = _experts(expert_num_per_rank, rank_size)
    if e is not None:
        _need(put_offset, "put_offset", e * num_src)
        _need(recv_base, "recv_base", rank_size)


def _need_scales(token_scale: torch.Tensor, rows: int, stride: int) -> None:
    if rows > 0 and stride >= 4:
        need = (rows - 1) * stride + 4
        have = token_scale.numel() * token_scale.element_size()
        if have < need:
            raise ValueError(f"token_scale holds {have} bytes, rows at stride {stride} need {need}")


def moe_recv_row_bytes(hidden: int, recv_type: int) -> int:
    out = _SZ(0)
    _check("moe_recv_row_bytes", _lib.moe_recv_row_bytes(hidden, recv_type, ctypes.byref(out)))
    return out.value


def moe_layout_workspace_bytes(bs: int, topk: int, num_experts: int) -> int:
    out = _SZ(0)
    _check("moe_layout_workspace_bytes",
           _lib.moe_layout_workspace_bytes(bs, topk, num_experts, ctypes.byref(out)))
    return out.value


def _need_layout(bs, topk, expert_num_per_rank, rank_size, token_per_expert, token_per_rank, send_token_idx,
                 bad_id_count) -> None:
    e = _experts(expert_num_per_rank, rank_size)
    if e is not None:
        _need(token_per_expert, "token_per_expert", e)
        _need(token_per_rank, "token_per_rank", rank_size)
    _need(send_token_idx, "send_token_idx", bs * topk)
    _need(bad_id_count, "bad_id_count", 1)


def moe_layout(topk_idx: torch.Tensor, expert_num_per_rank: int, rank_size: int,
               token_per_expert: torch.Tensor, token_per_rank: torch.Tensor,
               send_token_idx: torch.Tensor, bad_id_count: Optional[torch.Tensor] = None,
               workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    if topk_idx.dim() != 2:
        raise ValueError("topk_idx must be [bs, topk]")
    bs, topk = topk_idx.shape
    _need_layout(bs, topk, expert_num_per_rank, rank_size, token_per_expert, token_per_rank, send_token_idx,
                 bad_id_count)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("moe_layout", _lib.moe_layout(
        _dev(topk_idx, "topk_idx", torch.int32), bs, topk, expert_num_per_rank, rank_size,
        _dev(token_per_expert, "token_per_expert", torch.int32),
        _dev(token_per_rank, "token_per_rank", torch.int32),
        _dev(send_token_idx, "send_token_idx", torch.int32),
        _dev(bad_id_count, "bad_id_count", torch.int32, optional=True),
        _dev(workspace, "workspace", optional=True), ws_bytes, _stream(stream)))


def moe_layout_no_alloc(topk_idx: torch.Tensor, expert_num_per_rank: int, rank_size: int,
                        token_per_expert: torch.Tensor, token_per_rank: torch.Tensor,
                        send_token_idx: torch.Tensor, bad_id_count: Optional[torch.Tensor] = None,
                        stream=None) -> None:
    """moe_layout with the library's static workspace (no allocation)."""
    if topk_idx.dim() != 2:
        raise ValueError("topk_idx must be [bs, topk]")
    bs, topk = topk_idx.shape
    _need_layout(bs, topk, expert_num_per_rank, rank_size, token_per_expert, token_per_rank, send_token_idx,
                 bad_id_count)
    _check("moe_layout_no_alloc", _lib.moe_layout_no_alloc(
        _dev(topk_idx, "topk_idx", torch.int32), bs, topk, expert_num_per_rank, rank_size,
        _dev(token_per_expert, "token_per_expert", torch.int32),
        _dev(token_per_rank, "token_per_rank", torch.int32),
        _dev(send_token_idx, "send_token_idx", torch.int32),
        _dev(bad_id_count, "bad_id_count", torch.int32, optional=True), _stream(stream)))


def moe_notify(token_per_expert: torch.Tensor, expert_num_per_rank: int, rank_size: int,
               put_offset: torch.Tensor, recv_count: torch.Tensor, recv_base: torch.Tensor,
               recv_token_per_expert: torch.Tensor, stream=None) -> None:
    e = _experts(expert_num_per_rank, rank_size)
    if e is not None:
        for t, name in ((token_per_expert, "token_per_expert"), (recv_token_per_expert, "recv_token_per_expert")):
            _need(t, name, e)
        _need(recv_count, "recv_count", rank_size)
    _need_routes(expert_num_per_rank, rank_size, put_offset, recv_base)
    _check("moe_notify", _lib.moe_notify(
        _dev(token_per_expert, "token_per_expert", torch.int32), expert_num_per_rank, rank_size,
        _dev(put_offset, "put_offset", torch.int32), _dev(recv_count, "recv_count", torch.int32),
        _dev(recv_base, "recv_base", torch.int32),
        _dev(recv_token_per_expert, "recv_token_per_expert", torch.int32), _stream(stream)))


def moe_dispatch(x: torch.Tensor, topk_idx: torch.Tensor, send_token_idx: torch.Tensor,
                 put_offset: torch.Tensor, recv_base: torch.Tensor, expert_num_per_rank: int,
                 rank_size: int, quant_int8: bool, recv_x: torch.Tensor, stream=None) -> None:
    if x.dim() != 2 or topk_idx.dim() != 2:
        raise ValueError("x must be [bs, hidden] and topk_idx [bs, topk]")
    bs, hidden = x.shape
    topk = topk_idx.shape[1]
    _need(send_token_idx, "send_token_idx", bs * topk)
    _need_routes(expert_num_per_rank, rank_size, put_offset, recv_base)
    _check("moe_dispatch", _lib.moe_dispatch(
        _dev(x, "x"), dtype_code(x.dtype), bs, hidden, topk,
        _dev(topk_idx, "topk_idx", torch.int32), _dev(send_token_idx, "send_token_idx", torch.int32),
        _dev(put_offset, "put_offset", torch.int32), _dev(recv_base, "recv_base", torch.int32),
        expert_num_per_rank, rank_size, 1 if quant_int8 else 0, _dev(recv_x, "recv_x"),
        recv_x.numel() * recv_x.element_size(), _stream(stream)))


def moe_combine(recv_x: torch.Tensor, recv_type: int, hidden: int, topk_idx: torch.Tensor,
                topk_weights: torch.Tensor, send_token_idx: torch.Tensor, put_offset: torch.Tensor,
                recv_base: torch.Tensor, expert_num_per_rank: int, rank_size: int,
                out: torch.Tensor, stream=None) -> None:
    if topk_idx.dim() != 2:
        raise ValueError("topk_idx must be [bs, topk]")
    bs, topk = topk_idx.shape
    if out.dim() != 2 or tuple(out.shape) != (bs, hidden):
        raise ValueError("out must be [bs, hidden]")
    _need(topk_weights, "topk_weights", bs * topk)
    _need(send_token_idx, "send_token_idx", bs * topk)
    _need_routes(expert_num_per_rank, rank_size, put_offset, recv_base)
    _check("moe_combine", _lib.moe_combine(
        _dev(recv_x, "recv_x"), recv_type, recv_x.numel() * recv_x.element_size(), bs, hidden, topk,
        _dev(topk_idx, "topk_idx", torch.int32), _dev(topk_weights, "topk_weights", torch.float32),
        _dev(send_token_idx, "send_token_idx", torch.int32), _dev(put_offset, "put_offset", torch.int32),
        _dev(recv_base, "recv_base", torch.int32), expert_num_per_rank, rank_size, _dev(out, "out"),
        dtype_code(out.dtype), _stream(stream)))


def moe_notify_multi(token_per_expert: torch.Tensor, expert_num_per_rank: int, rank_size: int,
                     put_offset: torch.Tensor, recv_count: torch.Tensor, recv_base: torch.Tensor,
                     recv_token_per_expert: torch.Tensor, stream=None) -> None:
    """token_per_expert [S, E] -> put_offset [E, S] and the per-rank arrays."""
    if token_per_expert.dim() != 2:
        raise ValueError("token_per_expert must be [num_src, E]")
    num_src, e = token_per_expert.shape
    if tuple(put_offset.shape) != (e, num_src):
        raise ValueError("put_offset must be [E, num_src]")
    if _experts(expert_num_per_rank, rank_size) not in (None, e):
        raise ValueError("token_per_expert must have expert_num_per_rank * rank_size columns")
    _need(recv_count, "recv_count", rank_size)
    _need(recv_base, "recv_base", rank_size)
    _need(recv_token_per_expert, "recv_token_per_expert", e)
    _check("moe_notify_multi", _lib.moe_notify_multi(
        _dev(token_per_expert, "token_per_expert", torch.int32), num_src, expert_num_per_rank,
        rank_size, _dev(put_offset, "put_offset", torch.int32),
        _dev(recv_count, "recv_count", torch.int32), _dev(recv_base, "recv_base", torch.int32),
        _dev(recv_token_per_expert, "recv_token_per_expert", torch.int32), _stream(stream)))


def moe_dispatch_src(x: torch.Tensor, topk_idx: torch.Tensor, send_token_idx: torch.Tensor,
                     put_offset: torch.Tensor, recv_base: torch.Tensor, expert_num_per_rank: int,
                     rank_size: int, src_rank: int, quant_int8: bool, recv_x: torch.Tensor,
                     stream=None) -> None:
    """Dispatch of source ``src_rank``; put_offset is [E, num_src]."""
    if x.dim() != 2 or topk_idx.dim() != 2 or put_offset.dim() != 2:
        raise ValueError("x must be [bs, hidden], topk_idx [bs, topk], put_offset [E, num_src]")
    bs, hidden = x.shape
    topk = topk_idx.shape[1]
    _need(send_token_idx, "send_token_idx", bs * topk)
    _need_routes(expert_num_per_rank, rank_size, put_offset, recv_base, put_offset.shape[1])
    _check("moe_dispatch_src", _lib.moe_dispatch_src(
        _dev(x, "x"), dtype_code(x.dtype), bs, hidden, topk,
        _dev(topk_idx, "topk_idx", torch.int32), _dev(send_token_idx, "send_token_idx", torch.int32),
        _dev(put_offset, "put_offset", torch.int32), _dev(recv_base, "recv_base", torch.int32),
        expert_num_per_rank, rank_size, put_offset.shape[1], src_rank, 1 if quant_int8 else 0,
        _dev(recv_x, "recv_x"), recv_x.numel() * recv_x.element_size(), _stream(stream)))


def moe_combine_src(recv_x: torch.Tensor, recv_type: int, hidden: int, topk_idx: torch.Tensor,
                    topk_weights: torch.Tensor, send_token_idx: torch.Tensor, put_offset: torch.Tensor,
                    recv_base: torch.Tensor, expert_num_per_rank: int, rank_size: int, src_rank: int,
                    out: torch.Tensor, stream=None) -> None:
    """Combine of source ``src_rank``; put_offset is [E, num_src]."""
    if topk_idx.dim() != 2 or put_offset.dim() != 2:
        raise ValueError("topk_idx must be [bs, topk] and put_offset [E, num_src]")
    bs, topk = topk_idx.shape
    if out.dim() != 2 or tuple(out.shape) != (bs, hidden):
        raise ValueError("out must be [bs, hidden]")
    _need(topk_weights, "topk_weights", bs * topk)
    _need(send_token_idx, "send_token_idx", bs * topk)
    _need_routes(expert_num_per_rank, rank_size, put_offset, recv_base, put_offset.shape[1])
    _check("moe_combine_src", _lib.moe_combine_src(
        _dev(recv_x, "recv_x"), recv_type, recv_x.numel() * recv_x.element_size(), bs, hidden, topk,
        _dev(topk_idx, "topk_idx", torch.int32), _dev(topk_weights, "topk_weights", torch.float32),
        _dev(send_token_idx, "send_token_idx", torch.int32), _dev(put_offset, "put_offset", torch.int32),
        _dev(recv_base, "recv_base", torch.int32), expert_num_per_rank, rank_size, put_offset.shape[1],
        src_rank, _dev(out, "out"), dtype_code(out.dtype), _stream(stream)))


def moe_fused_supported(bs: int, hidden: int, topk: int, expert_num_per_rank: int, rank_size: int,
                        x_dtype: torch.dtype, quant_int8: bool) -> bool:
    out = _INT(0)
    _check("moe_fused_supported", _lib.moe_fused_supported(
        bs, hidden, topk, expert_num_per_rank, rank_size, dtype_code(x_dtype), 1 if quant_int8 else 0,
        ctypes.byref(out)))
    return bool(out.value)


def moe_layout_notify_dispatch(x: torch.Tensor, topk_idx: torch.Tensor, expert_num_per_rank: int,
                               rank_size: int, quant_int8: bool, token_per_expert: torch.Tensor,
                               token_per_rank: torch.Tensor, send_token_idx: torch.Tensor,
                               bad_id_count: Optional[torch.Tensor], put_offset: torch.Tensor,
                               recv_count: torch.Tensor, recv_base: torch.Tensor,
                               recv_token_per_expert: torch.Tensor, recv_x: torch.Tensor,
                               workspace: torch.Tensor, stream=None) -> None:
    if x.dim() != 2 or topk_idx.dim() != 2:
        raise ValueError("x must be [bs, hidden] and topk_idx [bs, topk]")
    bs, hidden = x.shape
    topk = topk_idx.shape[1]
    _need_layout(bs, topk, expert_num_per_rank, rank_size, token_per_expert, token_per_rank, send_token_idx,
                 bad_id_count)
    e = _experts(expert_num_per_rank, rank_size)
    if e is not None:
        _need(recv_token_per_expert, "recv_token_per_expert", e)
        _need(recv_count, "recv_count", rank_size)
    _need_routes(expert_num_per_rank, rank_size, put_offset, recv_base)
    i32 = torch.int32
    _check("moe_layout_notify_dispatch", _lib.moe_layout_notify_dispatch(
        _dev(x, "x"), dtype_code(x.dtype), bs, hidden, topk, _dev(topk_idx, "topk_idx", i32),
        expert_num_per_rank, rank_size, 1 if quant_int8 else 0,
        _dev(token_per_expert, "token_per_expert", i32), _dev(token_per_rank, "token_per_rank", i32),
        _dev(send_token_idx, "send_token_idx", i32), _dev(bad_id_count, "bad_id_count", i32, optional=True),
        _dev(put_offset, "put_offset", i32), _dev(recv_count, "recv_count", i32),
        _dev(recv_base, "recv_base", i32), _dev(recv_token_per_expert, "recv_token_per_expert", i32),
        _dev(recv_x, "recv_x"), recv_x.numel() * recv_x.element_size(), _dev(workspace, "workspace"),
        workspace.numel() * workspace.element_size(), _stream(stream)))


def moe_deq_swiglu_quant(acc: torch.Tensor, weight_scale: torch.Tensor, token_scale: torch.Tensor,
                         out: torch.Tensor, token_scale_stride: int = 4, rows: Optional[int] = None,
                         stream=None) -> None:
    """Expert-side epilogue: acc int32 [rows, 2n], weight_scale float32 [2n];
    the float scale of row m is read at byte m * token_scale_stride of
    ``token_scale`` (a float32 [rows] tensor with stride 4, or the int8
    receive buffer at its inverse-scale byte, see ``token_scales_of``); out is
    a uint8 buffer of at least rows * moe_recv_row_bytes(n, MOE_INT8_ROWSCALE)
    bytes, written as int8 rows (codes, inverse scale at byte align32(n))."""
    if acc.dim() != 2 or acc.shape[1] % 2:
        raise ValueError("acc must be [rows, 2n]")
    n_rows = acc.shape[0] if rows is None else rows
    n = acc.shape[1] // 2
    if weight_scale.numel() != 2 * n:
        raise ValueError("weight_scale must hold 2n floats")
    if n_rows > acc.shape[0]:
        raise ValueError("rows exceeds acc's rows")
    if not token_scale.is_cuda:
        raise ValueError("token_scale must be a device tensor")
    _need_scales(token_scale, n_rows, token_scale_stride)
    _check("moe_deq_swiglu_quant", _lib.moe_deq_swiglu_quant(
        _dev(acc, "acc", torch.int32), n_rows, n, _dev(weight_scale, "weight_scale", torch.float32),
        token_scale.data_ptr(), token_scale_stride, _dev(out, "out"), out.numel() * out.element_size(),
        _stream(stream)))


def moe_grouped_gemm_i8(a: torch.Tensor, a_row_bytes: int, rows: int, k: int,
                        group_count: torch.Tensor, w: torch.Tensor, out: torch.Tensor,
                        stream=None) -> None:
    """First expert matmul: ``a`` is a device byte buffer (uint8 or int8,
    e.g. the int8 receive buffer) whose row m starts at byte m * a_row_bytes
    and holds k int8 codes; group_count int32 [groups] (device) gives each
    expert's rows in order; w int8 [groups, n, k]; out int32 [rows, n] gets
    out[m][j] = sum_i a[m][i] * w[g][j][i] for the rows of expert g (rows of
    no expert are not written)."""
    if w.dim() != 3 or w.shape[2] != k or w.dtype not in (torch.int8, torch.uint8):
        raise ValueError("w must be int8 [groups, n, k]")
    groups, n = w.shape[0], w.shape[1]
    if group_count.numel() != groups:
        raise ValueError("group_count must hold one count per group")
    if a.dtype not in (torch.int8, torch.uint8):
        raise ValueError("a must be a byte buffer")
    if rows > 0 and a.numel() < (rows - 1) * a_row_bytes + k:
        raise ValueError("a is smaller than (rows - 1) * a_row_bytes + k bytes")
    _check("moe_grouped_gemm_i8", _lib.moe_grouped_gemm_i8(
        _dev(a, "a"), a_row_bytes, rows, k, _dev(group_count, "group_count", torch.int32), groups,
        _dev(w, "w"), n, _dev(out, "out", torch.int32), out.numel() * out.element_size(),
        _stream(stream)))


def moe_gemm_swiglu_quant_workspace_bytes(rows: int, n: int) -> int:
    out = _SZ(0)
    _check("moe_gemm_swiglu_quant_workspace_bytes",
           _lib.moe_gemm_swiglu_quant_workspace_bytes(rows, n, ctypes.byref(out)))
    return out.value


def moe_grouped_gemm_swiglu_quant_i8(a: torch.Tensor, a_row_bytes: int, rows: int, k: int,
                                     group_count: torch.Tensor, w: torch.Tensor, weight_scale: torch.Tensor,
                                     token_scale: torch.Tensor, out: torch.Tensor, workspace: torch.Tensor,
                                     token_scale_stride: int = 4, stream=None) -> None:
    """The first expert matmul with its epilogue fused: ``a``, a_row_bytes,
    rows, k and group_count as for ``moe_grouped_gemm_i8``; w int8 [groups,
    2n, k] (gate rows, then up rows); weight_scale float32 [groups, 2n];
    token_scale and token_scale_stride as for ``moe_deq_swiglu_quant``; out a
    uint8 buffer of int8 rows (moe_recv_row_bytes(n, MOE_INT8_ROWSCALE) bytes
    each; rows no expert owns are not written); workspace a device buffer of
    moe_gemm_swiglu_quant_workspace_bytes(rows, n) bytes."""
    if w.dim() != 3 or w.shape[2] != k or w.shape[1] % 2 or w.dtype not in (torch.int8, torch.uint8):
        raise ValueError("w must be int8 [groups, 2n, k]")
    groups, n = w.shape[0], w.shape[1] // 2
    if group_count.numel() != groups:
        raise ValueError("group_count must hold one count per group")
    if weight_scale.numel() != groups * 2 * n:
        raise ValueError("weight_scale must hold groups * 2n floats")
    if a.dtype not in (torch.int8, torch.uint8):
        raise ValueError("a must be a byte buffer")
    if rows > 0 and a.numel() < (rows - 1) * a_row_bytes + k:
        raise ValueError("a is smaller than (rows - 1) * a_row_bytes + k bytes")
    if not token_scale.is_cuda:
        raise ValueError("token_scale must be a device tensor")
    _need_scales(token_scale, rows, token_scale_stride)
    _check("moe_grouped_gemm_swiglu_quant_i8", _lib.moe_grouped_gemm_swiglu_quant_i8(
        _dev(a, "a"), a_row_bytes, rows, k, _dev(group_count, "group_count", torch.int32), groups,
        _dev(w, "w"), n, _dev(weight_scale, "weight_scale", torch.float32), token_scale.data_ptr(),
        token_scale_stride, _dev(out, "out"), out.numel() * out.element_size(), _dev(workspace, "workspace"),
        workspace.numel() * workspace.element_size(), _stream(stream)))


def token_scales_of(recv_x: torch.Tensor, hidden: int) -> Tuple[torch.Tensor, int]:
    """(base tensor view, byte stride) that addresses the inverse scales of an
    int8 receive buffer in place, for ``moe_deq_swiglu_quant``."""
    rb = moe_recv_row_bytes(hidden, MOE_INT8_ROWSCALE)
    off = (hidden + 31) // 32 * 32
    return recv_x[off:], rb


class EpBuffers:
    """Device buffers of one pipeline shape, allocated once through torch.

    ``run`` enqueues layout -> notify -> dispatch -> combine on the current
    stream and allocates nothing."""

    def __init__(self, bs: int, hidden: int, topk: int, expert_num_per_rank: int, rank_size: int,
                 x_dtype: torch.dtype = torch.bfloat16, quant_int8: bool = True,
                 out_dtype: Optional[torch.dtype] = None, device="cuda"):
        e = expert_num_per_rank * rank_size
        self.bs, self.hidden, self.topk = bs, hidden, topk
        self.epr, self.ranks, self.num_experts = expert_num_per_rank, rank_size, e
        self.quant_int8 = quant_int8
        self.x_dtype = x_dtype
        self.recv_type = MOE_INT8_ROWSCALE if quant_int8 else dtype_code(x_dtype)
        self.row_bytes = moe_recv_row_bytes(hidden, self.recv_type)
        i32 = dict(dtype=torch.int32, device=device)
        self.token_per_expert = torch.zeros(e, **i32)
        self.token_per_rank = torch.zeros(rank_size, **i32)
        self.send_token_idx = torch.zeros((bs, topk), **i32)
        self.bad_id_count = torch.zeros(1, **i32)
        ws = moe_layout_workspace_bytes(bs, topk, e)
        self.workspace = torch.zeros(max(ws, 4) // 4, **i32)
        self.put_offset = torch.zeros(e, **i32)
        self.recv_count = torch.zeros(rank_size, **i32)
        self.recv_base = torch.zeros(rank_size, **i32)
        self.recv_token_per_expert = torch.zeros(e, **i32)
        self.recv_x = torch.zeros(bs * topk * self.row_bytes, dtype=torch.uint8, device=device)
        self.out = torch.zeros((bs, hidden), dtype=out_dtype or x_dtype, device=device)

    def layout(self, topk_idx, stream=None):
        moe_layout(topk_idx, self.epr, self.ranks, self.token_per_expert, self.token_per_rank,
                   self.send_token_idx, self.bad_id_count, self.workspace, stream)

    def notify(self, stream=None):
        moe_notify(self.token_per_expert, self.epr, self.ranks, self.put_offset, self.recv_count,
                   self.recv_base, self.recv_token_per_expert, stream)

    def dispatch(self, x, topk_idx, stream=None):
        moe_dispatch(x, topk_idx, self.send_token_idx, self.put_offset, self.recv_base, self.epr,
                     self.ranks, self.quant_int8, self.recv_x, stream)

    def combine(self, topk_idx, topk_w, stream=None):
        moe_combine(self.recv_x, self.recv_type, self.hidden, topk_idx, topk_w, self.send_token_idx,
                    self.put_offset, self.recv_base, self.epr, self.ranks, self.out, stream)

    def layout_notify_dispatch(self, x, topk_idx, stream=None):
        moe_layout_notify_dispatch(x, topk_idx, self.epr, self.ranks, self.quant_int8, self.token_per_expert,
                                   self.token_per_rank, self.send_token_idx, self.bad_id_count,
                                   self.put_offset, self.recv_count, self.recv_base,
                                   self.recv_token_per_expert, self.recv_x, self.workspace, stream)

    def run(self, x, topk_idx, topk_w, stream=None, fused: bool = False):
        if fused:
            self.layout_notify_dispatch(x, topk_idx, stream)
        else:
            self.layout(topk_idx, stream)
            self.notify(stream)
            self.dispatch(x, topk_idx, stream)
        self.combine(topk_idx, topk_w, stream)
        return self.out


class EpMultiBuffers:
    """Device buffers for several source ranks sharing one receive buffer
    (one GPU standing in for the sources of an expert-parallel group).

    Source s has ``sizes[s]`` tokens; each source keeps its own layout
    outputs and combine output, the notify outputs and the receive buffer
    (sum of the sources' bs * topk rows) are shared.  ``run`` enqueues every
    source's layout, one notify over the [S, E] count matrix, every source's
    dispatch, then every source's combine, on one stream."""

    def __init__(self, sizes, hidden: int, topk: int, expert_num_per_rank: int, rank_size: int,
                 x_dtype: torch.dtype = torch.bfloat16, quant_int8: bool = True,
                 out_dtype: Optional[torch.dtype] = None, device="cuda"):
        sizes = [int(b) for b in sizes]
        if not sizes:
            raise ValueError("at least one source")
        e = expert_num_per_rank * rank_size
        self.sizes, self.hidden, self.topk = sizes, hidden, topk
        self.num_src = len(sizes)
        self.epr, self.ranks, self.num_experts = expert_num_per_rank, rank_size, e
        self.quant_int8 = quant_int8
        self.recv_type = MOE_INT8_ROWSCALE if quant_int8 else dtype_code(x_dtype)
        self.row_bytes = moe_recv_row_bytes(hidden, self.recv_type)
        i32 = dict(dtype=torch.int32, device=device)
        self.token_per_expert = torch.zeros((self.num_src, e), **i32)
        self.token_per_rank = torch.zeros((self.num_src, rank_size), **i32)
        self.send_token_idx = [torch.zeros((b, topk), **i32) for b in sizes]
        self.bad_id_count = torch.zeros(self.num_src, **i32)
        # one layout workspace per source, so the sources' layouts may run
        # concurrently on different streams
        self.workspace = [torch.zeros(max(moe_layout_workspace_bytes(b, topk, e), 4) // 4, **i32)
                          for b in sizes]
        self.put_offset = torch.zeros((e, self.num_src), **i32)
        self.recv_count = torch.zeros(rank_size, **i32)
        self.recv_base = torch.zeros(rank_size, **i32)
        self.recv_token_per_expert = torch.zeros(e, **i32)
        self.total_rows = sum(sizes) * topk
        self.recv_x = torch.zeros(self.total_rows * self.row_bytes, dtype=torch.uint8, device=device)
        self.out = [torch.zeros((b, hidden), dtype=out_dtype or x_dtype, device=device) for b in sizes]

    def layout(self, src: int, topk_idx, stream=None):
        moe_layout(topk_idx, self.epr, self.ranks, self.token_per_expert[src], self.token_per_rank[src],
                   self.send_token_idx[src], self.bad_id_count[src:src + 1], self.workspace[src], stream)

    def notify(self, stream=None):
        moe_notify_multi(self.token_per_expert, self.epr, self.ranks, self.put_offset, self.recv_count,
                         self.recv_base, self.recv_token_per_expert, stream)

    def dispatch(self, src: int, x, topk_idx, stream=None):
        moe_dispatch_src(x, topk_idx, self.send_token_idx[src], self.put_offset, self.recv_base, self.epr,
                         self.ranks, src, self.quant_int8, self.recv_x, stream)

    def combine(self, src: int, topk_idx, topk_w, stream=None):
        moe_combine_src(self.recv_x, self.recv_type, self.hidden, topk_idx, topk_w, self.send_token_idx[src],
                        self.put_offset, self.recv_base, self.epr, self.ranks, src, self.out[src], stream)

    def run(self, xs, idxs, ws, stream=None):
        for src in range(self.num_src):
            self.layout(src, idxs[src], stream)
        self.notify(stream)
        for src in range(self.num_src):
            self.dispatch(src, xs[src], idxs[src], stream)
        for src in range(self.num_src):
            self.combine(src, idxs[src], ws[src], stream)
        return self.out
