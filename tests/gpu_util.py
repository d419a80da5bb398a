"""Helpers for the GPU tests: move generated inputs to the device, run the HIP
library's stages through the C ABI (via the thin binding), and bring the
results back in the oracle's canonical form."""

from __future__ import annotations

import sys
from typing import Dict, Optional

import numpy as np
import torch


def log(msg: str) -> None:
    """Name the case before a GPU step, so a failing run says what it ran."""
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def align32(v: int) -> int:
    return (v + 31) // 32 * 32


def dev_i32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def dev_f32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def dev_half(bits: np.ndarray, kind: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).cuda()
    return t.view(torch.bfloat16 if kind == "bf16" else torch.float16)


def host_bits(t: torch.Tensor) -> np.ndarray:
    """16-bit tensor -> uint16 patterns on the host."""
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def int8_row_bytes(hidden: int) -> int:
    """Bytes of an int8 receive row, as the library sizes it (moe_recv_row_bytes)."""
    import combine_moe_layout_03_amd as M

    return M.moe_recv_row_bytes(hidden, M.MOE_INT8_ROWSCALE)


def unpack_recv(recv_x: torch.Tensor, hidden: int, kind: str) -> Dict[str, np.ndarray]:
    """Receive buffer bytes -> canonical rows (passthrough) or codes + inv.

    Layout (include/moe_ep.h): passthrough rows are 2*hidden bytes; int8 rows
    are moe_recv_row_bytes(hidden) bytes with the codes first and the float
    inverse scale at byte align32(hidden)."""
    raw = recv_x.cpu().numpy()
    if kind == "int8":
        rb = int8_row_bytes(hidden)
        m = raw.reshape(-1, rb)
        codes = np.ascontiguousarray(m[:, :hidden]).view(np.int8)
        off = align32(hidden)
        inv = np.ascontiguousarray(m[:, off:off + 4]).view(np.float32).reshape(-1)
        return dict(codes=codes, inv=inv)
    m = raw.reshape(-1, 2 * hidden)
    return dict(rows=np.ascontiguousarray(m).view(np.uint16))


def pack_recv(canon: Dict[str, np.ndarray], hidden: int, kind: str) -> np.ndarray:
    """Canonical receive rows -> the library's byte layout (for feeding the
    GPU combine an oracle-made buffer)."""
    if kind == "int8":
        rows = canon["codes"].shape[0]
        rb = int8_row_bytes(hidden)
        m = np.zeros((rows, rb), np.uint8)
        m[:, :hidden] = canon["codes"].view(np.uint8)
        off = align32(hidden)
        m[:, off:off + 4] = canon["inv"].astype(np.float32).view(np.uint8).reshape(rows, 4)
        return m.reshape(-1)
    return np.ascontiguousarray(canon["rows"]).view(np.uint8).reshape(-1)


class GpuRun:
    """One pass of the four stages on the GPU for a workload."""

    def __init__(self, w, quant: bool, out_kind: Optional[str] = None):
        import combine_moe_layout_03_amd as M

        self.M = M
        self.w = w
        self.quant = quant
        self.kind = w.x_dtype
        self.out_kind = out_kind or w.x_dtype
        out_dtype = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}[self.out_kind]
        x_dtype = torch.bfloat16 if self.kind == "bf16" else torch.float16
        self.buf = M.EpBuffers(w.bs, w.hidden, w.topk, w.expert_num_per_rank, w.rank_size,
                               x_dtype=x_dtype, quant_int8=quant, out_dtype=out_dtype)
        self.x = dev_half(w.x, self.kind)
        self.idx = dev_i32(w.topk_idx)
        self.wts = dev_f32(w.topk_w)

    def layout(self):
        self.buf.layout(self.idx)
        return self

    def notify(self):
        self.buf.notify()
        return self

    def dispatch(self):
        self.buf.dispatch(self.x, self.idx)
        return self

    def combine(self):
        self.buf.combine(self.idx, self.wts)
        return self

    def run_all(self, fused: bool = False):
        if fused:
            self.buf.layout_notify_dispatch(self.x, self.idx)
            return self.combine()
        return self.layout().notify().dispatch().combine()

    def host(self) -> Dict[str, object]:
        torch.cuda.synchronize()
        b = self.buf
        res = dict(
            token_per_expert=b.token_per_expert.cpu().numpy(),
            token_per_rank=b.token_per_rank.cpu().numpy(),
            send_token_idx=b.send_token_idx.cpu().numpy(),
            bad=int(b.bad_id_count.cpu().item()),
            put_offset=b.put_offset.cpu().numpy(),
            recv_count=b.recv_count.cpu().numpy(),
            recv_base=b.recv_base.cpu().numpy(),
            recv_token_per_expert=b.recv_token_per_expert.cpu().numpy(),
            recv=unpack_recv(b.recv_x, self.w.hidden, "int8" if self.quant else self.kind),
        )
        if self.out_kind == "fp32":
            res["out"] = b.out.cpu().numpy()
        else:
            res["out"] = host_bits(b.out)
        return res
