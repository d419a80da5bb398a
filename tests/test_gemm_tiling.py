"""CPU check of the grouped GEMM's grid and indexing (no GPU needed).

Replays, on the host, how the launch maps workgroups to (expert, row tile,
column tile) through the prefix sum over the per-expert counts, and which
rows, weight rows and output elements each workgroup touches, for the tile
shape the library launches (read from its headers).  Asserts that every
load stays inside the buffers the C ABI documents, and that every output
element of a row some expert owns is written exactly once and no other
element is written.
"""

import os
import re

import numpy as np
import pytest

import workloads as W

CSRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                    "combine_moe_layout_03_amd", "csrc")


def _shape():
    """Tile, waves, stage bytes and tile-order block of the library's GEMM, from its headers."""
    h = open(os.path.join(CSRC, "gemm.h")).read()
    tm, tn = map(int, re.search(r"kGemmTileM = (\d+), kGemmTileN = (\d+);", h).groups())
    wm, wn = map(int, re.search(r"kGemmWavesM = (\d+), kGemmWavesN = (\d+);", h).groups())
    groups_c = int(re.search(r"kGemmXcdColGroups = (\d+);", h).group(1))
    xrows = int(re.search(r"kGemmXcdRows = (\d+);", h).group(1))
    sel = open(os.path.join(CSRC, "select.h")).read()
    sk = int(re.search(r"kGemmStageK = (\d+);", sel).group(1))
    return tm, tn, wm, wn, sk, groups_c, xrows


def _tile_of(b, n_tiles, groups_c, xrows):
    """(row slot, column tile) of workgroup b, as the kernel maps it."""
    if n_tiles % groups_c == 0:
        x, l = b % 8, b // 8
        cols = n_tiles // groups_c
        per_block = xrows * cols
        blk = 2 * (l // per_block) + x // groups_c
        w = l % per_block
        return blk * xrows + w // cols, (x % groups_c) * cols + w % cols
    return divmod(b, n_tiles)


def _slot(counts, rows, slot, tm):
    """(expert, first row, end row) of a row slot, or None: the kernel's
    wave-wide prefix sums over chunks of 64 experts."""
    row_base = tile_base = 0
    found = None
    for g0 in range(0, len(counts), 64):
        c = np.array([max(int(v), 0) for v in counts[g0:g0 + 64]], np.int64)
        incl = np.cumsum(c)
        s = np.minimum(row_base + incl - c, rows)
        e = np.minimum(row_base + incl, rows)
        tiles = (e - s + tm - 1) // tm
        t0 = tile_base + np.cumsum(tiles) - tiles
        for lane in range(c.size):
            if t0[lane] <= slot < t0[lane] + tiles[lane]:
                assert found is None
                found = (g0 + lane, int(s[lane] + (slot - t0[lane]) * tm), int(e[lane]))
        row_base = min(row_base + int(incl[-1]), rows)
        tile_base += int(tiles.sum())
        if tile_base > slot:
            break
    return found


@pytest.mark.parametrize("rows,k,n,counts", [
    (1000, 320, 300, "owned:900:5"),
    (830, 128, 128, [0, 300, -5, 1, 0, 517]),
    (3, 16, 16, [0, 1, 0]),
    (2000, 64, 128, "owned:2000:130"),
    (1000, 96, 48, [400, 400, 400]),
    (257, 48, 1, [257]),
    (4096, 7168, 512, "owned:4096:16"),
    # 4, 8 and 28 column tiles: the XCD-aware order (whole blocks of row slots)
    (1000, 320, 1024, [0, 300, -5, 1, 0, 517]),
    (2000, 64, 2048, "owned:1990:130"),
    (300, 144, 7168, [100, 0, 200]),
    (900, 1008, 520, "owned:880:4"),
    (700, 384, 600, "owned:690:3"),
    (600, 1536, 260, [300, 290]),
    (300, 1392, 256, [300]),
    # counts whose sum passes 2^31: the slot search sums in 64 bits
    (300, 128, 512, [2 ** 31 - 1, 2 ** 31 - 1, 5]),
])
def test_grid_covers_owned_outputs_once_and_loads_stay_in_bounds(rows, k, n, counts):
    tm, tn, wm, wn, sk, groups_c, xrows = _shape()
    if isinstance(counts, str):
        _, owned, groups = counts.split(":")
        pick = (W.u64(1, 0, int(owned)) % np.uint64(int(groups))).astype(np.int64)
        counts = np.bincount(pick, minlength=int(groups))
    counts = list(counts)
    stride = (k + 31) // 32 * 32 + 32
    waves = wm * wn
    pieces = sk // 16
    rows_per_load = 64 // pieces
    lane = np.arange(64)
    slots = (rows + tm - 1) // tm + len(counts)
    n_tiles = (n + tn - 1) // tn
    if n_tiles % groups_c == 0:
        slots = (slots + 2 * xrows - 1) // (2 * xrows) * (2 * xrows)
    written = np.zeros((rows, n), np.int32)
    seen = set()
    a_end, w_end = (rows - 1) * stride + k, len(counts) * n * k
    stages = (k + sk - 1) // sk
    for b in range(slots * n_tiles):
        slot, col_tile = _tile_of(b, n_tiles, groups_c, xrows)
        assert 0 <= slot < slots and 0 <= col_tile < n_tiles and (slot, col_tile) not in seen
        seen.add((slot, col_tile))
        hit = _slot(counts, rows, slot, tm)
        if hit is None:
            continue
        g, row0, row_end = hit
        assert 0 <= row0 < row_end <= rows
        col0 = col_tile * tn
        for wave in range(waves):
            # every stage the kernel loads (the first, the last, and the last
            # again for the re-loads past the end)
            for s in sorted({0, stages - 1, stages}):
                k0 = min(s, stages - 1) * sk
                for q in range(tm // rows_per_load // waves):
                    r = rows_per_load * (q * waves + wave) + lane // pieces
                    p = (lane % pieces) ^ ((r // (16 // pieces)) & (pieces - 1))
                    row = np.minimum(row0 + r, row_end - 1)
                    addr = row * stride + np.where(k0 + p * 16 < k, p * 16 + k0, 0)
                    assert (addr >= 0).all() and (addr + 16 <= a_end).all()
                for q in range(tn // rows_per_load // waves):
                    r = rows_per_load * (q * waves + wave) + lane // pieces
                    p = (lane % pieces) ^ ((r // (16 // pieces)) & (pieces - 1))
                    col = np.minimum(col0 + r, n - 1)
                    addr = (g * n + col) * k + np.where(k0 + p * 16 < k, p * 16 + k0, 0)
                    assert (addr >= 0).all() and (addr + 16 <= w_end).all()
            wr, wc = wave // wn, wave % wn
            for i in range(tm // wm // 16):
                for j in range(tn // wn // 16):
                    col = col0 + wc * (tn // wn) + j * 16 + lane % 16
                    for r in range(4):
                        row = row0 + wr * (tm // wm) + i * 16 + (lane // 16) * 4 + r
                        m = (row < row_end) & (col < n)
                        np.add.at(written, (row[m], col[m]), 1)
    assert len(seen) == slots * n_tiles
    owner = np.full(rows, -1)
    start = 0
    for g, c in enumerate(counts):
        c = max(int(c), 0)
        owner[start:min(start + c, rows)] = g
        start += c
    assert (written[owner >= 0] == 1).all() and (written[owner < 0] == 0).all()
