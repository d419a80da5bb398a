"""Checks that pin the CPU oracle to things other than itself.

Each ``check_*`` function takes an ``oracle.Oracle`` and raises AssertionError
(or OracleError) when the oracle disagrees with the pin.  The oracle tests run
them on the real build; the mutation tests run them on deliberately broken
builds and expect a failure.  The pins are:

* brute force of the layout definition on every tiny input;
* equivalence with library routines (numpy stable argsort, cumsum, rint) and
  with torch / numpy dtype conversions (exhaustive on 16-bit patterns);
* the hand-worked rows in tests/golden/ (quantiser ties, scale values,
  order-sensitive combine sums, output rounding);
* exact rational arithmetic for the quantiser's scale, inverse and codes, and
  float64 error bounds for the combine sums;
* for the first expert matmul, numpy's int64 matrix product per expert,
  closed forms of constant and extreme operands, and column-picking weights.
"""

from __future__ import annotations

import itertools
import json
import os
from fractions import Fraction
from typing import Dict, Tuple

import numpy as np

import workloads as W

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# --------------------------------------------------------------------------
# exact helpers
# --------------------------------------------------------------------------

def f32_bits(x) -> int:
    return int(np.array([x], dtype=np.float32).view(np.uint32)[0])


def f32_from_bits(u: int) -> np.float32:
    return np.array([u], dtype=np.uint32).view(np.float32)[0]


def round_f32(q: Fraction) -> Fraction:
    """Round an exact rational to the nearest binary32 value, ties to even.

    Covers normal and subnormal results; overflow is not needed here."""
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    # now 2^(e-1) <= a < 2^(e+1); settle e so that 2^e <= a < 2^(e+1)
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)
    ulp = Fraction(2) ** (e - 23)
    m = a / ulp
    n = m.numerator // m.denominator
    rem = m - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return sign * n * ulp


def round_int_even(q: Fraction) -> int:
    n = q.numerator // q.denominator  # floor
    rem = q - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return n


def frac(x) -> Fraction:
    return Fraction(float(np.float32(x)))


def to_bits16(values, kind: str) -> np.ndarray:
    """Exact float -> 16-bit patterns; fails if a value is not representable."""
    import torch

    v = np.asarray(values, dtype=np.float64)
    if kind == "bf16":
        t = torch.tensor(v, dtype=torch.float64).to(torch.bfloat16)
        back = t.to(torch.float64).numpy()
        bits = t.view(torch.int16).numpy().view(np.uint16)
    else:
        h = v.astype(np.float16)
        back = h.astype(np.float64)
        bits = h.view(np.uint16)
    assert np.array_equal(back, v), "fixture value is not exact in " + kind
    return np.ascontiguousarray(bits)


def widen16(bits: np.ndarray, kind: str) -> np.ndarray:
    """16-bit patterns -> float32 through numpy/torch (library conversions)."""
    import torch

    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    if kind == "bf16":
        return torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    return bits.view(np.float16).astype(np.float32)


def load_golden(name: str) -> dict:
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# --------------------------------------------------------------------------
# conversions
# --------------------------------------------------------------------------

def _same_f32(a: np.ndarray, b: np.ndarray) -> bool:
    a = np.asarray(a, np.float32)
    b = np.asarray(b, np.float32)
    na, nb = np.isnan(a), np.isnan(b)
    if not np.array_equal(na, nb):
        return False
    return np.array_equal(a[~na].view(np.uint32), b[~nb].view(np.uint32))


def _f32_probe_values() -> np.ndarray:
    """Random bit patterns over every exponent plus hand-picked edges and ties."""
    rng = np.random.default_rng(12345)
    u = rng.integers(0, 2 ** 32, size=400_000, dtype=np.uint64).astype(np.uint32)
    # ties and near-ties for bf16 (low half 0x8000 +- 1) and for fp16 (13 low bits)
    hi = rng.integers(0, 2 ** 16, size=20_000, dtype=np.uint64).astype(np.uint32) << np.uint32(16)
    ties_bf = np.concatenate([hi | np.uint32(0x8000), hi | np.uint32(0x7FFF), hi | np.uint32(0x8001)])
    base = rng.integers(0, 2 ** 19, size=20_000, dtype=np.uint64).astype(np.uint32) << np.uint32(13)
    ties_h = np.concatenate([base | np.uint32(0x1000), base | np.uint32(0x0FFF), base | np.uint32(0x1001)])
    # the fp16 range [2^-25, 65520] on a dense grid
    exps = np.arange(-26, 17)
    grid = []
    for e in exps:
        m = rng.random(2000) + 1.0
        grid.append((m * 2.0 ** e).astype(np.float32))
    edges = np.array([0.0, -0.0, 65504.0, 65519.99, 65520.0, 65536.0, 6.1035156e-05, 5.9604645e-08,
                      2.9802322e-08, 2.9802326e-08, 1e-45, 3.4028235e38, -3.4028235e38,
                      np.inf, -np.inf], dtype=np.float32)
    vals = np.concatenate([u.view(np.float32), ties_bf.view(np.float32), ties_h.view(np.float32),
                           np.concatenate(grid), -np.concatenate(grid), edges])
    return vals.astype(np.float32)


def check_conversions(orc) -> None:
    import torch

    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    # widening: exhaustive over all 65536 patterns
    ref_bf = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    assert _same_f32(orc.bf16_to_f32(bits), ref_bf), "bf16 -> f32 differs from torch"
    ref_h = bits.view(np.float16).astype(np.float32)
    assert _same_f32(orc.f16_to_f32(bits), ref_h), "f16 -> f32 differs from numpy"
    # narrowing with round-half-even
    vals = _f32_probe_values()
    finite = ~np.isnan(vals)
    got_bf = orc.f32_to_bf16(vals)
    ref_bf16 = torch.from_numpy(vals.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got_bf[finite], ref_bf16[finite]), "f32 -> bf16 differs from torch"
    got_h = orc.f32_to_f16(vals)
    with np.errstate(over="ignore"):
        ref_h16 = vals.astype(np.float16).view(np.uint16)
    assert np.array_equal(got_h[finite], ref_h16[finite]), "f32 -> f16 differs from numpy"
    nan_in = np.array([np.nan, -np.nan], dtype=np.float32)
    assert np.all(np.isnan(widen16(orc.f32_to_bf16(nan_in), "bf16")))
    assert np.all(np.isnan(widen16(orc.f32_to_f16(nan_in), "fp16")))


# --------------------------------------------------------------------------
# layout (stage 1) and notify (stage 2)
# --------------------------------------------------------------------------

def brute_layout(idx: np.ndarray, epr: int, ranks: int):
    """The definition itself, by counting earlier equal entries (O(n^2))."""
    flat = [int(v) for v in idx.reshape(-1)]
    e_num = epr * ranks
    slots, bad = [], 0
    for i, e in enumerate(flat):
        if 0 <= e < e_num:
            slots.append(sum(1 for p in flat[:i] if p == e))
        else:
            slots.append(-1)
            bad += 1
    cnt = [sum(1 for p in flat if p == e) for e in range(e_num)]
    per_rank = [sum(cnt[r * epr:(r + 1) * epr]) for r in range(ranks)]
    return cnt, per_rank, slots, bad


def sort_layout(idx: np.ndarray, epr: int, ranks: int):
    """Layout through numpy's stable argsort: the receive order of a stable
    sort of the flat entries by expert id, minus each expert's start."""
    flat = idx.reshape(-1).astype(np.int64)
    e_num = epr * ranks
    valid = (flat >= 0) & (flat < e_num)
    keys = np.where(valid, flat, e_num)
    order = np.argsort(keys, kind="stable")
    pos = np.empty(flat.size, np.int64)
    pos[order] = np.arange(flat.size)
    cnt = np.bincount(flat[valid], minlength=e_num)
    start = np.concatenate([[0], np.cumsum(cnt)])
    slot = np.where(valid, pos - start[np.minimum(keys, e_num)], -1)
    return cnt, cnt.reshape(ranks, epr).sum(axis=1), slot.reshape(idx.shape), int((~valid).sum())


def check_layout_bruteforce(orc) -> None:
    """Every input with bs <= 3, k <= 2, E <= 4, ids in [-1, E] (bad ids included)."""
    shapes = [(0, 1), (1, 1), (1, 2), (2, 1), (2, 2), (3, 1), (3, 2)]
    for e_num, ranks in [(1, 1), (2, 1), (2, 2), (3, 3), (4, 2), (4, 4)]:
        epr = e_num // ranks
        values = list(range(-1, e_num + 1))
        for bs, k in shapes:
            n = bs * k
            if n > 4 and e_num == 4 and ranks == 4:
                continue  # (4, 2) already covers E = 4 at full size
            for combo in itertools.product(values, repeat=n):
                idx = np.array(combo, dtype=np.int32).reshape(bs, k)
                got = orc.layout(idx, epr, ranks)
                cnt, per_rank, slots, bad = brute_layout(idx, epr, ranks)
                assert got["token_per_expert"].tolist() == cnt, (idx.tolist(), "counts")
                assert got["token_per_rank"].tolist() == per_rank, (idx.tolist(), "per rank")
                assert got["send_token_idx"].reshape(-1).tolist() == slots, (idx.tolist(), "slots")
                assert got["bad"] == bad, (idx.tolist(), "bad")


def check_layout_sort(orc, idx: np.ndarray, epr: int, ranks: int) -> None:
    got = orc.layout(idx, epr, ranks)
    cnt, per_rank, slot, bad = sort_layout(idx, epr, ranks)
    assert np.array_equal(got["token_per_expert"], cnt), "counts vs bincount"
    assert np.array_equal(got["token_per_rank"], per_rank), "per-rank counts"
    assert np.array_equal(got["send_token_idx"], slot), "slots vs stable argsort"
    assert got["bad"] == bad


def check_layout_invariants(orc, idx: np.ndarray, epr: int, ranks: int) -> None:
    got = orc.layout(idx, epr, ranks)
    e_num = epr * ranks
    flat = idx.reshape(-1)
    slot = got["send_token_idx"].reshape(-1)
    cnt = got["token_per_expert"]
    valid = (flat >= 0) & (flat < e_num)
    assert cnt.sum() == flat.size - got["bad"], "sum of counts = entries - bad"
    assert np.all(slot[~valid] == -1)
    for e in np.unique(flat[valid]):
        s = slot[flat == e]
        assert np.array_equal(s, np.arange(cnt[e])), f"slots of expert {e} are 0..cnt-1 in order"
    assert np.array_equal(got["token_per_rank"], cnt.reshape(ranks, epr).sum(1))


def check_notify(orc, tpe: np.ndarray, epr: int, ranks: int) -> None:
    """Against numpy cumsum: the global exclusive scan G over experts gives
    recvBase[r] = G[r*EPR] and putOffset[e] = G[e] - G[rank(e)*EPR]."""
    tpe = np.asarray(tpe, np.int64)
    got = orc.notify(tpe.astype(np.int32), epr, ranks)
    g = np.concatenate([[0], np.cumsum(tpe)])
    e = np.arange(epr * ranks)
    assert np.array_equal(got["recv_base"], g[np.arange(ranks) * epr]), "recvBase"
    assert np.array_equal(got["put_offset"], g[e] - g[(e // epr) * epr]), "putOffset"
    assert np.array_equal(got["recv_count"], tpe.reshape(ranks, epr).sum(1)), "recvCount"
    assert np.array_equal(got["recv_token_per_expert"], tpe), "recvTokenPerExpert"
    # invariants: first expert of each rank at 0, regions tile [0, total)
    assert np.all(got["put_offset"].reshape(ranks, epr)[:, 0] == 0)
    total = int(tpe.sum())
    assert int(got["recv_base"][-1]) + int(got["recv_count"][-1]) == total


def check_notify_multi_golden(orc) -> None:
    """Hand-worked count matrices of several sources (golden/notify_multi.json)."""
    g = load_golden("notify_multi.json")
    for c in g["cases"]:
        got = orc.notify_multi(np.array(c["counts"], np.int32), c["epr"], c["ranks"])
        for key in ("put_offset", "recv_count", "recv_base", "recv_token_per_expert"):
            assert np.array_equal(got[key], np.array(c[key], np.int32)), (c["name"], key)


def check_notify_multi_single_source(orc, tpe: np.ndarray, epr: int, ranks: int) -> None:
    """With one source the multi-source notify is the single-source one
    (itself pinned against numpy cumsum)."""
    one = orc.notify(tpe, epr, ranks)
    multi = orc.notify_multi(np.asarray(tpe, np.int32).reshape(1, -1), epr, ranks)
    assert np.array_equal(multi["put_offset"][:, 0], one["put_offset"])
    for key in ("recv_count", "recv_base", "recv_token_per_expert"):
        assert np.array_equal(multi[key], one[key]), key


def multi_rows(idxs, layouts, no, epr: int):
    """Receive row of every valid entry of every source, from the oracle's
    outputs: recvBase[e / EPR] + putOffset[e][s] + slot_s[t, j]."""
    out = []
    for src, (idx, lay) in enumerate(zip(idxs, layouts)):
        idx = np.asarray(idx, np.int64)
        e_num = no["put_offset"].shape[0]
        valid = (idx >= 0) & (idx < e_num)
        ec = np.where(valid, idx, 0)
        rows = no["recv_base"][ec // epr].astype(np.int64) + no["put_offset"][ec, src] + \
            lay["send_token_idx"].astype(np.int64)
        out.append(np.where(valid, rows, -1))
    return out


def check_multi_receive_order(orc, idxs, epr: int, ranks: int) -> None:
    """Library-routine pin of the multi-source layout: sorting every valid
    (source, token, k) entry by the key (expert, source, token, k) with
    numpy's lexsort gives each entry's receive row (its position), and the
    rows tile [0, total) exactly once."""
    lays = [orc.layout(idx, epr, ranks) for idx in idxs]
    no = orc.notify_multi(np.stack([l["token_per_expert"] for l in lays]), epr, ranks)
    rows = multi_rows(idxs, lays, no, epr)
    e_num = epr * ranks
    keys_e, keys_s, keys_f, got = [], [], [], []
    for src, (idx, r) in enumerate(zip(idxs, rows)):
        flat = np.asarray(idx, np.int64).reshape(-1)
        valid = (flat >= 0) & (flat < e_num)
        keys_e.append(flat[valid])
        keys_s.append(np.full(int(valid.sum()), src, np.int64))
        keys_f.append(np.nonzero(valid)[0])
        got.append(r.reshape(-1)[valid])
    ke, ks, kf, got = (np.concatenate(a) for a in (keys_e, keys_s, keys_f, got))
    order = np.lexsort((kf, ks, ke))  # last key is the primary one
    expect = np.empty_like(order)
    expect[order] = np.arange(order.size)
    assert np.array_equal(got, expect), "multi-source receive rows = lexsort position"
    total = int(order.size)
    assert int(no["recv_base"][-1]) + int(no["recv_count"][-1]) == total
    counts = np.stack([l["token_per_expert"] for l in lays]).astype(np.int64)
    assert np.array_equal(no["recv_token_per_expert"], counts.sum(0)), "recvTokenPerExpert"
    assert np.array_equal(no["recv_count"], counts.sum(0).reshape(ranks, epr).sum(1)), "recvCount"


def check_pipeline_multi_vs_single(orc, xs, x_kind: str, idxs, ws, epr: int, ranks: int,
                                   quant: bool) -> None:
    """Closed form of the whole multi-source pipeline: each source's combine
    output equals that source's single-source pipeline (the rows it reads are
    the rows it wrote, wherever they sit), bit for bit; and every valid
    entry's receive row holds that source's token (passthrough) or its
    quantised copy (int8)."""
    m = orc.pipeline_multi(xs, x_kind, idxs, ws, epr, ranks, quant)
    rows = multi_rows(idxs, m["layouts"], m["notify"], epr)
    for src, (x, idx, w) in enumerate(zip(xs, idxs, ws)):
        single = orc.pipeline(x, x_kind, idx, w, epr, ranks, quant)
        assert np.array_equal(m["outs"][src], single["out"]), f"source {src} output"
        r = rows[src]
        t_of = np.broadcast_to(np.arange(idx.shape[0])[:, None], idx.shape)
        sel = r >= 0
        if quant:
            srow = single["dispatch"]["codes"]
            srows = multi_rows([idx], [single["layout"]],
                               dict(put_offset=single["notify"]["put_offset"][:, None],
                                    recv_base=single["notify"]["recv_base"]), epr)[0]
            assert np.array_equal(m["dispatch"]["codes"][r[sel]], srow[srows[sel]]), f"source {src} codes"
            assert np.array_equal(m["dispatch"]["inv"][r[sel]], single["dispatch"]["inv"][srows[sel]])
        else:
            assert np.array_equal(m["dispatch"]["rows"][r[sel]], np.asarray(x)[t_of[sel]]), f"source {src} rows"


# --------------------------------------------------------------------------
# dispatch (stage 3)
# --------------------------------------------------------------------------

def check_dispatch_passthrough(orc, x: np.ndarray, x_kind: str, idx: np.ndarray, epr: int,
                               ranks: int) -> None:
    """Closed form: the receive buffer is the expanded rows stably sorted by
    expert id (rank-major, then expert, then token order)."""
    lay = orc.layout(idx, epr, ranks)
    no = orc.notify(lay["token_per_expert"], epr, ranks)
    d = orc.dispatch(x, x_kind, idx, lay["send_token_idx"], no["put_offset"], no["recv_base"],
                     epr, ranks, quant=False)
    flat = idx.reshape(-1).astype(np.int64)
    e_num = epr * ranks
    valid = (flat >= 0) & (flat < e_num)
    order = np.argsort(np.where(valid, flat, e_num), kind="stable")[: int(valid.sum())]
    k = idx.shape[1]
    expect = np.zeros_like(d["rows"])
    expect[: order.size] = x[order // k]
    assert np.array_equal(d["rows"], expect), "receive rows = x expanded and sorted by expert"


def check_dispatch_int8_rows(orc, x: np.ndarray, x_kind: str, idx: np.ndarray, epr: int,
                             ranks: int) -> None:
    """Each received int8 row is the quantised source row, at the sorted position."""
    lay = orc.layout(idx, epr, ranks)
    no = orc.notify(lay["token_per_expert"], epr, ranks)
    d = orc.dispatch(x, x_kind, idx, lay["send_token_idx"], no["put_offset"], no["recv_base"],
                     epr, ranks, quant=True)
    flat = idx.reshape(-1).astype(np.int64)
    e_num = epr * ranks
    valid = (flat >= 0) & (flat < e_num)
    order = np.argsort(np.where(valid, flat, e_num), kind="stable")[: int(valid.sum())]
    k = idx.shape[1]
    for r, src in enumerate(order // k):
        codes, inv = quant_expected(x[src], x_kind)
        assert np.array_equal(d["codes"][r], codes), f"codes of receive row {r}"
        assert f32_bits(d["inv"][r]) == f32_bits(inv), f"inverse scale of receive row {r}"
    assert not d["codes"][order.size:].any() and not d["inv"][order.size:].any()


def quant_expected(x_bits: np.ndarray, x_kind: str) -> Tuple[np.ndarray, np.float32]:
    """The quantiser in exact rational arithmetic with an explicit binary32
    rounding after each operation of the page's formula."""
    f = widen16(x_bits, x_kind).astype(np.float64)
    amax = Fraction(float(np.max(np.abs(f)))) if f.size else Fraction(0)
    denom = round_f32(amax + frac(np.float32(1e-12)))
    s = round_f32(Fraction(127) / denom)
    codes = np.array([round_int_even(round_f32(Fraction(float(v)) * s)) for v in f], dtype=np.int64)
    inv = round_f32(Fraction(1) / s)
    return codes.astype(np.int8), np.float32(float(inv))


def check_quant_golden(orc) -> None:
    g = load_golden("quant_rows.json")
    for case in g["cases"]:
        bits = to_bits16(case["x"], case["x_kind"])
        codes, inv, s = orc.quant_row(bits, case["x_kind"])
        assert codes.tolist() == case["codes"], case["name"]
        if case["scale_hex"] is not None:
            assert f32_bits(s) == int(case["scale_hex"], 16), case["name"] + " scale"
            assert f32_bits(inv) == int(case["inv_hex"], 16), case["name"] + " inverse"
        else:
            exp_codes, exp_inv = quant_expected(bits, case["x_kind"])
            assert np.isfinite(s) and f32_bits(inv) == f32_bits(exp_inv), case["name"]


def check_quant_power_of_two(orc, seed: int = 7) -> None:
    """Rows whose max is 127 * 2^m: the scale is exactly 2^-m, so the codes
    are numpy.rint of an exact scaling and inv = 2^m."""
    rng = np.random.default_rng(seed)
    for m in range(-12, 13, 3):
        for kind in ("bf16", "fp16"):
            if kind == "fp16" and not (-8 <= m <= 8):
                continue
            h = 64
            peak = 127.0 * 2.0 ** m
            vals = np.clip(rng.normal(0, 40, h) * 2.0 ** m, -peak, peak)
            vals[rng.integers(h)] = peak if m % 2 else -peak
            bits = np.ascontiguousarray(to_bits16_round(vals, kind))
            f = widen16(bits, kind).astype(np.float64)
            codes, inv, s = orc.quant_row(bits, kind)
            assert float(s) == 2.0 ** -m and float(inv) == 2.0 ** m, (m, kind)
            assert np.array_equal(codes.astype(np.int64), np.rint(f * 2.0 ** -m).astype(np.int64)), (m, kind)


def to_bits16_round(vals: np.ndarray, kind: str) -> np.ndarray:
    import torch

    if kind == "bf16":
        return torch.tensor(vals, dtype=torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    return vals.astype(np.float16).view(np.uint16)


def check_quant_exact(orc, rows: np.ndarray, kind: str) -> None:
    """Scale, inverse and codes against exact rational arithmetic, plus the
    reconstruction error bound.  With q = rint(fl(f*s)) and inv = fl(1/s):
    |q - f*s| <= 1/2 + 127.5u and |inv - 1/s| <= u/s (u = 2^-24), so
    |inv*q - f| <= (1/2 + 255u) / s, and 1/s <= inv * (1 + 2u)."""
    for r in range(rows.shape[0]):
        codes, inv, s = orc.quant_row(rows[r], kind)
        exp_codes, exp_inv = quant_expected(rows[r], kind)
        assert np.array_equal(codes, exp_codes), f"codes row {r}"
        assert f32_bits(inv) == f32_bits(exp_inv), f"inverse scale row {r}"
        f = widen16(rows[r], kind).astype(np.float64)
        err = np.abs(codes.astype(np.float64) * float(inv) - f)
        u = 2.0 ** -24
        assert np.all(err <= (0.5 + 255 * u) * float(inv) * (1 + 2 * u)), f"error bound row {r}"
        amax = np.max(np.abs(f))
        if amax > 1e-9:
            assert np.max(np.abs(codes.astype(np.int64))) == 127, f"peak code row {r}"
        assert np.all(np.sign(codes) * np.sign(f) >= 0), f"sign row {r}"


# --------------------------------------------------------------------------
# combine (stage 4)
# --------------------------------------------------------------------------

def _one_token_case(rows_vals, weights, h: int = 8):
    """bs = 1, entry j -> expert j: receive row j holds rows_vals[j] in every column."""
    k = len(rows_vals)
    idx = np.arange(k, dtype=np.int32).reshape(1, k)
    w = np.asarray(weights, dtype=np.float32).reshape(1, k)
    x_rows = np.repeat(to_bits16(rows_vals, "bf16").reshape(k, 1), h, axis=1)
    return idx, w, np.ascontiguousarray(x_rows)


def check_combine_golden(orc) -> None:
    g = load_golden("combine_order.json")
    for case in g["cases"]:
        k = len(case["rows"])
        idx, w, rows = _one_token_case(case["rows"], case["weights"])
        slot = np.zeros((1, k), np.int32)
        put = np.zeros(k, np.int32)
        base = np.arange(k, dtype=np.int32)  # one expert per rank, one row each
        out32 = orc.combine(dict(rows=rows), "bf16", idx, w, slot, put, base, 1, k, "fp32")
        assert np.all(out32 == np.float32(case["out_fp32"])), case["name"]
        assert np.all(f32_bits(out32[0, 0]) == f32_bits(np.float32(case["out_fp32"]))), case["name"]
        if "out_bf16_hex" in case:
            outb = orc.combine(dict(rows=rows), "bf16", idx, w, slot, put, base, 1, k, "bf16")
            assert np.all(outb == int(case["out_bf16_hex"], 16)), case["name"]


def combine_terms(recv: Dict[str, np.ndarray], recv_kind: str, idx, w, slot, put, base, epr):
    """Per token, the k terms v_j * w_j in float64 (exact products of the
    binary32 inputs) and their rows; invalid entries give zero terms."""
    bs, k = idx.shape
    e_num = put.size
    if recv_kind == "int8":
        h = recv["codes"].shape[1]
    else:
        h = recv["rows"].shape[1]
    terms = np.zeros((bs, k, h), np.float64)
    for t in range(bs):
        for j in range(k):
            e = int(idx[t, j])
            if not (0 <= e < e_num) or slot[t, j] < 0:
                continue
            row = int(base[e // epr]) + int(put[e]) + int(slot[t, j])
            if recv_kind == "int8":
                v = recv["codes"][row].astype(np.float64) * float(recv["inv"][row])
                # the dequantised value is rounded to binary32 before the weight multiply
                v = v.astype(np.float32).astype(np.float64)
            else:
                v = widen16(recv["rows"][row], recv_kind).astype(np.float64)
            terms[t, j] = v * float(w[t, j])
    return terms


def check_combine_bound(orc, recv, recv_kind, idx, w, slot, put, base, epr, ranks) -> None:
    """fp32 output against the float64 sum of the terms: with k products and
    k additions each rounded once, |out - sum| <= (2k) * 2^-24 * sum|terms|
    (plus the dequantisation rounding, already inside the terms)."""
    out = orc.combine(recv, recv_kind, idx, w, slot, put, base, epr, ranks, "fp32")
    terms = combine_terms(recv, recv_kind, idx, w, slot, put, base, epr)
    exact = terms.sum(axis=1)
    mag = np.abs(terms).sum(axis=1)
    k = idx.shape[1]
    bound = (2 * k) * 2.0 ** -24 * mag + 1e-38
    err = np.abs(out.astype(np.float64) - exact)
    assert np.all(err <= bound), f"combine error {float((err - bound).max())} over bound"
    # the 16-bit outputs are the fp32 result rounded half-even (torch / numpy)
    outb = orc.combine(recv, recv_kind, idx, w, slot, put, base, epr, ranks, "bf16")
    assert np.array_equal(outb, to_bits16_round(out.astype(np.float32), "bf16")), "bf16 output rounding"
    outh = orc.combine(recv, recv_kind, idx, w, slot, put, base, epr, ranks, "fp16")
    with np.errstate(over="ignore"):
        assert np.array_equal(outh, out.astype(np.float16).view(np.uint16)), "fp16 output rounding"


def check_combine_identity(orc, x: np.ndarray, x_kind: str, epr: int, ranks: int) -> None:
    """k = 1 with weight 1 returns the dequantised row exactly (passthrough:
    the row itself; int8: float(q) * inv as numpy computes it)."""
    bs, h = x.shape
    e_num = epr * ranks
    idx = (np.arange(bs, dtype=np.int32) % e_num).reshape(bs, 1)
    w = np.ones((bs, 1), np.float32)
    for quant in (False, True):
        res = orc.pipeline(x, x_kind, idx, w, epr, ranks, quant, out_kind="fp32")
        if not quant:
            assert np.array_equal(res["out"], widen16(x, x_kind)), "passthrough identity"
            res16 = orc.pipeline(x, x_kind, idx, w, epr, ranks, quant, out_kind=x_kind)
            assert np.array_equal(res16["out"], x), "passthrough identity (16-bit out)"
        else:
            lay, no, d = res["layout"], res["notify"], res["dispatch"]
            rows = no["recv_base"][idx[:, 0] // epr] + no["put_offset"][idx[:, 0]] + lay["send_token_idx"][:, 0]
            deq = d["codes"][rows].astype(np.float32) * d["inv"][rows][:, None]
            assert np.array_equal(res["out"], deq.astype(np.float32)), "int8 identity"


def random_receive_buffer(seed: int, rows: int, h: int, kind: str) -> Dict[str, np.ndarray]:
    """A receive buffer whose rows all differ, as after a real expert step:
    N(0,1) rows for bf16/fp16, uniform codes in [-127, 127] with positive
    inverse scales for int8."""
    rng = np.random.default_rng(seed)
    if kind == "int8":
        codes = rng.integers(-127, 128, size=(rows, h)).astype(np.int8)
        inv = (rng.random(rows) * 0.05 + 1e-3).astype(np.float32)
        return dict(codes=codes, inv=inv)
    return dict(rows=np.ascontiguousarray(to_bits16_round(rng.normal(0, 1, (rows, h)), kind)))


def check_combine_random_rows(orc, seed: int = 5) -> None:
    """Combine over receive rows that differ per (token, k) entry, so a
    permuted weight, a dropped or repeated term, or a wrong row address
    moves the result far outside the float64 bound."""

    for kind in ("bf16", "int8"):
        w = W.random_case(seed, 37, 24, 6, 12, 3, routing="dup", bad_frac=0.05)
        lay = orc.layout(w.topk_idx, 4, 3)
        no = orc.notify(lay["token_per_expert"], 4, 3)
        recv = random_receive_buffer(seed + 1, w.bs * w.topk, 24, kind)
        check_combine_bound(orc, recv, kind, w.topk_idx, w.topk_w, lay["send_token_idx"],
                            no["put_offset"], no["recv_base"], 4, 3)


# --------------------------------------------------------------------------
# expert-side epilogue: dequantise, SwiGLU, requantise
# --------------------------------------------------------------------------

def ulp32(ref: np.ndarray) -> np.ndarray:
    """binary32 ulp at |ref| (float64), with the subnormal spacing below 2^-126."""
    a = np.abs(np.asarray(ref, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return 2.0 ** (e - 23)


def exp_probe_values() -> np.ndarray:
    """A dense grid over the finite range, random bit patterns inside it, and
    edges: zeros, tiny arguments, the overflow and underflow boundaries, and
    arguments whose result is subnormal."""
    grid = np.linspace(-104.0, 89.0, 400001).astype(np.float32)
    rng = np.random.default_rng(2024)
    pats = rng.integers(0, 2 ** 32, 400000, dtype=np.uint64).astype(np.uint32).view(np.float32)
    pats = pats[np.isfinite(pats) & (pats > -104.0) & (pats < 89.0)]
    edges = np.float32([0.0, -0.0, 1e-30, -1e-30, 2.0 ** -25, -(2.0 ** -25), 0.5, -0.5, 1.0, -1.0,
                        88.72283, 88.7228, 88.72284, -87.33654, -87.3366, -100.0, -103.27893,
                        -103.97207, -103.9721, 17.0, 16.0, -17.0, 0.34657359, -0.34657359])
    return np.concatenate([grid, pats, edges]).astype(np.float32)


def check_exp(orc) -> None:
    """The oracle's binary32 e^x against float64 exp (a library routine):
    within 1.25 ulp everywhere it is finite and nonzero, subnormal results
    within one subnormal step, exact at 0, monotone over the grid, +inf
    above ln(max float) and +0 far below the subnormal range, NaN kept."""
    x = exp_probe_values()
    y = orc.exp_f32(x).astype(np.float64)
    ref = np.exp(x.astype(np.float64))
    big = ref >= 3.4028235677973366e38  # rounds to +inf in binary32
    assert np.all(np.isinf(y[big])), "overflow to +inf"
    fin = ~big
    err = np.abs(y[fin] - ref[fin]) / ulp32(ref[fin])
    assert err.max() <= 1.25, f"exp error {err.max():.3f} ulp at x = {x[fin][np.argmax(err)]!r}"
    assert orc.exp_f32(np.float32([0.0, -0.0])).tolist() == [1.0, 1.0]
    grid = orc.exp_f32(np.linspace(-104.0, 88.7, 200001).astype(np.float32))
    assert np.all(np.diff(grid.astype(np.float64)) >= 0), "exp not monotone"
    far = orc.exp_f32(np.float32([89.5, 100.0, 1e30, -104.5, -200.0, -1e30, np.inf, -np.inf]))
    assert far[:3].tolist() == [np.inf] * 3 and np.isinf(far[6]) and far[7] == 0.0
    assert np.all(far[3:6] == 0.0)
    assert np.isnan(orc.exp_f32(np.float32([np.nan]))[0])


def quant_f32_expected(acts: np.ndarray) -> Tuple[np.ndarray, np.float32]:
    """The dispatch quantiser applied to a binary32 row, in exact rational
    arithmetic with a binary32 rounding after each operation."""
    a = np.asarray(acts, dtype=np.float32).astype(np.float64)
    amax = Fraction(float(np.max(np.abs(a)))) if a.size else Fraction(0)
    denom = round_f32(amax + frac(np.float32(1e-12)))
    s = round_f32(Fraction(127) / denom)
    codes = np.array([round_int_even(round_f32(Fraction(float(v)) * s)) for v in a], dtype=np.int64)
    inv = round_f32(Fraction(1) / s)
    return codes.astype(np.int8), np.float32(float(inv))


def check_swiglu_golden(orc) -> None:
    g = load_golden("swiglu_rows.json")
    for case in g["cases"]:
        codes, inv, _ = orc.swiglu_quant_row(np.array(case["acc"], np.int32),
                                             np.array(case["weight_scale"], np.float32),
                                             case["token_scale"])
        assert codes.tolist() == case["codes"], case["name"]
        assert f32_bits(inv) == int(case["inv_hex"], 16), case["name"] + " inverse scale"


def swiglu_exact_case(seed: int, n: int):
    """A row whose dequantisation is exact: |acc| < 2^24 and power-of-two
    scales, so the gate and up values are known exactly in float64."""
    rng = np.random.default_rng(seed)
    acc = rng.integers(-(2 ** 23), 2 ** 23, 2 * n).astype(np.int32)
    ws = (2.0 ** -rng.integers(18, 24, 2 * n)).astype(np.float32)
    ts = np.float32(2.0 ** -int(rng.integers(0, 4)))
    # a few gates pushed to the extremes: exp overflow, exp underflow, near 0
    k = max(1, n // 16)
    pos = rng.choice(n, size=3 * k, replace=False)
    acc[pos[:k]] = -(2 ** 23) + 1
    ws[pos[:k]] = np.float32(2.0 ** -15)  # gate about -256: e^-g overflows
    acc[pos[k:2 * k]] = 2 ** 23 - 1
    ws[pos[k:2 * k]] = np.float32(2.0 ** -15)  # gate about +256: e^-g underflows
    acc[pos[2 * k:]] = rng.integers(-3, 4, k)
    g = acc[:n].astype(np.float64) * ws[:n] * float(ts)
    u = acc[n:].astype(np.float64) * ws[n:] * float(ts)
    return acc, ws, ts, g, u


def check_swiglu_bound(orc, seeds=(1, 2, 3), n: int = 200) -> None:
    """Activations within 4 binary32 roundings (relative) of the float64
    g / (1 + e^-g) * u on rows with exact dequantisation (e^x within 1.25 ulp,
    then add, divide, multiply); codes and inverse scale exactly the
    quantiser of those activations in rational arithmetic."""
    for seed in seeds:
        acc, ws, ts, g, u = swiglu_exact_case(seed, n)
        codes, inv, act = orc.swiglu_quant_row(acc, ws, ts)
        with np.errstate(over="ignore"):
            ref = g / (1.0 + np.exp(-g)) * u
        tol = 4.5 * 2.0 ** -24 * np.abs(ref) + 2.0 ** -149
        assert np.all(np.abs(act.astype(np.float64) - ref) <= tol), f"activation bound, seed {seed}"
        exp_codes, exp_inv = quant_f32_expected(act)
        assert np.array_equal(codes, exp_codes), f"codes, seed {seed}"
        assert f32_bits(inv) == f32_bits(exp_inv), f"inverse scale, seed {seed}"


def check_swiglu_dequant_exact(orc, seed: int = 9, n: int = 64) -> None:
    """Rows whose gates are all >= 17 after dequantisation (e^-g below half an
    ulp of 1, so SwiGLU reduces to g * u exactly), with accumulators beyond
    2^24 and scales that are not powers of two: every activation must equal
    fl(fl(fl(fl(acc_g) * ws_g) * ts) * fl(fl(fl(acc_u) * ws_u) * ts)),
    evaluated in rational arithmetic (int32 -> binary32 rounds half-even)."""
    rng = np.random.default_rng(seed)
    for trial in range(4):
        ws = rng.uniform(0.5, 2.0, 2 * n).astype(np.float32) * np.float32(2.0 ** -22)
        ts = np.float32(rng.uniform(0.9, 1.1))
        acc = np.empty(2 * n, np.int64)
        acc[:n] = rng.integers(2 ** 28, 2 ** 31 - 1, n)  # gate >= 2^28 * 2^-23 * 0.9 > 17
        acc[n:] = rng.integers(-(2 ** 31), 2 ** 31 - 1, n)
        acc[n] = 2 ** 24 + 1  # ties in the int32 -> binary32 cast
        acc[n + 1] = 2 ** 24 + 3
        acc = acc.astype(np.int32)
        codes, inv, act = orc.swiglu_quant_row(acc, ws, ts)
        tsf = frac(ts)
        for i in range(n):
            gq = round_f32(round_f32(round_f32(Fraction(int(acc[i]))) * frac(ws[i])) * tsf)
            assert gq >= 17, "fixture: gate below 17"
            uq = round_f32(round_f32(round_f32(Fraction(int(acc[n + i]))) * frac(ws[n + i])) * tsf)
            a = round_f32(gq * uq)
            assert f32_bits(act[i]) == f32_bits(np.float32(float(a))), (trial, i)
        exp_codes, exp_inv = quant_f32_expected(act)
        assert np.array_equal(codes, exp_codes) and f32_bits(inv) == f32_bits(exp_inv), trial


# --------------------------------------------------------------------------
# first expert matmul (GMM1: int8 x int8 -> int32 over per-expert row ranges)
# --------------------------------------------------------------------------

def gemm_owners(counts, rows: int) -> np.ndarray:
    """Owner of each row: expert g holds the next max(c_g, 0) rows, in
    expert order; rows past the experts' total belong to nobody (-1)."""
    owner = np.full(rows, -1, np.int64)
    start = 0
    for g, c in enumerate(np.asarray(counts, dtype=np.int64)):
        c = max(int(c), 0)
        owner[start:min(start + c, rows)] = g
        start += c
    return owner


def check_gemm_per_expert_matmul(orc, seed: int = 3) -> None:
    """Each expert's rows equal numpy's int64 product of those rows with the
    transposed weights of that expert; rows of no expert are left alone.
    Rows are read at a stride larger than k (padding bytes are random)."""
    c = W.gemm_case(seed, rows=45, k=80, n=24, groups=5, stride=112,
                    counts=[7, 0, 13, 1, 16])
    out, grp = orc.grouped_gemm_i8(c.a, c.k, c.group_count, c.w)
    owner = gemm_owners(c.group_count, c.rows)
    assert np.array_equal(grp, owner)
    start = 0
    for g, cnt in enumerate(c.group_count):
        ref = c.a[start:start + cnt, :c.k].astype(np.int64) @ c.w[g].astype(np.int64).T
        assert np.array_equal(out[start:start + cnt].astype(np.int64), ref), g
        start += int(cnt)
    assert not out[start:].any()


def check_gemm_closed_forms(orc) -> None:
    """Constant operands: all-ones rows against weights g+1 give k*(g+1);
    the int8 extremes at k = 8192 give 8192 * (-128)^2 = 2^27 and
    8192 * 127 * (-128) = -133169152, both exact."""
    k, n = 40, 16
    a = np.ones((9, k), np.int8)
    w = np.stack([np.full((n, k), g + 1, np.int8) for g in range(3)])
    out, grp = orc.grouped_gemm_i8(a, k, np.array([2, 3, 4], np.int32), w)
    assert np.array_equal(out, (k * (grp[:, None] + 1)) * np.ones((1, n), np.int64))
    k = 8192
    a = np.full((2, k), -128, np.int8)
    a[1] = 127
    w = np.full((1, 16, k), -128, np.int8)
    out, _ = orc.grouped_gemm_i8(a, k, np.array([2], np.int32), w)
    assert (out[0] == 2 ** 27).all() and (out[1] == -133169152).all()


def check_gemm_permutation(orc, seed: int = 4) -> None:
    """Weights that pick one input column per output column: w[g][j][i] = 1
    exactly when i = p_g(j), so out[m][j] = a[m][p_g(j)].  With k != n and
    permutations that are not their own inverses, a transposed weight read
    or a swapped operand gives other columns."""
    k, n, rows = 48, 32, 12
    a = W.gemm_case(seed, rows=rows, k=k, n=1, groups=1).a
    perms = [(np.arange(n) * 5 + g * 7 + 3) % k for g in range(3)]
    w = np.zeros((3, n, k), np.int8)
    for g, p in enumerate(perms):
        w[g, np.arange(n), p] = 1
    counts = np.array([5, 4, 3], np.int32)
    out, grp = orc.grouped_gemm_i8(a, k, counts, w)
    for m in range(rows):
        assert np.array_equal(out[m], a[m, perms[grp[m]]].astype(np.int32)), m


def check_gemm_ownership(orc, seed: int = 5) -> None:
    """Negative counts own no rows, empty experts are skipped, rows past the
    total belong to nobody, and a row list returns the same rows as the full
    call."""
    c = W.gemm_case(seed, rows=20, k=16, n=16, groups=4, counts=[-3, 6, 0, 9])
    out, grp = orc.grouped_gemm_i8(c.a, c.k, c.group_count, c.w)
    assert np.array_equal(grp, [1] * 6 + [3] * 9 + [-1] * 5)
    ref3 = c.a[6:15].astype(np.int64) @ c.w[3].astype(np.int64).T
    assert np.array_equal(out[6:15], ref3)
    sel = np.array([19, 0, 7, 14, 5])
    out_s, grp_s = orc.grouped_gemm_i8(c.a, c.k, c.group_count, c.w, rows=sel)
    assert np.array_equal(grp_s, grp[sel]) and np.array_equal(out_s, out[sel])
