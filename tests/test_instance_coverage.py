"""Every compiled kernel instance is reached by a GPU parity case (CPU only).

Three sources are tied together:
  * the selection rules and width tables of csrc/select.h, compiled here with
    the system C++ compiler into a small driver that the launchers' own
    functions answer for each case;
  * the kernel instances the library ships, as hipcc reports them when it
    compiles csrc/*.hip with the library's flags;
  * the GPU cases of tests/instance_cases.py (run by test_gpu_instances.py).
The tables must list exactly the compiled instances, and the cases must
reach all of them.  A new width, element type or mode without a GPU case
fails here.
"""

import os
import re
import subprocess
import tempfile

import pytest

import instance_cases as IC
import kernel_remarks

CSRC = kernel_remarks.CSRC

_DRIVER = r"""
#include <cstdio>
#include "select.h"
using namespace moe::select;
template <size_t N> static void table(const char* name, const int (&t)[N]) {
  std::printf("%s", name);
  for (size_t i = 0; i < N; ++i) std::printf(" %d", t[i]);
  std::printf("\n");
}
int main() {
  table("fused_vpl", kFusedVpl);
  table("dispatch_vpl", kDispatchVpl);
  table("rows_max_k", kCombineRowsMaxK);
  table("rows_chunks", kCombineRowsChunks);
  std::printf("epilogue");
  for (const EpilogueShape& s : kEpilogueShapes) std::printf(" %d:%d", s.it, s.waves);
  std::printf("\n");
  std::printf("layout %d:%d %d:%d\n", layout_waves(1), layout_rounds(1), layout_waves(2048),
              layout_rounds(2048));
  char kind;
  while (std::scanf(" %c", &kind) == 1) {
    if (kind == 'p') {
      long long bs, h, k, e;
      if (std::scanf("%lld %lld %lld %lld", &bs, &h, &k, &e) != 4) return 1;
      std::printf("p %d %d %d %d %d %d %d %lld\n", fused_applies(int(bs), int(h), int(k)) ? 1 : 0,
                  fused_vpl(int(h)), dispatch_vpl(int(h)), combine_rows_max_k(int(k)),
                  combine_rows_chunks(int(h)), layout_waves(int(e)), layout_rounds(int(e)),
                  (long long)layout_num_tiles(bs * k, int(e)));
    } else if (kind == 'g') {
      int k;
      if (std::scanf("%d", &k) != 1) return 1;
      std::printf("g %d\n", gemm_k_tail(k) ? 1 : 0);
    } else if (kind == 'e') {
      int n;
      if (std::scanf("%d", &n) != 1) return 1;
      const int i = epilogue_shape_index(n);
      std::printf("e %d %d\n", i < 0 ? 0 : kEpilogueShapes[i].it, i < 0 ? 0 : kEpilogueShapes[i].waves);
    }
  }
  return 0;
}
"""

RECV = {"bf16": 0, "fp16": 1, "int8": 2}
OUT = {"bf16": 0, "fp16": 1, "fp32": 2}


@pytest.fixture(scope="module")
def selection():
    """(tables, answers for the pipeline cases, answers for the epilogue cases)."""
    with tempfile.TemporaryDirectory() as d:
        src = os.path.join(d, "driver.cpp")
        exe = os.path.join(d, "driver")
        with open(src, "w") as f:
            f.write(_DRIVER)
        subprocess.run(["g++", "-std=c++17", "-O1", f"-I{CSRC}", src, "-o", exe], check=True)
        lines = [f"p {c[1]} {c[2]} {c[3]} {c[4]}" for c in IC.PIPELINE_CASES]
        lines += [f"e {n}" for _, n in IC.EPILOGUE_NS]
        lines += [f"g {c[1]}" for c in IC.GEMM_CASES + IC.FUSED_GEMM_CASES]
        r = subprocess.run([exe], input="\n".join(lines) + "\n", capture_output=True, text=True, check=True)
    out = r.stdout.splitlines()
    tables = {}
    for line in out[:6]:
        name, *vals = line.split()
        tables[name] = [tuple(int(p) for p in v.split(":")) if ":" in v else int(v) for v in vals]
    pipe = [list(map(int, line.split()[1:])) for line in out[6:] if line.startswith("p ")]
    epi = [tuple(map(int, line.split()[1:])) for line in out[6:] if line.startswith("e ")]
    gemm = [int(line.split()[1]) for line in out[6:] if line.startswith("g ")]
    assert len(pipe) == len(IC.PIPELINE_CASES) and len(epi) == len(IC.EPILOGUE_NS)
    assert len(gemm) == len(IC.GEMM_CASES) + len(IC.FUSED_GEMM_CASES)
    return tables, pipe, epi, gemm


def _arg(v: str) -> int:
    v = v.strip()
    if v in ("true", "false"):
        return int(v == "true")
    m = re.fullmatch(r"(?:\([\w:]+\))?(-?\d+)", v)
    assert m, v
    return int(m.group(1))


@pytest.fixture(scope="module")
def compiled():
    """{kernel family: set of template-argument tuples} shipped by the library."""
    if not kernel_remarks.hipcc_available():
        pytest.skip("hipcc not available")
    names = kernel_remarks.demangle(kernel_remarks.kernel_remarks())
    fam = {}
    for full in names.values():
        m = re.search(r"::(\w+)<(.*)>\(", full)
        if not m:
            continue
        fam.setdefault(m.group(1), set()).add(tuple(_arg(a) for a in m.group(2).split(",")))
    return fam


def expected(tables):
    t = tables
    exp = {
        "fused_kernel": {(f, q, v) for f in (0, 1) for q in (0, 1) for v in t["fused_vpl"]},
        "dispatch_kernel": {(f, q, v) for f in (0, 1) for q in (0, 1) for v in t["dispatch_vpl"]},
        "combine_rows_kernel": {(r, o, c, k) for r in range(3) for o in range(3) for c in t["rows_chunks"]
                                for k in t["rows_max_k"]},
        "combine_kernel": {(r, o) for r in range(3) for o in range(3)},
        "deq_swiglu_quant_kernel": set(t["epilogue"]),
        "layout_count_kernel": set(t["layout"]),
        "layout_rank_kernel": set(t["layout"]),
        "grouped_gemm_kernel": {(t, f) for t in (0, 1) for f in (0, 1)},
    }
    return exp


def reached(selection):
    _, pipe, epi, gemm = selection
    got = {k: set() for k in ("fused_kernel", "dispatch_kernel", "combine_rows_kernel", "combine_kernel",
                              "deq_swiglu_quant_kernel", "layout_count_kernel", "layout_rank_kernel",
                              "grouped_gemm_kernel")}
    for i, tail in enumerate(gemm):  # the plain cases, then the fused ones
        got["grouped_gemm_kernel"].add((tail, int(i >= len(IC.GEMM_CASES))))
    for case, ans in zip(IC.PIPELINE_CASES, pipe):
        seed, bs, h, k, e, r, route, bad, xk, q = case
        applies, fvpl, dvpl, kmax, chunks, lw, lr, tiles = ans
        f16 = int(xk == "fp16")
        # the fused entry point: the one kernel, or the three stages
        if applies:
            got["fused_kernel"].add((f16, int(q), fvpl))
        # the separate stages (run for every case; also the fused fallback)
        got["layout_rank_kernel"].add((lw, lr))
        if tiles > 1:
            got["layout_count_kernel"].add((lw, lr))
        got["dispatch_kernel"].add((f16, int(q), dvpl))
        recv = RECV["int8" if q else xk]
        for ok in IC.OUT_KINDS:
            if kmax:
                got["combine_rows_kernel"].add((recv, OUT[ok], chunks, kmax))
            else:
                got["combine_kernel"].add((recv, OUT[ok]))
    for it_w in epi:
        got["deq_swiglu_quant_kernel"].add(it_w)
    return got


def test_tables_list_exactly_the_compiled_instances(selection, compiled):
    tables = selection[0]
    for family, want in expected(tables).items():
        have = compiled.get(family, set())
        if family == "combine_kernel":  # <Recv, Out, 32 entries, 8 elements, 4 waves, nt load, nt store>
            have = {a[:2] for a in have}
        elif family == "grouped_gemm_kernel":  # <tile M, tile N, waves M, waves N, k tail, fused>
            have = {a[-2:] for a in have}
        elif family == "dispatch_kernel":
            assert all(len(a) == 3 for a in have), f"dispatch_kernel template arguments changed: {have}"
        assert have == want, f"{family}: compiled {sorted(have)} but the tables give {sorted(want)}"


def test_every_instance_has_a_gpu_case(selection):
    tables = selection[0]
    got = reached(selection)
    for family, want in expected(tables).items():
        missing = sorted(want - got[family])
        assert not missing, f"{family}: no GPU case reaches {missing}"


def test_benchmarked_instance_is_reached():
    """The large shape (h = 7168, k = 8) in both modes is among the GPU cases
    of its own file as well: fused_kernel<bf16, *, 14> and combine at 4 chunks
    per lane, 8 entries."""
    assert any(c[2] == 7168 and c[3] == 8 and c[8] == "bf16" and not c[9] for c in IC.PIPELINE_CASES)
    assert any(c[2] == 7168 and c[3] == 8 and c[8] == "bf16" and c[9] for c in IC.PIPELINE_CASES)
