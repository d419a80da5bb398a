"""Every compiled instance of the row kernels against the oracle, through the
C ABI (the cases of instance_cases.py; test_instance_coverage.py checks on
the CPU that they reach every instance the library ships).

Each case runs the fused entry point (the one kernel, or the three stages
when it does not apply) and the separate stages, and combine into every
output type; everything is compared bit for bit with the oracle.
"""

import numpy as np
import pytest
import torch

import instance_cases as IC
import workloads as W
from gpu_util import GpuRun, log
from test_gpu_parity import compare, oracle_run

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible MI355X")


@pytest.mark.parametrize("case", IC.PIPELINE_CASES, ids=[IC.case_id(c) for c in IC.PIPELINE_CASES])
def test_instance_pipeline(case):
    seed, bs, h, k, e, r, route, bad, xk, quant = case
    w = W.random_case(seed, bs, h, k, e, r, x_dtype=xk, routing=route, bad_frac=bad, zero_rows=1)
    for i, out_kind in enumerate(IC.OUT_KINDS):
        fused = i == 0
        log(f"instance case {IC.case_id(case)} {'fused entry' if fused else 'separate stages'} out={out_kind}")
        g = GpuRun(w, quant, out_kind).run_all(fused=fused).host()
        compare(w, quant, out_kind, g, oracle_run(w, quant, out_kind))


@pytest.mark.parametrize("rows,n", IC.EPILOGUE_NS, ids=[f"n{n}" for _, n in IC.EPILOGUE_NS])
def test_instance_epilogue(rows, n):
    from test_gpu_epilogue import assert_same, run_gpu

    case = W.epilogue_case(900 + n, rows, n)
    log(f"instance epilogue rows={rows} n={n}")
    out = run_gpu(case, guard_rows=1)
    assert_same(case, out, f"rows={rows} n={n}")


@pytest.mark.parametrize("rows,k,n,groups,counts", IC.GEMM_CASES, ids=[f"k{c[1]}" for c in IC.GEMM_CASES])
def test_instance_grouped_gemm(rows, k, n, groups, counts):
    from test_gpu_gemm import assert_same, run_gpu

    case = W.gemm_case(950 + k, rows, k, n, groups, stride=(k + 31) // 32 * 32 + 32, counts=counts)
    log(f"instance grouped gemm rows={rows} k={k} n={n}")
    assert_same(case, run_gpu(case), f"k={k}")


@pytest.mark.parametrize("rows,k,n,groups,counts", IC.FUSED_GEMM_CASES,
                         ids=[f"k{c[1]}" for c in IC.FUSED_GEMM_CASES])
def test_instance_grouped_gemm_swiglu(rows, k, n, groups, counts):
    from test_gpu_gemm_swiglu import assert_rows, make_case, run_fused

    case, ws, ts = make_case(960 + k, rows, k, n, groups, counts)
    log(f"instance grouped gemm + swiglu rows={rows} k={k} n={n}")
    assert_rows(case, ws, ts, run_fused(case, ws, ts), np.arange(rows), f"k={k}")
