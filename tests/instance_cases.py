"""Cases that reach every compiled instance of the library's kernels.

The kernels that hold a token's row in registers are compiled once per
register-array width, element type and mode; which instance a call runs is a
function of its sizes (combine_moe_layout_03_amd/csrc/select.h).  Instances
differ in more than a constant: one of them once kept its row in scratch
memory and ran at half speed.  So every shipped instance needs a GPU parity
case of its own.  The lists below are those cases; test_gpu_instances.py
runs them against the oracle, and test_instance_coverage.py (CPU) checks,
with the selection rules compiled from select.h and the instance list read
from the compiler, that together they reach every instance.

Plain data only (no torch), so the CPU check can import it.
"""

# (xkind, quant): passthrough rows keep x's type, quantised rows are int8
X_MODES = [("bf16", False), ("fp16", False), ("bf16", True), ("fp16", True)]

# (hidden, topk): hidden picks the register widths of the fused, dispatch and
# combine kernels, topk picks combine's entry bound (4, 8, or the k > 8
# kernel).  Per x mode these reach fused widths 1, 2, 4, 8, 12, 14, 16 (and
# the three-stage form above 8192), dispatch widths 1-32, and combine's
# (chunks per lane, entry bound) pairs (1,4) (1,8) (2,4) (2,8) (4,4) (4,8)
# (8,4) (8,8) plus the k > 8 kernel.
HIDDEN_TOPK = [(512, 3), (1024, 8), (2048, 12), (3072, 4), (4096, 8), (6144, 2), (7168, 8),
               (8192, 5), (12288, 4), (16384, 8)]

# Per hidden: tokens, experts, ranks, routing, fraction of bad ids.  Tokens
# shrink as rows grow so the oracle stays fast; two shapes have more than
# 2048 entries (several layout tiles) and two have more than 512 experts
# (the layout's 4-wave tiles).
_SHAPE = {
    512: (1000, 64, 8, "dup", 0.01),       # 3000 entries: two layout tiles
    1024: (300, 1024, 8, "uniform", 0.0),  # 2400 entries, E = 1024: two 4-wave tiles
    2048: (130, 256, 16, "zipf1.2", 0.0),
    3072: (97, 32, 4, "dup", 0.02),
    4096: (80, 64, 8, "hot", 0.0),
    6144: (70, 2048, 16, "uniform", 0.0),  # E = 2048, one tile
    7168: (64, 256, 16, "uniform", 0.0),
    8192: (45, 24, 3, "dup", 0.05),
    12288: (33, 128, 16, "zipf1.2", 0.0),
    16384: (24, 16, 2, "dup", 0.0),
}

# seed, bs, hidden, topk, experts, ranks, routing, bad fraction, xkind, quant
PIPELINE_CASES = []
for _m, (_xk, _q) in enumerate(X_MODES):
    for _i, (_h, _k) in enumerate(HIDDEN_TOPK):
        _bs, _e, _r, _route, _bad = _SHAPE[_h]
        PIPELINE_CASES.append((700 + 20 * _m + _i, _bs, _h, _k, _e, _r, _route, _bad, _xk, _q))

# combine runs once per output type on every case
OUT_KINDS = ["bf16", "fp16", "fp32"]

# Epilogue widths n (columns of the int8 output): one per launch shape, each
# with a ragged tail where possible.
EPILOGUE_NS = [(40, 200), (30, 500), (25, 1020), (20, 2044), (12, 4092)]  # (rows, n)

# Grouped GEMM: k a whole number of 128-byte stages, and k ending inside one
# (rows, k, n, groups, counts)
GEMM_CASES = [(700, 1024, 1024, 4, [100, 0, 350, 240]), (650, 336, 512, 3, [300, -2, 340])]

# The matmul with its fused epilogue, the same two k: (rows, k, n, groups,
# counts), n the activation columns (the weights have 2n rows per expert)
FUSED_GEMM_CASES = [(700, 1024, 512, 4, [100, 0, 350, 240]), (650, 336, 260, 3, [300, -2, 340])]


def case_id(case) -> str:
    seed, bs, h, k, e, r, route, bad, xk, q = case
    return f"{seed}-{xk}-{'int8' if q else 'pass'}-h{h}-k{k}-E{e}"
