"""The operand repack (rows that are not whole 16-byte multiples are copied
into the workspace, zero padded) in each combination: A only, B only, both,
neither, for every input dtype (4-, 2- and 1-byte elements: 4, 8 and 16
elements per 16-byte chunk), short rows (fewer chunks than a workgroup has
threads) and rows spanning several workgroups, against the oracle.  Both
repacks run as one launch over a flat chunk index, so an operand's first
chunk follows the other's last.
"""
import pytest

import oracle
from gpu_util import compare, run_gemm, to_device
from persistent_stream_tiling_amd import inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

DIST = {"f32": "uniform", "f16": "normal", "bf16": "normal", "i8": "int8"}
V = {"f32": 4, "f16": 8, "bf16": 8, "i8": 16}


def _shapes(dt):
    v = V[dt]
    # (M, N, K) with K (A's rows) and N (B's rows) whole chunks or not
    return {
        "A-only": (150, 32 * v, 5 * v + 3),
        "B-only": (130, 9 * v + 5, 24 * v),
        "both": (203, 7 * v + 1, 3 * v + 1),
        "neither": (96, 16 * v, 8 * v),
        "long-rows": (67, 300 * v + 3, 290 * v + 5),
        "one-col": (77, 1, 41),
    }


CASES = [(dt, name) for dt in ("f32", "f16", "bf16", "i8") for name in _shapes(dt)]


@pytest.mark.parametrize("dt,name", CASES, ids=[f"{d}-{n}" for d, n in CASES])
def test_repack_combinations(dt, name):
    M, N, K = _shapes(dt)[name]
    a, b = inputs.operands(M, N, K, dt, DIST[dt], seed=M * 3 + N + 7 * K)
    ref, scale = oracle.gemm(a, b, dt)
    da, db = to_device(a, dt), to_device(b, dt)
    for schedule in ("dp", "hybrid"):
        plan, ws, c = run_gemm(da, db, M, N, K, dt, schedule)
        info = plan.info
        assert info["pack_a"] == int((K * {"f32": 4, "i8": 1}.get(dt, 2)) % 16 != 0)
        assert info["pack_b"] == int((N * {"f32": 4, "i8": 1}.get(dt, 2)) % 16 != 0)
        compare(c.cpu().numpy(), ref, scale, dt, exact=dt == "i8", what=plan.describe())
        # a second run over the same workspace rewrites the packed copies
        a2, b2 = inputs.operands(M, N, K, dt, DIST[dt], seed=M * 3 + N + 7 * K + 1)
        ref2, scale2 = oracle.gemm(a2, b2, dt)
        c2 = torch.empty_like(c)
        plan.run(to_device(a2, dt), to_device(b2, dt), c2, ws)
        torch.cuda.synchronize()
        compare(c2.cpu().numpy(), ref2, scale2, dt, exact=dt == "i8", what=plan.describe())
