"""The planner's default Stream-K / hybrid plans (fp16/bf16, no tile, grid 0)
against the oracle: the cost model picks tiles of 256x256, 256x128 or 128x128
and g = s*T aligned splits (up to 16 pieces per tile) or one workgroup per CU.

Shapes: log-sampled ones (the distribution the model was fitted on) and
ragged ones (repacked operands, partial tiles), small enough for the full
oracle, in both schedules and both input dtypes.
"""
import pytest

import oracle
from gpu_util import compare, run_gemm, to_device
from persistent_stream_tiling_amd import grid_model, inputs
from persistent_stream_tiling_amd.inputs import log_sampled_shapes

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)


def _shapes():
    # the smallest log-sampled shapes (whole-matrix oracle in well under a
    # second each; four of them pick 64x64 tiles), then ragged ones
    small = sorted(set(log_sampled_shapes(200, seed=11)), key=lambda s: (s[0] * s[1] * s[2], s))[:8]
    # larger ones whose picks are 256x256 tiles, 128x128 at g = CUs or crossing ranges
    larger = [(1536, 1536, 8192), (3328, 768, 1792), (2048, 2048, 1024), (768, 256, 5632)]
    return small + larger + [(257, 203, 701), (1000, 300, 4100), (130, 2050, 640),
                             (520, 260, 9000)]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("shape", _shapes(), ids=lambda s: "x".join(map(str, s)))
def test_default_plans_match_the_oracle(shape, dtype):
    M, N, K = shape
    a, b = inputs.operands(M, N, K, dtype, "normal", seed=M * 7 + N * 3 + K)
    ref, scale = oracle.gemm(a, b, dtype)
    da, db = to_device(a, dtype), to_device(b, dtype)
    pick = grid_model.choose(M, N, K)
    for schedule in ("streamk", "hybrid"):
        plan, ws, c = run_gemm(da, db, M, N, K, dtype, schedule)
        if pick is not None:
            assert (plan.info["bm"], plan.info["bn"], plan.info["g"]) == pick, plan.describe()
        compare(c.cpu().numpy(), ref, scale, dtype, what=plan.describe())
        if ws is not None:
            assert plan.workspace_status(ws) == 0


@pytest.mark.parametrize("shape", [(4352, 4352, 640), (4160, 4224, 1000), (6400, 6208, 320)],
                         ids=lambda s: "x".join(map(str, s)))
def test_default_hybrid_above_the_model(shape):
    # more than 256 tiles for every tile shape: the default hybrid keeps one
    # Stream-K wave (T mod g tiles) and cuts each of its tiles into its own pieces
    M, N, K = shape
    a, b = inputs.operands(M, N, K, "f16", "normal", seed=M + N + K)
    ref, scale = oracle.gemm(a, b, "f16")
    plan, ws, c = run_gemm(to_device(a, "f16"), to_device(b, "f16"), M, N, K, "f16", "hybrid")
    info = plan.info
    assert grid_model.choose(M, N, K) is None
    assert 0 < info["tiles_sk"] <= info["g"] and info["pieces_per_tile"] >= 2, plan.describe()
    compare(c.cpu().numpy(), ref, scale, "f16", what=plan.describe())
    assert plan.workspace_status(ws) == 0
