"""gemm_run_noalloc (the entry point for callers that cannot allocate) against
gemm_run with a caller-owned workspace, through the C ABI.

Two calls in a row on the library's per-device array, the second with a
smaller input, each compared bit for bit with gemm_run on the same plan and
element by element with the oracle; plus the size limit, the status read of
the array, and a lost signal on the array followed by a clean call.
"""
import numpy as np
import pytest

import oracle
from gpu_util import compare, to_device
from persistent_stream_tiling_amd import inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import persistent_stream_tiling_amd as gsk  # noqa: E402


def _both(M, N, K, dtype, schedule, **tiles):
    a, b = inputs.operands(M, N, K, dtype, "normal", seed=M + N + K)
    ref, scale = oracle.gemm(a, b, dtype)
    da, db = to_device(a, dtype), to_device(b, dtype)
    plan = gsk.GemmPlan(M, N, K, dtype, schedule, **tiles)
    assert 0 < plan.workspace_bytes <= gsk._lib.NOALLOC_MAX_WORKSPACE
    ws = plan.new_workspace()
    c_ref = torch.full((M, N), float("nan"), device="cuda")
    plan.run(da, db, c_ref, ws)
    c = torch.full((M, N), float("nan"), device="cuda")
    plan.run_noalloc(da, db, c)
    torch.cuda.synchronize()
    assert plan.workspace_status(None) == 0
    return plan, c, c_ref, ref, scale


def test_two_calls_in_a_row_match_gemm_run():
    # first call: many split tiles and a repacked B; second: smaller, fewer
    # workgroups, a different workspace layout over the same array
    first = _both(1000, 777, 1500, "f16", "hybrid", grid=24, bm=128, bn=128,
                  flags=gsk.FLAG_FIXUP_SPLIT)
    second = _both(300, 200, 704, "bf16", "streamk", grid=37, bm=64, bn=64,
                   flags=gsk.FLAG_FIXUP_HEAD)
    for plan, c, c_ref, ref, scale in (first, second):
        assert plan.info["max_pieces"] >= 2
        assert torch.equal(c.view(torch.int32), c_ref.view(torch.int32)), plan.describe()
        compare(c.cpu().numpy(), ref, scale, plan.dtype, what=plan.describe())


def test_plans_without_workspace_and_the_size_limit():
    # a data-parallel plan needs no workspace at all
    M, N, K = 256, 320, 512
    a, b = inputs.operands(M, N, K, "f16", "normal", seed=3)
    ref, scale = oracle.gemm(a, b, "f16")
    plan = gsk.GemmPlan(M, N, K, "f16", "dp", bm=128, bn=128)
    assert plan.workspace_bytes == 0
    c = torch.full((M, N), float("nan"), device="cuda")
    plan.run_noalloc(to_device(a, "f16"), to_device(b, "f16"), c)
    torch.cuda.synchronize()
    compare(c.cpu().numpy(), ref, scale, "f16", what=plan.describe())
    # 256x256 split pieces at g = 256 need 128 MiB of slots: refused, nothing run
    big = gsk.GemmPlan(512, 512, 65536, "bf16", "streamk", bm=256, bn=256,
                       flags=gsk.FLAG_FIXUP_SPLIT)
    assert big.workspace_bytes > gsk._lib.NOALLOC_MAX_WORKSPACE
    with pytest.raises(RuntimeError, match=r"gemm_run_noalloc failed \(-2\)"):
        big.run_noalloc(0, 0, 0)


def test_a_failed_call_leaves_no_state_behind():
    # a lost signal (forced from the host, bounded waits) sets the array's
    # status word; the next call clears it and is exact again
    M, N, K = 256, 512, 16384
    a, b = inputs.operands(M, N, K, "bf16", "int4", seed=41)
    rows, cols = inputs.sample_positions(M, N, 1024, seed=42, tails=True)
    ref, _ = oracle.gemm_sampled(a, b, "bf16", rows, cols)
    da, db = to_device(a, "bf16"), to_device(b, "bf16")
    bad = gsk.GemmPlan(M, N, K, "bf16", "streamk", bm=128, bn=128,
                       flags=gsk.FLAG_FIXUP_SPLIT | gsk.FLAG_DEBUG_DROP_SIGNAL)
    good = gsk.GemmPlan(M, N, K, "bf16", "streamk", bm=128, bn=128, flags=gsk.FLAG_FIXUP_SPLIT)
    c = torch.empty((M, N), device="cuda")
    with pytest.raises(gsk.FixupError):
        bad.run_noalloc(da, db, c)
    assert bad.workspace_status(None) == 1
    good.run_noalloc(da, db, c)
    torch.cuda.synchronize()
    assert good.workspace_status(None) == 0
    compare(c.cpu().numpy()[rows, cols], ref, None, "bf16", exact=True, what=good.describe())
