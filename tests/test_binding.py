"""The Python binding's run() logic on the CPU, with the library's launch and
status calls replaced by stubs: a run of a plan whose workgroups wait on each
other reads the workspace status and raises when a fixup wait gave up; a
plan that cannot wait, or check=False, never reads it."""
import pytest

import persistent_stream_tiling_amd as gsk


class _StubLib:
    """Forwards to the real library, except the launch and the status read."""

    def __init__(self, real, status):
        self._real, self.status, self.status_reads, self.runs = real, status, 0, 0

    def gemm_run(self, *args):
        self.runs += 1
        return 0

    def gemm_workspace_status(self, plan, ws, stream, out):
        self.status_reads += 1
        out._obj.value = self.status  # out is ctypes.byref(c_int32)
        return 0

    def __getattr__(self, name):
        return getattr(self._real, name)


def _plan(**kw):
    return gsk.plan_for_device(256, 512, 65536, "bf16", "streamk", bm=128, bn=128, **kw)


def test_run_raises_when_the_status_says_a_wait_gave_up():
    plan = _plan(flags=gsk.FLAG_FIXUP_SPLIT)
    assert plan.may_wait
    stub = _StubLib(plan._lib, status=1)
    plan._lib = stub
    with pytest.raises(gsk.FixupError, match="gave up"):
        plan.run(0x1000, 0x2000, 0x3000, 0x4000, stream=0)
    assert stub.status_reads == 1
    stub.status = 0
    plan.run(0x1000, 0x2000, 0x3000, 0x4000, stream=0)
    assert stub.status_reads == 2
    # check=False keeps the call asynchronous: no status read
    stub.status = 1
    plan.run(0x1000, 0x2000, 0x3000, 0x4000, stream=0, check=False)
    assert stub.status_reads == 2 and stub.runs == 3
    plan._lib = stub._real


@pytest.mark.parametrize("kw", [dict(schedule="dp"), dict(flags=gsk.FLAG_FIXUP_TWO_KERNEL)],
                         ids=["no-split", "two-kernel"])
def test_plans_that_never_wait_skip_the_status_read(kw):
    sched = kw.pop("schedule", "streamk")
    plan = gsk.plan_for_device(256, 512, 65536, "bf16", sched, bm=128, bn=128, **kw)
    assert not plan.may_wait
    stub = _StubLib(plan._lib, status=1)
    plan._lib = stub
    plan.run(0x1000, 0x2000, 0x3000, 0x4000, stream=0)
    assert stub.status_reads == 0
    plan._lib = stub._real
