"""Helpers for the GPU parity tests: device tensors from seeded bits, one
library run, and the element-wise comparison with the oracle."""
import numpy as np

TOL = {"f32": 1e-5, "f16": 4e-3, "bf16": 4e-3, "i8": 0.0}


def to_device(bits, dtype):
    import torch
    if dtype == "f32":
        t = torch.from_numpy(np.ascontiguousarray(bits).view(np.float32))
    elif dtype == "i8":
        t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int8))
    else:
        t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
        t = t.view(torch.float16 if dtype == "f16" else torch.bfloat16)
    return t.to("cuda")


def run_gemm(a, b, M, N, K, dtype, schedule, ws_cache=None, stream=None, **tiles):
    """C (torch fp32, or int32 for int8, on the GPU) = a @ b through the C ABI for one plan."""
    import torch
    import persistent_stream_tiling_amd as gsk
    plan = gsk.GemmPlan(M, N, K, dtype, schedule, **tiles)
    ws = plan.new_workspace()
    if dtype == "i8":  # int32 C; a sentinel no int8 product of these sizes reaches
        c = torch.full((M, N), -(2 ** 31), dtype=torch.int32, device="cuda")
    else:
        c = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    plan.run(a, b, c, ws, stream=stream)
    torch.cuda.synchronize()
    return plan, ws, c


def compare(c_gpu, ref, scale, dtype, exact=False, what=""):
    """Element-wise check: exact equality, or |C - C_ref| <= tol * S."""
    c = np.asarray(c_gpu, dtype=np.float64)
    assert c.shape == ref.shape
    assert not np.isnan(c).any(), f"{what}: NaN in the output (element not written?)"
    if exact:
        bad = c != ref
        assert not bad.any(), f"{what}: {bad.sum()} elements differ from the exact result, " \
                              f"first at {np.argwhere(bad)[0]}"
        return 0.0
    err = np.abs(c - ref)
    bound = TOL[dtype] * scale
    bad = err > bound
    assert not bad.any(), (f"{what}: {bad.sum()} elements exceed {TOL[dtype]} * S; worst "
                           f"{np.max(err / np.maximum(scale, 1e-300)):.3e}, first at "
                           f"{np.argwhere(bad)[0]}")
    return float(np.max(err / np.maximum(scale, 1e-300)))
