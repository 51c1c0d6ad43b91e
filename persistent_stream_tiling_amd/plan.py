"""Plan objects and the ``matmul`` convenience call (argument marshalling only)."""
import ctypes

from ._lib import (DTYPES, FLAG_C_INPUT_DTYPE, SCHEDULES, DeviceDesc, PlanInfo, Segment, Tiles,
                   last_error, load)


class FixupError(RuntimeError):
    """A Stream-K fixup wait gave up: the run's C is not valid, and the
    workspace must be zero-filled before it serves another run."""

_TORCH_DTYPES = None


def _torch_dtypes():
    global _TORCH_DTYPES
    if _TORCH_DTYPES is None:
        import torch
        _TORCH_DTYPES = {torch.float32: "f32", torch.float16: "f16", torch.bfloat16: "bf16",
                         torch.int8: "i8"}
    return _TORCH_DTYPES


def _code(table, key, what):
    if isinstance(key, int):
        return key
    try:
        return table[key]
    except KeyError:
        raise ValueError(f"unknown {what} {key!r}; expected one of {sorted(table)}") from None


class GemmPlan:
    """A plan for C = A.B (M x K times K x N) under one schedule.

    ``schedule`` is "dp", "persistent", "streamk" or "hybrid"; ``dtype`` is
    "f32", "f16", "bf16" (fp32 accumulate; C fp32, or the input dtype with
    ``flags=FLAG_C_INPUT_DTYPE``) or "i8" (exact int32 accumulate, int32 C).
    Tile knobs default to the library's choice.  With ``device`` =
    (cus, xcds, wg_per_cu) the plan is made for a described device without
    touching a GPU (inspection only).
    """

    def __init__(self, M, N, K, dtype, schedule="hybrid", bm=0, bn=0, bk=0, grid=0, group_m=0,
                 flags=0, wave_m=0, wave_n=0, stages=0, device=None):
        self._lib = load()
        self._h = None
        tiles = Tiles(bm, bn, bk, grid, group_m, flags, wave_m, wave_n, stages)
        d = _code(DTYPES, dtype, "dtype")
        s = _code(SCHEDULES, schedule, "schedule")
        if device is not None:
            desc = DeviceDesc(*device)
            h = self._lib.gemm_plan_create_for_device(M, N, K, d, s, ctypes.byref(tiles),
                                                      ctypes.byref(desc))
        else:
            h = self._lib.gemm_plan_create(M, N, K, d, s, ctypes.byref(tiles))
        if not h:
            raise ValueError(f"gemm_plan_create failed: {last_error()}")
        self._h = h
        info = PlanInfo()
        if self._lib.gemm_plan_get_info(h, ctypes.byref(info)) != 0:
            raise RuntimeError(last_error())
        self.info = info.as_dict()
        self.M, self.N, self.K = M, N, K
        self.dtype = dtype if isinstance(dtype, str) else {v: k for k, v in DTYPES.items()}[d]
        self.schedule = schedule
        self.workspace_bytes = int(self._lib.gemm_plan_workspace_size(h))
        # a run can end with a fixup wait that gave up only when workgroups
        # wait on each other's pieces: some tile split, in-kernel fixup
        self.may_wait = (self.info["tiles_sk"] > 0 and self.info["max_pieces"] >= 2
                         and self.info["split_fixup"] != 2)

    # -- introspection --------------------------------------------------
    def describe(self):
        n = self._lib.gemm_plan_describe(self._h, None, 0)
        buf = ctypes.create_string_buffer(n + 1)
        self._lib.gemm_plan_describe(self._h, buf, n + 1)
        return buf.value.decode()

    def segments(self, wg):
        """[(tile, k_begin, k_end, role, peer_last), ...] of logical workgroup wg."""
        n = self._lib.gemm_plan_segments(self._h, wg, None, 0)
        if n < 0:
            raise ValueError(last_error())
        arr = (Segment * max(n, 1))()
        self._lib.gemm_plan_segments(self._h, wg, arr, n)
        return [(s.tile, s.k_begin, s.k_end, s.role, s.peer_last) for s in arr[:n]]

    def tile_coords(self, t):
        tm, tn = ctypes.c_int32(), ctypes.c_int32()
        if self._lib.gemm_plan_tile_coords(self._h, t, ctypes.byref(tm), ctypes.byref(tn)):
            raise ValueError(last_error())
        return tm.value, tn.value

    def logical_wg(self, hw):
        v = self._lib.gemm_plan_logical_wg(self._h, hw)
        if v < 0:
            raise ValueError(last_error())
        return v

    # -- execution ------------------------------------------------------
    def new_workspace(self, device=None):
        """A zero-filled workspace tensor (None when the plan needs none)."""
        if self.workspace_bytes == 0:
            return None
        import torch
        return torch.zeros(self.workspace_bytes, dtype=torch.uint8,
                           device=device or torch.device("cuda"))

    def run(self, A, B, C, workspace=None, stream=None, check=True):
        """Enqueue C = A.B on ``stream`` (default: torch's current stream).

        A, B, C and workspace are torch tensors (or raw device addresses).
        With ``check`` (the default) and a plan whose workgroups wait on each
        other (``may_wait``), the workspace status is read after the run,
        which synchronizes the stream, and a fixup wait that gave up raises
        FixupError.  ``check=False`` keeps the call asynchronous (the caller
        then reads ``workspace_status`` itself)."""
        import torch

        def ptr(x):
            if x is None:
                return None
            return x.data_ptr() if isinstance(x, torch.Tensor) else int(x)

        if stream is None:
            stream = torch.cuda.current_stream().cuda_stream
        elif isinstance(stream, torch.cuda.Stream):
            stream = stream.cuda_stream
        rc = self._lib.gemm_run(self._h, ptr(A), ptr(B), ptr(C), ptr(workspace), stream)
        if rc != 0:
            raise RuntimeError(f"gemm_run failed ({rc}): {last_error()}")
        if check and self.may_wait:
            st = self._status(ptr(workspace), stream)
            if st != 0:
                raise FixupError(f"a Stream-K fixup wait gave up (workspace status {st}): C is "
                                 "not valid and the workspace must be zero-filled again; "
                                 f"plan: {self.describe()}")

    def run_noalloc(self, A, B, C, stream=None, check=True):
        """Enqueue C = A.B through gemm_run_noalloc: no workspace argument, no
        allocation (the library's fixed per-device array serves as the
        workspace; calls that overlap in time on one device race).  ``check``
        as in ``run``."""
        import torch

        def ptr(x):
            return x.data_ptr() if isinstance(x, torch.Tensor) else int(x)

        if stream is None:
            stream = torch.cuda.current_stream().cuda_stream
        elif isinstance(stream, torch.cuda.Stream):
            stream = stream.cuda_stream
        rc = self._lib.gemm_run_noalloc(self._h, ptr(A), ptr(B), ptr(C), stream)
        if rc != 0:
            raise RuntimeError(f"gemm_run_noalloc failed ({rc}): {last_error()}")
        if check and self.may_wait:
            st = self._status(None, stream)
            if st != 0:
                raise FixupError(f"a Stream-K fixup wait gave up (status {st}): C is not valid; "
                                 f"plan: {self.describe()}")

    def _status(self, ws_ptr, stream_handle):
        st = ctypes.c_int32()
        rc = self._lib.gemm_workspace_status(self._h, ws_ptr, stream_handle, ctypes.byref(st))
        if rc:
            raise RuntimeError(last_error())
        return st.value

    def workspace_status(self, workspace, stream=None):
        """Synchronously read the workspace status word (0 ok, 1 a fixup wait gave up)."""
        import torch
        if stream is None:
            stream = torch.cuda.current_stream().cuda_stream
        elif isinstance(stream, torch.cuda.Stream):
            stream = stream.cuda_stream
        ws = workspace.data_ptr() if workspace is not None else None
        return self._status(ws, stream)

    def close(self):
        if self._h:
            self._lib.gemm_plan_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def plan_for_device(M, N, K, dtype, schedule, cus=256, xcds=8, wg_per_cu=1, **tiles):
    """A plan for a described device (no GPU needed); for inspecting schedules."""
    return GemmPlan(M, N, K, dtype, schedule, device=(cus, xcds, wg_per_cu), **tiles)


_PLANS = {}


def matmul(a, b, schedule="hybrid", out_dtype=None, **tiles):
    """C = a @ b for contiguous CUDA tensors a (M x K) and b (K x N) of
    float32, float16, bfloat16 or int8, through the library's kernels.  C is
    fp32, or a's dtype when ``out_dtype`` is a's dtype (fp32 sums rounded to
    nearest even as they are stored); int32 for int8 inputs.

    Plans and their zero-filled workspaces are cached per shape, dtype,
    schedule, knobs, device and stream, so calls on different streams never
    share a workspace.  The call reads the workspace status after any run
    whose workgroups wait on each other (it then synchronizes the stream) and
    raises FixupError if a fixup wait gave up; the cached workspace is
    zero-filled again first, so the next call starts clean."""
    import torch
    if a.dim() != 2 or b.dim() != 2 or a.shape[1] != b.shape[0]:
        raise ValueError(f"incompatible shapes {tuple(a.shape)} and {tuple(b.shape)}")
    if a.dtype != b.dtype or a.dtype not in _torch_dtypes():
        raise ValueError(f"unsupported dtypes {a.dtype}, {b.dtype}")
    if not (a.is_cuda and b.is_cuda):
        raise ValueError("a and b must be on the GPU")
    if a.dtype == torch.int8:
        if out_dtype not in (None, torch.int32):
            raise ValueError("int8 products are int32")
    elif out_dtype not in (None, torch.float32, a.dtype):
        raise ValueError(f"out_dtype must be float32 or {a.dtype}, got {out_dtype}")
    if out_dtype == a.dtype and a.dtype != torch.float32:
        tiles["flags"] = tiles.get("flags", 0) | FLAG_C_INPUT_DTYPE
    a, b = a.contiguous(), b.contiguous()
    M, K = a.shape
    N = b.shape[1]
    stream = torch.cuda.current_stream(a.device)
    key = (M, N, K, a.dtype, schedule, tuple(sorted(tiles.items())), a.device.index,
           stream.cuda_stream)
    entry = _PLANS.get(key)
    if entry is None:
        plan = GemmPlan(M, N, K, _torch_dtypes()[a.dtype], schedule, **tiles)
        entry = (plan, plan.new_workspace(a.device))
        _PLANS[key] = entry
    plan, ws = entry
    c_half = tiles.get("flags", 0) & FLAG_C_INPUT_DTYPE
    c_type = torch.int32 if a.dtype == torch.int8 else (a.dtype if c_half else torch.float32)
    c = torch.empty((M, N), dtype=c_type, device=a.device)
    try:
        plan.run(a, b, c, ws, stream=stream)
    except FixupError:
        ws.zero_()
        raise
    return c
