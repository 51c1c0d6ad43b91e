"""ctypes declarations for libgemmsk.so (the C ABI in include/gemm_sk.h)."""
import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libgemmsk.so")

F32, F16, BF16, I8 = 0, 1, 2, 3
DP, PERSISTENT, STREAMK, HYBRID = 0, 1, 2, 3
FLAG_ONE_TILE = 1 << 0
FLAG_NO_XCD_REMAP = 1 << 1
FLAG_FIXUP_HEAD = 1 << 3
FLAG_FIXUP_SPLIT = 1 << 4
FLAG_C_INPUT_DTYPE = 1 << 6
FLAG_DEBUG_DROP_SIGNAL = 1 << 7
FLAG_FIXUP_TWO_KERNEL = 1 << 8
FLAG_STREAM_COPIES = 1 << 9
FLAG_HILBERT_ORDER = 1 << 10
FLAG_PING_PONG = 1 << 11
FLAG_RING_KERNEL = 1 << 12
FLAG_TILE_SPLIT = 1 << 13
ROLE_FULL, ROLE_CONTRIB, ROLE_OWNER = 0, 1, 2
NOALLOC_MAX_WORKSPACE = 80 << 20  # GEMM_NOALLOC_MAX_WORKSPACE

SCHEDULES = {"dp": DP, "persistent": PERSISTENT, "streamk": STREAMK, "hybrid": HYBRID}
DTYPES = {"f32": F32, "f16": F16, "bf16": BF16, "i8": I8}


class Tiles(ctypes.Structure):
    _fields_ = [("bm", ctypes.c_int32), ("bn", ctypes.c_int32), ("bk", ctypes.c_int32),
                ("grid", ctypes.c_int32), ("group_m", ctypes.c_int32), ("flags", ctypes.c_uint32),
                ("wave_m", ctypes.c_int32), ("wave_n", ctypes.c_int32),
                ("stages", ctypes.c_int32)]


class DeviceDesc(ctypes.Structure):
    _fields_ = [("cus", ctypes.c_int32), ("xcds", ctypes.c_int32), ("wg_per_cu", ctypes.c_int32)]


class PlanInfo(ctypes.Structure):
    _fields_ = [("M", ctypes.c_int64), ("N", ctypes.c_int64), ("K", ctypes.c_int64),
                ("dtype", ctypes.c_int32), ("schedule", ctypes.c_int32),
                ("bm", ctypes.c_int32), ("bn", ctypes.c_int32), ("bk", ctypes.c_int32),
                ("group_m", ctypes.c_int32), ("flags", ctypes.c_uint32),
                ("wave_m", ctypes.c_int32), ("wave_n", ctypes.c_int32),
                ("kernel_kind", ctypes.c_int32), ("stages", ctypes.c_int32),
                ("split_fixup", ctypes.c_int32), ("max_pieces", ctypes.c_int32),
                ("tiles_m", ctypes.c_int32), ("tiles_n", ctypes.c_int32),
                ("tiles", ctypes.c_int32), ("iters_per_tile", ctypes.c_int32),
                ("tiles_sk", ctypes.c_int32), ("tiles_dp", ctypes.c_int32),
                ("iters_sk", ctypes.c_int64), ("q", ctypes.c_int32), ("r", ctypes.c_int32),
                ("g", ctypes.c_int32), ("launch_grid", ctypes.c_int32),
                ("threads", ctypes.c_int32), ("cus", ctypes.c_int32), ("xcds", ctypes.c_int32),
                ("wg_capacity", ctypes.c_int32), ("pack_a", ctypes.c_int32),
                ("pack_b", ctypes.c_int32), ("workspace", ctypes.c_size_t),
                ("lds_bytes", ctypes.c_size_t), ("pieces_per_tile", ctypes.c_int32)]

    def as_dict(self):
        return {name: getattr(self, name) for name, _ in self._fields_}


class VariantInfo(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("bm", ctypes.c_int32), ("bn", ctypes.c_int32),
                ("bk", ctypes.c_int32), ("wave_m", ctypes.c_int32), ("wave_n", ctypes.c_int32),
                ("kind", ctypes.c_int32), ("stages", ctypes.c_int32),
                ("stream_copies", ctypes.c_int32), ("threads", ctypes.c_int32),
                ("lds_bytes", ctypes.c_size_t)]

    def as_dict(self):
        return {name: getattr(self, name) for name, _ in self._fields_}


class Segment(ctypes.Structure):
    _fields_ = [("tile", ctypes.c_int32), ("k_begin", ctypes.c_int32), ("k_end", ctypes.c_int32),
                ("role", ctypes.c_int32), ("peer_last", ctypes.c_int32)]


EXPORTS = ("gemm_plan_create", "gemm_plan_create_for_device", "gemm_run", "gemm_run_noalloc",
           "gemm_plan_destroy",
           "gemm_plan_workspace_size", "gemm_plan_describe", "gemm_last_error",
           "gemm_plan_get_info", "gemm_plan_segments", "gemm_plan_tile_coords",
           "gemm_plan_logical_wg", "gemm_workspace_status", "gemm_variant_count",
           "gemm_variant_get")

_lib = None


def load(path=None):
    """Load libgemmsk.so; raises if it has not been built (there is no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    path = path or LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with persistent_stream_tiling_amd._build "
                           "(or __graft_entry__.build()); there is no CPU fallback")
    lib = ctypes.CDLL(path)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    lib.gemm_plan_create.argtypes = [i64, i64, i64, ctypes.c_int, ctypes.c_int,
                                     ctypes.POINTER(Tiles)]
    lib.gemm_plan_create.restype = vp
    lib.gemm_plan_create_for_device.argtypes = [i64, i64, i64, ctypes.c_int, ctypes.c_int,
                                                ctypes.POINTER(Tiles), ctypes.POINTER(DeviceDesc)]
    lib.gemm_plan_create_for_device.restype = vp
    lib.gemm_run.argtypes = [vp, vp, vp, vp, vp, vp]
    lib.gemm_run.restype = ctypes.c_int
    lib.gemm_run_noalloc.argtypes = [vp, vp, vp, vp, vp]
    lib.gemm_run_noalloc.restype = ctypes.c_int
    lib.gemm_plan_destroy.argtypes = [vp]
    lib.gemm_plan_destroy.restype = None
    lib.gemm_plan_workspace_size.argtypes = [vp]
    lib.gemm_plan_workspace_size.restype = ctypes.c_size_t
    lib.gemm_plan_describe.argtypes = [vp, ctypes.c_char_p, ctypes.c_size_t]
    lib.gemm_plan_describe.restype = ctypes.c_int
    lib.gemm_last_error.argtypes = []
    lib.gemm_last_error.restype = ctypes.c_char_p
    lib.gemm_plan_get_info.argtypes = [vp, ctypes.POINTER(PlanInfo)]
    lib.gemm_plan_get_info.restype = ctypes.c_int
    lib.gemm_plan_segments.argtypes = [vp, i32, ctypes.POINTER(Segment), i32]
    lib.gemm_plan_segments.restype = ctypes.c_int
    lib.gemm_plan_tile_coords.argtypes = [vp, i32, ctypes.POINTER(i32), ctypes.POINTER(i32)]
    lib.gemm_plan_tile_coords.restype = ctypes.c_int
    lib.gemm_plan_logical_wg.argtypes = [vp, i32]
    lib.gemm_plan_logical_wg.restype = i32
    lib.gemm_workspace_status.argtypes = [vp, vp, vp, ctypes.POINTER(i32)]
    lib.gemm_workspace_status.restype = ctypes.c_int
    lib.gemm_variant_count.argtypes = []
    lib.gemm_variant_count.restype = i32
    lib.gemm_variant_get.argtypes = [i32, ctypes.POINTER(VariantInfo)]
    lib.gemm_variant_get.restype = ctypes.c_int
    _lib = lib
    return lib


def variants():
    """The compiled kernel table, as dicts (see gemm_variant_info)."""
    lib = load()
    out = []
    for i in range(lib.gemm_variant_count()):
        v = VariantInfo()
        if lib.gemm_variant_get(i, ctypes.byref(v)) != 0:
            raise RuntimeError(last_error())
        out.append(v.as_dict())
    return out


def last_error():
    return load().gemm_last_error().decode(errors="replace")
