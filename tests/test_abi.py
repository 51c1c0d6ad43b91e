"""The C-ABI library builds, loads and exports every symbol its header declares (no GPU)."""
import ctypes
import os
import re
import subprocess

import pytest

import persistent_stream_tiling_amd as gsk
from persistent_stream_tiling_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gemm_sk.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gemm_\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("gemm_plan_create", "gemm_run", "gemm_plan_destroy",
                     "gemm_plan_workspace_size", "gemm_plan_describe", "gemm_last_error"):
        assert required in names
    assert set(names) == set(_lib.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(_lib.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_structs_match_header_layout(tmp_path):
    # the ctypes mirrors against what a C compiler makes of the header
    src = tmp_path / "sizes.c"
    src.write_text("""#include <stdio.h>
#include <stddef.h>
#include "gemm_sk.h"
int main(void) {
  printf("%zu %zu %zu %zu %zu %zu %zu\\n", sizeof(gemm_tiles), sizeof(gemm_device_desc),
         sizeof(gemm_segment), sizeof(gemm_plan_info), offsetof(gemm_plan_info, iters_sk),
         offsetof(gemm_plan_info, workspace), offsetof(gemm_plan_info, lds_bytes));
  return 0;
}
""")
    exe = tmp_path / "sizes"
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)],
                   check=True)
    got = [int(v) for v in subprocess.run([str(exe)], capture_output=True, text=True,
                                          check=True).stdout.split()]
    want = [ctypes.sizeof(_lib.Tiles), ctypes.sizeof(_lib.DeviceDesc),
            ctypes.sizeof(_lib.Segment), ctypes.sizeof(_lib.PlanInfo),
            _lib.PlanInfo.iters_sk.offset, _lib.PlanInfo.workspace.offset,
            _lib.PlanInfo.lds_bytes.offset]
    assert got == want


def test_no_gpu_means_no_plan_and_a_message():
    # on a machine without a GPU gemm_plan_create must fail cleanly, never fall back
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    with pytest.raises(ValueError, match="gemm_plan_create failed"):
        gsk.GemmPlan(64, 64, 64, "f16", "dp")


def test_destroy_null_and_describe_null_are_safe():
    lib = gsk.load()
    lib.gemm_plan_destroy(None)
    assert lib.gemm_plan_describe(None, None, 0) == -1
    assert lib.gemm_plan_workspace_size(None) == 0


def test_header_flag_values_match_the_binding():
    # every GEMM_FLAG_* in the header has the same bit in the Python binding
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    flags = dict(re.findall(r"GEMM_FLAG_(\w+)\s*=\s*1u\s*<<\s*(\d+)", text))
    assert flags
    for name, bit in flags.items():
        assert getattr(_lib, "FLAG_" + name) == 1 << int(bit), name


def test_plan_describes_its_output_dtype():
    plan = gsk.plan_for_device(300, 200, 704, "f16", "hybrid", bm=128, bn=128)
    assert " C=f32 " in plan.describe()
    plan = gsk.plan_for_device(300, 200, 704, "bf16", "hybrid", bm=128, bn=128,
                               flags=gsk.FLAG_C_INPUT_DTYPE)
    assert " C=bf16 " in plan.describe()
    assert plan.info["flags"] & gsk.FLAG_C_INPUT_DTYPE


def test_variant_table_is_exported_and_each_entry_selectable():
    vs = gsk.variants()
    assert len(vs) == gsk.load().gemm_variant_count() > 0
    names = {0: "f32", 1: "f16", 2: "bf16", 3: "i8"}
    seen = set()
    for v in vs:
        key = (v["dtype"], v["bm"], v["bn"], v["wave_m"], v["wave_n"], v["stream_copies"],
               v["kind"])
        assert key not in seen, f"two table entries for {key}"
        seen.add(key)
        flags = (gsk.FLAG_STREAM_COPIES if v["stream_copies"] else 0) | \
            (gsk.FLAG_PING_PONG if v["kind"] == 3 else 0) | \
            (gsk.FLAG_RING_KERNEL if v["kind"] == 2 else 0)
        plan = gsk.plan_for_device(1000, 1000, 1000, names[v["dtype"]], "dp", bm=v["bm"],
                                   bn=v["bn"], wave_m=v["wave_m"], wave_n=v["wave_n"],
                                   stages=v["stages"], flags=flags)
        info = plan.info
        assert (info["bm"], info["bn"], info["bk"], info["wave_m"], info["wave_n"],
                info["kernel_kind"], info["stages"], info["threads"]) == \
            (v["bm"], v["bn"], v["bk"], v["wave_m"], v["wave_n"], v["kind"], v["stages"],
             v["threads"])
    lib = gsk.load()
    assert lib.gemm_variant_get(len(vs), None) == -1
    assert lib.gemm_variant_get(-1, None) == -1


def test_reserved_flag_bits_are_refused():
    for bit in (2, 5):
        with pytest.raises(ValueError, match="reserved"):
            gsk.plan_for_device(300, 200, 704, "f16", "dp", flags=1 << bit)


def test_output_offsets_stay_within_32_bits():
    # one tile's rows of C are addressed with 32-bit byte offsets, kept below
    # 2^30: 256 rows of 2^20 fp32 values reach it and are refused, 2^20 - 256
    # columns stay below it
    with pytest.raises(ValueError, match="32-bit"):
        gsk.plan_for_device(256, 1 << 22, 64, "f16", "dp", bm=256, bn=256)
    with pytest.raises(ValueError, match="32-bit"):
        gsk.plan_for_device(256, 1 << 20, 64, "f16", "dp", bm=256, bn=256)
    ok = gsk.plan_for_device(256, (1 << 20) - 256, 64, "f16", "dp", bm=256, bn=256)
    assert ok.info["N"] == (1 << 20) - 256
    # with fp16 C the same row block holds twice the columns
    ok = gsk.plan_for_device(256, (1 << 21) - 256, 64, "f16", "dp", bm=256, bn=256,
                             flags=gsk.FLAG_C_INPUT_DTYPE)
    assert ok.info["N"] == (1 << 21) - 256


def test_ping_pong_is_the_256x256_default():
    for dt in ("f16", "bf16"):
        p = gsk.plan_for_device(4096, 4096, 4096, dt, "dp", bm=256, bn=256)
        assert p.info["kernel_kind"] == 3 and "pingpong" in p.describe()
        assert gsk.plan_for_device(4096, 4096, 4096, dt, "dp", bm=256, bn=256,
                                   flags=gsk.FLAG_RING_KERNEL).info["kernel_kind"] == 2
        # other tiles, the non-temporal copies and other wave layouts: the ring kernel
        assert gsk.plan_for_device(4096, 4096, 4096, dt, "dp", bm=256, bn=128).info["kernel_kind"] == 2
        assert gsk.plan_for_device(4096, 4096, 4096, dt, "dp", bm=256, bn=256,
                                   flags=gsk.FLAG_STREAM_COPIES).info["kernel_kind"] == 2
        with pytest.raises(ValueError, match="no kernel"):
            gsk.plan_for_device(4096, 4096, 4096, dt, "dp", bm=128, bn=128,
                                flags=gsk.FLAG_PING_PONG)
    with pytest.raises(ValueError, match="exclude"):
        gsk.plan_for_device(4096, 4096, 4096, "f16", "dp", bm=256, bn=256,
                            flags=gsk.FLAG_PING_PONG | gsk.FLAG_RING_KERNEL)
    # int8 at 256x256: the ping-pong kernel; its other tile and GEMM_FLAG_RING_KERNEL
    # (no int8 ring kernel) take the register-staged one, as fp32 always does
    p = gsk.plan_for_device(1024, 1024, 1024, "i8", "dp", bm=256, bn=256)
    assert p.info["kernel_kind"] == 3 and p.info["bk"] == 128
    assert gsk.plan_for_device(1024, 1024, 1024, "i8", "dp", bm=128, bn=128).info["kernel_kind"] == 0
    assert gsk.plan_for_device(1024, 1024, 1024, "i8", "dp", bm=256, bn=256,
                               flags=gsk.FLAG_RING_KERNEL).info["kernel_kind"] == 0
