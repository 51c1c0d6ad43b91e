"""Static checks on the HIP sources (no GPU)."""
import glob
import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SOURCES = sorted(glob.glob(os.path.join(ROOT, "persistent_stream_tiling_amd", "csrc", "*.hip")) +
                 glob.glob(os.path.join(ROOT, "persistent_stream_tiling_amd", "csrc", "*.h")))


def test_no_bit_cast_of_subscripted_vector_element():
    # hipcc lowered __builtin_bit_cast(T, v[i]) on a vector lvalue to a read of
    # v[0]; this produced wrong fp32 MFMA operands and wrong stores before.
    bad = re.compile(r"__builtin_bit_cast\(\s*[\w:]+\s*,\s*[\w.]+(\[[^\]]*\])+\s*\)")
    hits = []
    for path in SOURCES:
        for n, line in enumerate(open(path), 1):
            if bad.search(line):
                hits.append(f"{os.path.basename(path)}:{n}: {line.strip()}")
    assert not hits, "\n".join(hits)
