"""The built-in schedule table's entries, parsed from its source file."""
import os
import re

import mixed_precision_quantized_prepack_amd as w4

TABLE = os.path.join(os.path.dirname(w4.LIB_PATH), "csrc", "w4_schedule_table.inc")
_ENTRY = re.compile(r"\s*\{(\w+), " + ", ".join([r"(\d+)"] * 9) + r"\},")


def builtin_schedule_entries():
    """(a_dtype, grouped, N, K, m_lo, m_hi, path, splitk, tile_m, strips) tuples."""
    names = {"W4_I8": w4.I8, "W4_FP8_E4M3": w4.FP8_E4M3, "W4_F16": w4.F16, "W4_BF16": w4.BF16}
    out = []
    with open(TABLE) as f:
        for line in f:
            m = _ENTRY.match(line)
            if m:
                out.append((names[m.group(1)], *map(int, m.groups()[1:])))
    return out
