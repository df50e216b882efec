"""The pins catch plausible mistakes in the oracle.

Each case copies ``oracle/oracle.c``, plants one mistake by text substitution,
builds the copy with the oracle's own flags into a temporary directory, and
requires that at least one quick pin fails on it.  The unmodified source must
pass the same battery.  Nothing here touches the GPU or the HIP library.
"""
import shutil
from pathlib import Path

import pytest

import oracle
import pins

SRC = Path(oracle.SOURCE).read_text()

BF16_LOOP = ("            for (int j = 1; j < nranks; ++j)\n"
             "                a = a + oracle_widen_bf16(((const uint16_t *)send[j])[i]);")
FP16_LOOP = ("            for (int j = 1; j < nranks; ++j)\n"
             "                a = a + oracle_widen_fp16(((const uint16_t *)send[j])[i]);")
FP32_LOOP = ("            for (int j = 1; j < nranks; ++j)\n"
             "                a = a + ((const float *)send[j])[i];")
BF16_START = "            float a = oracle_widen_bf16(((const uint16_t *)send[0])[i]);"
BF16_OUT = ("            for (int r = 0; r < nranks; ++r)\n"
            "                ((uint16_t *)recv[r])[i] = y;")
BF16_TIE = "    if (dropped > 0x8000u || (dropped == 0x8000u && (kept & 1u)))"
FP16_TIE = "        if (rem > half || (rem == half && (q & 1u)))"

MUTANTS = {
    # summation order and terms
    "bf16 order 0,R-1..1": (BF16_LOOP, BF16_LOOP.replace("send[j]", "send[nranks - j]")),
    "fp32 reversed order": (FP32_LOOP, FP32_LOOP.replace("send[j]", "send[nranks - j]")),
    "bf16 drops last rank": (BF16_LOOP, BF16_LOOP.replace("j < nranks", "j < nranks - 1")),
    "fp16 drops last rank": (FP16_LOOP, FP16_LOOP.replace("j < nranks", "j < nranks - 1")),
    "bf16 subtracts": (BF16_LOOP, BF16_LOOP.replace("a = a +", "a = a -")),
    "fp32 subtracts": (FP32_LOOP, FP32_LOOP.replace("a = a +", "a = a -")),
    "bf16 neighbour index": (BF16_LOOP, BF16_LOOP.replace("send[j])[i]",
                                                          "send[j])[i > 0 ? i - 1 : 0]")),
    "bf16 reads rank 0 twice": (BF16_LOOP, BF16_LOOP.replace("send[j]", "send[j - 1]")),
    # accumulator
    "bf16 starts from +0": (BF16_START, BF16_START.replace("float a = ", "float a = 0.0f + ")),
    "bf16 double accumulator": (BF16_START, BF16_START.replace("float a", "double a")),
    "bf16 accumulates in bf16": (BF16_LOOP, BF16_LOOP.replace(
        "a = a + oracle_widen_bf16(((const uint16_t *)send[j])[i]);",
        "a = oracle_widen_bf16(oracle_rne_bf16(a + oracle_widen_bf16("
        "((const uint16_t *)send[j])[i])));")),
    # output
    "bf16 writes rank 0 only": (BF16_OUT, "            ((uint16_t *)recv[0])[i] = y;"),
    # narrowing
    "bf16 truncates": (BF16_TIE, "    if (0)"),
    "bf16 ties away from zero": (BF16_TIE, "    if (dropped >= 0x8000u)"),
    "bf16 NaN not quieted": ("        return (uint16_t)((u >> 16) | 0x0040u);",
                             "        return (uint16_t)(u >> 16);"),
    "fp16 ties away from zero": (FP16_TIE, "        if (rem >= half)"),
    "fp16 truncates": (FP16_TIE, "        if (0)"),
    "fp16 no gradual underflow": ("    int Q = (E > -14 ? E : -14) - 10;", "    int Q = E - 10;"),
    "fp16 overflow threshold": ("    if (E > 15)", "    if (E >= 15)"),
    "fp16 widening exponent": ("mag = ldexpf((float)(m | 0x400u), (int)e - 25);",
                               "mag = ldexpf((float)(m | 0x400u), (int)e - 24);"),
    "fp16 subnormal widening": ("mag = ldexpf((float)m, -24);", "mag = ldexpf((float)m, -25);"),
    # the hierarchical order
    "grouped partial from +0": ("            part = (l == 0) ? x : part + x;",
                                "            part = (l == 0) ? 0.0f + x : part + x;"),
    "grouped sums groups in reverse": ("    for (int g = 0; g < nranks / group; ++g) {",
                                       "    for (int g = nranks / group - 1; g >= 0; --g) {"),
    "grouped drops the last group": ("    for (int g = 0; g < nranks / group; ++g) {",
                                     "    for (int g = 0; g < nranks / group - 1; ++g) {"),
    "grouped reverses ranks in a node": ("            const int j = g * group + l;",
                                         "            const int j = g * group + (group - 1 - l);"),
    "grouped nodes strided, not consecutive": ("            const int j = g * group + l;",
                                               "            const int j = l * (nranks / group) + g;"),
    "grouped total from +0": ("        total = (g == 0) ? part : total + part;",
                              "        total = total + part;"),
}


def quick_battery(orc):
    """Fast pins; raises AssertionError on the first failure."""
    pins.pin_hand_cases(orc)
    for dtype in ("bf16", "fp16", "fp32"):
        pins.pin_bruteforce_exhaustive(orc, dtype, R=3)
        pins.pin_bruteforce_random(orc, dtype, 8, 3000)
        pins.pin_integer_closed_form(orc, dtype, 8)
        pins.pin_invariants(orc, dtype)
    pins.pin_converters(orc, pins.converter_patterns_sample(n=1 << 18))
    pins.pin_widen_fp16(orc)
    pins.pin_grouped_hand_cases(orc)
    for dtype in ("bf16", "fp32"):
        pins.pin_grouped_random(orc, dtype, 16, 8, 1500)
    pins.pin_grouped_exhaustive(orc, "fp32")


def _build_variant(tmp_path: Path, text: str) -> "oracle.Oracle":
    src = tmp_path / "oracle.c"
    src.write_text(text)
    lib = oracle.build(src, tmp_path / "liboracle_variant.so")
    return oracle.Oracle(lib)


def test_unmodified_source_passes_quick_battery(tmp_path):
    quick_battery(_build_variant(tmp_path, SRC))


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(tmp_path, name):
    find, repl = MUTANTS[name]
    assert SRC.count(find) >= 1, f"mutation anchor for {name!r} not found in oracle.c"
    mutated = SRC.replace(find, repl, 1)
    assert mutated != SRC
    orc = _build_variant(tmp_path, mutated)
    with pytest.raises(AssertionError):
        quick_battery(orc)
    shutil.rmtree(tmp_path, ignore_errors=True)
