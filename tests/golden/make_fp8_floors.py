"""Writes tests/golden/fp8_quantisation_floors.txt: for each case of tests/fp8_cases.py, the O RMSE
of exact fp64 attention on the e4m3-dequantised inputs against exact fp64 attention on the
unquantised inputs, over the rows the GPU test checks.  Calls only oracle/ (through
tests/fp8_cases.py) and seeded_inputs/.  Run from the repository root:
    python tests/golden/make_fp8_floors.py"""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from tests import fp8_cases  # noqa: E402

HEADER = """# Quantisation floor of the FP8 parity cases (tests/fp8_cases.py): O RMSE of exact fp64 attention
# on the e4m3-dequantised inputs (the oracle's pre-pass: Hadamard rotation where the case has one,
# per-64-token-block power-of-two scales) against exact fp64 attention on the unquantised bf16
# inputs, over the rows the GPU test checks.  The error measure is the FlashAttention-3 digest's
# (section 3.5, Table 3).  Written by tests/golden/make_fp8_floors.py from oracle/ only.
"""


def main():
    lines = [HEADER]
    for name in fp8_cases.CASES:
        m = fp8_cases.quantisation_floor(*fp8_cases.case(name))
        lines.append(f"{name} {m['rmse']!r}\n")
        print(name, m, flush=True)
    with open(fp8_cases.FLOORS_FILE, "w") as f:
        f.writelines(lines)


if __name__ == "__main__":
    main()
