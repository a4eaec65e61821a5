"""Writes swiglu.txt: hand-worked SwiGLU values from the closed form.

h = silu(g) * u = g * u / (1 + e^(-g)) (SGLang PR #7762, "Cutlass W4A8 MoE":
SiLU and Mul between the two grouped GEMMs; DeepGEMM PR #53, "Changes": L1
GEMM -> SwiGLU).  Each value is evaluated with 60-digit decimal arithmetic
(no floating point, no oracle code) and printed to 25 significant digits;
the test rounds it to fp64 and fp32 itself.

    python tests/golden/make_swiglu_golden.py > tests/golden/swiglu.txt
"""
from decimal import Decimal, getcontext

getcontext().prec = 60

CASES = [("1", "2"), ("-1", "3"), ("0", "5"), ("0.5", "-4"), ("-0.25", "-8"), ("20", "-0.5"),
         ("-30", "1"), ("60", "1"), ("-60", "1"), ("-88", "1000"), ("7.75", "0.125")]


def main():
    print("# SwiGLU h = silu(g) * u = g * u / (1 + exp(-g)), gate g and up u as exact decimals.")
    print("# SGLang PR #7762 \"Cutlass W4A8 MoE\" (SiLU and Mul between the grouped GEMMs);")
    print("# DeepGEMM PR #53 \"Changes\" (L1 GEMM -> SwiGLU).  Evaluated with 60-digit decimal")
    print("# arithmetic by make_swiglu_golden.py; printed to 25 significant digits.")
    print("# g u h")
    for g, u in CASES:
        gd, ud = Decimal(g), Decimal(u)
        h = gd * ud / (1 + (-gd).exp())
        print("%s %s %s" % (g, u, format(h, ".24e")))


if __name__ == "__main__":
    main()
