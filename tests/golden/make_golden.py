"""Writes the exact closed-form fixtures in this folder (standard library only).

Uniform causal attention (all queries zero) gives A[q, k] = 1/(q+1) for k <= q,
so at a = 0 (w = 1/2, the H2O limit of the WAITS README's introduction) a KV
head with G query heads scores s[k] = (G/2) (H_N - H_k), H_n the harmonic
numbers; at a -> inf with window b the score is the sum of 1/(q+1) over the
last b rows q >= k.  Values are written as exact fractions.

Run: python tests/golden/make_golden.py
"""
import os
from fractions import Fraction

HERE = os.path.dirname(os.path.abspath(__file__))


def harmonic(n):
    return sum((Fraction(1, i) for i in range(1, n + 1)), Fraction(0))


def main():
    n, group = 12, 4
    with open(os.path.join(HERE, "uniform_h2o_n12_g4.txt"), "w") as f:
        f.write("# uniform attention, a=0 (any b), N=12, G=4: s[k] = (G/2)(H_N - H_k)\n")
        f.write("# written by make_golden.py; one line per key: k numerator/denominator\n")
        hn = harmonic(n)
        for k in range(n):
            v = Fraction(group, 2) * (hn - harmonic(k))
            f.write(f"{k} {v.numerator}/{v.denominator}\n")
    n, window = 12, 5
    with open(os.path.join(HERE, "uniform_snap_n12_w5.txt"), "w") as f:
        f.write("# uniform attention, a=inf, b=5, N=12, G=1: s[k] = sum_{q>=max(k,N-b)} 1/(q+1)\n")
        f.write("# written by make_golden.py; one line per key: k numerator/denominator\n")
        for k in range(n):
            v = sum((Fraction(1, q + 1) for q in range(max(k, n - window), n)), Fraction(0))
            f.write(f"{k} {v.numerator}/{v.denominator}\n")


if __name__ == "__main__":
    main()
