"""Independent brute-force references for tiny inputs (exact arithmetic).

Nothing here shares code with the oracle or the HIP library.  These are the
definitions written out with Python integers / Fractions and exhaustive
enumeration, used to pin the oracle on inputs small enough to enumerate.
"""
from fractions import Fraction
from itertools import combinations

import numpy as np


def bf16_bits_to_fraction(h: int) -> Fraction:
    """Exact value of a bf16 bit pattern (finite)."""
    u = (int(h) & 0xFFFF) << 16
    return Fraction(float(np.array([u], dtype=np.uint32).view(np.float32)[0]))


def f32_to_fraction(x) -> Fraction:
    return Fraction(float(np.float32(x)))


def exact_nearest(x_bits, beacons):
    """Argmax of cosine(x, b_j) with exact rationals; ties -> lowest j.

    Zero norm on either side counts as cosine 0.  Comparison of
    a/sqrt(A) with c/sqrt(C) (A, C > 0) is done on signs and squares.
    """
    x = [bf16_bits_to_fraction(v) for v in x_bits]
    xx = sum(v * v for v in x)
    best_j, best = None, None          # best = (dot, norm2) or zero

    def cos_key(j):
        b = [f32_to_fraction(v) for v in beacons[j]]
        bb = sum(v * v for v in b)
        if xx == 0 or bb == 0:
            return (Fraction(0), Fraction(1))
        return (sum(p * q for p, q in zip(x, b)), bb)

    def greater(a, c):
        """cos a > cos c, each given as (dot, norm2) with cos = dot/sqrt(norm2)."""
        (da, na), (dc, nc) = a, c
        if da >= 0 and dc < 0:
            return da > 0 or dc < 0
        if da < 0 and dc >= 0:
            return False
        if da >= 0:       # both non-negative
            return da * da * nc > dc * dc * na
        return da * da * nc < dc * dc * na   # both negative

    for j in range(len(beacons)):
        k = cos_key(j)
        if best is None or greater(k, best):
            best_j, best = j, k
    return best_j


def topk_by_dominance(scores, P, B):
    """All B-P subsets S of candidates [P, N) such that every member beats
    every non-member under (higher score, then lower slot).  For a strict
    total order exactly one such subset exists; returns the list of them."""
    N = P + len(scores)
    k = B - P
    cands = list(range(P, N))

    def beats(a, b):
        sa, sb = scores[a - P], scores[b - P]
        return sa > sb or (sa == sb and a < b)

    found = []
    for S in combinations(cands, k):
        sset = set(S)
        if all(beats(a, b) for a in S for b in cands if b not in sset):
            found.append(sorted(S))
    return found
