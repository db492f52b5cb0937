"""Pure-Python brute-force checkers used to pin the oracle.

Nothing here imports the oracle or the HIP library: these are independent,
deliberately naive formulations of what the W12 pages fix (a 16-binade window
per output channel with the fewest out-of-window weights; an exact GEMM), fed
the same inputs.
"""
from fractions import Fraction


def bf16_exponent(u: int) -> int:
    return (u >> 7) & 0xFF


def bf16_fraction(u: int) -> Fraction:
    """Exact rational value of a finite bfloat16 bit pattern."""
    s = -1 if (u >> 15) & 1 else 1
    e = (u >> 7) & 0xFF
    m = u & 0x7F
    if e == 255:
        raise ValueError("non-finite")
    if e == 0:
        return s * Fraction(m, 128) * Fraction(2) ** -126
    return s * (1 + Fraction(m, 128)) * Fraction(2) ** (e - 127)


def misses(row, b: int) -> int:
    """Weights of ``row`` whose exponent field lies outside [b, b+15], or that are not normal."""
    n = 0
    for u in row:
        e = bf16_exponent(u)
        if not (1 <= e <= 254 and b <= e <= b + 15):
            n += 1
    return n


def best_window(row):
    """(smallest b in 1..239 with the fewest misses, that number): a literal double loop."""
    best_b, best_n = None, None
    for b in range(1, 240):
        n = misses(row, b)
        if best_n is None or n < best_n:
            best_b, best_n = b, n
    return best_b, best_n


def exact_gemm(x_rows, w_rows):
    """y[m][n] = sum_k x[m][k] * W[n][k] as exact Fractions (finite bf16 inputs)."""
    xs = [[bf16_fraction(u) for u in r] for r in x_rows]
    ws = [[bf16_fraction(u) for u in r] for r in w_rows]
    return [[sum((a * b for a, b in zip(xr, wr)), Fraction(0)) for wr in ws] for xr in xs]


def truncate_mantissa_3(u: int) -> Fraction:
    """Value of a normal bf16 weight with its mantissa cut to 3 bits, computed arithmetically:
    sign * floor(|w| / 2^(e-127-3)) * 2^(e-127-3)."""
    v = bf16_fraction(u)
    e = bf16_exponent(u)
    ulp = Fraction(2) ** (e - 127 - 3)
    mag = abs(v)
    q = (mag // ulp) * ulp
    return q if v >= 0 else -q
