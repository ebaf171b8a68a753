"""Host model of the tau kernel's histogram packing (CPU only).

Per row and bin the kernel keeps two 64-bit words of integer moments of
y = x - lo in fixed point Y = floor(min(y, 1) (2^S - 1)) (so Y < 2^S):
    word 1 = (count << 40) + sum Y,     word 2 = sum Y^2    (both mod 2^64),
and for alpha = 1.5 reads f exactly at every bin edge e from the moments of
the bins above it: f(e) = S2 - 2 e S1 + e^2 C - 1.  tau's bin is the highest
edge with f >= 0 ("AdaSplash-2: The Transformer Revolution We Didn't See
Coming", "Sparse Attention Makes Waves": a coarse histogram of scores kept
on chip starts tau).  With S = 24 a bin holding 65536 or more entries near
y = 1 carries sum Y into the count and wraps sum Y^2; the library takes
S = 24 for N <= 65536 and S = 40 - ceil(log2 N) beyond, which this model
checks never overflows for N <= 2^20 and picks the right bin on a row with
150000 tied scores.
"""
import math

import numpy as np

from oracle import entmax_oracle as O

BINS = 16
M64 = (1 << 64) - 1


def shift_rule(n: int) -> int:
    L = max(1, math.ceil(math.log2(max(n, 2))))
    return 24 if L <= 16 else 40 - L


def packed_bins(y, width, S):
    """The two words per bin as the kernel's integer atomics leave them."""
    w1 = [0] * BINS
    w2 = [0] * BINS
    for yy in y:
        if yy <= 0.0:
            continue
        Y = int(math.floor(min(yy, 1.0) * ((1 << S) - 1)))
        b = min(int(yy * BINS / width), BINS - 1)
        w1[b] = (w1[b] + (1 << 40) + Y) & M64
        w2[b] = (w2[b] + Y * Y) & M64
    return w1, w2


def tau_bin(w1, w2, width, S):
    """Highest bin b whose lower edge has f >= 0 (f exact at the edges)."""
    u = 1.0 / ((1 << S) - 1)
    C = S1 = S2 = 0.0
    for b in range(BINS - 1, -1, -1):
        C += w1[b] >> 40
        S1 += (w1[b] & ((1 << 40) - 1)) * u
        S2 += w2[b] * u * u
        e = b * width / BINS
        if S2 - 2 * e * S1 + e * e * C - 1.0 >= 0.0 or b == 0:
            return b
    return 0


def test_shift_rule_never_overflows():
    for L in range(1, 21):
        n = 1 << L
        S = shift_rule(n)
        assert n * ((1 << S) - 1) < (1 << 40), L          # sum Y stays below the count bits
        assert n * ((1 << S) - 1) ** 2 < (1 << 64), L     # sum Y^2 fits its word
        assert n < (1 << 24)                              # the count fits its 24 bits
    assert shift_rule(65536) == 24 and shift_rule(65537) == 23 and shift_rule(1 << 20) == 20


def test_tied_bin_overflow_and_fix():
    """150000 tied scores just above the lower edge of bin 14 plus ten at the
    row maximum (alpha = 1.5).  The exact tau (sort-based oracle) lies in
    bin 13; a packing with S = 24 overflows and picks another bin, the packing
    with the library's shift picks bin 13."""
    n_tie, n_top = 150000, 10
    n = n_tie + n_top
    width = 1.0 - n ** (1.0 - 1.5)           # hi - lo of the provable bracket
    e14 = 14 * width / BINS
    y = np.concatenate([np.ones(n_top), np.full(n_tie, e14 + 1e-4)])
    x = (y - 1.0)[None, :]                    # x - max x; lo = max x - 1 -> y = x - lo
    tau = O.tau_sort(x, 1.5)[0]
    true_bin = int((tau + 1.0) * BINS / width)
    assert true_bin == 13
    wrapped = tau_bin(*packed_bins(y, width, 24), width, 24)
    assert wrapped != true_bin                # S = 24 overflows at this n
    S = shift_rule(n)
    assert S == 22
    assert tau_bin(*packed_bins(y, width, S), width, S) == true_bin
