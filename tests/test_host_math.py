"""The division by multiplication the attention kernels use for the piece of a
slot (no integer division before their first loads): for n * d <= 2^32 the
high half of n * m, m = floor((2^32 - 1) / d) + 1, is floor(n / d).  The
host computes m (magic_of in csrc/tree_attn.hip); the kernels take the high
half (div_magic).  Checked here over the whole admissible range by sampling,
at its edges, and for the divisors the configurations use."""
import numpy as np


def magic_of(d):
    return 0 if d <= 1 else (0xFFFFFFFF // d + 1)


def div_magic(n, d):
    return n if d == 1 else (n * magic_of(d)) >> 32


def test_magic_division_exact_on_admissible_range():
    rng = np.random.default_rng(7)
    for d in list(range(1, 300)) + [1023, 1024, 1025, 4095, 65535, 65536, 65537, 1 << 20]:
        nmax = (1 << 32) // d  # n * d <= 2^32
        ns = set(int(x) for x in rng.integers(0, nmax + 1, size=400))
        ns |= {0, 1, d - 1, d, d + 1, nmax - 1, nmax}
        for n in ns:
            if 0 <= n <= nmax:
                assert div_magic(n, d) == n // d, (n, d)


def test_magic_division_fails_far_past_the_bound():
    # the bound matters: near 2^32 the rounding error of m adds up to a whole unit
    d = 7
    wrong = [n for n in range((1 << 32) - 64, 1 << 32) if div_magic(n, d) != n // d]
    assert wrong
