"""Seeded cold-start initialisation for k-means (test infrastructure only).

The pages start each chunk's clustering either from the previous chunk's
centroids or, with no cache, from a seeded initial set (163.com article,
section 5; gist.science German summary section 2C).  They do not say how the
seeded set is drawn; the reading taken here is Forgy's method: K distinct token
rows chosen uniformly without replacement.

Random numbers come from SplitMix64 (G. L. Steele, D. Lea, C. H. Flood,
"Fast splittable pseudorandom number generators", OOPSLA 2014): the state
advances by the odd constant 0x9E3779B97F4A7C15 and each output is the state
passed through the 64-bit finaliser (xor-shift 30, multiply by
0xBF58476D1CE4E5B9, xor-shift 27, multiply by 0x94D049BB133111EB,
xor-shift 31).  The K rows are the first K entries of a Fisher-Yates shuffle of
0..N-1 in which step i swaps entry i with entry i + (r_i mod (N - i)).
"""
from __future__ import annotations

from typing import List

MASK64 = (1 << 64) - 1
GAMMA = 0x9E3779B97F4A7C15


def splitmix64_next(state: int):
    """Advance a SplitMix64 state; returns (new_state, 64-bit output)."""
    state = (state + GAMMA) & MASK64
    z = state
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK64
    return state, z ^ (z >> 31)


def forgy_key(seed: int, head: int, stage: int) -> int:
    """Stream key of one (codec seed, head, stage); stage counts from 1."""
    return ((seed * 65536 + head) * 64 + stage) & MASK64


def shuffle_prefix(n: int, k: int, key: int) -> List[int]:
    """First k entries of the keyed partial Fisher-Yates shuffle of 0..n-1.
    When n < k the whole permutation is drawn and entry i is a[i mod n]."""
    a = list(range(n))
    state = key & MASK64
    for i in range(min(k, n)):
        state, r = splitmix64_next(state)
        j = i + r % (n - i)
        a[i], a[j] = a[j], a[i]
    return [a[i % n] for i in range(k)]


def forgy_indices(n: int, k: int, seed: int, head: int, stage: int) -> List[int]:
    """Token rows that seed the k centroids of (head, stage) on a cold start."""
    return shuffle_prefix(n, k, forgy_key(seed, head, stage))
