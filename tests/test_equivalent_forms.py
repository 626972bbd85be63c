"""The GPU path computes some sums in a different form from the oracle's
eager one; each form must give the very same fp results, i.e. the same
grouping of the same operands.  Checked here on the CPU, independently of
both implementations:

- worker counts that are not powers of two: values pushed one at a time into
  a binary-counter stack, the remaining levels folded lowest first, group
  exactly like the pairwise-by-levels sum with an odd tail passing up;
- the server's 8-worker subtree tables: for n = 8, 16, 32, 64, the pairwise
  sum over groups of 8 (each group summed pairwise) is the pairwise sum over
  all n;
- block partials: folding each aligned quad of segment partials as
  ((p0 + p1) + (p2 + p3)) and then summing the quads pairwise (zero padded to
  a power of two) equals the pairwise sum over the segment partials zero
  padded to a power of two, bit for bit.
"""
import random
import struct

import pytest


def pairwise_levels(vals):
    """Pairs (2i, 2i+1) level by level; an odd tail passes up."""
    vals = list(vals)
    while len(vals) > 1:
        nxt = [(vals[2 * i], vals[2 * i + 1]) for i in range(len(vals) // 2)]
        if len(vals) % 2:
            nxt.append(vals[-1])
        vals = nxt
    return vals[0]


def binary_counter_stack(vals):
    """Value w merges with the stack levels given by the trailing one bits of
    w (stack level first, then the carry); the levels left at the end (the set
    bits of n) are folded from the lowest up (higher level first)."""
    stack = {}
    for w, v in enumerate(vals):
        level, x = 0, w
        while x & 1:
            v = (stack.pop(level), v)
            level += 1
            x >>= 1
        stack[level] = v
    acc = None
    for level in sorted(stack):
        acc = stack[level] if acc is None else (stack[level], acc)
    return acc


@pytest.mark.parametrize("n", range(1, 65))
def test_binary_counter_stack_groups_like_pairwise_levels(n):
    assert binary_counter_stack(range(n)) == pairwise_levels(range(n))


@pytest.mark.parametrize("n", [8, 16, 32, 64])
def test_subtree_groups_of_eight(n):
    groups = [pairwise_levels(range(8 * g, 8 * g + 8)) for g in range(n // 8)]
    assert pairwise_levels(groups) == pairwise_levels(range(n))


def pairwise_padded(vals):
    """Pairwise sum (pairs (2i, 2i+1)) over vals zero padded to a power of two."""
    width = 1
    while width < len(vals):
        width *= 2
    v = list(vals) + [0.0] * (width - len(vals))
    while len(v) > 1:
        v = [v[2 * i] + v[2 * i + 1] for i in range(len(v) // 2)]
    return v[0]


def bits(x):
    return struct.pack("<d", x)


@pytest.mark.parametrize("seed", range(8))
def test_block_partials_fold_like_segment_partials(seed):
    rng = random.Random(seed)
    for nseg in list(range(1, 70)) + [rng.randrange(70, 5000) for _ in range(40)]:
        # sums of squares: non-negative, spread over many binades, some zeros
        p = [0.0 if rng.random() < 0.05 else rng.random() * 2.0 ** rng.randrange(-40, 40)
             for _ in range(nseg)]
        padded = p + [0.0] * (-nseg % 4)
        quads = [(padded[4 * i] + padded[4 * i + 1]) + (padded[4 * i + 2] + padded[4 * i + 3])
                 for i in range(len(padded) // 4)]
        assert bits(pairwise_padded(quads)) == bits(pairwise_padded(p)), nseg
