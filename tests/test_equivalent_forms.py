"""The GPU path computes some sums in a different form from the oracle's
eager one; each form must give the very same fp results, i.e. the same
grouping of the same operands.  Checked here on the CPU, independently of
both implementations:

- worker counts that are not powers of two: values pushed one at a time into
  a binary-counter stack, the remaining levels folded lowest first, group
  exactly like the pairwise-by-levels sum with an odd tail passing up;
- the server's subtree tables: for n = 8, 16, 32, 64, the pairwise sum over
  groups of 8, each group the sum of its two quads (each quad summed
  pairwise), is the pairwise sum over all n;
- the server's 64x64 bit transpose as the kernel builds it from gfx950's
  cross-lane operations (permlane32/16 swaps, DPP row_ror:8, row_half_mirror
  and quad_perm, byte permutes with per-lane selectors), emulated with the
  lane semantics those operations showed on the device: it is the
  transpose;
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


@pytest.mark.parametrize("n", [8, 16, 32, 64])
def test_group_of_eight_is_its_two_quads(n):
    quads = [pairwise_levels(range(4 * t, 4 * t + 4)) for t in range(n // 4)]
    groups = [(quads[2 * g], quads[2 * g + 1]) for g in range(n // 8)]
    assert pairwise_levels(groups) == pairwise_levels(range(n))


# --- the bit transpose, one 32-bit register per lane per list entry ---

M32 = 0xFFFFFFFF


def permlane32_swap(a, b):
    """(a', b'): a's upper 32 lanes trade places with b's lower 32 lanes."""
    return ([a[i] if i < 32 else b[i - 32] for i in range(64)],
            [a[i + 32] if i < 32 else b[i] for i in range(64)])


def permlane16_swap(a, b):
    """(a', b'): a's odd 16-lane rows trade places with b's even rows."""
    return ([b[i - 16] if i & 16 else a[i] for i in range(64)],
            [b[i] if i & 16 else a[i + 16] for i in range(64)])


def dpp_row_ror8(x):
    return [x[(i & ~15) | ((i + 8) & 15)] for i in range(64)]


def dpp_half_mirror(x):
    return [x[(i & ~7) | (7 - (i & 7))] for i in range(64)]


def dpp_quad(x, sel):
    return [x[(i & ~3) | sel[i & 3]] for i in range(64)]


def perm_b32(s0, s1, sel):
    """v_perm_b32: selector bytes 0-3 take s1's bytes, 4-7 s0's."""
    src = (s0 << 32) | s1
    return sum(((src >> (8 * ((sel >> (8 * k)) & 0xFF))) & 0xFF) << (8 * k) for k in range(4))


def rotr(x, k):
    return ((x >> k) | (x << (32 - k))) & M32


def stage(x, k):
    if k == 16:
        a, b = permlane16_swap(x, x)
        return [perm_b32(b[i], a[i], 0x07060302 if i & 16 else 0x05040100) for i in range(64)]
    if k == 8:
        p = dpp_row_ror8(x)
        return [perm_b32(p[i], x[i], 0x03070105 if i & 8 else 0x06020400) for i in range(64)]
    high = {4: 0xF0F0F0F0, 2: 0xCCCCCCCC, 1: 0xAAAAAAAA}[k]
    if k == 4:
        p = dpp_quad(dpp_half_mirror(x), [3, 2, 1, 0])
    elif k == 2:
        p = dpp_quad(x, [2, 3, 0, 1])
    else:
        p = dpp_quad(x, [1, 0, 3, 2])
    out = []
    for i in range(64):
        up = bool(i & k)
        r = rotr(p[i], k if up else 32 - k)
        keep = high if up else ~high & M32
        out.append((x[i] & keep) | (r & ~keep & M32))
    return out


def transpose64(lo, hi):
    lo, hi = permlane32_swap(lo, hi)
    for k in (16, 8, 4, 2, 1):
        lo, hi = stage(lo, k), stage(hi, k)
    return lo, hi


@pytest.mark.parametrize("seed", range(4))
def test_cross_lane_bit_transpose(seed):
    rng = random.Random(seed)
    rows = [rng.getrandbits(64) for _ in range(64)]  # lane L holds row L
    lo, hi = transpose64([r & M32 for r in rows], [r >> 32 for r in rows])
    for e in range(64):
        col = lo[e] | (hi[e] << 32)
        assert col == sum(((rows[L] >> e) & 1) << L for L in range(64)), "column %d" % e


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
