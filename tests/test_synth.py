"""Seeded input generator (host side): published Philox known answers,
distribution sanity, bf16 rounding."""
import numpy as np
import pytest

import synth


@pytest.mark.parametrize("ctr,key,want", [
    # Known-answer vectors of Philox4x32-10 distributed with Random123
    # (Salmon et al., "Parallel random numbers: as easy as 1, 2, 3", SC'11).
    ((0, 0, 0, 0), (0, 0), (0x6627e8d5, 0xe169c58d, 0xbc57ac4c, 0x9b00dbd8)),
    ((0xffffffff,) * 4, (0xffffffff,) * 2, (0x408f276d, 0x41c83b0e, 0xa20bc7c6, 0x6d5451fd)),
    ((0x243f6a88, 0x85a308d3, 0x13198a2e, 0x03707344), (0xa4093822, 0x299f31d0),
     (0xd16cfe09, 0x94fdcceb, 0x5001e420, 0x24126ea1)),
])
def test_philox_known_answers(ctr, key, want):
    assert tuple(synth.philox_block(ctr, key)) == want


def test_normal_moments():
    g = synth.fill_cpu(1 << 20, 0, 0, 0, sigma=1e-2).astype(np.float64)
    assert abs(g.mean()) < 3e-5
    assert abs(g.std() / 1e-2 - 1) < 3e-3


def test_student_t3_is_heavy_tailed():
    g = synth.fill_cpu(1 << 20, 0, 0, 0, dist=synth.STUDENT_T3, sigma=1e-3).astype(np.float64)
    # t(3): median |t| ~ 0.765, and far more mass beyond 5 than a normal
    assert 0.7e-3 < np.median(np.abs(g)) < 0.83e-3
    assert np.mean(np.abs(g) > 5e-3) > 1e-3


def test_counter_based_slices_agree():
    full = synth.fill_cpu(4096, 0, 3, 2, sigma=1e-3)
    part = synth.fill_cpu(1000, 1234, 3, 2, sigma=1e-3)
    np.testing.assert_array_equal(full[1234:2234], part)
    idx = np.array([5, 77, 4095, 1234], dtype=np.uint64)
    np.testing.assert_array_equal(synth.gather_cpu(idx, 3, 2, sigma=1e-3), full[idx.astype(np.int64)])
    assert not np.array_equal(full, synth.fill_cpu(4096, 0, 3, 3, sigma=1e-3))
    assert not np.array_equal(full, synth.fill_cpu(4096, 0, 4, 2, sigma=1e-3))


def test_bf16_round_to_nearest_even():
    f = synth.fill_cpu(1 << 16, 0, 0, 0, sigma=1e-3)
    b = synth.fill_cpu(1 << 16, 0, 0, 0, sigma=1e-3, bf16=True)
    up = (b.astype(np.uint32) << 16).view(np.float32)
    err = np.abs(up.astype(np.float64) - f)
    # nearest: no other bf16 value is closer
    for nb in (b - 1, b + 1):
        other = (nb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        assert np.all(err <= np.abs(other - f))


def test_workloads_have_the_stated_shapes():
    """The five workloads' padded sizes, worker counts, tensor counts, step
    splits and c5's learning-rate decay, as the workload list states them
    (architecture shapes of BERT-Base/Large and GPT-2-XL; 15 % of 200 steps
    of warm-up for c5)."""
    import numpy as np
    from synth import workloads as W
    want = {  # d, n, tensors, raw elements, warm-up, compressed, bf16, staged
        "c1": (1 << 20, 4, 1, 1 << 20, 3, 7, False, False),
        "c2": (110_000_128, 8, 1, 110_000_000, 2, 20, True, False),
        "c3": (334_123_008, 16, 390, 334_122_810, 3, 7, False, False),
        "c4": (1_557_611_520, 8, 580, 1_557_611_200, 3, 50, False, False),
        "c5": (340_000_768, 64, 1, 340_000_000, 30, 170, False, True),
    }
    for name, (d, n, tensors, raw, warm, comp, bf16, staged) in want.items():
        w = W.make(name)
        assert (w.d, w.n, w.tensors, w.raw, w.warmup, w.compressed, w.bf16, w.staged) == \
            (d, n, tensors, raw, warm, comp, bf16, staged), name
        assert w.d % (64 * w.n) == 0, name
        # the padding ranges cover exactly d - raw elements
        assert sum(b - a for a, b in w.pads) == w.d - w.raw, name
    c5 = W.make("c5")
    assert c5.lr_at(29) == np.float32(1e-3) and c5.lr_at(30) == np.float32(1e-3)
    assert c5.lr_at(199) == np.float32(1e-3 / 170)
    assert W.make("c4").dist == W.STUDENT_T3
