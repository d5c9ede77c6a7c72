"""Pins of the toy arrival simulator (CPU only).

The page prints no readouts for its toy machine [F55 §实验台], so the
simulator is tied down by cases with a closed form: memory large enough for
everyone, one-token blocks, the row reservation's concurrency bound, and two
small cases worked by hand (one preempts, one shows strict first come,
first served).
"""
import numpy as np
import pytest

from oracle.arrivals import simulate, toy_pool


def _random_case(seed, n=12, max_len=20, spread=10):
    rng = np.random.default_rng(seed)
    return rng.integers(0, spread, n).tolist(), rng.integers(1, max_len + 1, n).tolist()


@pytest.mark.parametrize("bs", [1, 2, 4, 8, 16])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_unlimited_memory_matches_interval_closed_forms(bs, seed):
    arr, lens = _random_case(seed)
    nb = sum(-(-n // bs) for n in lens)  # everyone at full length at once still fits
    out = simulate(nb, bs, arr, lens)
    assert out["preemptions"] == 0
    assert out["rounds"] == max(a + n for a, n in zip(arr, lens))
    for r, (c, held, reserved) in enumerate(out["trace"]):
        live = [r - a + 1 for a, n in zip(arr, lens) if a <= r < a + n]  # tokens written by round r
        assert c == len(live)
        assert held == sum(live)
        assert reserved == sum(bs * -(-k // bs) for k in live)  # less than one block of waste each
    assert out["max_concurrent"] == max(
        sum(1 for a, n in zip(arr, lens) if a <= r < a + n) for r in range(out["rounds"]))


@pytest.mark.parametrize("nb", [20, 23, 30, 44])
@pytest.mark.parametrize("seed", [0, 3])
def test_one_token_blocks_waste_nothing(nb, seed):
    arr, lens = _random_case(seed, n=20, spread=4)
    out = simulate(nb, 1, arr, lens)
    assert all(held == reserved for _, held, reserved in out["trace"])
    samples = [h for _, h, v in out["trace"] if v]
    assert samples and out["utilisation"] == 1.0


@pytest.mark.parametrize("seed", [0, 1])
def test_row_reservation_bounds_concurrency(seed):
    """A whole row of 20 slots per sequence: 176 // 20 = 8 at once, never a
    preemption, and with 12 sequences waiting at round 0 exactly 8 run."""
    nb, bs = toy_pool(176, None, 20)
    assert (nb, bs) == (8, 20)
    rng = np.random.default_rng(seed)
    lens = rng.integers(1, 21, 12).tolist()
    out = simulate(nb, bs, [0] * 12, lens)
    assert out["preemptions"] == 0 and out["max_concurrent"] == 8
    for c, held, reserved in out["trace"]:
        assert reserved == 20 * c and held <= reserved


def test_hand_worked_preemption():
    """2 blocks of 2 slots; two 3-token sequences arrive at round 0.
    r0: both admitted (2 tokens in 4 slots).  r1: both write (4/4).
    r2: sequence 0 needs a second block; sequence 1, the latest arrival, is
    swapped out; sequence 0 writes its last token (3/4) and leaves.
    r3: sequence 1 resumes with 2 blocks and writes its last token (3/4)."""
    out = simulate(2, 2, [0, 0], [3, 3])
    assert out["trace"] == [(2, 2, 4), (2, 4, 4), (1, 3, 4), (1, 3, 4)]
    assert out["rounds"] == 4 and out["max_concurrent"] == 2 and out["preemptions"] == 1
    assert out["utilisation"] == pytest.approx((0.5 + 1 + 0.75 + 0.75) / 4)


def test_hand_worked_head_of_line_wait():
    """6 one-token blocks.  Sequences 0 (6 tokens) and 1 (4 tokens) arrive at
    round 0, sequence 2 (1 token) at round 4.
    r0-r2: both write (6 of 6 blocks at r2).  r3: sequence 0 needs a block;
    sequence 1 (3 tokens written) is swapped out.  r4: one block is free and
    sequence 2 would fit, but the head of the queue, sequence 1, needs 4; both
    wait.  r5: sequence 0 writes its last token and leaves.  r6: sequence 1
    resumes with 4 blocks, then sequence 2 is admitted; both finish."""
    out = simulate(6, 1, [0, 0, 4], [6, 4, 1])
    assert out["trace"] == [(2, 2, 2), (2, 4, 4), (2, 6, 6), (1, 4, 4), (1, 5, 5), (1, 6, 6), (2, 5, 5)]
    assert out["rounds"] == 7 and out["preemptions"] == 1 and out["max_concurrent"] == 2


def test_invalid_inputs():
    with pytest.raises(ValueError):
        simulate(2, 4, [0], [9])  # needs 3 blocks of a 2-block pool
    with pytest.raises(ValueError):
        simulate(4, 4, [0], [0])
