"""Pins for the oracle's pair plane (one byte per group of 8 for masks keeping
at most 2 of 8): the round trip through the effective weight of 2:8 and 1:8
masks, hand-worked group bytes, injectivity over every representable group,
the size (d_in / 8 bytes per row, half the 2-bit code plane), and the refusal
of a group with 3 non-zeros."""
import itertools

import numpy as np
import pytest

import oracle
from sbl_inputs import weight


@pytest.mark.parametrize("n", [1, 2])
def test_round_trip_through_effective_weight(n):
    W = weight(41, n, 96, 256)
    w_eff, _, _ = oracle.effective_weight(W, n)
    plane = oracle.pack_pairs(w_eff)
    assert plane.shape == (96, 32) and plane.dtype == np.uint8
    assert plane.nbytes * 2 == oracle.pack_codes(w_eff).nbytes   # 1 bit per weight against 2
    assert np.array_equal(oracle.unpack_pairs(plane), w_eff)
    assert plane.max() < oracle.PAIR_CODES


def test_worked_groups():
    """By hand: +1 at 1 and -1 at 5: pair (1, 5) has rank 7 + 3 = 10 (the 7 pairs
    starting at 0 come first), digits (1, 2): 9 * 10 + 3 + 2 = 95.  -1 alone at
    7 pads to (0, 7): rank 6, digits (0, 2): 56.  +1 alone at 0 pads to (0, 1):
    digits (1, 0): 3.  -1 at 0 and +1 at 7: rank 6, digits (2, 1): 54 + 7 = 61.
    All zero: 0.  +1 at 6 and +1 at 7: the last pair, rank 27: 243 + 4 = 247."""
    groups = [[0, 1, 0, 0, 0, -1, 0, 0], [0, 0, 0, 0, 0, 0, 0, -1], [1, 0, 0, 0, 0, 0, 0, 0],
              [-1, 0, 0, 0, 0, 0, 0, 1], [0] * 8, [0, 0, 0, 0, 0, 0, 1, 1]]
    w = np.array([sum(groups, [])], np.int8)
    assert list(oracle.pack_pairs(w)[0]) == [95, 56, 3, 61, 0, 247]
    assert oracle.pair_index(1, 5) == 10 and oracle.pair_index(6, 7) == 27 and oracle.pair_index(0, 1) == 0


def test_injective_over_all_representable_groups():
    seen = {}
    for nz in (0, 1, 2):
        for pos in itertools.combinations(range(8), nz):
            for vals in itertools.product((1, -1), repeat=nz):
                g = [0] * 8
                for p, v in zip(pos, vals):
                    g[p] = v
                b = int(oracle.pack_pairs(np.array([g], np.int8))[0, 0])
                assert b not in seen, (g, seen.get(b))
                seen[b] = g
                assert oracle.unpack_pairs(np.array([[b]], np.uint8))[0].tolist() == g
    assert len(seen) == 1 + 8 * 2 + 28 * 4


def test_three_nonzeros_refused():
    with pytest.raises(AssertionError):
        oracle.pack_pairs(np.array([[1, 0, -1, 0, 1, 0, 0, 0]], np.int8))
