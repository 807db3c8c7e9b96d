"""Pins for the oracle's kept-only 2:4 operand plane (2:8 and 2:4 masks): the
round trip to W_eff, a hand-worked group layout, the padding rule, its size
(2 bits per weight like the code plane), and that a group with 3 non-zeros is
refused."""
import numpy as np
import pytest

import oracle
from sbl_inputs import weight


@pytest.mark.parametrize("n,m", [(2, 8), (2, 4), (1, 4), (1, 8)])
def test_round_trip(n, m):
    W = weight(61, n * 10 + m, 48, 256)
    w_eff, _, _ = oracle.effective_weight(W, n, m)
    plane = oracle.pack_sparse24(w_eff)
    assert plane.shape == (48, 4, 16) and plane.nbytes == 48 * 256 // 4   # 2 bits per weight
    np.testing.assert_array_equal(oracle.unpack_sparse24(plane), w_eff)


def test_worked_groups():
    # row of 64: group 0 = [0, -1, 0, 1] -> positions (1, 3), codes (11, 01);
    # group 1 = [0, 0, 0, 1] -> one non-zero at 3 -> (2, 3), codes (00, 01);
    # group 2 = [1, 0, 0, 0] -> (0, 1), codes (01, 00); everything else zero -> (0, 1), (00, 00)
    w = np.zeros((1, 64), np.int8)
    w[0, 0:4] = [0, -1, 0, 1]
    w[0, 4:8] = [0, 0, 0, 1]
    w[0, 8:12] = [1, 0, 0, 0]
    plane = oracle.pack_sparse24(w)
    cw0 = int(np.frombuffer(plane[0, 0, 0:4].tobytes(), np.uint32)[0])
    iw0 = int(np.frombuffer(plane[0, 0, 8:12].tobytes(), np.uint32)[0])
    # codes: slots 0,1 = 11, 01; slots 2,3 = 00, 01; slots 4,5 = 01, 00; rest 00
    assert cw0 == (0b11 | 0b01 << 2 | 0b00 << 4 | 0b01 << 6 | 0b01 << 8)
    # positions: group 0 (1,3) -> 1 | 3 << 2 = 0xD; group 1 (2,3) -> 2 | 3 << 2 = 0xE; others (0,1) -> 0x4
    assert iw0 == 0xD | 0xE << 4 | 0x4 << 8 | 0x4 << 12 | 0x4 << 16 | 0x4 << 20 | 0x4 << 24 | 0x4 << 28
    assert int(np.frombuffer(plane[0, 0, 4:8].tobytes(), np.uint32)[0]) == 0                # half 1: zeros
    assert int(np.frombuffer(plane[0, 0, 12:16].tobytes(), np.uint32)[0]) == 0x44444444


def test_three_nonzeros_refused():
    w = np.zeros((1, 64), np.int8)
    w[0, 0:3] = [1, -1, 1]
    with pytest.raises(AssertionError):
        oracle.pack_sparse24(w)
