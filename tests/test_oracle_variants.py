"""Pins for the oracle's variant rows: N:4 groups inside the 8-slot planes, the
"mask from quantized weight" ablation, and the "mask without grad" ablation.

Pinned against: brute force over every candidate subset (the unique size-N
subset whose every kept key beats every dropped key, lower index winning ties),
hand-worked groups, and counting properties of the packed planes.
"""
import itertools

import numpy as np
import pytest

import oracle
from sbl_inputs import f32_to_bf16_bits, weight


def _brute_keep(keys, n):
    m = len(keys)
    outranks = lambda a, b: keys[a] > keys[b] or (keys[a] == keys[b] and a < b)
    found = [S for S in itertools.combinations(range(m), n)
             if all(outranks(a, b) for a in S for b in range(m) if b not in S)]
    assert len(found) == 1
    keep = np.zeros(m, bool)
    keep[list(found[0])] = True
    return keep


@pytest.mark.parametrize("m", [4, 8])
def test_mask_from_quantized_brute_force(m):
    g = np.random.default_rng(21)
    for _ in range(40):
        wq = g.choice([-1, 0, 1], size=(2, 2 * m), p=[0.3, 0.4, 0.3]).astype(np.int8)
        for n in range(1, m + 1):
            got = oracle.mask_from_quantized(wq, n, m)
            for r in range(2):
                for gi in range(2):
                    keys = [abs(int(v)) for v in wq[r, gi * m:(gi + 1) * m]]
                    assert np.array_equal(got[r, gi * m:(gi + 1) * m], _brute_keep(keys, n))


def test_mask_from_quantized_worked_groups():
    # worked by hand: non-zero slots first in index order, then zero slots in index order
    cases = [
        ([1, 0, -1, 1, 0, 1, -1, 1], 6, 8, [0, 2, 3, 5, 6, 7]),
        ([1, 1, 1, -1, 1, 1, 1, 1], 6, 8, [0, 1, 2, 3, 4, 5]),
        ([0, -1, 0, 0, 0, 0, 0, 1], 6, 8, [0, 1, 2, 3, 4, 7]),
        ([0, 0, 0, 0, 0, 0, 0, 0], 2, 8, [0, 1]),
        ([0, -1, 0, 1, 1, 1, -1, 0], 2, 4, [1, 3, 4, 5]),
    ]
    for row, n, m, kept in cases:
        got = oracle.mask_from_quantized(np.array([row], np.int8), n, m)[0]
        assert sorted(np.nonzero(got)[0].tolist()) == kept, (row, n, m)


@pytest.mark.parametrize("n", [1, 2, 3, 4])
def test_pack_n_of_4_planes(n):
    # N:4 inside the 8-slot words: every nibble of the mask plane holds n kept bits,
    # codes are zero outside the mask, and the planes equal the N:4 definition packed
    W = weight(31, n, 48, 64)
    codes, mplane, g = oracle.quant_mask_pack(W, n, 4)
    for nib in (mplane & 0xF, mplane >> 4):
        assert np.all(np.vectorize(lambda b: bin(int(b)).count("1"))(nib) == n)
    w_eff = oracle.unpack_codes(codes)
    keep = oracle.nm_mask(W, n, 4)
    assert not np.any(w_eff[~keep])
    assert np.array_equal(w_eff[keep], oracle.ternary(W, g)[keep])
    assert np.array_equal(mplane, oracle.pack_mask(keep))


@pytest.mark.parametrize("n,m", [(6, 8), (2, 8), (2, 4)])
def test_pack_from_quantized_counts(n, m):
    # per group: the kept non-zero codes are the first min(n, nnz) non-zero W_q slots
    W = weight(33, n + m, 40, 128)
    codes, mplane, g = oracle.quant_mask_pack(W, n, m, from_quantized=True)
    wq = oracle.ternary(W, g)
    w_eff = oracle.unpack_codes(codes)
    for r in range(W.shape[0]):
        for c in range(0, W.shape[1], m):
            nz = np.nonzero(wq[r, c:c + m])[0]
            want = np.zeros(m, np.int8)
            want[nz[:n]] = wq[r, c:c + m][nz[:n]]
            assert np.array_equal(w_eff[r, c:c + m], want)
    # the magnitude mask of the same matrix differs somewhere (the ablation is a different rule)
    codes_mag, _, _ = oracle.quant_mask_pack(W, n, m)
    assert not np.array_equal(codes, codes_mag)


def test_mask_grad_zeroes_masked_slots_only():
    g = np.random.default_rng(5)
    dW = g.standard_normal((8, 32))
    dW[0, 0] = -0.0
    mask = g.random((8, 32)) < 0.75
    mask[0, 1] = False
    dW[0, 1] = -1.5
    out = oracle.mask_grad(dW, mask)
    assert np.array_equal(out[mask].view(np.int64), dW[mask].view(np.int64))   # kept: bit for bit
    assert np.all(out[~mask].view(np.int64) == 0)                                # masked: +0.0
