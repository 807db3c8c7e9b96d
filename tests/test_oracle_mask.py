"""Pins for the oracle's N:M top-N mask.

Pinned against: brute force over every candidate subset (exactly one subset of
size N has every kept key beating every dropped key, with the lower index
winning ties), an exhaustive tie-heavy alphabet, the explainer page's worked
2:4 example, and invariances (sign, powers of two).
"""
import itertools
import os

import numpy as np
import pytest

import oracle
from sbl_inputs import f32_to_bf16_bits, tie_heavy_weight, weight

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _brute_force_mask(values, n, m):
    """For one group: the unique size-n subset whose every member outranks every non-member.

    Rank key: larger |value| first; equal |value| -> lower index first.
    """
    idx = range(m)
    outranks = lambda a, b: abs(values[a]) > abs(values[b]) or (abs(values[a]) == abs(values[b]) and a < b)
    found = []
    for S in itertools.combinations(idx, n):
        rest = [j for j in idx if j not in S]
        if all(outranks(a, b) for a in S for b in rest):
            found.append(S)
    assert len(found) == 1
    keep = np.zeros(m, bool)
    keep[list(found[0])] = True
    return keep


@pytest.mark.parametrize("m", [4, 8])
def test_mask_brute_force_random_groups(m):
    g = np.random.default_rng(11)
    for trial in range(60):
        # mix of continuous values and a small alphabet so ties occur
        if trial % 2:
            vals = g.choice([-0.5, -0.25, 0.0, 0.25, 0.5, -0.0], size=(3, m * 2)).astype(np.float32)
        else:
            vals = g.standard_normal((3, m * 2)).astype(np.float32)
        bits = f32_to_bf16_bits(vals)
        dec = oracle.bf16_to_f64(bits)
        for n in range(1, m + 1):
            got = oracle.nm_mask(bits, n, m)
            for r in range(3):
                for gi in range(2):
                    want = _brute_force_mask(list(dec[r, gi * m:(gi + 1) * m]), n, m)
                    assert np.array_equal(got[r, gi * m:(gi + 1) * m], want)


@pytest.mark.parametrize("n", [2, 4, 6, 8])
def test_mask_exhaustive_small_alphabet(n):
    # All 5^8 groups over {-2,-1,0,1,2}.  Vectorised brute force: integer keys
    # key_j = |v_j| * 8 + (7 - j) are distinct and order slots exactly as the rule does;
    # a subset is the mask iff min(key over kept) > max(key over dropped).
    alphabet = np.array([-2, -1, 0, 1, 2], dtype=np.float32)
    combos = np.array(list(itertools.product(range(5), repeat=8)), dtype=np.int64)
    vals = alphabet[combos]
    bits = f32_to_bf16_bits(vals)
    got = oracle.nm_mask(bits, n, 8)
    keys = np.abs(vals).astype(np.int64) * 8 + (7 - np.arange(8))
    want = np.zeros_like(got)
    hits = np.zeros(len(vals), np.int64)
    for S in itertools.combinations(range(8), n):
        inS = np.zeros(8, bool)
        inS[list(S)] = True
        kmin = keys[:, inS].min(axis=1)
        kmax = keys[:, ~inS].max(axis=1) if (~inS).any() else np.full(len(vals), -1)
        ok = kmin > kmax
        hits += ok
        want[ok] = inS
    assert np.all(hits == 1)
    assert np.array_equal(got, want)


def test_mask_popcount_and_dense():
    W = weight(0, 0, 64, 256)
    for n in range(1, 9):
        k = oracle.nm_mask(W, n, 8)
        assert np.all(k.reshape(64, 32, 8).sum(-1) == n)
    assert oracle.nm_mask(W, 8, 8).all()


def test_mask_invariances():
    W = weight(0, 2, 32, 128)
    x = oracle.bf16_to_f64(W).astype(np.float32)
    for n in (2, 4, 6):
        base = oracle.nm_mask(W, n, 8)
        assert np.array_equal(oracle.nm_mask(W ^ np.uint16(0x8000), n, 8), base)     # negation
        for k in (-3, 4):
            Wk = f32_to_bf16_bits(x * np.float32(2.0 ** k))
            assert np.array_equal(oracle.nm_mask(Wk, n, 8), base)


def test_mask_signed_zero_and_sign_ties():
    # +x and -x tie, +0 and -0 tie; ties go to the lower index
    vals = np.array([[0.0, -0.0, 0.5, -0.5, 0.25, -0.25, 0.0, 1.0]], np.float32)
    bits = f32_to_bf16_bits(vals)
    bits[0, 1] = 0x8000
    assert np.array_equal(oracle.nm_mask(bits, 6, 8)[0], [1, 0, 1, 1, 1, 1, 0, 1])
    assert np.array_equal(oracle.nm_mask(bits, 2, 8)[0], [0, 0, 1, 0, 0, 0, 0, 1])
    assert np.array_equal(oracle.nm_mask(bits, 3, 8)[0], [0, 0, 1, 1, 0, 0, 0, 1])


def _read_golden(name):
    d = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            k, *v = line.split()
            d[k] = v
    return d


def test_explainer_worked_example_2of4():
    d = _read_golden("explainer_nm_2of4_example.txt")
    m, n = int(d["m"][0]), int(d["n"][0])
    vals = np.array([[float(v) for v in d["input"]]], np.float32)
    bits = f32_to_bf16_bits(vals)
    keep = oracle.nm_mask(bits, n, m)[0]
    assert keep.astype(int).tolist() == [int(v) for v in d["kept"]]
    result = np.where(keep, vals[0], 0.0)
    assert np.allclose(result, [float(v) for v in d["result"]])


def test_explainer_values_with_groups_of_8():
    # Same 8 weights, one group of 8.  |w| order: 1.2 (3) > 0.9 (6) > 0.8 (0) > 0.7 (4)
    # > 0.5 (2) > 0.4 (7) > 0.3 (1) > 0.2 (5); keep the first N.
    bits = f32_to_bf16_bits(np.array([[0.8, -0.3, 0.5, 1.2, -0.7, 0.2, 0.9, -0.4]], np.float32))
    assert oracle.nm_mask(bits, 6, 8)[0].astype(int).tolist() == [1, 0, 1, 1, 1, 0, 1, 1]
    assert oracle.nm_mask(bits, 4, 8)[0].astype(int).tolist() == [1, 0, 0, 1, 1, 0, 1, 0]
    assert oracle.nm_mask(bits, 2, 8)[0].astype(int).tolist() == [0, 0, 0, 1, 0, 0, 1, 0]


def test_mask_tie_heavy_matches_brute_force():
    W = tie_heavy_weight(0, 16, 64)
    dec = oracle.bf16_to_f64(W)
    for n in (2, 4, 6):
        got = oracle.nm_mask(W, n, 8)
        for r in range(16):
            for gi in range(8):
                want = _brute_force_mask(list(dec[r, gi * 8:(gi + 1) * 8]), n, 8)
                assert np.array_equal(got[r, gi * 8:(gi + 1) * 8], want)
