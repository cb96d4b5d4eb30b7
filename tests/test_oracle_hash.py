"""Pins of the oracle's context, key and hash steps (CPU only).

The pages name a hashed bigram + trigram table with a sign trick
(modded-nanogpt README, technique list) but give no hash.  The oracle takes
the SplitMix64 finaliser + Lemire multiply-shift; these tests pin it to things
other than itself: SplitMix64's published output sequence, closed forms of
the range reduction, hand-derived context/key fixtures, and statistics.
Whether this matches the speedrun's own hash is unpinned (the pages are
silent).
"""
import json
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
GAMMA = 0x9E3779B97F4A7C15
M64 = (1 << 64) - 1


def test_splitmix64_published_sequence():
    # SplitMix64 from state 0 (Steele, Lea & Flood, OOPSLA 2014; the same
    # generator as java.util.SplittableRandom seeded with 0) outputs
    # 0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F.  The oracle's
    # hash of key n*gamma with seed 0 is output n+1.
    expected = [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]
    for n, e in enumerate(expected):
        assert oracle.hash64((n * GAMMA) & M64, 0) == e


def test_seed_enters_by_xor():
    # hash(k, s) depends on k ^ s only: key gamma^s with seed s is state
    # gamma, i.e. SplitMix64's second output from state 0.
    assert oracle.hash64(GAMMA ^ 0x1234, 0x1234) == 0x6E789E6AA1B965F4


@pytest.mark.parametrize("m", [1, 5, 12, 20, 26, 30])
def test_multiply_shift_power_of_two(m):
    # For R = 2^m, ((z >> 32) * 2^m) >> 32 is the top m bits of z.
    rs = np.random.default_rng(m)
    for z in rs.integers(0, 2**63, size=200, dtype=np.uint64):
        z = int(z) * 2 + 1
        assert oracle.row_of(z & M64, 1 << m) == (z & M64) >> (64 - m)


def test_multiply_shift_bounds_and_extremes():
    for R in (1, 3, 4096, 5_287_500, 42_300_000, 2**31 - 1):
        assert oracle.row_of(0, R) == 0
        assert oracle.row_of(M64, R) == R - 1
        rs = np.random.default_rng(R)
        for z in rs.integers(0, 2**63, size=100, dtype=np.uint64):
            r = oracle.row_of(int(z) * 2, R)
            assert 0 <= r < R
    # monotone in the upper 32 bits: floor(hi * R / 2^32)
    R = 42_300_000
    for hi in (0, 1, 2**31, 2**32 - 1, 123456789):
        assert oracle.row_of(hi << 32, R) == (hi * R) // 2**32


def test_context_and_keys_golden():
    with open(os.path.join(GOLDEN, "context_keys.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        tok = np.array(c["tokens"], np.int32)
        p1, p2 = oracle.context(tok, c["vocab"], c["eos"])
        assert p1.tolist() == c["p1"]
        assert p2.tolist() == c["p2"]
        for i, t in enumerate(c["tokens"]):
            kb, kt = oracle.keys(c["vocab"], c["p2"][i], c["p1"][i], t)
            assert kb == c["kb"][i]
            assert kt == c["kt"][i]


def test_rows_compose_keys_hash_and_reduction():
    # orc_ngram_rows must be: bigram row from seeds[0], trigram from seeds[1],
    # sign from bit 0 -- checked on the golden keys.
    with open(os.path.join(GOLDEN, "context_keys.json")) as f:
        c = json.load(f)["cases"][3]
    R = (4096, 1000)
    seeds = (11, 22)
    rb, nb, rt, nt, bad = oracle.ngram_rows(np.array(c["tokens"], np.int32), c["vocab"],
                                            c["eos"], R, seeds)
    assert bad == 0
    for i in range(len(c["tokens"])):
        zb = oracle.hash64(c["kb"][i], seeds[0])
        zt = oracle.hash64(c["kt"][i], seeds[1])
        assert rb[i] == oracle.row_of(zb, R[0]) and nb[i] == (zb & 1)
        assert rt[i] == oracle.row_of(zt, R[1]) and nt[i] == (zt & 1)


def test_invalid_ids_counted():
    tok = np.array([50256, 5, -1, 50304, 7], np.int32)
    *_, bad = oracle.ngram_rows(tok, 50304, 50256, (100, 100))
    assert bad == 2


def test_uniformity_sign_balance_and_distinct_count():
    # 10^6 distinct trigram keys into R = 4096 rows: chi-square on row counts,
    # sign balance, and the occupancy closed form R (1 - (1 - 1/R)^n).
    R = 4096
    n = 1_000_000
    L = oracle.lib()
    rows = np.empty(n, np.int64)
    signs = np.empty(n, np.int64)
    for k in range(n):
        z = L.orc_hash64(k * 7919 + 3, 2)
        rows[k] = L.orc_row_of(z, R)
        signs[k] = z & 1
    cnt = np.bincount(rows, minlength=R)
    exp = n / R
    chi2 = float(((cnt - exp) ** 2 / exp).sum())
    # dof 4095: mean 4095, sd ~ 90.5; allow 6 sd
    assert abs(chi2 - (R - 1)) < 6 * math.sqrt(2 * (R - 1))
    frac = signs.mean()
    assert abs(frac - 0.5) < 5 * 0.5 / math.sqrt(n)
    m = 20_000
    distinct = len(np.unique(rows[:m]))
    expect = R * (1 - (1 - 1 / R) ** m)
    sd = math.sqrt(R * (1 - 1 / R) ** m * (1 - (1 - 1 / R) ** m))
    assert abs(distinct - expect) < 6 * max(sd, 1.0)
