"""Pins of the oracle's sampler: Philox, the candidate filter, and the accept / resample rule."""
import numpy as np
import pytest
import scipy.special
import scipy.stats

from oracle import sampling as S

RNG = np.random.default_rng(99)


def test_philox_matches_numpy():
    # numpy's Philox (4x64, 10 rounds) increments its 256-bit counter before producing a block,
    # so its first block for counter c is the Philox function of c + 1.
    for _ in range(20):
        c = [int(x) for x in RNG.integers(0, 2 ** 63, size=4, dtype=np.uint64)]
        k = [int(x) for x in RNG.integers(0, 2 ** 63, size=2, dtype=np.uint64)]
        got = np.random.Philox(counter=c, key=k).random_raw(4)
        want = S.philox4x64_10([c[0] + 1, c[1], c[2], c[3]], k)
        assert [int(x) for x in got] == list(want)


def test_uniforms_are_24_bit_and_distinct_per_counter():
    seen = set()
    for t in range(200):
        ua, us = S.uniforms(1, t, 0)
        assert ua.dtype == np.float32 and 0.0 <= ua < 1.0 and 0.0 <= us < 1.0
        assert float(ua) * 2 ** 24 == int(float(ua) * 2 ** 24)
        seen.add((float(ua), float(us)))
    assert len(seen) == 200
    assert S.uniforms(1, 5, 0) != S.uniforms(1, 5, 1)  # request is part of the counter
    assert S.uniforms(1, 5, 0) != S.uniforms(2, 5, 0)  # seed is the key


def _brute_order(s):
    return sorted(range(len(s)), key=lambda i: (-float(s[i]), i))


@pytest.mark.parametrize("T", [0.7, 1.0, 1.3])
@pytest.mark.parametrize("top_k", [0, 1, 5, 20, 64])
@pytest.mark.parametrize("top_p", [0.5, 0.95, 1.0])
def test_filter_against_brute_force(T, top_k, top_p):
    V = 64
    for trial in range(5):
        z = (RNG.standard_normal(V) * 2).astype(np.float32)
        z[RNG.integers(0, V, 6)] = z[3]  # plant ties
        ids, p = S.sample_dist(z, T, top_k, top_p)
        s = z / np.float32(T)
        order = _brute_order(s)
        k = V if top_k <= 0 else min(top_k, V)
        assert list(ids) == order[:len(ids)]
        q64 = scipy.special.softmax(s[order[:k]].astype(np.float64))
        c64 = np.cumsum(q64)
        if top_p < 1.0:
            cut = int(np.nonzero(c64 >= top_p)[0][0]) + 1 if (c64 >= top_p).any() else k
            if np.min(np.abs(c64 - top_p)) > 1e-5:
                assert len(ids) == cut
        else:
            assert len(ids) == k
        np.testing.assert_allclose(p, q64[:len(ids)] / q64[:len(ids)].sum(), rtol=2e-6, atol=1e-7)
        assert p.dtype == np.float32 and abs(float(p.astype(np.float64).sum()) - 1.0) < 1e-5


def test_filter_greedy_is_argmax_lowest_id():
    z = np.array([0.1, 3.0, -1.0, 3.0, 2.9], dtype=np.float32)
    ids, p = S.sample_dist(z, 0.0, 20, 0.95)
    assert list(ids) == [1] and list(p) == [1.0]


def _dist(V, zero_tail=0):
    p = RNG.dirichlet(np.ones(V) * 0.8)
    if zero_tail:
        p[np.argsort(p)[:zero_tail]] = 0.0
        p /= p.sum()
    ids = np.array(sorted(range(V), key=lambda i: (-p[i], i)))
    ids = ids[p[ids] > 0]
    return ids.astype(np.int64), p[ids].astype(np.float32), p


@pytest.mark.parametrize("which", ["argmax", "mid", "absent"])
def test_accept_rate_and_resample_law(which):
    """A deterministic draft x is accepted with probability p(x); a rejected position follows p with x
    removed and renormalised; the first emitted token follows p."""
    V = 8
    ids, p32, p = _dist(V, zero_tail=2)
    if which == "argmax":
        x = int(ids[0])
    elif which == "mid":
        x = int(ids[len(ids) // 2])
    else:
        x = int([t for t in range(V) if t not in set(ids.tolist())][0])
    bonus = (ids, p32)
    N = 60000
    acc = 0
    resample = np.zeros(V)
    first = np.zeros(V)
    for t in range(N):
        out = S.decide([(ids, p32), bonus], [x], 10 * t, seed=7, request=3)
        first[out[0]] += 1
        if len(out) == 2:
            assert out[0] == x
            acc += 1
        else:
            assert out[0] != x
            resample[out[0]] += 1
    px = float(p[x])
    if px in (0.0, 1.0):
        assert acc == round(px * N)
    else:
        z = (acc / N - px) / np.sqrt(px * (1 - px) / N)
        assert abs(z) < 4.5, z
    if N - acc > 0:
        r = p.copy()
        r[x] = 0
        r /= r.sum()
        sup = r > 0
        assert resample[~sup].sum() == 0
        assert scipy.stats.chisquare(resample[sup], r[sup] * resample.sum()).pvalue > 1e-4
    sup = p > 0
    assert first[~sup].sum() == 0
    assert scipy.stats.chisquare(first[sup], p[sup] * N).pvalue > 1e-4


def test_decide_greedy_rows():
    # T = 0 rows are point masses: accept iff the draft is the argmax, else emit the argmax.
    rows = [(np.array([4]), np.array([1.0], np.float32)), (np.array([2]), np.array([1.0], np.float32)),
            (np.array([9]), np.array([1.0], np.float32))]
    assert S.decide(rows, [4, 2], 0, 1, 0) == [4, 2, 9]
    assert S.decide(rows, [4, 3], 0, 1, 0) == [4, 2]
    assert S.decide(rows, [5, 2], 0, 1, 0) == [4]


def test_decide_law_is_a_distribution_and_matches_closed_form():
    ids, p32, p = _dist(6)
    ids2, p32b, pb = _dist(6)
    x = int(ids[1])
    law = S.decide_law([(ids, p32), (ids2, p32b)], [x])
    tot = sum(pr for _, pr in law)
    assert abs(tot - 1.0) < 1e-6
    d = {tuple(k): v for k, v in law}
    for y in range(6):
        if y != x and p[y] > 0:
            assert abs(d[(y,)] - float(p32[ids == y][0])) < 1e-7
    for y in range(6):
        if pb[y] > 0:
            assert abs(d[(x, y)] - float(p32[ids == x][0]) * float(p32b[ids2 == y][0])) < 1e-7


def test_inverse_cdf_extremes():
    ids = np.array([3, 1, 2])
    p = np.array([0.5, 0.5, 0.0], dtype=np.float32)
    assert S.inverse_cdf(ids, p, np.float32(0.0), None) == 3
    assert S.inverse_cdf(ids, p, np.float32(1 - 2 ** -24), None) == 1
    assert S.inverse_cdf(ids, p, np.float32(0.3), exclude=3) == 1
