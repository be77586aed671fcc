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


# ---- stochastic drafts: accept min(1, p/q), resample from max(0, p - q)

def test_decide_q_with_point_mass_q_equals_decide():
    """q a point mass at the draft is the deterministic case: decide_q takes decide's decisions exactly."""
    for t in range(400):
        V = int(RNG.integers(3, 9))
        nd = int(RNG.integers(1, 4))
        rows = [_dist(V, zero_tail=int(RNG.integers(0, 2)))[:2] for _ in range(nd + 1)]
        drafts = [int(RNG.integers(0, V)) for _ in range(nd)]
        qrows = [(np.array([d]), np.array([1.0], np.float32)) for d in drafts]
        assert S.decide_q(rows, qrows, drafts, 5 * t, 11, 2) == S.decide(rows, drafts, 5 * t, 11, 2)


def test_decide_q_law_closed_form():
    """Drawing the draft from q and applying the rule gives the target's p exactly; the draft is kept
    with probability sum_x min(p(x), q(x))."""
    for _ in range(20):
        V = 7
        ids, p32, p = _dist(V, zero_tail=1)
        qids, q32, q = _dist(V, zero_tail=2)
        bonus = _dist(V)[:2]
        marg = np.zeros(V)
        keep = 0.0
        for x, qx in zip(qids, q32.astype(np.float64)):
            for em, pr in S.decide_q_law([(ids, p32), bonus], [(qids, q32)], [int(x)]):
                marg[em[0]] += qx * pr
                if len(em) == 2:
                    keep += qx * pr
        p64 = np.zeros(V)
        p64[ids] = p32
        q64 = np.zeros(V)
        q64[qids] = q32
        assert np.abs(marg - p64 / p64.sum()).max() < 1e-6
        assert abs(keep - np.minimum(p64, q64).sum()) < 1e-6


@pytest.mark.parametrize("overlap", ["disjoint_tail", "shared"])
def test_stochastic_draft_monte_carlo(overlap):
    """The float32 rule with drafts drawn by sample_draft: the emitted token follows p (chi-square) and
    the acceptance rate is sum_x min(p, q) (binomial z-test)."""
    V = 8
    ids, p32, p = _dist(V, zero_tail=2)
    qids, q32, q = _dist(V, zero_tail=2 if overlap == "disjoint_tail" else 0)
    pf = np.zeros(V)
    pf[ids] = p32
    qf = np.zeros(V)
    qf[qids] = q32
    bonus = (ids, p32)
    N = 60000
    first = np.zeros(V)
    acc = 0
    for t in range(N):
        n = 10 * t
        d = S.sample_draft(qids, q32, 7, n + 1, 3)
        out = S.decide_q([(ids, p32), bonus], [(qids, q32)], [d], n, 7, 3)
        first[out[0]] += 1
        acc += len(out) == 2
    a = float(np.minimum(pf, qf).sum())
    z = (acc / N - a) / np.sqrt(a * (1 - a) / N)
    assert abs(z) < 4.5, z
    sup = pf > 0
    assert first[~sup].sum() == 0
    assert scipy.stats.chisquare(first[sup], pf[sup] / pf[sup].sum() * N).pvalue > 1e-4


def test_sample_draft_uses_stream_one():
    ids = np.array([2, 0, 1])
    q = np.array([0.5, 0.25, 0.25], dtype=np.float32)
    for t in range(50):
        u, _ = S.uniforms(5, t, 1, stream=1)
        assert S.sample_draft(ids, q, 5, t, 1) == S.inverse_cdf(ids, q, u, None)


def _brute_dist64(z, T, top_k, top_p):
    """The filter written out with Python floats: order by (logit desc, id asc), keep the top k, weights
    exp(s - s_max) normalised with fsum, keep the shortest prefix whose running sum reaches top_p
    (inclusive), renormalise."""
    import math
    s = [float(v) / T for v in z]
    order = sorted(range(len(s)), key=lambda i: (-s[i], i))
    k = len(s) if top_k <= 0 else min(top_k, len(s))
    ids = order[:k]
    w = [math.exp(s[i] - s[ids[0]]) for i in ids]
    tot = math.fsum(w)
    q = [x / tot for x in w]
    keep = k
    if top_p < 1.0:
        run = 0.0
        for j, x in enumerate(q):
            run += x
            if run >= top_p:
                keep = j + 1
                break
    kept = q[:keep]
    t2 = math.fsum(kept)
    return ids[:keep], [x / t2 for x in kept]


@pytest.mark.parametrize("T", [0.6, 1.0, 1.7])
@pytest.mark.parametrize("top_k", [0, 1, 7, 20, 100])
@pytest.mark.parametrize("top_p", [0.3, 0.8, 0.95, 1.0])
def test_filter64_against_brute_force(T, top_k, top_p):
    """sample_dist64 (the float64 filter the law enumerations use) against the filter written out in
    Python floats, ties planted: same ids in the same order, probabilities to 1e-12."""
    V = 48
    for trial in range(4):
        z = RNG.standard_normal(V) * 2.0
        z[RNG.integers(0, V, 5)] = z[7]  # plant ties
        ids, p = S.sample_dist64(z, T, top_k, top_p)
        bid, bp = _brute_dist64(z, T, top_k, top_p)
        assert list(ids) == bid
        np.testing.assert_allclose(p, bp, rtol=1e-12, atol=1e-15)
        assert p.dtype == np.float64 and abs(float(p.sum()) - 1.0) < 1e-12


def test_filter64_edge_cases():
    """The top-p cut is inclusive (a prefix whose sum equals top_p exactly stops there), ties keep the
    lower id first, top_k <= 0 keeps the whole vocabulary, top_k past the vocabulary clamps, and
    temperature 0 is the argmax with the lowest id."""
    z = np.array([1.0, 1.0, -40.0, -40.0])  # two equal heads hold half the mass each (to 1e-30)
    ids, p = S.sample_dist64(z, 1.0, 0, 0.5)
    assert list(ids) == [0] and list(p) == [1.0]
    ids, p = S.sample_dist64(z, 1.0, 0, 0.5000001)
    assert list(ids) == [0, 1] and np.allclose(p, [0.5, 0.5])
    ids, p = S.sample_dist64(np.array([0.3, 2.0, 2.0, -1.0]), 1.0, 0, 1.0)
    assert list(ids) == [1, 2, 0, 3]
    ids, p = S.sample_dist64(np.array([0.3, 2.0, 2.0, -1.0]), 1.0, 10, 1.0)
    assert list(ids) == [1, 2, 0, 3] and abs(p.sum() - 1.0) < 1e-15
    ids, p = S.sample_dist64(np.array([0.3, 2.0, 2.0, -1.0]), 0.0, 20, 0.95)
    assert list(ids) == [1] and list(p) == [1.0]
