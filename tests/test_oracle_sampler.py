"""Pins for oracle.sampler (CPU only).

Philox4x64-10 is checked against numpy's own implementation of the same
generator (numpy.random.Philox, which advances its counter by one before each
block of four words).  The Gumbel-max sampler is checked against the target
distribution softmax(logits / T) with a chi-square test.
"""
import numpy as np
import pytest
from scipy import stats

from oracle import sampler

KEYS = [(0, 0), (5, 0), (0x1234567890ABCDEF, 0x0FEDCBA987654321), (2 ** 64 - 1, 2 ** 64 - 1)]
CTRS = [(1, 0, 0, 0), (5, 7, 11, 13), (2 ** 64 - 1, 3, 2 ** 63, 1), (99, 0, 15, 0)]


@pytest.mark.parametrize("key", KEYS)
@pytest.mark.parametrize("ctr", CTRS)
def test_philox_matches_numpy(key, ctr):
    c = list(ctr)
    # numpy increments the 256-bit counter before generating; start one below
    if c[0] == 0:
        pytest.skip("needs a borrow")
    prev = np.array([c[0] - 1, c[1], c[2], c[3]], dtype=np.uint64)
    bg = np.random.Philox(counter=prev, key=np.array(key, dtype=np.uint64))
    want = [int(x) for x in bg.random_raw(4)]
    got = [int(x) for x in sampler.philox4x64_10([np.uint64(x) for x in c], key)]
    assert got == want


def test_philox_vectorised_equals_scalar():
    ctr0 = np.arange(10, dtype=np.uint64)
    vec = sampler.philox4x64_10((ctr0, np.uint64(3), np.uint64(4), np.uint64(0)), (9, 0))
    for i in range(10):
        sc = sampler.philox4x64_10((np.uint64(i), np.uint64(3), np.uint64(4), np.uint64(0)), (9, 0))
        assert [int(v[i]) for v in vec] == [int(s) for s in sc]


def test_uniforms_layout_and_range():
    u = sampler.uniforms(37, seed=5, step=2, seq=3)
    assert u.dtype == np.float32 and u.shape == (37,)
    assert (u > 0).all() and (u < 1).all()
    # the extreme words map strictly inside (0, 1) in float32
    lo, hi = np.float32(0.5 * 2.0 ** -23), np.float32((2 ** 23 - 0.5) * 2.0 ** -23)
    assert 0 < lo and hi < 1
    # element v takes word v % 4 of counter (v // 4, step, seq, 0)
    w = sampler.philox4x64_10((np.uint64(6), np.uint64(2), np.uint64(3), np.uint64(0)), (5, 0))
    r = int(w[1])
    assert u[25] == np.float32(((r >> 41) + 0.5) * 2.0 ** -23)
    ub = sampler.uniforms_batch(37, 5, [0, 2], 3)
    assert np.array_equal(ub[1], u)


def test_uniforms_are_uniform():
    u = sampler.uniforms_batch(64, 5, np.arange(2000), 0).reshape(-1).astype(np.float64)
    assert stats.kstest(u, "uniform").pvalue > 1e-3


@pytest.mark.parametrize("temperature", [1.0, 0.5])
def test_gumbel_max_samples_softmax(temperature):
    logits = np.array([0.3, -1.0, 2.0, 0.0, 1.1, -0.4, 0.9, 1.6])
    n = 100_000
    u = sampler.uniforms_batch(8, 5, np.arange(n), 1).astype(np.float64)
    draws = np.argmax(logits / temperature - np.log(-np.log(u)), axis=1)
    p = np.exp(logits / temperature - np.max(logits / temperature))
    p /= p.sum()
    obs = np.bincount(draws, minlength=8)
    chi2 = stats.chisquare(obs, p * n)
    assert chi2.pvalue > 1e-4
    # the scalar path takes the same decision as the batched one
    for s in range(5):
        assert sampler.sample(logits, temperature, 5, s, 1) == draws[s]


def test_low_temperature_is_greedy_and_reproducible():
    logits = np.array([0.1, 3.0, 2.0, -1.0, 2.9])
    for s in range(20):
        assert sampler.sample(logits, 1e-3, 5, s, 0) == 1
    assert sampler.sample(logits, 1.0, 5, 7, 2) == sampler.sample(logits, 1.0, 5, 7, 2)
    draws = {sampler.sample(np.zeros(16), 1.0, 5, s, 0) for s in range(60)}
    assert len(draws) > 8  # flat logits: many different tokens over steps


def test_greedy_ties_lowest_index():
    assert sampler.greedy([2.0, 5.0, 5.0]) == 1
    assert sampler.sample([2.0, 5.0, 5.0], 0.0, 1, 1, 1) == 1


# ---------------------------------------------------------------- top-p
@pytest.mark.parametrize("probs,top_p,kept", [
    # running sums of exact binary fractions: 0.5, 0.75, 0.875, 1
    ([0.5, 0.25, 0.125, 0.125], 0.75, [0, 1]),   # reaching top_p exactly stops there
    ([0.5, 0.25, 0.125, 0.125], 0.7, [0, 1]),
    ([0.5, 0.25, 0.125, 0.125], 0.76, [0, 1, 2]),
    ([0.5, 0.25, 0.125, 0.125], 0.5, [0]),
    ([0.5, 0.25, 0.125, 0.125], 0.4, [0]),
    ([0.125, 0.5, 0.125, 0.25], 0.75, [1, 3]),   # order comes from the probabilities
    ([0.25, 0.25, 0.25, 0.25], 0.5, [0, 1]),     # ties: lower index first
    ([0.25, 0.25, 0.25, 0.25], 0.51, [0, 1, 2]),
    ([0.125, 0.375, 0.375, 0.125], 0.5, [1, 2]),
    ([0.125, 0.375, 0.375, 0.125], 0.8, [0, 1, 2]),   # tie at the boundary: index 0 kept, 3 dropped
    ([0.125, 0.375, 0.375, 0.125], 0.9, [0, 1, 2, 3]),
])
def test_nucleus_hand_values(probs, top_p, kept):
    keep = sampler.nucleus_from_probs(probs, top_p)
    assert sorted(np.flatnonzero(keep).tolist()) == kept


def test_nucleus_is_the_smallest_set_reaching_top_p_brute_force():
    """Over every subset of a 6-token vocabulary: the kept set's size is the
    least size of any subset with mass >= top_p, and among subsets of that size
    it has the largest mass."""
    import itertools
    rng = np.random.default_rng(7)
    for trial in range(40):
        p = rng.dirichlet(np.ones(6))
        for top_p in (0.1, 0.5, 0.8, 0.95, 0.999):
            keep = sampler.nucleus_from_probs(p, top_p)
            best_size = min(r for r in range(1, 7) for s in itertools.combinations(range(6), r)
                            if p[list(s)].sum() >= top_p)
            assert keep.sum() == best_size, (trial, top_p)
            best_mass = max(p[list(s)].sum() for s in itertools.combinations(range(6), best_size))
            assert p[keep].sum() == pytest.approx(best_mass, rel=0, abs=1e-15)


def test_nucleus_limits():
    lg = np.random.default_rng(3).standard_normal(300)
    assert sampler.nucleus(lg, 1.0, 1.0).all()
    assert sampler.nucleus(lg, 0.0, 0.5).all()            # greedy ignores top_p
    tiny = sampler.nucleus(lg, 0.8, 1e-12)
    assert np.flatnonzero(tiny).tolist() == [int(np.argmax(lg))]


@pytest.mark.parametrize("temperature,top_p", [(1.0, 0.9), (0.7, 0.5), (1.5, 0.99), (1.0, 0.05)])
def test_nucleus_invariants(temperature, top_p):
    lg = 2.0 * np.random.default_rng(int(100 * top_p)).standard_normal(5000)
    p = sampler.softmax_t(lg, temperature)
    keep = sampler.nucleus(lg, temperature, top_p)
    assert p[keep].sum() >= top_p                               # reaches top_p
    assert p[keep].sum() - p[keep].min() < top_p                # minimal
    assert p[keep].min() >= p[~keep].max()                      # the most probable tokens


def test_top_p_one_equals_plain_sampling():
    lg = np.random.default_rng(11).standard_normal(700)
    for step in range(20):
        assert sampler.sample(lg, 0.9, 4, step, 1, top_p=1.0) == int(
            np.argmax(lg / 0.9 + sampler.gumbel(lg.size, 4, step, 1)))


def test_top_p_draws_follow_the_renormalised_nucleus():
    """Chi-square: over 20,000 steps the Gumbel-max draws restricted to the
    nucleus match p / p(nucleus); nothing outside the nucleus is drawn."""
    lg = np.array([2.0, 1.5, 1.2, 0.4, 0.3, -0.5, -1.0, -2.0])
    T, top_p = 1.0, 0.8
    keep = sampler.nucleus(lg, T, top_p)
    assert 2 <= keep.sum() < lg.size
    steps = np.arange(20000)
    u = sampler.uniforms_batch(lg.size, 17, steps, 0).astype(np.float64)
    sc = lg[None, :] / T - np.log(-np.log(u))
    sc[:, ~keep] = -np.inf
    draws = np.argmax(sc, axis=1)
    # the vectorised draws equal the sampler's own for a few steps
    for s in range(5):
        assert draws[s] == sampler.sample(lg, T, 17, s, 0, top_p)
    counts = np.bincount(draws, minlength=lg.size)
    assert counts[~keep].sum() == 0
    p = sampler.softmax_t(lg, T)[keep]
    exp = p / p.sum() * steps.size
    assert stats.chisquare(counts[keep], exp).pvalue > 1e-3


def test_top_p_non_finite_row_keeps_every_token():
    lg = np.array([0.1, np.nan, 0.3, np.nan])
    assert sampler.nucleus(lg, 1.0, 0.5).all()
    assert sampler.sample(lg, 1.0, 1, 0, 0, top_p=0.5) == 1   # first NaN ranks above every number
