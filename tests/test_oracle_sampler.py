"""Pins for the oracle's sampling rule (CPU only): the element step on its own, the special
group sizes that reduce the two-level rule to the textbook Gumbel-max trick, and the
distribution of the two-level draw on a vocabulary of 16 groups.

The rule (the pages leave the sampler open; the reading is a two-level Gumbel-max over groups
of 64 consecutive candidates) must draw exactly from softmax(l).  What pins it here:
* the Gumbel transform -log(-log u) is strictly increasing in u, so among equal log-weights
  the element step must take the member with the largest uniform (lowest position on ties);
* within one group the element step is a Gumbel-max draw, so its frequencies follow the
  softmax of that group's log-weights (chi-square);
* with groups of one candidate the group step alone is the flat Gumbel-max draw on the group
  uniforms, and with one group holding every candidate the element step alone is the flat
  Gumbel-max draw on the element uniforms (Gumbel, 1954; the "Gumbel-max trick");
* on V = 1024 (sixteen groups) the two-level draw follows softmax(l) (chi-square).
"""
import numpy as np
import pytest
import scipy.special
import scipy.stats

from oracle import philox, sampler


def _eu(seed, off, purpose=1):
    return lambda i: philox.uniforms(seed, off, purpose, 0, i)


def _merged_chi2_pvalue(counts, probs, min_expected=20.0):
    """Chi-square p-value of counts against probs, rare cells merged (expected >= 20)."""
    N = counts.sum()
    order = np.argsort(probs)
    cp, cc, acc_p, acc_c = [], [], 0.0, 0.0
    for i in order:
        acc_p += probs[i]
        acc_c += counts[i]
        if acc_p * N >= min_expected:
            cp.append(acc_p)
            cc.append(acc_c)
            acc_p = acc_c = 0.0
    if acc_p > 0:
        cp[-1] += acc_p
        cc[-1] += acc_c
    cp, cc = np.array(cp), np.array(cc)
    stat = float(np.sum((cc - cp * N) ** 2 / (cp * N)))
    return scipy.stats.chi2.sf(stat, len(cp) - 1)


@pytest.mark.parametrize("n,g", [(300, 0), (300, 2), (300, 4), (64, 0), (65, 1), (1000, 15)])
def test_pick_in_group_with_equal_weights_takes_largest_uniform(n, g):
    # equal log-weights: the Gumbel keys order exactly as the uniforms do
    ell = np.full(n, -1.25)
    lo, hi = g * sampler.GROUP, min(n, (g + 1) * sampler.GROUP)
    for off in range(40):
        eu = _eu(3, off)
        u = eu(np.arange(lo, hi))
        pos, es = sampler.pick_in_group(ell, g, eu)
        assert lo <= pos < hi
        assert pos == lo + int(np.argmax(u))          # numpy: first maximum
        assert es.shape == (hi - lo,)


def test_pick_in_group_ties_and_masked_members():
    n, g = 200, 1
    lo = g * sampler.GROUP
    const = lambda i: np.full(np.shape(i), 0.5)      # every member gets the same uniform
    ell = np.zeros(n)
    ell[lo + 9] = ell[lo + 40] = ell[lo + 41] = 2.0   # a three-way tie on the largest weight
    assert sampler.pick_in_group(ell, g, const)[0] == lo + 9
    # a member with weight -inf (zero probability) is never taken, whatever its uniform
    ell = np.full(n, -np.inf)
    ell[lo + 63] = 0.0
    for off in range(30):
        assert sampler.pick_in_group(ell, g, _eu(5, off))[0] == lo + 63
    # the short last group of a ragged vocabulary only offers positions below n
    ell = np.zeros(130)
    for off in range(30):
        pos, es = sampler.pick_in_group(ell, 2, _eu(6, off))
        assert 128 <= pos < 130 and es.shape == (2,)


@pytest.mark.parametrize("n,g", [(200, 0), (200, 3)])
def test_pick_in_group_follows_softmax_of_the_group(n, g):
    rng = np.random.default_rng(n + g)
    ell = rng.standard_normal(n) * 1.3
    lo, hi = g * sampler.GROUP, min(n, (g + 1) * sampler.GROUP)
    p = np.exp(ell[lo:hi] - scipy.special.logsumexp(ell[lo:hi]))
    N = 20000
    counts = np.zeros(hi - lo)
    for off in range(N):
        counts[sampler.pick_in_group(ell, g, _eu(17, off))[0] - lo] += 1
    assert _merged_chi2_pvalue(counts, p) > 1e-4


def test_pick_in_group_is_the_element_step_of_the_two_level_draw():
    rng = np.random.default_rng(2)
    n = 333
    for off in range(300):
        ell = rng.standard_normal(n) * 2.0
        ell[rng.integers(0, n, 20)] = -np.inf
        gu = lambda j, off=off: philox.uniforms(8, off, 0, 0, j)
        eu = _eu(8, off)
        tok, diag = sampler.two_level_sample(ell, gu, eu)
        assert tok // sampler.GROUP == diag["group"]
        pos, es = sampler.pick_in_group(ell, diag["group"], eu)
        assert pos == tok
        np.testing.assert_array_equal(es, diag["elem_scores"])


def _textbook_gumbel_max(ell, u):
    """argmax_i (l_i + G_i) with G_i = -log(-log u_i) (first maximum)."""
    return int(np.argmax(np.asarray(ell) - np.log(-np.log(u))))


@pytest.mark.parametrize("n", [1, 7, 64, 200])
def test_groups_of_one_candidate_are_flat_gumbel_max_on_group_uniforms(n):
    rng = np.random.default_rng(n)
    for off in range(50):
        ell = rng.standard_normal(n) * 1.7
        gu = lambda j, off=off: philox.uniforms(4, off, 0, 0, j)
        tok, _ = sampler.two_level_sample(ell, gu, _eu(4, off), group=1)
        assert tok == _textbook_gumbel_max(ell, gu(np.arange(n)))


@pytest.mark.parametrize("n", [1, 7, 64, 200])
def test_one_group_of_every_candidate_is_flat_gumbel_max_on_element_uniforms(n):
    rng = np.random.default_rng(100 + n)
    for off in range(50):
        ell = rng.standard_normal(n) * 1.7
        eu = _eu(4, off)
        tok, diag = sampler.two_level_sample(ell, lambda j, off=off: philox.uniforms(4, off, 0, 0, j), eu, group=n)
        assert diag["group"] == 0
        assert tok == _textbook_gumbel_max(ell, eu(np.arange(n)))


def test_two_level_sampler_matches_softmax_over_sixteen_groups():
    V = 1024
    rng = np.random.default_rng(V)
    y = rng.standard_normal(V) * 1.5
    p = np.exp(y - scipy.special.logsumexp(y))
    N = 20000
    counts = np.zeros(V)
    for off in range(N):
        tok, _ = sampler.two_level_sample(y, lambda g, off=off: philox.uniforms(12, off, 0, 0, g), _eu(12, off))
        counts[tok] += 1
    assert _merged_chi2_pvalue(counts, p) > 1e-4
