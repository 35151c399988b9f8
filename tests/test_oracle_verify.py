"""Pins for the oracle's verification (CPU only): the pages' worked examples and table,
closed forms, special cases and Monte Carlo against exact distributions."""
import json
import os

import numpy as np
import pytest
import scipy.stats

from oracle import verify

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _onehot_logits(argmaxes, V):
    z = np.zeros((len(argmaxes), V), np.float32)
    for t, g in enumerate(argmaxes):
        z[t, g] = 5.0
    return z


def test_closed_form_matches_printed_table():
    g = json.load(open(os.path.join(GOLDEN, "closed_form_gamma4.json")))
    for row in g["rows"]:
        val = verify.expected_tokens_per_step(row["alpha"], g["gamma"])
        assert round(val, g["decimals"]) == row["tokens_per_step"]
    # limits: alpha -> 0 gives exactly one token, alpha = 1 gives gamma + 1
    assert verify.expected_tokens_per_step(0.0, 4) == 1.0
    assert verify.expected_tokens_per_step(1.0, 4) == 5.0


def test_greedy_worked_examples():
    g = json.load(open(os.path.join(GOLDEN, "greedy_worked_examples.json")))
    for case in g["cases"]:
        draft = np.array([case["draft"]], np.int32)
        gamma = draft.shape[1]
        V = 128
        z = _onehot_logits(case["target_argmax"], V)[None]
        assert z.shape == (1, gamma + 1, V)
        acc, out = verify.verify_greedy(z, draft, "f32")
        assert acc[0] == case["accept_len"], case["name"]
        emitted = [int(t) for t in out[0] if t >= 0]
        assert emitted == case["emitted"], case["name"]
        assert 1 <= len(emitted) <= gamma + 1


def test_greedy_ties_use_lowest_index():
    V, gamma = 16, 2
    z = np.zeros((1, gamma + 1, V), np.float32)
    z[0, :, 3] = 1.0
    z[0, :, 9] = 1.0                      # exact tie with id 3
    acc, out = verify.verify_greedy(z, np.array([[9, 3]], np.int32), "f32")
    assert acc[0] == 0 and out[0, 0] == 3
    acc, out = verify.verify_greedy(z, np.array([[3, 3]], np.int32), "f32")
    assert acc[0] == 2 and list(out[0]) == [3, 3, 3]


def test_acceptance_rate_identity():
    rng = np.random.default_rng(0)
    for _ in range(20):
        p = rng.dirichlet(np.ones(50))
        q = rng.dirichlet(np.ones(50))
        # sum_x min(p,q) = 1 - total variation distance
        assert abs(verify.acceptance_rate(p, q) - (1 - 0.5 * np.abs(p - q).sum())) < 1e-12
        assert verify.acceptance_rate(p, p) == pytest.approx(1.0)


def _fixed_rounds(p_rows, q_rows, B, seed):
    """B independent rounds with the same per-position p_t, q_t; x_t ~ q_t, u ~ U(0,1)."""
    rng = np.random.default_rng(seed)
    gamma = len(q_rows)
    lp = np.log(np.array(p_rows, np.float64))
    lq = np.log(np.array(q_rows, np.float64))
    target = np.broadcast_to(lp, (B,) + lp.shape).astype(np.float32)
    draft = np.broadcast_to(lq, (B,) + lq.shape).astype(np.float32)
    V = lp.shape[1]
    x = np.stack([rng.choice(V, size=B, p=np.array(q_rows[t]) / np.sum(q_rows[t])) for t in range(gamma)], 1)
    u = ((rng.integers(0, 1 << 23, size=(B, gamma)) + 0.5) * 2.0 ** -23).astype(np.float32)
    return target, draft, x.astype(np.int32), u


@pytest.mark.parametrize("p,q,alpha", [
    ([.7, .1, .1, .1], [.2, .4, .2, .2], 0.5),
    ([.5, .3, .2], [.3, .5, .2], 0.8),
])
def test_mean_emitted_tokens_matches_closed_form(p, q, alpha):
    gamma = 4
    assert verify.acceptance_rate(p, q) == pytest.approx(alpha)
    B = 8000
    target, draft, x, u = _fixed_rounds([p] * (gamma + 1), [q] * gamma, B, seed=int(alpha * 10))
    acc, out, _ = verify.verify_sample(target, draft, x, u, "f32", seed=77, offset=0)
    emitted = acc + 1
    want = verify.expected_tokens_per_step(alpha, gamma)
    sd = emitted.std() / np.sqrt(B)
    assert abs(emitted.mean() - want) < 4 * sd, (emitted.mean(), want, sd)
    # accept frequency at the first position is alpha
    f0 = np.mean(acc >= 1)
    assert abs(f0 - alpha) < 4 * np.sqrt(alpha * (1 - alpha) / B)


def test_output_distribution_is_the_target_distribution():
    # position 0: accepted draft or residual draw; the emitted token must follow p_0 exactly.
    # all accepted: the bonus token must follow p_gamma.
    p0 = np.array([.05, .3, .25, .15, .25])
    q0 = np.array([.4, .1, .2, .2, .1])
    p1 = np.array([.2, .2, .2, .2, .2])
    q1 = np.array([.2, .2, .2, .2, .2])          # always accepted
    p2 = np.array([.6, .1, .1, .1, .1])          # bonus distribution
    gamma = 2
    B = 12000
    target, draft, x, u = _fixed_rounds([p0, p1, p2], [q0, q1], B, seed=5)
    acc, out, _ = verify.verify_sample(target, draft, x, u, "f32", seed=123, offset=9)
    c0 = np.bincount(out[:, 0], minlength=5)
    assert scipy.stats.chisquare(c0, p0 * B).pvalue > 1e-4
    bonus = out[acc == gamma, gamma]
    assert len(bonus) > 1000
    assert scipy.stats.chisquare(np.bincount(bonus, minlength=5), p2 * len(bonus)).pvalue > 1e-4
    # positions after the first rejection are padding
    for b in range(200):
        assert np.all(out[b, acc[b] + 1:] == -1)


def test_sampling_special_cases():
    V, gamma, B = 40, 3, 50
    rng = np.random.default_rng(8)
    z = rng.standard_normal((B, gamma + 1, V)).astype(np.float32)
    x = rng.integers(0, V, size=(B, gamma)).astype(np.int32)
    u = ((rng.integers(0, 1 << 23, size=(B, gamma)) + 0.5) * 2.0 ** -23).astype(np.float32)
    # p == q: every draft accepted for every u
    acc, out, _ = verify.verify_sample(z, z[:, :gamma].copy(), x, u, "f32", seed=1)
    assert np.all(acc == gamma)
    # draft almost certain of x while the target almost excludes it: first draft rejected,
    # and the correction is never x (residual is p with x removed)
    d = np.zeros((B, gamma, V), np.float32)
    t = np.zeros((B, gamma + 1, V), np.float32)
    for b in range(B):
        d[b, :, x[b, 0]] = 60.0
        t[b, 0, x[b, 0]] = -60.0
    acc, out, _ = verify.verify_sample(t, d, x, u, "f32", seed=2)
    assert np.all(acc == 0)
    assert np.all(out[:, 0] != x[:, 0])


def test_greedy_verify_equals_sampling_limit_structure():
    # greedy: accept iff equal to the target argmax; output always has a+1 tokens
    rng = np.random.default_rng(3)
    B, gamma, V = 30, 5, 64
    z = rng.standard_normal((B, gamma + 1, V)).astype(np.float32)
    g = z.argmax(-1)
    x = g[:, :gamma].copy()
    flip = rng.integers(0, gamma + 1, size=B)
    for b in range(B):
        if flip[b] < gamma:
            x[b, flip[b]] = (x[b, flip[b]] + 1) % V
    acc, out = verify.verify_greedy(z, x.astype(np.int32), "f32")
    np.testing.assert_array_equal(acc, flip)
    for b in range(B):
        assert out[b, acc[b]] == g[b, acc[b]]
