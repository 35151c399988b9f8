"""Pins of the static trimmed-vocabulary head and its acceptance ceiling (CPU)."""
import numpy as np
import pytest

from drafter_lm_head_slimspec_amd import synth
from oracle import fp, heads, verify


@pytest.mark.parametrize("mode", ["greedy", "sample"])
def test_keeping_every_id_is_the_dense_head(mode):
    h = synth.hidden(4, 64, "bf16", 1)
    W = synth.dense_weights(300, 64, "bf16", 1)
    a = heads.head_trimmed(h, W, np.arange(300), "bf16", mode, 0.9, 5, 2)
    b = heads.head_dense(h, W, "bf16", mode, 0.9, 5, 2)
    np.testing.assert_array_equal(a["token"], b["token"])
    np.testing.assert_array_equal(a["lse"], b["lse"])


def test_greedy_is_the_argmax_over_the_kept_ids():
    # brute force: the full dense logits with every trimmed id excluded
    rng = np.random.default_rng(2)
    h = synth.hidden(6, 32, "f32", 2)
    W = synth.dense_weights(500, 32, "f32", 2)
    ids = np.sort(rng.choice(500, 120, replace=False))
    out = heads.head_trimmed(h, np.ascontiguousarray(W[ids]), ids, "f32")
    z = fp.decode(h, "f32") @ fp.decode(W, "f32").T
    for m in range(6):
        masked = np.full(500, -np.inf)
        masked[ids] = z[m, ids]
        assert out["token"][m] == int(np.argmax(masked))
        assert out["token"][m] in set(ids.tolist())


def test_sampled_ids_follow_the_trimmed_distribution():
    # many rows of the same hidden state: the sampled ids follow softmax over the kept rows
    import scipy.stats
    rng = np.random.default_rng(3)
    V, d, n = 40, 16, 12
    W = synth.dense_weights(V, d, "f32", 3)
    ids = np.sort(rng.choice(V, n, replace=False))
    h1 = synth.hidden(1, d, "f32", 3)
    counts = np.zeros(V)
    for off in range(3000):
        counts[heads.head_trimmed(h1, np.ascontiguousarray(W[ids]), ids, "f32", "sample", 1.0, 7, off)["token"][0]] += 1
    z = (fp.decode(W, "f32") @ fp.decode(h1, "f32")[0])[ids]
    p = np.exp(z - z.max())
    p /= p.sum()
    assert counts[np.setdiff1d(np.arange(V), ids)].sum() == 0
    assert scipy.stats.chisquare(counts[ids], p * 3000).pvalue > 1e-4


def test_acceptance_ceiling():
    rng = np.random.default_rng(4)
    V = 64
    p = rng.dirichlet(np.ones(V))
    ids = np.sort(rng.choice(V, 20, replace=False))
    ceil = heads.trimmed_acceptance_ceiling(p, ids)
    assert ceil == pytest.approx(p[ids].sum())
    for _ in range(50):   # any draft supported on the kept ids stays under the ceiling
        q = np.zeros(V)
        q[ids] = rng.dirichlet(np.ones(ids.size))
        assert verify.acceptance_rate(p, q) <= ceil + 1e-12
    q = np.zeros(V)        # the renormalised restriction of p reaches it
    q[ids] = p[ids] / p[ids].sum()
    assert verify.acceptance_rate(p, q) == pytest.approx(ceil)
