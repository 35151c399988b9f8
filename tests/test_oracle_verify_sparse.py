"""Pins of sampling verification against a sparse (top-k) draft distribution (CPU)."""
import numpy as np
import pytest
import scipy.stats

from oracle import verify


def test_full_support_equals_dense_verification():
    # K = every id and q = softmax(draft logits): the dense verification, draw for draw
    rng = np.random.default_rng(1)
    B, gamma, V = 24, 4, 40
    target = (2.0 * rng.standard_normal((B, gamma + 1, V))).astype(np.float32)
    draft = (target[:, :gamma] + rng.standard_normal((B, gamma, V))).astype(np.float32)
    q = np.exp(draft.astype(np.float64) - draft.max(-1, keepdims=True))
    q /= q.sum(-1, keepdims=True)
    x = np.stack([[rng.choice(V, p=q[b, t]) for t in range(gamma)] for b in range(B)]).astype(np.int32)
    u = ((rng.integers(0, 1 << 23, size=(B, gamma)) + 0.5) * 2.0 ** -23).astype(np.float32)
    idx = np.tile(np.arange(V), (B, gamma, 1))
    a1, o1, d1 = verify.verify_sample(target, draft, x, u, "f32", 1.0, 9, 2)
    a2, o2, d2 = verify.verify_sample_sparse(target, idx, q, x, u, "f32", 1.0, 9, 2)
    np.testing.assert_array_equal(a1, a2)
    np.testing.assert_array_equal(o1, o2)


def _sparse_rounds(p_rows, K_rows, qK_rows, B, seed):
    rng = np.random.default_rng(seed)
    gamma = len(K_rows)
    lp = np.log(np.array(p_rows, np.float64))
    target = np.broadcast_to(lp, (B,) + lp.shape).astype(np.float32)
    idx = np.broadcast_to(np.array(K_rows), (B, gamma, len(K_rows[0])))
    prob = np.broadcast_to(np.array(qK_rows, np.float64), idx.shape)
    x = np.stack([np.array(K_rows[t])[rng.choice(len(K_rows[t]), size=B, p=qK_rows[t])] for t in range(gamma)], 1)
    u = ((rng.integers(0, 1 << 23, size=(B, gamma)) + 0.5) * 2.0 ** -23).astype(np.float32)
    return target, idx, prob, x.astype(np.int32), u


def test_sparse_draft_acceptance_rate_and_target_distribution():
    # q lives on K = {1, 2, 4}; p has mass outside K, which only the residual can emit
    p0 = np.array([.1, .3, .2, .15, .15, .1])
    K = [1, 2, 4]
    qK = [.5, .3, .2]
    q_full = np.zeros(6)
    q_full[K] = qK
    alpha = verify.acceptance_rate(p0, q_full)
    assert alpha == pytest.approx(min(.3, .5) + min(.2, .3) + min(.15, .2))
    # the acceptance rate of a draft supported on K is at most p(K) (SlimSpec write-up, 四)
    assert alpha <= p0[K].sum() + 1e-12
    p1 = np.array([.6, .1, .1, .1, .05, .05])
    B = 12000
    target, idx, prob, x, u = _sparse_rounds([p0, p1], [K], [qK], B, seed=4)
    acc, out, _ = verify.verify_sample_sparse(target, idx, prob, x, u, "f32", 1.0, 31, 5)
    f0 = np.mean(acc >= 1)
    assert abs(f0 - alpha) < 4 * np.sqrt(alpha * (1 - alpha) / B)
    assert scipy.stats.chisquare(np.bincount(out[:, 0], minlength=6), p0 * B).pvalue > 1e-4
    bonus = out[acc == 1, 1]
    assert scipy.stats.chisquare(np.bincount(bonus, minlength=6), p1 * len(bonus)).pvalue > 1e-4


def test_token_outside_the_candidate_set():
    # a draft token with q(x) = 0 but p(x) > 0 is accepted (ratio infinite)
    V = 8
    target = np.zeros((1, 2, V), np.float32)
    idx = np.array([[[0, 1, 2]]])
    prob = np.array([[[.5, .25, .25]]])
    acc, out, d = verify.verify_sample_sparse(target, idx, prob, np.array([[5]], np.int32),
                                              np.array([[0.999]], np.float32), "f32")
    assert acc[0] == 1 and out[0, 0] == 5 and np.isinf(d["ratio"][0, 0])
