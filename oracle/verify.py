"""Batched verification of gamma draft tokens against the target's gamma+1 distributions.

Greedy (explainer, "小模型起草，大模型批改" and "为什么答案不会变"; phrase-level page:
a candidate is accepted only when it equals the target's own argmax):
  g_t = argmax z^p_t (ties -> lowest id), a = first t < gamma with x_t != g_t (else gamma),
  emitted tokens = x_0..x_{a-1}, g_a  (1 .. gamma+1 tokens per round).

Sampling (explainer, "为什么答案不会变"; SpecTr-GBV page, "为什么重新设计…" and "第三步"):
  accept x_t with probability min(1, p_t(x_t) / q_t(x_t)), i.e. accept iff u_t < p/q;
  the first rejection at position a ends the block and a token is drawn from
  norm(max(0, p_a - q_a)); if all gamma drafts are accepted a bonus token is drawn from
  p_gamma.  Both p and q are softmax(z / T) over the full vocabulary (SpecVocab page 3.3:
  verification keeps the full vocabulary).

Readings: u_t are given inputs in (0,1); a draft id outside [0, V) is never accepted; the residual and bonus draws use the two-level
Gumbel rule with Philox purposes 3/4 (residual group/element) and 5/6 (bonus), row = b;
if the residual mass is exactly zero the draw falls back to p_a (unreachable for finite,
distinct logits).  Output rows are padded with -1 after the last emitted token.
"""
import numpy as np

from . import fp
from .philox import (uniforms, PURPOSE_RESID_GROUP, PURPOSE_RESID_ELEM, PURPOSE_BONUS_GROUP,
                     PURPOSE_BONUS_ELEM)
from .sampler import two_level_sample, logsumexp


def argmax_lowest(z):
    return int(np.argmax(np.asarray(z)))


def verify_greedy(target_logits, draft_tokens, dtype):
    """target_logits: [B, gamma+1, V]; draft_tokens: [B, gamma] -> (accept_len, out_tokens)."""
    tl = fp.decode(target_logits, dtype)
    x = np.asarray(draft_tokens, dtype=np.int64)
    B, gamma = x.shape
    acc = np.zeros(B, np.int64)
    out = np.full((B, gamma + 1), -1, np.int64)
    for b in range(B):
        g = [argmax_lowest(tl[b, t]) for t in range(gamma + 1)]
        a = 0
        while a < gamma and x[b, a] == g[a]:
            a += 1
        out[b, :a] = x[b, :a]
        out[b, a] = g[a]
        acc[b] = a
    return acc, out


def _softmax(y):
    lse = logsumexp(y)
    return np.exp(y - lse), lse


def verify_sample(target_logits, draft_logits, draft_tokens, u_accept, dtype, temperature=1.0,
                  seed=0, offset=0):
    """Speculative-sampling verification.  Returns (accept_len, out_tokens, diag)."""
    tl = fp.decode(target_logits, dtype) / temperature
    dl = fp.decode(draft_logits, dtype) / temperature
    x = np.asarray(draft_tokens, dtype=np.int64)
    u = np.asarray(u_accept, dtype=np.float64)
    B, gamma = x.shape
    acc = np.zeros(B, np.int64)
    out = np.full((B, gamma + 1), -1, np.int64)
    diag = {"ratio": np.zeros((B, gamma)), "sample": []}
    for b in range(B):
        a = gamma
        for t in range(gamma):
            if not (0 <= x[b, t] < tl.shape[2]):
                a = t
                break
            lp = tl[b, t, x[b, t]] - logsumexp(tl[b, t])
            lq = dl[b, t, x[b, t]] - logsumexp(dl[b, t])
            ratio = np.exp(lp - lq)
            diag["ratio"][b, t] = ratio
            if not (u[b, t] < ratio):
                a = t
                break
        if a < gamma:
            p, _ = _softmax(tl[b, a])
            q, _ = _softmax(dl[b, a])
            r = p - q
            with np.errstate(divide="ignore"):
                ell = np.where(r > 0, np.log(np.where(r > 0, r, 1.0)), -np.inf)
            tok, dg = two_level_sample(
                ell,
                lambda g: uniforms(seed, offset, PURPOSE_RESID_GROUP, b, g),
                lambda i: uniforms(seed, offset, PURPOSE_RESID_ELEM, b, i),
            )
            if tok is None:  # zero residual mass: fall back to the target distribution
                tok, dg = two_level_sample(
                    tl[b, a],
                    lambda g: uniforms(seed, offset, PURPOSE_RESID_GROUP, b, g),
                    lambda i: uniforms(seed, offset, PURPOSE_RESID_ELEM, b, i),
                )
            dg["kind"] = "residual"
            dg["p"], dg["q"] = p, q
        else:
            tok, dg = two_level_sample(
                tl[b, gamma],
                lambda g: uniforms(seed, offset, PURPOSE_BONUS_GROUP, b, g),
                lambda i: uniforms(seed, offset, PURPOSE_BONUS_ELEM, b, i),
            )
            dg["kind"] = "bonus"
        out[b, :a] = x[b, :a]
        out[b, a] = tok
        acc[b] = a
        dg["a"] = a
        diag["sample"].append(dg)
    return acc, out, diag


def acceptance_rate(p, q):
    """Per-position acceptance probability alpha = sum_x min(p(x), q(x)) ("SlimSpec"
    write-up, section 四)."""
    return float(np.sum(np.minimum(np.asarray(p, np.float64), np.asarray(q, np.float64))))


def expected_tokens_per_step(alpha, gamma):
    """Mean emitted tokens per round, (1 - alpha^(gamma+1)) / (1 - alpha) (explainer,
    "这笔账划不划算，看一个数"), with the alpha -> 1 limit gamma + 1."""
    if alpha == 1.0:
        return float(gamma + 1)
    return (1.0 - alpha ** (gamma + 1)) / (1.0 - alpha)


def verify_sample_sparse(target_logits, draft_idx, draft_prob, draft_tokens, u_accept, dtype,
                         temperature=1.0, seed=0, offset=0):
    """Speculative-sampling verification against a sparse draft distribution: q_t is given
    on a candidate set K_t (draft_idx [B, gamma, k], ascending ids, draft_prob [B, gamma, k]:
    the SpecVocab head's probabilities over its top-k, section 2.2.3) and is zero outside it
    (reading: SpecVocab section 3.3 keeps the full vocabulary for verification, so the
    residual max(0, p - q) equals p outside K).  The acceptance test, residual, bonus and
    uniforms are those of verify_sample.  Returns (accept_len, out_tokens, diag)."""
    tl = fp.decode(target_logits, dtype) / temperature
    idx = np.asarray(draft_idx, dtype=np.int64)
    qk = np.asarray(draft_prob, dtype=np.float64)
    x = np.asarray(draft_tokens, dtype=np.int64)
    u = np.asarray(u_accept, dtype=np.float64)
    B, gamma = x.shape
    V = tl.shape[2]
    acc = np.zeros(B, np.int64)
    out = np.full((B, gamma + 1), -1, np.int64)
    diag = {"ratio": np.zeros((B, gamma)), "sample": []}

    def q_row(b, t):
        q = np.zeros(V)
        q[idx[b, t]] = qk[b, t]
        return q

    for b in range(B):
        a = gamma
        for t in range(gamma):
            if not (0 <= x[b, t] < V):
                a = t
                break
            p, _ = _softmax(tl[b, t])
            qx = q_row(b, t)[x[b, t]]
            ratio = p[x[b, t]] / qx if qx > 0 else (np.inf if p[x[b, t]] > 0 else 0.0)
            diag["ratio"][b, t] = ratio
            if not (u[b, t] < ratio):
                a = t
                break
        if a < gamma:
            p, _ = _softmax(tl[b, a])
            q = q_row(b, a)
            r = p - q
            with np.errstate(divide="ignore"):
                ell = np.where(r > 0, np.log(np.where(r > 0, r, 1.0)), -np.inf)
            tok, dg = two_level_sample(
                ell,
                lambda g: uniforms(seed, offset, PURPOSE_RESID_GROUP, b, g),
                lambda i: uniforms(seed, offset, PURPOSE_RESID_ELEM, b, i),
            )
            if tok is None:
                tok, dg = two_level_sample(
                    tl[b, a],
                    lambda g: uniforms(seed, offset, PURPOSE_RESID_GROUP, b, g),
                    lambda i: uniforms(seed, offset, PURPOSE_RESID_ELEM, b, i),
                )
            dg["kind"] = "residual"
            dg["p"], dg["q"] = p, q
        else:
            tok, dg = two_level_sample(
                tl[b, gamma],
                lambda g: uniforms(seed, offset, PURPOSE_BONUS_GROUP, b, g),
                lambda i: uniforms(seed, offset, PURPOSE_BONUS_ELEM, b, i),
            )
            dg["kind"] = "bonus"
        out[b, :a] = x[b, :a]
        out[b, a] = tok
        acc[b] = a
        dg["a"] = a
        diag["sample"].append(dg)
    return acc, out, diag
