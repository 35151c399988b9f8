"""The drafter LM head in its three forms, plus selection (argmax / sampling).

* dense: z = W h with W in R^{V x d} ("SlimSpec" write-up, section 三: the head projects
  the d-dim hidden state to V scores through a V x d matrix, cost O(V d)).
* low-rank (SlimSpec, section 三 and Q&A Q1): h_r = W_down h (d -> r), z = W_up h_r
  (r -> V); every one of the V tokens keeps a score.  Layout reading: W_down is stored as
  [r, d] and W_up as [V, r] so both products are row dot products.  Position-adaptive rank
  (section 七): row m uses nested prefixes of rank r_m of the same pair.
* SpecVocab (2kiu.com write-up, sections 2.2.1-2.2.3): h' = W_down h (d' = d/16),
  s = W_vocab h' (approximate scores), K = top-k(s), z' = U[K,:] h (exact logits from
  the full hidden state), q = softmax(z') over the k candidates; q is 0 outside K.

Readings where the pages are silent (each one also used by the HIP path):
* dot products accumulate in float64 here (fp32 on the GPU);
* h_r and h' are rounded once, RNE, to the storage dtype (bf16, or f32 for f32 inputs);
* temperature: y = z / T; lse and logprob refer to y; greedy picks argmax z;
* ties: argmax and top-k boundary ties go to the lowest index; top-k is returned sorted
  by ascending vocabulary id; sampling uses the two-level Gumbel rule in ``sampler``
  with Philox uniforms (purpose 0 = group, 1 = element, row = row of the call).
  For SpecVocab the sampled positions are candidate positions 0..k-1 in ascending-id order.
"""
import numpy as np

from . import fp
from .philox import uniforms, PURPOSE_DRAFT_GROUP, PURPOSE_DRAFT_ELEM
from .sampler import two_level_sample, logsumexp, _argmax_lowest

GREEDY = "greedy"
SAMPLE = "sample"


def select(z, mode, temperature, seed, offset, row):
    """Token selection on one row of logits z (float64) plus lse / logprob of y = z / T."""
    z = np.asarray(z, dtype=np.float64)
    y = z / temperature
    lse = logsumexp(y)
    if mode == GREEDY:
        token, margin = _argmax_lowest(z)
        diag = {"margin": margin}
    elif mode == SAMPLE:
        token, diag = two_level_sample(
            y,
            lambda g: uniforms(seed, offset, PURPOSE_DRAFT_GROUP, row, g),
            lambda i: uniforms(seed, offset, PURPOSE_DRAFT_ELEM, row, i),
        )
    else:
        raise ValueError(mode)
    return int(token), lse, float(y[token] - lse), diag


def _finish(Z, mode, temperature, seed, offset):
    M = Z.shape[0]
    out = {"logits": Z, "token": np.zeros(M, np.int64), "lse": np.zeros(M), "logprob": np.zeros(M),
           "diag": []}
    for m in range(M):
        t, lse, lp, dg = select(Z[m], mode, temperature, seed, offset, m)
        out["token"][m], out["lse"][m], out["logprob"][m] = t, lse, lp
        out["diag"].append(dg)
    return out


def head_dense(h, W, dtype, mode=GREEDY, temperature=1.0, seed=0, offset=0):
    """Dense head. h: [M, d], W: [V, d] (bf16 bits or f32).  Returns dict of outputs."""
    hd = fp.decode(h, dtype)
    Wd = fp.decode(W, dtype)
    Z = hd @ Wd.T                      # [M, V], float64
    return _finish(Z, mode, temperature, seed, offset)


def lowrank_down(h, W_down, dtype):
    """h_r before and after the one rounding step: returns (exact float64, rounded)."""
    hd = fp.decode(h, dtype)
    Wd = fp.decode(W_down, dtype)
    pre = hd @ Wd.T                    # [M, r]
    return pre, fp.round_to_dtype(pre, dtype)


def head_lowrank(h, W_down, W_up, dtype, mode=GREEDY, temperature=1.0, seed=0, offset=0):
    """SlimSpec head: z = W_up (round(W_down h)).  W_down: [r, d], W_up: [V, r]."""
    pre, hr = lowrank_down(h, W_down, dtype)
    Wu = fp.decode(W_up, dtype)
    Z = hr @ Wu.T                      # [M, V]
    out = _finish(Z, mode, temperature, seed, offset)
    out["h_r_exact"] = pre
    out["h_r"] = hr
    return out


def head_lowrank_adaptive(h, W_down, W_up, ranks, dtype, mode=GREEDY, temperature=1.0, seed=0,
                          offset=0):
    """Position-adaptive rank ("SlimSpec" write-up, section 七, the second future direction:
    earlier draft positions get a larger rank, later ones a smaller one).  Reading: one factor
    pair of rank r_max serves every position through nested prefixes, so row m of rank r_m uses
    the first r_m rows of W_down and the first r_m columns of W_up:
        z_m = W_up[:, :r_m] round(W_down[:r_m] h_m),   1 <= r_m <= r_max.
    Selection, rounding and uniforms are those of head_lowrank (Philox row = m)."""
    pre, hr = lowrank_down(h, W_down, dtype)          # [M, r_max]; row m keeps its first r_m
    Wu = fp.decode(W_up, dtype)
    ranks = [int(r) for r in np.asarray(ranks).reshape(-1)]
    M = hr.shape[0]
    if len(ranks) != M or min(ranks) < 1 or max(ranks) > Wu.shape[1]:
        raise ValueError("ranks must hold one value in [1, r_max] per row")
    Z = np.empty((M, Wu.shape[0]))
    for m, r in enumerate(ranks):
        Z[m] = Wu[:, :r] @ hr[m, :r]
    out = _finish(Z, mode, temperature, seed, offset)
    mask = np.arange(hr.shape[1])[None, :] < np.array(ranks)[:, None]
    out["h_r_exact"] = np.where(mask, pre, 0.0)
    out["h_r"] = np.where(mask, hr, 0.0)
    return out


def head_trimmed(h, W_S, ids, dtype, mode=GREEDY, temperature=1.0, seed=0, offset=0):
    """Static trimmed-vocabulary head ("SlimSpec" write-up, section 二: static vocabulary
    trimming scores only a fixed reduced vocabulary, and a trimmed-away token can never be
    proposed).  W_S [n_S, d] holds the kept rows W[ids] (trimmed once, offline); the head is the
    dense head over those n_S rows, and the chosen position j maps back to the id ids[j].
    Reading: sampling groups, lse and logprob are over the n_S kept positions in the given
    order (Philox row = m)."""
    out = head_dense(h, W_S, dtype, mode, temperature, seed, offset)
    ids = np.asarray(ids, dtype=np.int64)
    out["position"] = out["token"].copy()
    out["token"] = ids[out["token"]]
    return out


def trimmed_acceptance_ceiling(p, ids):
    """Largest acceptance rate any draft supported on the kept ids can reach against the target
    distribution p: sum_x min(p(x), q(x)) <= p(S) for every q with q = 0 outside S, with equality
    for q = p restricted to S and renormalised (SlimSpec write-up, section 二: the ceiling)."""
    p = np.asarray(p, dtype=np.float64)
    return float(p[np.asarray(ids, dtype=np.int64)].sum())


def topk_ascending(s, k):
    """Indices of the k largest entries of s (ties -> lowest index), sorted ascending."""
    s = np.asarray(s, dtype=np.float64)
    n = s.size
    order = np.lexsort((np.arange(n), -s))   # primary key -s (descending s), then index
    return np.sort(order[:k])


def head_specvocab(h, W_down, W_vocab, U, k, dtype, mode=GREEDY, temperature=1.0, seed=0,
                   offset=0):
    """SpecVocab head.  W_down: [d', d], W_vocab: [V, d'], U: [V, d].

    Returns per row: approximate scores s, ascending top-k ids K, exact logits z'[K],
    q = softmax(z'/T) over K, the token (a vocabulary id), lse and logprob over K.
    """
    hd = fp.decode(h, dtype)
    pre = hd @ fp.decode(W_down, dtype).T
    hp = fp.round_to_dtype(pre, dtype)
    S = hp @ fp.decode(W_vocab, dtype).T          # [M, V]
    M = hd.shape[0]
    out = {"scores": S, "h_prime_exact": pre, "h_prime": hp,
           "topk_idx": np.zeros((M, k), np.int64), "topk_logit": np.zeros((M, k)),
           "topk_prob": np.zeros((M, k)), "token": np.zeros(M, np.int64),
           "lse": np.zeros(M), "logprob": np.zeros(M), "diag": []}
    for m in range(M):
        K = topk_ascending(S[m], k)
        rows = fp.decode(np.asarray(U)[K], dtype)  # gathered rows U[K,:]
        zp = rows @ hd[m]
        y = zp / temperature
        lse = logsumexp(y)
        q = np.exp(y - lse)
        if mode == GREEDY:
            j, margin = _argmax_lowest(zp)
            dg = {"margin": margin}
        else:
            j, dg = two_level_sample(
                y,
                lambda g: uniforms(seed, offset, PURPOSE_DRAFT_GROUP, m, g),
                lambda i: uniforms(seed, offset, PURPOSE_DRAFT_ELEM, m, i),
            )
        out["topk_idx"][m] = K
        out["topk_logit"][m] = zp
        out["topk_prob"][m] = q
        out["token"][m] = K[j]
        out["lse"][m] = lse
        out["logprob"][m] = y[j] - lse
        dg["position"] = int(j)
        out["diag"].append(dg)
    return out
