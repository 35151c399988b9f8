"""Sampling rule of the oracle: two-level Gumbel-max over groups of 64 candidates.

The pages say a drafter samples from its softmax and that a rejected draft is replaced by a
draw from the normalised positive part of (p - q) (explainer, "为什么答案不会变"), but not
how the draw is made.  Reading used (and implemented independently by the HIP path):

  given log-weights l_i over candidate positions i = 0..n-1 (-inf allowed),
  1. split positions into groups of G = 64 consecutive ones (last group may be short);
  2. L_g = log sum_{i in g} exp(l_i);  group score L_g + Gumbel(u_g);  g* = argmax,
     ties -> lowest g;
  3. inside g*: token = argmax_i (l_i + Gumbel(u_i)), ties -> lowest i.

By the Gumbel-max property applied twice, P(g) = e^{L_g} / sum e^{L} and
P(i | g) = e^{l_i - L_g}, so P(i) = e^{l_i} / sum_j e^{l_j}: an exact draw from softmax(l).
"""
import numpy as np

from .philox import gumbel

GROUP = 64


def logsumexp(x):
    """log(sum(exp(x))) in float64, -inf for an empty or all -inf input."""
    x = np.asarray(x, dtype=np.float64)
    if x.size == 0:
        return -np.inf
    m = np.max(x)
    if m == -np.inf:
        return -np.inf
    return float(m + np.log(np.sum(np.exp(x - m))))


def _argmax_lowest(scores):
    """Index of the maximum, lowest index on ties, plus the gap to the runner-up."""
    s = np.asarray(scores, dtype=np.float64)
    i = int(np.argmax(s))            # numpy returns the first maximum
    if s.size > 1:
        rest = np.delete(s, i)
        gap = float(s[i] - np.max(rest))
    else:
        gap = np.inf
    return i, gap


def two_level_sample(ell, group_uniforms, elem_uniforms, group=GROUP):
    """Draw one position from softmax(ell).

    group_uniforms(g_idx) -> uniforms for group ids; elem_uniforms(i_idx) -> uniforms for
    candidate positions.  Returns (position, diag) or (None, diag) if every weight is 0.
    diag holds the decision margins (winner minus runner-up) used by parity tests.
    """
    ell = np.asarray(ell, dtype=np.float64)
    n = ell.size
    ng = (n + group - 1) // group
    L = np.array([logsumexp(ell[g * group:(g + 1) * group]) for g in range(ng)])
    gs = L + gumbel(group_uniforms(np.arange(ng)))
    if np.all(gs == -np.inf):
        return None, {"group_margin": np.inf, "elem_margin": np.inf, "group": -1}
    g_star, g_gap = _argmax_lowest(gs)
    lo, hi = g_star * group, min(n, (g_star + 1) * group)
    pos = np.arange(lo, hi)
    es = ell[lo:hi] + gumbel(elem_uniforms(pos))
    i_star, e_gap = _argmax_lowest(es)
    diag = {
        "group": g_star,
        "group_margin": g_gap,
        "group_score": float(gs[g_star]),
        "group_scores": gs,
        "elem_margin": e_gap,
        "elem_score": float(es[i_star]),
        "elem_scores": es,
        "group_lse": L,
    }
    return lo + i_star, diag


def pick_in_group(ell, g, elem_uniforms, group=GROUP):
    """The element step of the rule applied to group g: (position, scores of its members)."""
    ell = np.asarray(ell, dtype=np.float64)
    lo, hi = g * group, min(ell.size, (g + 1) * group)
    pos = np.arange(lo, hi)
    es = ell[lo:hi] + gumbel(elem_uniforms(pos))
    i_star, _ = _argmax_lowest(es)
    return lo + i_star, es
