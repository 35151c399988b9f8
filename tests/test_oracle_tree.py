"""Pins of the greedy tree verification oracle (CPU)."""
import itertools

import numpy as np

from oracle import tree, verify


def _logits_with_argmax(g, V, rng):
    """Random fp32 logits [N, V] whose row n has its unique maximum at g[n]."""
    z = rng.standard_normal((len(g), V)).astype(np.float32)
    for n, t in enumerate(g):
        z[n, t] = np.max(z[n]) + 1.0
    return z


def test_chain_tree_is_linear_greedy_verification():
    # a chain (node n's parent is n-1) is the linear case: gamma = N-1 drafts
    rng = np.random.default_rng(1)
    B, N, V = 16, 6, 50
    tl = rng.standard_normal((B, N, V)).astype(np.float32)
    g = tl.argmax(-1)
    tok = np.zeros((B, N), np.int64)
    for b in range(B):
        k = b % N   # first k drafts match the argmax chain, then a mismatch
        for n in range(1, N):
            tok[b, n] = g[b, n - 1] if n <= k else (g[b, n - 1] + 1) % V
    par = np.tile(np.arange(-1, N - 1), (B, 1))
    a, node, out = tree.verify_tree_greedy(tl, tok, par, "f32")
    la, lout = verify.verify_greedy(tl, tok[:, 1:], "f32")
    np.testing.assert_array_equal(a, la)
    np.testing.assert_array_equal(out, lout)
    np.testing.assert_array_equal(node, la)   # on a chain the deepest node's index is its depth


def _brute_force(tl, tok, par):
    """Every node's root path checked prefix by prefix (no propagation)."""
    N = tok.shape[0]
    g = tl.argmax(-1)
    best, best_path = 0, []
    for n in range(1, N):
        path, m, ok = [], n, True
        while m != 0:
            p = par[m]
            if not (0 <= p < m):
                ok = False
                break
            path.append(m)
            m = p
        if not ok:
            continue
        path.reverse()
        prev = 0
        for m in path:
            if tok[m] != g[prev]:
                ok = False
                break
            prev = m
        if ok and len(path) > len(best_path):
            best, best_path = n, path
    return len(best_path), best, [int(tok[m]) for m in best_path] + [int(g[best])]


def test_random_trees_match_brute_force():
    rng = np.random.default_rng(2)
    for trial in range(200):
        N = int(rng.integers(1, 14))
        V = int(rng.integers(2, 5))    # small V: many matches and duplicate siblings
        par = np.array([-1] + [int(rng.integers(0, n)) for n in range(1, N)])
        g = rng.integers(0, V, N)
        tl = _logits_with_argmax(g, V, rng)
        tok = rng.integers(0, V, N)
        a, node, out = tree.verify_tree_greedy(tl[None], tok[None], par[None], "f32")
        ba, bn, bpath = _brute_force(tl, tok, par)
        assert a[0] == ba and node[0] == bn, (trial, par, tok, g)
        np.testing.assert_array_equal(out[0, :ba + 1], bpath)
        assert np.all(out[0, ba + 1:] == -1)


def test_duplicate_siblings_take_lowest_index_and_bad_parents_are_rejected():
    V = 4
    g = [2, 1, 1, 3, 0]
    rng = np.random.default_rng(3)
    tl = _logits_with_argmax(g, V, rng)
    # nodes 1 and 2 both carry token 2 (= argmax after the root); node 3 under node 2 matches
    tok = np.array([0, 2, 2, 1, 3])
    par = np.array([-1, 0, 0, 2, 3])
    a, node, out = tree.verify_tree_greedy(tl[None], tok[None], par[None], "f32")
    assert a[0] == 3 and node[0] == 4
    np.testing.assert_array_equal(out[0], [2, 1, 3, 0, -1])
    # equal depth: nodes 1 and 2 alone -> the lower index wins
    a, node, out = tree.verify_tree_greedy(tl[None, :3], tok[None, :3], par[None, :3], "f32")
    assert a[0] == 1 and node[0] == 1
    # a parent index that does not precede the node is never accepted
    par_bad = np.array([-1, 0, 5, 2, 3])
    a, node, out = tree.verify_tree_greedy(tl[None], tok[None], par_bad[None], "f32")
    assert a[0] == 1 and node[0] == 1
