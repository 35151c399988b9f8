"""Greedy verification of a tree of candidate continuations.

Phrase-level speculation page ("短语级投机解码", section "更换单元：从 token 到短语"): the
candidates drafted in one round share prefixes and are organised as a prefix tree; the target
scores every node in one pass (a prefix-tree attention mask), and a candidate is kept only
where it equals the target's own argmax, so the output equals greedy decoding.

Tree layout (reading: the pages fix no format): nodes 0..N-1 of tree b; node 0 is the root
(the last accepted token, not itself verified); parent[n] < n for n >= 1; node_token[n] is the
token node n proposes; target_logits[b, n] are the target's scores for the token that follows
node n's prefix.  A node is accepted when its parent is accepted and its token equals the
argmax (ties -> lowest id) of its parent's target scores.  The deepest accepted node (ties ->
lowest index) ends the accepted path; the target's argmax after it is emitted as well (the
correction when the path stops early, the bonus when it reaches a leaf).  A node whose parent
index is not in [0, n) is never accepted.
"""
import numpy as np

from . import fp


def verify_tree_greedy(target_logits, node_token, parent, dtype):
    """target_logits [B, N, V], node_token [B, N], parent [B, N] ->
    (accept_len [B], accept_node [B], out_tokens [B, N] with -1 padding)."""
    tl = fp.decode(target_logits, dtype)
    tok = np.asarray(node_token, dtype=np.int64)
    par = np.asarray(parent, dtype=np.int64)
    B, N = tok.shape
    acc_len = np.zeros(B, np.int64)
    acc_node = np.zeros(B, np.int64)
    out = np.full((B, N), -1, np.int64)
    for b in range(B):
        g = [int(np.argmax(tl[b, n])) for n in range(N)]
        accepted = [False] * N
        depth = [0] * N
        accepted[0] = True
        for n in range(1, N):
            p = int(par[b, n])
            if 0 <= p < n and accepted[p] and tok[b, n] == g[p]:
                accepted[n] = True
                depth[n] = depth[p] + 1
        best = 0
        for n in range(1, N):
            if accepted[n] and depth[n] > depth[best]:
                best = n
        path = []
        n = best
        while n != 0:
            path.append(int(tok[b, n]))
            n = int(par[b, n])
        path.reverse()
        acc_len[b] = len(path)
        acc_node[b] = best
        out[b, :len(path)] = path
        out[b, len(path)] = g[best]
    return acc_len, acc_node, out
