"""Planted winners for each streaming pass of the heads, through the C ABI.

The tile pass (low-rank rows of at most 512 elements, at most 64 activation rows) hands
64-row vocabulary groups to waves in a stride over the grid; the wide pass (65-256 rows) and
the K-chunked pass (rows longer than 512 elements) give each workgroup a consecutive range
of groups.  A mistake in that bookkeeping (a group skipped or read twice, a wrong owner of
the winning group's logits, the short last group) shows only when the winner sits there, so
these cases move the winner of each activation row onto such a group: the first group, the
short last group, the ends of the ranges of workgroups 1, 128 and 255 (for a 256-workgroup
grid), and the tile pass's wave-stride seams (groups 3 / 4, 1023 / 1024).

Greedy: one vocabulary row per activation row gets the logit ~beta by a weight row parallel
to that row's activations.  Sampling: all rows of the planted group get logits beta + N(0, 1),
so that group carries nearly all the mass and the element draw inside it is not trivial.
Expected values are the oracle's on the planted inputs (planting uses only the oracle's h_r).
"""
import numpy as np
import pytest
import torch

from drafter_lm_head_slimspec_amd import spechead as sh, synth
from oracle import fp, heads
from tests import parity as P
from tests.test_gpu_heads import _check_outputs, _lowrank_check

pytestmark = pytest.mark.gpu
G = 64


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    sh.load()


def boundary_groups(NG):
    cand = [0, NG - 1, 3, 4, 1023, 1024]
    for p in (1, 128, 255):
        b = p * NG // 256
        cand += [b, b - 1]
    out = []
    for g in cand:
        if 0 <= g < NG and g not in out:
            out.append(g)
    return out


def plant(W, X, mode, seed, beta):
    """W: [V, K] weights in storage format; X: [M, K] float64 activations of the final
    product.  Returns (planted weights, {row: planted id (greedy) or group (sampling)})."""
    W = W.copy()
    V = W.shape[0]
    NG = (V + G - 1) // G
    groups = boundary_groups(NG)
    rng = np.random.default_rng(seed)
    dt = "bf16" if W.dtype == np.uint16 else "f32"
    planted, used = {}, set()
    for m in range(X.shape[0]):
        g = groups[m % len(groups)]
        lo, hi = g * G, min(V, g * G + G)
        u = X[m] / np.dot(X[m], X[m])
        if mode == "greedy":
            i = lo + (13 * m + 5 * (m // len(groups))) % (hi - lo)
            if m == 1:
                i = hi - 1   # the last row of the vocabulary
            if i in used:
                continue
            used.add(i)
            W[i] = synth.store((beta * u).astype(np.float32), dt)
            planted[m] = i
        else:
            if m >= len(groups):
                continue
            c = beta + rng.standard_normal(hi - lo)
            W[lo:hi] = synth.store((c[:, None] * u[None, :]).astype(np.float32), dt)
            planted[m] = g
    return W, planted


def _hits(o_tok, planted, mode):
    if mode == "greedy":
        return sum(int(o_tok[m]) == i for m, i in planted.items())
    return sum(int(o_tok[m]) // G == g for m, g in planted.items())


TILE = [
    # d, V, r, M         tile pass: V past 1024 groups (two groups for the first waves), short last group
    (512, 100000, 512, 48),
    (512, 100000, 128, 6),
    (520, 70001, 384, 64),
    (512, 100000, 256, 1),
]
WIDE = [
    # d, V, r, M         wide pass (65-256 activation rows)
    (512, 100000, 360, 192),
    (256, 70001, 512, 100),
]


@pytest.mark.parametrize("mode,want_lse", [("greedy", True), ("greedy", False), ("sample", True)])
@pytest.mark.parametrize("case", TILE + WIDE, ids=lambda c: "d%d-V%d-r%d-M%d" % c)
def test_lowrank_planted(case, mode, want_lse):
    d, V, r, M = case
    seed, offset, T = 31, 6, (0.7 if M > 64 else 1.0)
    P.log(f"planted lowrank d={d} V={V} r={r} M={M} {mode} lse={want_lse}")
    h = synth.hidden(M, d, "bf16", seed)
    Wd, Wu = synth.lowrank_weights(V, d, r, "bf16", seed)
    _, hr_o = heads.lowrank_down(h, Wd, "bf16")
    Wu, planted = plant(Wu, hr_o, mode, seed, 10.0 if mode == "greedy" else 12.0)
    out = sh.draft_head_lowrank(P.to_device(h, "bf16"), P.to_device(Wd, "bf16"), P.to_device(Wu, "bf16"),
                                mode=mode, temperature=T, seed=seed, offset=offset, want_lse=want_lse,
                                want_intermediate=True)
    torch.cuda.synchronize()
    o = _lowrank_check(out, h, Wd, Wu, "bf16", mode, T, seed, offset, f"planted lowrank M={M}")
    hits = _hits(o["token"], planted, mode)
    P.log(f"  oracle picks the planted winner in {hits} of {len(planted)} rows")
    assert hits >= 0.9 * len(planted)


KCHUNK = [
    # d, V, M            K-chunked pass (rows longer than 512 elements)
    (1024, 100000, 48),
    (4096, 70001, 6),
    (2048, 100000, 64),
    (1024, 100000, 1),
]


@pytest.mark.parametrize("mode,want_lse", [("greedy", True), ("greedy", False), ("sample", True)])
@pytest.mark.parametrize("case", KCHUNK, ids=lambda c: "d%d-V%d-M%d" % c)
def test_dense_planted(case, mode, want_lse):
    d, V, M = case
    seed, offset, T = 37, 2, 1.0
    P.log(f"planted dense d={d} V={V} M={M} {mode} lse={want_lse}")
    h = synth.hidden(M, d, "bf16", seed)
    W = synth.dense_weights(V, d, "bf16", seed)
    W, planted = plant(W, fp.decode(h, "bf16"), mode, seed, 10.0 if mode == "greedy" else 12.0)
    out = sh.draft_head_dense(P.to_device(h, "bf16"), P.to_device(W, "bf16"), mode=mode, temperature=T,
                              seed=seed, offset=offset, want_lse=want_lse)
    torch.cuda.synchronize()
    o = heads.head_dense(h, W, "bf16", mode, T, seed, offset)
    _check_outputs(out, o, "bf16", mode, T, seed, offset, f"planted dense M={M}")
    hits = _hits(o["token"], planted, mode)
    P.log(f"  oracle picks the planted winner in {hits} of {len(planted)} rows")
    assert hits >= 0.9 * len(planted)
