"""Pins of the position-adaptive-rank low-rank head (CPU): the nested-prefix reading reduces
to the fixed-rank head on sliced factors, rows are independent, and rank 1 has a closed form."""
import numpy as np
import pytest

from drafter_lm_head_slimspec_amd import synth
from oracle import fp, heads


def _inputs(M, d, V, r, dtype, seed):
    h = synth.hidden(M, d, dtype, seed)
    Wd, Wu = synth.lowrank_weights(V, d, r, dtype, seed)
    return h, Wd, Wu


@pytest.mark.parametrize("mode", ["greedy", "sample"])
def test_full_rank_everywhere_is_the_fixed_rank_head(mode):
    h, Wd, Wu = _inputs(5, 96, 300, 32, "bf16", 1)
    a = heads.head_lowrank_adaptive(h, Wd, Wu, [32] * 5, "bf16", mode, 1.0, 4, 2)
    b = heads.head_lowrank(h, Wd, Wu, "bf16", mode, 1.0, 4, 2)
    np.testing.assert_array_equal(a["token"], b["token"])
    np.testing.assert_allclose(a["logits"], b["logits"], rtol=1e-12, atol=1e-12)   # fp64 summation order
    np.testing.assert_allclose(a["lse"], b["lse"], rtol=1e-12)


@pytest.mark.parametrize("r", [1, 7, 16])
def test_uniform_rank_is_the_head_of_the_sliced_pair(r):
    # nested prefixes: rank r uses W_down[:r] and W_up[:, :r]
    h, Wd, Wu = _inputs(4, 64, 200, 24, "f32", 2)
    a = heads.head_lowrank_adaptive(h, Wd, Wu, [r] * 4, "f32", "sample", 0.8, 3, 1)
    b = heads.head_lowrank(h, np.ascontiguousarray(Wd[:r]), np.ascontiguousarray(Wu[:, :r]), "f32", "sample",
                           0.8, 3, 1)
    np.testing.assert_array_equal(a["token"], b["token"])
    np.testing.assert_allclose(a["logits"], b["logits"], rtol=1e-12, atol=1e-12)   # fp64 summation order


def test_mixed_ranks_rows_are_independent():
    h, Wd, Wu = _inputs(6, 64, 500, 32, "bf16", 3)
    ranks = [32, 32, 24, 16, 8, 8]
    mixed = heads.head_lowrank_adaptive(h, Wd, Wu, ranks, "bf16", "sample", 1.0, 9, 5)
    for m, r in enumerate(ranks):
        one = heads.head_lowrank_adaptive(h, Wd, Wu, [r] * 6, "bf16", "sample", 1.0, 9, 5)
        assert mixed["token"][m] == one["token"][m]
        np.testing.assert_array_equal(mixed["logits"][m], one["logits"][m])
    # the masked h_r keeps exactly the first r_m entries of each row
    assert np.all(mixed["h_r"][4, 8:] == 0) and np.any(mixed["h_r"][4, :8] != 0)


def test_rank_one_closed_form():
    # z[v] = W_up[v, 0] * c with c = round(W_down[0] . h): greedy picks the extreme of column 0
    h, Wd, Wu = _inputs(3, 32, 100, 8, "f32", 4)
    out = heads.head_lowrank_adaptive(h, Wd, Wu, [1, 1, 1], "f32", "greedy")
    col = fp.decode(Wu, "f32")[:, 0]
    for m in range(3):
        c = float(np.float32(fp.decode(Wd, "f32")[0] @ fp.decode(h, "f32")[m]))
        want = int(np.argmax(col)) if c > 0 else int(np.argmin(col))
        assert out["token"][m] == want


def test_rank_outside_range_is_rejected():
    h, Wd, Wu = _inputs(2, 32, 64, 8, "f32", 5)
    with pytest.raises(ValueError):
        heads.head_lowrank_adaptive(h, Wd, Wu, [0, 4], "f32")
    with pytest.raises(ValueError):
        heads.head_lowrank_adaptive(h, Wd, Wu, [9, 4], "f32")
