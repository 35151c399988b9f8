"""GPU parity of greedy tree verification with the oracle's verify_tree_greedy, through the C
ABI (bit-exact: every output is an integer decided by argmaxes)."""
import numpy as np
import pytest
import torch

from drafter_lm_head_slimspec_amd import configs, spechead as sh, synth
from oracle import tree, verify
from tests import parity as P

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    sh.load()


def _run(inp, dtype):
    acc, node, out = sh.spec_verify_tree(P.to_device(inp["target"], dtype),
                                         torch.from_numpy(np.ascontiguousarray(inp["tokens"])).cuda(),
                                         torch.from_numpy(np.ascontiguousarray(inp["parent"])).cuda())
    torch.cuda.synchronize()
    return acc.cpu().numpy(), node.cpu().numpy(), out.cpu().numpy()


def _check(inp, dtype):
    acc, node, out = _run(inp, dtype)
    oa, on, oo = tree.verify_tree_greedy(inp["target"], inp["tokens"], inp["parent"], dtype)
    np.testing.assert_array_equal(acc, oa)
    np.testing.assert_array_equal(node, on)
    np.testing.assert_array_equal(out, oo)
    P.log(f"  mean accepted depth {oa.mean():.3f} (max {oa.max()})")
    return oa


SEEDS = {"logits": 71, "tokens": 72, "uniforms": 73}


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("sigma", [0.3, 1.0])
def test_random_trees(dtype, sigma):
    P.log(f"tree B=16 N=32 V=1000 sigma={sigma} {dtype}")
    inp = synth.tree_inputs(16, 32, 1000, sigma, dtype, SEEDS)
    oa = _check(inp, dtype)
    if sigma == 0.3:
        assert oa.max() >= 2   # the recipe produces accepted paths, not only roots


def test_chain_tree_equals_linear_greedy_verification():
    # a chain of N nodes is the linear case with gamma = N - 1 drafts
    w = configs.VERIFY
    B, N = 8, w.gamma + 1
    inp = synth.verify_inputs(B, w.gamma, w.V, 0.5, w.dtype, w.seeds, mode="greedy")
    tok = np.zeros((B, N), np.int32)
    tok[:, 1:] = inp["tokens"]
    par = np.tile(np.arange(-1, N - 1, dtype=np.int32), (B, 1))
    acc, node, out = _run({"target": inp["target"], "tokens": tok, "parent": par}, w.dtype)
    la, lo = sh.spec_verify(P.to_device(inp["target"], w.dtype), None, torch.from_numpy(inp["tokens"]).cuda(),
                            None, mode="greedy")
    torch.cuda.synchronize()
    np.testing.assert_array_equal(acc, la.cpu().numpy())
    np.testing.assert_array_equal(out, lo.cpu().numpy())
    np.testing.assert_array_equal(node, acc)
    oa, oo = verify.verify_greedy(inp["target"], inp["tokens"], w.dtype)
    np.testing.assert_array_equal(acc, oa)


def test_bad_parents_single_node_and_ties():
    V, N = 64, 6
    rng = np.random.default_rng(5)
    z = rng.standard_normal((3, N, V)).astype(np.float32)
    g = z.argmax(-1)
    par = np.tile(np.array([-1, 0, 1, 2, 3, 4], np.int32), (3, 1))
    tok = np.zeros((3, N), np.int32)
    for b in range(3):
        for n in range(1, N):
            tok[b, n] = g[b, n - 1]
    par[0, 3] = 7       # not before the node: nodes 3.. are cut off
    par[1, 2] = -4
    z[2, 0, 10] = z[2, 0, 20] = z[2, 0].max() + 1.0   # tie in the root row -> lowest id (10)
    tok[2, 1] = 20
    inp = {"target": z, "tokens": tok, "parent": par}
    acc, node, out = _run(inp, "f32")
    oa, on, oo = tree.verify_tree_greedy(z, tok, par, "f32")
    np.testing.assert_array_equal(acc, oa)
    np.testing.assert_array_equal(node, on)
    np.testing.assert_array_equal(out, oo)
    assert acc[0] == 2 and acc[1] == 1 and acc[2] == 0 and out[2, 0] == 10
    # one node: only the root, its argmax is emitted
    one = {"target": z[:, :1].copy(), "tokens": tok[:, :1].copy(), "parent": par[:, :1].copy()}
    acc, node, out = _run(one, "f32")
    assert np.all(acc == 0) and np.all(node == 0)
    np.testing.assert_array_equal(out[:, 0], z[:, 0].argmax(-1))


def test_largest_tree():
    P.log("tree B=3 N=1024 V=256")
    inp = synth.tree_inputs(3, 1024, 256, 0.2, "bf16", SEEDS, chain=0.9)
    _check(inp, "bf16")


def test_tree_full_vocabulary():
    P.log("tree B=16 N=16 V=151936")
    w = configs.VERIFY
    inp = synth.tree_inputs(16, 16, w.V, 0.5, w.dtype, w.seeds)
    _check(inp, w.dtype)
