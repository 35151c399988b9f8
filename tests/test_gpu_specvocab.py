"""GPU parity of the SpecVocab head and its top-k building block against the oracle."""
import numpy as np
import pytest
import torch

from drafter_lm_head_slimspec_amd import configs, spechead as sh, synth
from oracle import fp, heads, philox
from tests import parity as P

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    sh.load()


@pytest.mark.parametrize("V,k", [(1000, 1), (1000, 7), (1000, 64), (1000, 1000), (151936, 2048), (5000, 4999)])
def test_topk_on_given_scores_is_exact(V, k):
    M = 3
    rng = np.random.default_rng(V + k)
    s = rng.standard_normal((M, V)).astype(np.float32)
    s[1] = np.round(s[1] * 4) / 4                 # many exact ties
    s[2, : V // 2] = 0.0                          # a large tied block, including -0.0
    s[2, 1::7] = -0.0
    P.log(f"topk M={M} V={V} k={k}")
    got = sh.topk(torch.from_numpy(s).cuda(), k).cpu().numpy()
    for m in range(M):
        want = heads.topk_ascending(s[m].astype(np.float64), k)
        np.testing.assert_array_equal(got[m], want)


def _specvocab(d, V, dprime, k, M, dtype, mode, T, seed, offset=2):
    P.log(f"specvocab d={d} V={V} d'={dprime} k={k} M={M} {dtype} {mode}")
    h = synth.hidden(M, d, dtype, seed)
    Wd, Wv, U = synth.specvocab_weights(V, d, dprime, dtype, seed)
    out = sh.draft_head_specvocab(P.to_device(h, dtype), P.to_device(Wd, dtype), P.to_device(Wv, dtype),
                                  P.to_device(U, dtype), k, mode=mode, temperature=T, seed=seed, offset=offset)
    torch.cuda.synchronize()
    o = heads.head_specvocab(h, Wd, Wv, U, k, dtype, mode, T, seed, offset)
    idx = out["topk_idx"].cpu().numpy()
    zl = out["topk_logit"].cpu().numpy()
    q = out["topk_prob"].cpu().numpy()
    tok = out["token"].cpu().numpy()
    terms = np.abs(fp.decode(h, dtype)) @ np.abs(fp.decode(Wd, dtype)).T
    bound = P.rounding_flip_bound(o["h_prime_exact"], terms, dtype, np.abs(fp.decode(Wv, dtype)))
    ex = P.Excusals(f"specvocab M={M} top-k boundary")
    Ud = None
    for m in range(M):
        s = o["scores"][m]
        assert np.all(np.diff(idx[m]) > 0), "top-k ids must be strictly ascending"
        gs, os_ = set(idx[m].tolist()), set(o["topk_idx"][m].tolist())
        same = gs == os_
        if not same:
            kth = np.sort(s)[::-1][k - 1]
            for i in gs ^ os_:
                tol = P.DEC_TOL * (1 + abs(kth)) + 2 * np.max(bound[m]) + 1e-6 * (1 + abs(kth))
                assert abs(s[i] - kth) <= tol, f"row {m}: id {i} score {s[i]} vs k-th {kth}"
            ex.add(("boundary", m, len(gs ^ os_) // 2))
        # exact logits of the GPU's candidates from the oracle's exact arithmetic
        if Ud is None:
            Ud = fp.decode(U, dtype)
        zo = Ud[idx[m]] @ fp.decode(h, dtype)[m]
        P.assert_logits_close(zl[m][None], zo[None], dtype, f"row {m} exact logits")
        np.testing.assert_allclose(q[m].sum(), 1.0, rtol=1e-4)
        if not same:
            continue
        np.testing.assert_allclose(q[m], o["topk_prob"][m], rtol=P.RTOL[dtype], atol=1e-7)
        if mode == "greedy":
            P.check_greedy_tokens(np.searchsorted(idx[m], tok[m:m + 1]), o["topk_logit"][m][None], ex)
        else:
            y = o["topk_logit"][m] / T
            jg = int(np.searchsorted(idx[m], tok[m]))
            assert idx[m][jg] == tok[m]
            P.check_sampled_token(jg, int(o["diag"][m]["position"]), y,
                                  lambda g, m=m: philox.uniforms(seed, offset, 0, m, g),
                                  lambda i, m=m: philox.uniforms(seed, offset, 1, m, i),
                                  o["diag"][m], lambda i, j: 0.0, ex, f"row{m}")
    ex.report(M, max_frac=0.1)


@pytest.mark.parametrize("mode", ["greedy", "sample"])
def test_tiny_specvocab(mode):
    w = configs.TINY
    _specvocab(w.d, w.V, w.dprime, w.k, w.Ms[0], w.dtype, mode, 1.0, seed=w.seeds["weights"])


@pytest.mark.parametrize("M", [1, 3, 12])
def test_small_bf16_specvocab(M):
    _specvocab(512, 3000, 32, 128, M, "bf16", "sample" if M != 3 else "greedy", 0.9, seed=21)


@pytest.mark.parametrize("M", configs.QWEN.Ms)
@pytest.mark.parametrize("mode", ["greedy", "sample"])
def test_qwen_specvocab_full(M, mode):
    w = configs.QWEN
    _specvocab(w.d, w.V, w.dprime, w.k, M, w.dtype, mode, 1.0, seed=w.seeds["weights"])


@pytest.mark.parametrize("V,k", [(5, 3), (64, 64), (2049, 100), (4097, 2048), (30000, 1)])
def test_topk_edge_shapes(V, k):
    """Shapes at the chunk and 64-score segment boundaries, a single score, k = V."""
    M = 4
    rng = np.random.default_rng(7 * V + k)
    s = rng.standard_normal((M, V)).astype(np.float32)
    s[1] = -np.abs(s[1]) * 1e30                    # negative only, large magnitudes
    s[2] = 1.5                                     # every score equal: the lowest k ids
    s[3, ::3] = s[3, 0]                            # a third of the row tied with one value
    P.log(f"topk edge M={M} V={V} k={k}")
    got = sh.topk(torch.from_numpy(s).cuda(), k).cpu().numpy()
    for m in range(M):
        np.testing.assert_array_equal(got[m], heads.topk_ascending(s[m].astype(np.float64), k))


def test_topk_on_a_dirty_workspace_repeats():
    """The workspace's contents on entry do not matter: calls on a workspace filled with
    junk, and repeated calls on one workspace, give the same ids."""
    M, V, k = 16, 151936, 2048
    rng = np.random.default_rng(5)
    s = torch.from_numpy(rng.standard_normal((M, V)).astype(np.float32)).cuda()
    first = sh.topk(s, k)
    ws = sh.workspace(sh.load().sh_topk_workspace_bytes(M, V, k), s.device, "topk")
    ws.fill_(0xA5)
    for _ in range(3):
        assert torch.equal(sh.topk(s, k), first)
    want = heads.topk_ascending(s[0].cpu().numpy().astype(np.float64), k)
    np.testing.assert_array_equal(first[0].cpu().numpy(), want)
