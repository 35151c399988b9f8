"""GPU parity of the SpecVocab head and its top-k building block against the oracle."""
import numpy as np
import pytest
import torch

from drafter_lm_head_slimspec_amd import configs, spechead as sh, synth
from oracle import fp, heads, philox, sampler
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
    """Each stage against the oracle on the inputs the GPU stage actually used: h' against the
    oracle's single rounding; the candidate set against the oracle's top-k of W_vocab h'_gpu
    (swaps only at a near-tie with the k-th score); the exact logits, softmax, lse, logprob and
    token against the oracle's arithmetic on the GPU's own candidate set."""
    P.log(f"specvocab d={d} V={V} d'={dprime} k={k} M={M} {dtype} {mode}")
    h = synth.hidden(M, d, dtype, seed)
    Wd, Wv, U = synth.specvocab_weights(V, d, dprime, dtype, seed)
    out = sh.draft_head_specvocab(P.to_device(h, dtype), P.to_device(Wd, dtype), P.to_device(Wv, dtype),
                                  P.to_device(U, dtype), k, mode=mode, temperature=T, seed=seed, offset=offset,
                                  want_intermediate=True)
    torch.cuda.synchronize()
    idx = out["topk_idx"].cpu().numpy()
    zl = out["topk_logit"].cpu().numpy()
    q = out["topk_prob"].cpu().numpy()
    tok = out["token"].cpu().numpy()
    lse = out["lse"].cpu().numpy()
    lp = out["logprob"].cpu().numpy()
    hd = fp.decode(h, dtype)
    pre = hd @ fp.decode(Wd, dtype).T
    terms = np.abs(hd) @ np.abs(fp.decode(Wd, dtype)).T
    hp = fp.decode(_bits(out["h_prime"], dtype), dtype)
    P.check_intermediate(hp, pre, terms, dtype, f"specvocab M={M} h'")
    scores = hp @ fp.decode(Wv, dtype).T
    Ud = fp.decode(U, dtype)
    ex = P.Excusals(f"specvocab M={M} top-k boundary")
    ext = P.Excusals(f"specvocab M={M} tokens")
    lse_o, ytok = np.zeros(M), np.zeros(M)
    for m in range(M):
        s = scores[m]
        assert np.all(np.diff(idx[m]) > 0), "top-k ids must be strictly ascending"
        K_o = heads.topk_ascending(s, k)
        gs, os_ = set(idx[m].tolist()), set(K_o.tolist())
        if gs != os_:
            kth = np.sort(s)[::-1][k - 1]
            for i in gs ^ os_:
                tol = P.DEC_TOL * (1 + abs(kth))
                assert abs(s[i] - kth) <= tol, f"row {m}: id {i} score {s[i]} vs k-th {kth}"
            ex.add(("boundary", m, len(gs ^ os_) // 2))
        # exact logits of the GPU's candidates (full-precision h), then softmax and the draw
        zo = Ud[idx[m]] @ hd[m]
        P.assert_logits_close(zl[m][None], zo[None], dtype, f"row {m} exact logits")
        y = zo / T
        lse_o[m] = sampler.logsumexp(y)
        qo = np.exp(y - lse_o[m])
        tolq = P.LSE_RTOL * (1 + abs(lse_o[m]) + np.abs(y)) * qo + 1e-9
        assert np.all(np.abs(q[m] - qo) <= tolq), f"row {m}: softmax off by {np.max(np.abs(q[m] - qo) / tolq)} tol"
        jg = int(np.searchsorted(idx[m], tok[m]))
        assert jg < k and idx[m][jg] == tok[m], "the token is one of the candidates"
        ytok[m] = y[jg]
        if mode == "greedy":
            P.check_greedy_tokens(np.array([jg]), zo[None], ext)
        else:
            jo, dg = sampler.two_level_sample(y, lambda g, m=m: philox.uniforms(seed, offset, 0, m, g),
                                              lambda i, m=m: philox.uniforms(seed, offset, 1, m, i))
            P.check_sampled_token(jg, int(jo), y, lambda g, m=m: philox.uniforms(seed, offset, 0, m, g),
                                  lambda i, m=m: philox.uniforms(seed, offset, 1, m, i), dg,
                                  lambda i, j: 0.0, ext, f"row{m}")
    ex.report(M, max_frac=0.1)
    ext.report(M)
    P.check_lse_logprob(lse, lp, lse_o, ytok, f"specvocab M={M}")


def _bits(t, dtype):
    if dtype == "bf16":
        return t.cpu().view(torch.int16).numpy().view(np.uint16)
    return t.cpu().numpy()


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
    """Shapes at the chunk and 64-score segment boundaries, a single score, k = V; a row whose
    scores share their top 12 key bits and differ in every lower bit (each level of the threshold
    search decides)."""
    M = 5
    rng = np.random.default_rng(7 * V + k)
    s = rng.standard_normal((M, V)).astype(np.float32)
    s[1] = -np.abs(s[1]) * 1e30                    # negative only, large magnitudes
    s[2] = 1.5                                     # every score equal: the lowest k ids
    s[3, ::3] = s[3, 0]                            # a third of the row tied with one value
    s[4] = rng.permutation(np.float32(1.0) + np.arange(V, dtype=np.float32) * np.float32(2.0 ** -23))
    P.log(f"topk edge M={M} V={V} k={k}")
    got = sh.topk(torch.from_numpy(s).cuda(), k).cpu().numpy()
    for m in range(M):
        np.testing.assert_array_equal(got[m], heads.topk_ascending(s[m].astype(np.float64), k))


@pytest.mark.parametrize("V,k", [(5, 3), (64, 64), (2049, 100), (4097, 2048), (30000, 1), (20000, 9000),
                                 (151936, 2048)])
def test_topk_one_and_two_rows(V, k):
    """One or two rows take the one-workgroup selection (threshold bin, the row streamed into
    LDS, the finish): each kind of row alone and in pairs, among them every score equal (all V
    keys inside the threshold bin, so the candidate list spills past LDS to the global list),
    rounded scores with many exact ties, a tied block of zeros including -0.0, and scores that
    share their top 12 key bits and differ below."""
    rng = np.random.default_rng(11 * V + k)
    s = rng.standard_normal((8, V)).astype(np.float32)
    s[1] = np.round(s[1] * 4) / 4
    s[2, : V // 2] = 0.0
    s[2, 1::7] = -0.0
    s[3] = -np.abs(s[3]) * 1e30
    s[4] = 1.5
    s[5, ::3] = s[5, 0]
    s[6] = rng.permutation(np.float32(1.0) + np.arange(V, dtype=np.float32) * np.float32(2.0 ** -23))
    want = [heads.topk_ascending(s[m].astype(np.float64), k) for m in range(8)]
    P.log(f"topk one/two rows V={V} k={k}")
    for m in range(8):
        got = sh.topk(torch.from_numpy(s[m:m + 1].copy()).cuda(), k).cpu().numpy()
        np.testing.assert_array_equal(got[0], want[m])
    for m in range(0, 8, 2):
        got = sh.topk(torch.from_numpy(s[m:m + 2].copy()).cuda(), k).cpu().numpy()
        np.testing.assert_array_equal(got[0], want[m])
        np.testing.assert_array_equal(got[1], want[m + 1])


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
