"""GPU parity of sampling verification against a sparse draft distribution (the SpecVocab head's
top-k probabilities) with the oracle's verify_sample_sparse, through the C ABI."""
import numpy as np
import pytest
import torch

from drafter_lm_head_slimspec_amd import configs, spechead as sh, synth
from oracle import fp, philox, verify
from tests import parity as P

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    sh.load()


def _run(inp, dtype, T, seed, offset):
    d = {"target": P.to_device(inp["target"], dtype),
         "idx": torch.from_numpy(np.ascontiguousarray(inp["idx"])).cuda(),
         "prob": torch.from_numpy(np.ascontiguousarray(inp["prob"])).cuda(),
         "tokens": torch.from_numpy(np.ascontiguousarray(inp["tokens"])).cuda(),
         "u": torch.from_numpy(inp["u"]).cuda()}
    acc, out = sh.spec_verify_sparse(d["target"], d["idx"], d["prob"], d["tokens"], d["u"], temperature=T,
                                     seed=seed, offset=offset)
    torch.cuda.synchronize()
    return acc.cpu().numpy(), out.cpu().numpy()


def _sparse(B, gamma, V, k, sigma, dtype, seeds, T=1.0, seed=99, offset=7, mutate=None):
    P.log(f"verify sparse B={B} gamma={gamma} V={V} k={k} sigma={sigma} {dtype} T={T}")
    inp = synth.verify_sparse_inputs(B, gamma, V, k, sigma, dtype, seeds, temperature=T)
    if mutate is not None:
        mutate(inp)
    acc, out = _run(inp, dtype, T, seed, offset)
    oa, oo, diag = verify.verify_sample_sparse(inp["target"], inp["idx"], inp["prob"], inp["tokens"], inp["u"],
                                               dtype, T, seed, offset)
    ex = P.Excusals(f"verify sparse k={k} sigma={sigma}")
    u = inp["u"].astype(np.float64)
    for b in range(B):
        if acc[b] != oa[b]:
            # only an accept decision within float32 error of u = p/q may differ
            t = min(acc[b], oa[b])
            r = diag["ratio"][b, t]
            assert np.isfinite(r) and abs(u[b, t] - r) < 1e-5 * max(1.0, r), \
                f"seq {b}: accept {acc[b]} vs {oa[b]}, u={u[b, t]}, p/q={r}"
            ex.add(("accept", b, int(acc[b]), int(oa[b])))
            continue
        np.testing.assert_array_equal(out[b, :acc[b]], oo[b, :oa[b]])
        assert np.all(out[b, acc[b] + 1:] == -1)
        tg, to = int(out[b, acc[b]]), int(oo[b, oa[b]])
        dg = diag["sample"][b]
        a = int(oa[b])
        tl = fp.decode(inp["target"][b], dtype) / T
        if dg["kind"] == "bonus":
            ell = tl[gamma]
            gp, ep = philox.PURPOSE_BONUS_GROUP, philox.PURPOSE_BONUS_ELEM
            tol_fn = lambda i, j: 0.0
        else:
            p, q = dg["p"], dg["q"]
            r = p - q
            with np.errstate(divide="ignore"):
                ell = np.where(r > 0, np.log(np.where(r > 0, r, 1.0)), -np.inf)
            gp, ep = philox.PURPOSE_RESID_GROUP, philox.PURPOSE_RESID_ELEM
            # float32 error of p (q is an exact input) relative to the residual itself
            err = 4e-6 * p + 1e-30

            def tol_fn(i, j, r=r, err=err):
                if isinstance(i, slice):
                    si, sj = np.sum(np.maximum(r[i], 0)), np.sum(np.maximum(r[j], 0))
                    return np.sum(err[i]) / max(si, 1e-300) + np.sum(err[j]) / max(sj, 1e-300)
                return err[i] / max(abs(r[i]), 1e-300) + err[j] / max(abs(r[j]), 1e-300)
        P.check_sampled_token(tg, to, ell, lambda g, b=b: philox.uniforms(seed, offset, gp, b, g),
                              lambda i, b=b: philox.uniforms(seed, offset, ep, b, i), dg, tol_fn, ex,
                              f"seq{b}-{dg['kind']}")
    ex.report(B, max_frac=0.05)
    P.log(f"  mean accepted {oa.mean():.3f}")
    return inp, acc, out


SEEDS = {"logits": 61, "tokens": 62, "uniforms": 63}


@pytest.mark.parametrize("sigma", [0.5, 2.0])
def test_tiny_sparse(sigma):
    w = configs.TINY_VERIFY
    _sparse(8, w.gamma, w.V, 64, sigma, w.dtype, w.seeds)


def test_bf16_ragged_groups_and_temperature():
    # V not a multiple of 64; candidates straddle group boundaries
    _sparse(6, 3, 1000, 100, 1.0, "bf16", SEEDS, T=0.8)


def test_single_candidate():
    # k = 1: q is a point mass; p/q = p(x) at the one candidate
    _sparse(6, 4, 1024, 1, 1.0, "f32", SEEDS)


def test_full_support():
    # k = V: q is positive everywhere, the residual is max(0, p - q) on every id
    _sparse(4, 3, 512, 512, 1.0, "f32", SEEDS)


def test_token_outside_candidates_is_accepted():
    # q(x) = 0 < p(x): the ratio is infinite, every such draft is accepted
    B, gamma, V, k = 5, 4, 1024, 32

    def outside(inp):
        for b in range(B):
            for t in range(gamma):
                cand = set(inp["idx"][b, t].tolist())
                x = next(i for i in range(V) if i not in cand)
                inp["tokens"][b, t] = x
        inp["tokens"][0, 2] = V   # an id outside the vocabulary is still rejected

    inp, acc, out = _sparse(B, gamma, V, k, 1.0, "f32", SEEDS, mutate=outside)
    assert acc[0] == 2 and np.all(acc[1:] == gamma)


def test_many_candidates():
    # k = 5000: the candidate scans take several batches, and the residual pass reads the
    # candidate list from memory instead of holding it in registers
    _sparse(4, 3, 8000, 5000, 1.0, "bf16", SEEDS)


def test_sparse_full_shape():
    # the verification workload (B = 64, gamma = 5, V = 151936) with the SpecVocab k = 2048
    w = configs.VERIFY
    _sparse(w.B, w.gamma, w.V, 2048, 1.0, w.dtype, w.seeds)


def test_sparse_dirty_workspace_and_repeat():
    w = configs.VERIFY
    B, k = 16, 2048
    inp = synth.verify_sparse_inputs(B, w.gamma, w.V, k, 1.0, w.dtype, w.seeds)
    a1, o1 = _run(inp, w.dtype, 1.0, 5, 1)
    need = sh.load().sh_verify_sparse_workspace_bytes(B, w.gamma, w.V, k)
    sh.workspace(need, torch.device("cuda:0"), "verify").fill_(0x5A)
    a2, o2 = _run(inp, w.dtype, 1.0, 5, 1)
    np.testing.assert_array_equal(a1, a2)
    np.testing.assert_array_equal(o1, o2)
