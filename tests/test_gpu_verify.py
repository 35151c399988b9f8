"""GPU parity of batched verification (greedy and rejection sampling) against the oracle."""
import numpy as np
import pytest
import torch

from drafter_lm_head_slimspec_amd import configs, spechead as sh, synth
from oracle import fp, philox, sampler, verify
from tests import parity as P

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    sh.load()


def _dev(inp, dtype):
    return {"target": P.to_device(inp["target"], dtype), "draft": P.to_device(inp["draft"], dtype),
            "tokens": torch.from_numpy(inp["tokens"]).cuda(), "u": torch.from_numpy(inp["u"]).cuda()}


def _greedy(B, gamma, V, sigma, dtype, seeds):
    P.log(f"verify greedy B={B} gamma={gamma} V={V} sigma={sigma} {dtype}")
    inp = synth.verify_inputs(B, gamma, V, sigma, dtype, seeds, mode="greedy")
    d = _dev(inp, dtype)
    acc, out = sh.spec_verify(d["target"], None, d["tokens"], None, mode="greedy")
    torch.cuda.synchronize()
    oa, oo = verify.verify_greedy(inp["target"], inp["tokens"], dtype)
    np.testing.assert_array_equal(acc.cpu().numpy(), oa)
    np.testing.assert_array_equal(out.cpu().numpy(), oo)
    P.log(f"  mean accepted {oa.mean():.3f}")


def _sample(B, gamma, V, sigma, dtype, seeds, T=1.0, seed=99, offset=7, tokens=None, mutate=None):
    P.log(f"verify sample B={B} gamma={gamma} V={V} sigma={sigma} {dtype} T={T}")
    inp = synth.verify_inputs(B, gamma, V, sigma, dtype, seeds, mode="sample", temperature=T)
    if tokens is not None:
        inp["tokens"] = tokens
    if mutate is not None:
        mutate(inp)
    d = _dev(inp, dtype)
    acc, out = sh.spec_verify(d["target"], d["draft"], d["tokens"], d["u"], mode="sample", temperature=T,
                              seed=seed, offset=offset)
    torch.cuda.synchronize()
    acc, out = acc.cpu().numpy(), out.cpu().numpy()
    oa, oo, diag = verify.verify_sample(inp["target"], inp["draft"], inp["tokens"], inp["u"], dtype, T, seed, offset)
    ex = P.Excusals(f"verify sigma={sigma}")
    u = inp["u"].astype(np.float64)
    for b in range(B):
        if acc[b] != oa[b]:
            t = min(acc[b], oa[b])
            r = diag["ratio"][b, t]
            assert abs(u[b, t] - r) < 1e-6, f"seq {b}: accept {acc[b]} vs {oa[b]}, |u - p/q| = {abs(u[b, t] - r)}"
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
        elif not np.any(dg["p"] - dg["q"] > 0):
            # no residual mass: the draw falls back to p at the rejected position
            ell = tl[a]
            gp, ep = philox.PURPOSE_RESID_GROUP, philox.PURPOSE_RESID_ELEM
            tol_fn = lambda i, j: 0.0
        else:
            p, q = dg["p"], dg["q"]
            r = p - q
            with np.errstate(divide="ignore"):
                ell = np.where(r > 0, np.log(np.where(r > 0, r, 1.0)), -np.inf)
            gp, ep = philox.PURPOSE_RESID_GROUP, philox.PURPOSE_RESID_ELEM
            # fp32 error of p - q relative to the residual itself
            err = 4e-6 * (p + q) + 1e-30

            def tol_fn(i, j, r=r, err=err):
                if isinstance(i, slice):
                    si, sj = np.sum(np.maximum(r[i], 0)), np.sum(np.maximum(r[j], 0))
                    return np.sum(err[i]) / max(si, 1e-300) + np.sum(err[j]) / max(sj, 1e-300)
                return err[i] / max(abs(r[i]), 1e-300) + err[j] / max(abs(r[j]), 1e-300)
        P.check_sampled_token(tg, to, ell, lambda g, b=b: philox.uniforms(seed, offset, gp, b, g),
                              lambda i, b=b: philox.uniforms(seed, offset, ep, b, i), dg, tol_fn, ex,
                              f"seq{b}-{dg['kind']}")
    ex.report(B, max_frac=0.05)
    P.log(f"  mean accepted {oa.mean():.3f}, emitted {oa.mean() + 1:.3f}")
    return acc


@pytest.mark.parametrize("sigma", [0.5, 1.0, 2.0])
def test_tiny_verify(sigma):
    w = configs.TINY_VERIFY
    _greedy(8, w.gamma, w.V, sigma, w.dtype, w.seeds)
    _sample(8, w.gamma, w.V, sigma, w.dtype, w.seeds)


def test_small_bf16_ragged_groups():
    # V not a multiple of 64: last group is partial
    seeds = {"logits": 31, "tokens": 32, "uniforms": 33}
    _greedy(5, 3, 1000, 1.0, "bf16", seeds)
    _sample(5, 3, 1000, 1.0, "bf16", seeds, T=0.8)


def test_invalid_draft_ids_are_rejected():
    seeds = {"logits": 41, "tokens": 42, "uniforms": 43}
    B, gamma, V = 4, 3, 1024
    inp = synth.verify_inputs(B, gamma, V, 1.0, "f32", seeds)
    tok = inp["tokens"].copy()
    tok[0, 0] = -1
    tok[1, 1] = V
    tok[2, 2] = 1 << 30
    acc = _sample(B, gamma, V, 1.0, "f32", seeds, tokens=tok)
    assert acc[0] == 0 and acc[1] <= 1 and acc[2] <= 2


def test_zero_residual_falls_back_to_target():
    """Draft equal to target makes p - q vanish; a rejected (invalid) draft id then leaves no
    residual mass and the token is drawn from p at that position."""
    seeds = {"logits": 51, "tokens": 52, "uniforms": 53}
    B, gamma, V = 6, 3, 1000

    def same_draft(inp):
        inp["draft"] = inp["target"][:, :gamma].copy()
        for b in range(B):
            inp["tokens"][b, b % gamma] = -5

    acc = _sample(B, gamma, V, 1.0, "bf16", seeds, mutate=same_draft)
    assert np.all(acc == np.arange(B) % gamma)


def test_verify_on_a_dirty_workspace():
    w = configs.VERIFY
    B = 32
    inp = synth.verify_inputs(B, w.gamma, w.V, 1.0, "bf16", w.seeds)
    d = _dev(inp, "bf16")
    a1, o1 = sh.spec_verify(d["target"], d["draft"], d["tokens"], d["u"], seed=5, offset=1)
    need = sh.load().sh_verify_workspace_bytes(sh.SAMPLE, B, w.gamma, w.V)
    sh.workspace(need, d["target"].device, "verify").fill_(0x5A)
    a2, o2 = sh.spec_verify(d["target"], d["draft"], d["tokens"], d["u"], seed=5, offset=1)
    torch.cuda.synchronize()
    assert torch.equal(a1, a2) and torch.equal(o1, o2)


@pytest.mark.parametrize("sigma", configs.VERIFY.sigmas)
def test_full_verify(sigma):
    w = configs.VERIFY
    _greedy(w.B, w.gamma, w.V, sigma, w.dtype, w.seeds)
    _sample(w.B, w.gamma, w.V, sigma, w.dtype, w.seeds)


def test_verify_bit_identical_runs():
    w = configs.VERIFY
    inp = synth.verify_inputs(16, w.gamma, w.V, 1.0, "bf16", w.seeds)
    d = _dev(inp, "bf16")
    a1, o1 = sh.spec_verify(d["target"], d["draft"], d["tokens"], d["u"], seed=5, offset=1)
    a2, o2 = sh.spec_verify(d["target"], d["draft"], d["tokens"], d["u"], seed=5, offset=1)
    torch.cuda.synchronize()
    assert torch.equal(a1, a2) and torch.equal(o1, o2)


@pytest.mark.parametrize("dtype,V", [("bf16", 4096), ("f32", 1000)])
def test_draft_excluding_tokens(dtype, V):
    """A draft that gives some tokens zero probability (-inf scores, as a drafter over a trimmed
    vocabulary does for every token outside it; SlimSpec write-up, section 二): three quarters
    of the vocabulary masked in every draft row, whole 8-element chunks of it included, and a
    few masked target scores.  Draft tokens come from the masked draft distribution."""
    B, gamma = 48, 4
    seeds = {"logits": 61, "tokens": 62, "uniforms": 63}
    rng = np.random.default_rng(64)
    keep = np.sort(rng.choice(V, V // 4, replace=False))
    masked = np.setdiff1d(np.arange(V), keep)
    ninf = synth.store(np.array([-np.inf], np.float32), dtype)[0]

    def mask(inp):
        inp["draft"][:, :, masked] = ninf
        inp["target"][:, :, masked[:5]] = ninf
        d = fp.decode(inp["draft"], dtype)
        g = np.random.default_rng(65).gumbel(size=d.shape)
        inp["tokens"] = np.argmax(d + g, axis=-1).astype(np.int32)
        assert np.all(np.isin(inp["tokens"], keep))

    acc = _sample(B, gamma, V, 0.5, dtype, seeds, mutate=mask)
    assert np.all(acc >= 0)
