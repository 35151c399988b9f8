"""GPU parity of the static trimmed-vocabulary head (dense head over kept rows W[ids], token
mapped to the vocabulary id) against the oracle's head_trimmed, through the C ABI."""
import numpy as np
import pytest
import torch

from drafter_lm_head_slimspec_amd import spechead as sh, synth
from oracle import heads
from tests import parity as P
from tests.test_gpu_heads import _check_outputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    sh.load()


def _trimmed(d, V, n, M, dtype, mode, T, seed=17, offset=4, want_logits=True):
    P.log(f"trimmed d={d} V={V} kept={n} M={M} {dtype} {mode} T={T}")
    rng = np.random.default_rng(seed)
    ids = np.sort(rng.choice(V, n, replace=False)).astype(np.int32)
    h = synth.hidden(M, d, dtype, seed)
    W = synth.dense_weights(V, d, dtype, seed)
    W_S = np.ascontiguousarray(W[ids])
    out = sh.draft_head_trimmed(P.to_device(h, dtype), P.to_device(W_S, dtype), torch.from_numpy(ids).cuda(),
                                mode=mode, temperature=T, seed=seed, offset=offset, want_logits=want_logits)
    torch.cuda.synchronize()
    o = heads.head_trimmed(h, W_S, ids, dtype, mode, T, seed, offset)
    tok = out["token"].cpu().numpy()
    assert np.all(np.isin(tok, ids)), "every token is a kept id"
    pos = np.searchsorted(ids, tok)
    got = dict(out)
    got["token"] = torch.from_numpy(pos.astype(np.int32))
    want = dict(o)
    want["token"] = o["position"]
    _check_outputs(got, want, dtype, mode, T, seed, offset, f"trimmed M={M}")


CASES = [
    # d, V, kept, M, dtype       path exercised
    (256, 1024, 300, 4, "f32"),     # fp32 VALU stream
    (512, 8000, 3000, 6, "bf16"),   # tile pass (rows of 512)
    (512, 8000, 3001, 48, "bf16"),  # tile pass, ragged last group
    (4096, 6000, 2000, 6, "bf16"),  # VALU stream, long rows
    (4096, 6000, 2000, 40, "bf16"), # MFMA stream
]


@pytest.mark.parametrize("mode,T", [("greedy", 1.0), ("sample", 1.0), ("sample", 0.6), ("greedy", 0.6)])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "d%d-V%d-n%d-M%d-%s" % c)
def test_trimmed(case, mode, T):
    # raw logits z (not z / T) are compared at every temperature
    _trimmed(*case, mode, T)


KCHUNK_CASES = [
    # d, V, kept, M, dtype       without raw logits: the K-chunked pass, tokens mapped
    (4096, 6000, 2000, 6, "bf16"),   # one column block
    (4096, 40000, 20001, 40, "bf16"),  # three column blocks, ragged last group, several groups
                                       # per workgroup
]


@pytest.mark.parametrize("mode,T", [("greedy", 1.0), ("sample", 1.0), ("sample", 0.6)])
@pytest.mark.parametrize("case", KCHUNK_CASES, ids=lambda c: "d%d-V%d-n%d-M%d-%s" % c)
def test_trimmed_kchunk(case, mode, T):
    _trimmed(*case, mode, T, want_logits=False)


@pytest.mark.parametrize("mode", ["greedy", "sample"])
def test_trimmed_kchunk_vocabulary_ends(mode):
    # kept ids include the first and the last vocabulary entry; 1001 kept rows leave a last
    # group of 41 rows
    d, V, n, M, seed = 2048, 9000, 1001, 24, 23
    rng = np.random.default_rng(seed)
    ids = np.sort(np.concatenate([[0, V - 1], rng.choice(np.arange(1, V - 1), n - 2, replace=False)])).astype(np.int32)
    h = synth.hidden(M, d, "bf16", seed)
    W = synth.dense_weights(V, d, "bf16", seed)
    # make the two end rows the best scores of every row, so that greedy picks them
    W[[0, V - 1]] = synth.store(np.sign(synth.as_f32(h[:2], "bf16")) * np.float32(0.05), "bf16")
    W_S = np.ascontiguousarray(W[ids])
    out = sh.draft_head_trimmed(P.to_device(h, "bf16"), P.to_device(W_S, "bf16"), torch.from_numpy(ids).cuda(),
                                mode=mode, seed=seed, offset=1)
    torch.cuda.synchronize()
    o = heads.head_trimmed(h, W_S, ids, "bf16", mode, 1.0, seed, 1)
    tok = out["token"].cpu().numpy()
    assert np.all(np.isin(tok, ids))
    got = dict(out)
    got["token"] = torch.from_numpy(np.searchsorted(ids, tok).astype(np.int32))
    want = dict(o)
    want["token"] = o["position"]
    _check_outputs(got, want, "bf16", mode, 1.0, seed, 1, f"trimmed ends {mode}")
    if mode == "greedy":
        assert tok[0] == 0 and tok[1] == V - 1


def test_acceptance_ceiling_through_verification():
    """SlimSpec write-up, section 二: a drafter that can only propose the kept ids S is accepted
    at most with probability p(S) -- with equality for the best such drafter, q = p restricted
    to S and renormalised.  Target scores are the dense head's logits (the library's kernel),
    the draft scores equal them on S (minus infinity elsewhere), the draft tokens are sampled by
    the trimmed head over S, and spec_verify decides.  The acceptance frequency over B
    sequences must match the mean p(S) (exact, from the oracle's float64 softmax of the same
    target scores) within four binomial standard deviations."""
    d, V, n, B, seed = 256, 4096, 1024, 4096, 29
    rng = np.random.default_rng(seed)
    ids = np.sort(rng.choice(V, n, replace=False)).astype(np.int32)
    h = synth.hidden(2 * B, d, "bf16", seed)                    # positions 0 and 1 of B sequences
    W = synth.dense_weights(V, d, "bf16", seed)
    Wt = P.to_device(W, "bf16")
    z = sh.draft_head_dense(P.to_device(h, "bf16"), Wt, want_logits=True, want_lse=False)["logits"]
    target = z.to(torch.bfloat16).view(B, 2, V).contiguous()
    ids_t = torch.from_numpy(ids).cuda()
    draft = torch.full((B, 1, V), float("-inf"), dtype=torch.bfloat16, device="cuda")
    draft[:, :, ids_t.long()] = target[:, :1, ids_t.long()]
    h0 = P.to_device(np.ascontiguousarray(h.reshape(B, 2, d)[:, 0]), "bf16")
    W_S = P.to_device(np.ascontiguousarray(W[ids]), "bf16")
    toks = sh.draft_head_trimmed(h0, W_S, ids_t, mode="sample", seed=seed, offset=1)["token"]
    assert np.all(np.isin(toks.cpu().numpy(), ids))
    u = torch.from_numpy(synth.uniforms_open((B, 1), seed + 1)).cuda()
    acc, _ = sh.spec_verify(target, draft.contiguous(), toks.view(B, 1).contiguous(), u, mode="sample", seed=seed)
    torch.cuda.synchronize()
    a = acc.cpu().numpy()
    t0 = target[:, 0].float().cpu().numpy().astype(np.float64)
    p = np.exp(t0 - t0.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    pS = p[:, ids].sum(axis=1)
    ceiling = [heads.trimmed_acceptance_ceiling(p[b], ids) for b in range(4)]
    np.testing.assert_allclose(ceiling, pS[:4], rtol=1e-12)
    alpha = a.mean()
    sd = np.sqrt(np.mean(pS * (1 - pS)) / B)
    P.log(f"trimmed ceiling: accept frequency {alpha:.4f}, mean p(S) {pS.mean():.4f} (sd {sd:.4f})")
    assert abs(alpha - pS.mean()) < 4 * sd + 2e-3
