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
