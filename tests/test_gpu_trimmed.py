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
    _check_outputs(got, want, dtype, mode, T, seed, offset, None, f"trimmed M={M}")


CASES = [
    # d, V, kept, M, dtype       path exercised
    (256, 1024, 300, 4, "f32"),     # fp32 VALU stream
    (512, 8000, 3000, 6, "bf16"),   # tile pass (rows of 512)
    (512, 8000, 3001, 48, "bf16"),  # tile pass, ragged last group
    (4096, 6000, 2000, 6, "bf16"),  # VALU stream, long rows
    (4096, 6000, 2000, 40, "bf16"), # MFMA stream
]


@pytest.mark.parametrize("mode,T", [("greedy", 1.0), ("sample", 1.0)])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "d%d-V%d-n%d-M%d-%s" % c)
def test_trimmed(case, mode, T):
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
