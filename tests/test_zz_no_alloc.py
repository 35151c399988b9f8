"""The no-allocation low-rank entry point against draft_head_lowrank, through the C ABI.

draft_head_lowrank_noalloc runs the same kernels as draft_head_lowrank on the library's
static device scratch instead of a caller workspace.  Two calls in a row (the second with a
smaller input, so the scratch holds the first call's leftovers) must each give outputs
bit-identical to the workspace entry point's on the same inputs, and sizes beyond the
scratch are refused before any launch.
"""
import numpy as np
import pytest
import torch

from drafter_lm_head_slimspec_amd import configs, spechead as sh, synth
from tests import parity as P

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    sh.load()


def _inputs(d, V, r, M, seed):
    h = P.to_device(synth.hidden(M, d, "bf16", seed), "bf16")
    Wd, Wu = synth.lowrank_weights(V, d, r, "bf16", seed)
    return h, P.to_device(Wd, "bf16"), P.to_device(Wu, "bf16")


def _outputs(M, V, want_logits):
    dev = torch.device("cuda")
    return (torch.full((M,), -7, dtype=torch.int32, device=dev),
            torch.full((M,), np.nan, dtype=torch.float32, device=dev),
            torch.full((M,), np.nan, dtype=torch.float32, device=dev),
            torch.full((M, V), np.nan, dtype=torch.float32, device=dev) if want_logits else None)


@pytest.mark.parametrize("mode", ["sample", "greedy"])
def test_noalloc_matches_workspace_entry_point_twice(mode):
    w = configs.LLAMA
    cases = [
        # the Llama-shaped head at 48 rows, then a smaller call on the scratch it left behind
        (w.d, w.V, w.r, 48, 0.9, False),
        (1024, 20000, 256, 6, 1.0, True),
    ]
    for i, (d, V, r, M, T, want_logits) in enumerate(cases):
        P.log(f"noalloc call {i}: d={d} V={V} r={r} M={M} {mode}")
        h, Wd, Wu = _inputs(d, V, r, M, 40 + i)
        tok, lse, lp, logits = _outputs(M, V, want_logits)
        sh.draft_head_lowrank_noalloc(h, Wd, Wu, tok, lse, lp, logits, mode=mode, temperature=T, seed=5, offset=i)
        ref = sh.draft_head_lowrank(h, Wd, Wu, mode=mode, temperature=T, seed=5, offset=i, want_logits=want_logits)
        torch.cuda.synchronize()
        assert torch.equal(tok, ref["token"])
        assert torch.equal(lse, ref["lse"])
        assert torch.equal(lp, ref["logprob"])
        if want_logits:
            assert torch.equal(logits, ref["logits"])


def test_noalloc_refuses_more_than_its_scratch():
    lib = sh.load()
    M, d, r, V = 64, 4096, 512, 1 << 21
    assert lib.sh_head_workspace_bytes(sh.OP_LOWRANK, M, d, r, V, 0) > (8 << 20)
    h, Wd, _ = _inputs(d, 1000, r, M, 3)
    # W_up is never read: validation refuses the call before any launch
    tok, lse, lp, _ = _outputs(M, 1, False)
    rc = lib.draft_head_lowrank_noalloc(sh._p(h), M, d, sh._p(Wd), r, sh._p(Wd), V, sh.SH_BF16, sh.GREEDY, 1.0, 0, 0,
                                        sh._p(tok), sh._p(lse), sh._p(lp), None, sh._stream(h.device))
    assert rc == sh.SH_ERR_UNSUPPORTED, rc
    assert b"static scratch" in lib.sh_last_error()
