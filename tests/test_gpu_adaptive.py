"""GPU parity of the position-adaptive-rank low-rank head (nested prefixes of one factor pair)
against the oracle's head_lowrank_adaptive, through the C ABI."""
import numpy as np
import pytest
import torch

from drafter_lm_head_slimspec_amd import spechead as sh, synth
from oracle import fp, heads
from tests import parity as P
from tests.test_gpu_heads import _check_outputs, _hr_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    sh.load()


def _adaptive(d, V, r, ranks, mode, T, seed=13, offset=2, want_logits=False):
    M = len(ranks)
    P.log(f"adaptive d={d} V={V} r_max={r} M={M} ranks={sorted(set(ranks))} {mode} T={T}")
    h = synth.hidden(M, d, "bf16", seed)
    Wd, Wu = synth.lowrank_weights(V, d, r, "bf16", seed)
    out = sh.draft_head_lowrank_adaptive(P.to_device(h, "bf16"), P.to_device(Wd, "bf16"), P.to_device(Wu, "bf16"),
                                         ranks, mode=mode, temperature=T, seed=seed, offset=offset,
                                         want_logits=want_logits, want_intermediate=True)
    torch.cuda.synchronize()
    # the GPU's h_r: row m holds round(W_down[:r_m] h_m) and zeros past r_m
    o_ref = heads.head_lowrank_adaptive(h, Wd, Wu, ranks, "bf16", mode, T, seed, offset)
    mask = np.arange(r)[None, :] < np.array(ranks)[:, None]
    terms = np.where(mask, np.abs(fp.decode(h, "bf16")) @ np.abs(fp.decode(Wd, "bf16")).T, 0.0)
    hr = _hr_bits(out["h_r"], "bf16")
    P.check_intermediate(fp.decode(hr, "bf16"), o_ref["h_r_exact"], terms, "bf16", f"adaptive M={M} h_r")
    assert np.all(hr[~mask] == 0), "h_r is zero past each row's rank"
    # up-projection and selection: the oracle's nested-prefix head on the GPU's h_r
    o = heads.head_dense(hr, Wu, "bf16", mode, T, seed, offset)
    _check_outputs(out, o, "bf16", mode, T, seed, offset, f"adaptive M={M}")
    return out, o


CASES = [
    # d, V, r_max, ranks                                   columns read
    (520, 8200, 256, [256, 256, 192, 128, 64, 32]),        # 256 (all of r_max)
    (512, 20000, 512, [512, 512, 384, 384, 256, 256] * 8),  # 512, the Llama-shaped schedule
    (512, 8200, 512, [128, 96, 64, 32, 17, 1]),            # 128 of 512: a prefix of every row
    (512, 8200, 384, [200, 160, 120, 80]),                 # 256 of 384
]


@pytest.mark.parametrize("mode,T", [("greedy", 1.0), ("sample", 1.0), ("sample", 0.7)])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "d%d-V%d-r%d-M%d" % (c[0], c[1], c[2], len(c[3])))
def test_adaptive(case, mode, T):
    _adaptive(*case, mode, T)


def test_adaptive_logits_and_uniform_rank_equals_fixed_rank_head():
    d, V, r, M = 512, 8200, 256, 5
    out, o = _adaptive(d, V, r, [256] * M, "sample", 1.0, want_logits=True)
    h = synth.hidden(M, d, "bf16", 13)
    Wd, Wu = synth.lowrank_weights(V, d, r, "bf16", 13)
    fixed = sh.draft_head_lowrank(P.to_device(h, "bf16"), P.to_device(Wd, "bf16"), P.to_device(Wu, "bf16"),
                                  mode="sample", temperature=1.0, seed=13, offset=2, want_logits=True)
    torch.cuda.synchronize()
    assert torch.equal(out["token"], fixed["token"])
    assert torch.equal(out["logits"], fixed["logits"])   # the same kernels on the same bits


def test_adaptive_rejects_unsupported():
    h = P.to_device(synth.hidden(2, 64, "f32", 1), "f32")
    Wd, Wu = synth.lowrank_weights(128, 64, 16, "f32", 1)
    with pytest.raises(sh.SpecHeadError):
        sh.draft_head_lowrank_adaptive(h, P.to_device(Wd, "f32"), P.to_device(Wu, "f32"), [16, 8])
