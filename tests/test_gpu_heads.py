"""GPU parity of the dense and SlimSpec low-rank heads against the oracle (via the C ABI)."""
import numpy as np
import pytest
import torch

from drafter_lm_head_slimspec_amd import configs, spechead as sh, synth
from oracle import fp, heads
from tests import parity as P

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    sh.load()


def _check_outputs(out, o, dtype, mode, T, seed, offset, name=""):
    """GPU outputs against the oracle run on the same inputs the GPU's final product used
    (for the low-rank head: the GPU's own rounded h_r), so no rounding-flip allowance is
    needed: tokens bit-exact up to counted near-ties, lse / logprob to LSE_RTOL."""
    M = o["logits"].shape[0]
    tok = out["token"].cpu().numpy()
    if out.get("logits") is not None:
        r = P.assert_logits_close(out["logits"].cpu().numpy(), o["logits"], dtype, name + " logits")
        P.log(f"  {name} logits ok (max err / tol = {r:.3g})")
    ex = P.Excusals(name + " tokens")
    if mode == "greedy":
        P.check_greedy_tokens(tok, o["logits"], ex)
    else:
        P.head_sample_check(tok, o, seed, offset, T, ex)
    ex.report(M)
    assert np.all((tok >= 0) & (tok < o["logits"].shape[1]))
    y_tok = o["logits"][np.arange(M), tok] / T
    lse = None if out["lse"] is None else out["lse"].cpu().numpy()
    lp = None if out["logprob"] is None else out["logprob"].cpu().numpy()
    P.check_lse_logprob(lse, lp, o["lse"], y_tok, name)


def _hr_bits(t, dtype):
    if dtype == "bf16":
        return t.cpu().view(torch.int16).numpy().view(np.uint16)
    return t.cpu().numpy()


def _lowrank_check(out, h, Wd, Wu, dtype, mode, T, seed, offset, name):
    """Down-projection: the GPU's h_r against the oracle's single rounding; up-projection and
    selection: the oracle's head on the GPU's h_r."""
    pre, _ = heads.lowrank_down(h, Wd, dtype)
    terms = np.abs(fp.decode(h, dtype)) @ np.abs(fp.decode(Wd, dtype)).T
    hr = _hr_bits(out["h_r"], dtype)
    P.check_intermediate(fp.decode(hr, dtype), pre, terms, dtype, name + " h_r")
    o = heads.head_dense(hr, Wu, dtype, mode, T, seed, offset)
    _check_outputs(out, o, dtype, mode, T, seed, offset, name)
    return o


def _lowrank(d, V, r, M, dtype, mode, T, seed=7, offset=3, want_logits=True, want_lse=True, plant=None):
    P.log(f"lowrank d={d} V={V} r={r} M={M} {dtype} {mode} T={T} lse={want_lse} plant={plant is not None}")
    h = synth.hidden(M, d, dtype, seed)
    Wd, Wu = synth.lowrank_weights(V, d, r, dtype, seed)
    if plant is not None:
        _, hr_o = heads.lowrank_down(h, Wd, dtype)
        Wu = plant(Wu, hr_o)
    out = sh.draft_head_lowrank(P.to_device(h, dtype), P.to_device(Wd, dtype), P.to_device(Wu, dtype),
                                mode=mode, temperature=T, seed=seed, offset=offset, want_logits=want_logits,
                                want_lse=want_lse, want_intermediate=True)
    torch.cuda.synchronize()
    return _lowrank_check(out, h, Wd, Wu, dtype, mode, T, seed, offset, f"lowrank M={M}")


def _dense(d, V, M, dtype, mode, T, seed=11, offset=5, want_logits=True, want_lse=True, plant=None):
    P.log(f"dense d={d} V={V} M={M} {dtype} {mode} T={T} lse={want_lse} plant={plant is not None}")
    h = synth.hidden(M, d, dtype, seed)
    W = synth.dense_weights(V, d, dtype, seed)
    if plant is not None:
        W = plant(W, fp.decode(h, dtype))
    out = sh.draft_head_dense(P.to_device(h, dtype), P.to_device(W, dtype), mode=mode, temperature=T,
                              seed=seed, offset=offset, want_logits=want_logits, want_lse=want_lse)
    torch.cuda.synchronize()
    o = heads.head_dense(h, W, dtype, mode, T, seed, offset)
    _check_outputs(out, o, dtype, mode, T, seed, offset, f"dense M={M}")
    return o


LOWRANK_SMALL = [
    # d, V, r, M, dtype          path exercised
    (256, 1024, 32, 4, "f32"),     # the tiny fp32 configuration (VALU, 8 lanes per row)
    (512, 1000, 64, 1, "bf16"),    # ragged last group, VALU
    (512, 1000, 64, 3, "bf16"),
    (512, 1000, 64, 6, "bf16"),
    (512, 1000, 64, 8, "bf16"),
    (512, 1000, 120, 5, "bf16"),   # 15 chunks per row, 16-lane rows with one masked lane
    (360, 777, 360, 2, "bf16"),    # 45 chunks per row, masked lanes
    (512, 1000, 64, 9, "bf16"),    # MFMA, one column block
    (512, 1000, 64, 33, "bf16"),   # MFMA, two column blocks, ragged
    (512, 2000, 360, 70, "bf16"),  # MFMA, k not a multiple of 16
    (512, 1000, 64, 300, "bf16"),  # MFMA, rows split over two passes (192 + 108)
]


@pytest.mark.parametrize("mode,T", [("greedy", 1.0), ("sample", 1.0), ("sample", 0.7)])
@pytest.mark.parametrize("case", LOWRANK_SMALL, ids=lambda c: "d%d-V%d-r%d-M%d-%s" % c)
def test_lowrank_small(case, mode, T):
    _lowrank(*case, mode, T)


# shapes of the tile-streaming pass (bf16, r = 128..512 in steps of 32, at most 64 rows) with
# several groups per wave: ragged V, d not a multiple of 32, 1..64 rows
LOWRANK_TILE = [
    (520, 8200, 128, 1, "bf16"),
    (520, 8200, 128, 6, "bf16"),
    (512, 8200, 256, 17, "bf16"),
    (520, 20000, 384, 48, "bf16"),
    (1024, 20000, 512, 64, "bf16"),
]


@pytest.mark.parametrize("mode,T", [("greedy", 1.0), ("sample", 1.0), ("sample", 0.7)])
@pytest.mark.parametrize("case", LOWRANK_TILE, ids=lambda c: "d%d-V%d-r%d-M%d-%s" % c)
def test_lowrank_tile(case, mode, T):
    _lowrank(*case, mode, T, want_logits=False)


# shapes of the wide pass (bf16, rows of at most 512 elements, 65..256 activation rows):
# r = 360 (rows not a multiple of 32), ragged V, every column-block count, the longest rows
LOWRANK_WIDE = [
    (520, 8200, 360, 192, "bf16"),
    (512, 20000, 128, 65, "bf16"),
    (512, 9000, 256, 130, "bf16"),
    (256, 5000, 512, 100, "bf16"),
    (512, 7000, 200, 256, "bf16"),
    (384, 6000, 384, 180, "bf16"),
]


@pytest.mark.parametrize("mode,T", [("greedy", 1.0), ("sample", 1.0), ("sample", 0.7)])
@pytest.mark.parametrize("case", LOWRANK_WIDE, ids=lambda c: "d%d-V%d-r%d-M%d-%s" % c)
def test_lowrank_wide(case, mode, T):
    _lowrank(*case, mode, T, want_logits=False)


# rows of 512 elements leave room for six Philox blocks of group draws in the wide pass's LDS
# table; with 400000 rows (24-25 groups per workgroup) some workgroups' ranges span seven
# blocks and draw them as the walk reaches them, the others from the table
def test_lowrank_wide_long_range():
    _lowrank(256, 400000, 512, 65, "bf16", "sample", 1.0, want_logits=False)


DENSE_SMALL = [
    (256, 1024, 4, "f32"),
    (520, 1000, 3, "bf16"),    # 65 chunks per row: two chunks per lane, masked
    (1024, 700, 6, "bf16"),
    (520, 1000, 40, "bf16"),   # MFMA
    (4096, 600, 40, "bf16"),   # MFMA with B fragments read from global memory (K too large for LDS)
]


@pytest.mark.parametrize("mode,T", [("greedy", 1.0), ("sample", 1.0)])
@pytest.mark.parametrize("case", DENSE_SMALL, ids=lambda c: "d%d-V%d-M%d-%s" % c)
def test_dense_small(case, mode, T):
    _dense(*case, mode, T)


DENSE_KCHUNK = [
    # d, V, M, dtype        rows of more than 512 elements, at most 64 activation rows, no raw
    #                       logits: the K-chunked pass
    (1024, 3000, 1, "bf16"),      # one activation row: the four waves split each group's tiles
    (520, 5000, 16, "bf16"),      # K just above one chunk (a second chunk of 8 elements)
    (4096, 20000, 6, "bf16"),     # the dense head's K, one or two groups per workgroup
    (776, 1000, 9, "bf16"),       # ragged chunk and ragged last group
    (1024, 1000, 17, "bf16"),     # two waves (one with a single valid row), ragged last group
    (1032, 3000, 33, "bf16"),     # last chunk of 8 elements, three waves
    (2048, 40000, 64, "bf16"),    # four waves, two or three groups per workgroup
    (1536, 100000, 20, "bf16"),   # six or seven groups per workgroup
    (1024, 151936, 24, "bf16"),   # more groups than eight per CU: more workgroups than CUs
    (1024, 1, 5, "bf16"),         # a one-row vocabulary: one workgroup, one partial group
    (2048, 65, 64, "bf16"),       # 64 activation rows, a last group of one row
    (8184, 700, 40, "bf16"),      # sixteen chunks (the longest rows accepted), the last of 504 elements
]


@pytest.mark.parametrize("mode,T", [("greedy", 1.0), ("sample", 1.0), ("sample", 0.7)])
@pytest.mark.parametrize("case", DENSE_KCHUNK, ids=lambda c: "d%d-V%d-M%d-%s" % c)
def test_dense_kchunk(case, mode, T):
    _dense(*case, mode, T, want_logits=False)


@pytest.mark.parametrize("case", LOWRANK_TILE + LOWRANK_WIDE, ids=lambda c: "d%d-V%d-r%d-M%d-%s" % c)
def test_lowrank_argmax_only(case):
    # greedy without lse / logprob: the argmax-only instances of the tile and wide passes
    _lowrank(*case, "greedy", 1.0, want_logits=False, want_lse=False)


@pytest.mark.parametrize("case", DENSE_KCHUNK, ids=lambda c: "d%d-V%d-M%d-%s" % c)
def test_dense_kchunk_argmax_only(case):
    # greedy without lse / logprob: the argmax-only instances of the K-chunked pass
    _dense(*case, "greedy", 1.0, want_logits=False, want_lse=False)


@pytest.mark.parametrize("mode", ["greedy", "sample"])
def test_lowrank_rank_above_one_chunk(mode):
    # r > 512: the up-projection runs on the K-chunked pass
    _lowrank(1024, 5000, 520, 40, "bf16", mode, 1.0, want_logits=False)


def test_lowrank_without_lse_outputs():
    d, V, r, M = 512, 1000, 64, 6
    h = synth.hidden(M, d, "bf16", 1)
    Wd, Wu = synth.lowrank_weights(V, d, r, "bf16", 1)
    out = sh.draft_head_lowrank(P.to_device(h, "bf16"), P.to_device(Wd, "bf16"), P.to_device(Wu, "bf16"),
                                want_lse=False)
    o = heads.head_lowrank(h, Wd, Wu, "bf16")
    ex = P.Excusals("no-lse greedy")
    P.check_greedy_tokens(out["token"].cpu().numpy(), o["logits"], ex)
    ex.report(M)


def test_identity_down_projection_equals_dense():
    # r = d and W_down = I: the low-rank head is the dense head with W = W_up (fp32)
    d, V, M = 256, 1024, 4
    h = synth.hidden(M, d, "f32", 2)
    W = synth.dense_weights(V, d, "f32", 2)
    eye = np.eye(d, dtype=np.float32)
    a = sh.draft_head_lowrank(P.to_device(h, "f32"), P.to_device(eye, "f32"), P.to_device(W, "f32"),
                              mode="sample", seed=4, offset=1, want_logits=True)
    b = sh.draft_head_dense(P.to_device(h, "f32"), P.to_device(W, "f32"), mode="sample", seed=4, offset=1,
                            want_logits=True)
    torch.cuda.synchronize()
    np.testing.assert_allclose(a["logits"].cpu().numpy(), b["logits"].cpu().numpy(), rtol=1e-5, atol=1e-6)
    assert torch.equal(a["token"], b["token"])


# ----- full-size shapes ----------------------------------------------------------------------

@pytest.mark.parametrize("M", configs.LLAMA.Ms)
@pytest.mark.parametrize("mode", ["greedy", "sample"])
def test_llama_lowrank_full(M, mode):
    w = configs.LLAMA
    _lowrank(w.d, w.V, w.r, M, w.dtype, mode, w.temperature, seed=w.seeds["weights"], offset=1,
             want_logits=(M == 6))


@pytest.mark.parametrize("M", configs.LLAMA.Ms)
def test_llama_dense_full(M):
    w = configs.LLAMA
    _dense(w.d, w.V, M, w.dtype, "sample" if M == 48 else "greedy", 1.0, seed=w.seeds["weights"],
           want_logits=False)


@pytest.mark.parametrize("kind,M", [("lowrank", 6), ("lowrank", 48), ("dense", 48)])
def test_llama_argmax_only_full(kind, M):
    w = configs.LLAMA
    if kind == "lowrank":
        _lowrank(w.d, w.V, w.r, M, w.dtype, "greedy", 1.0, seed=w.seeds["weights"], offset=1, want_logits=False,
                 want_lse=False)
    else:
        _dense(w.d, w.V, M, w.dtype, "greedy", 1.0, seed=w.seeds["weights"], want_logits=False, want_lse=False)


@pytest.mark.parametrize("mode", ["sample", "greedy"])
def test_gptoss_lowrank_full(mode):
    w = configs.GPTOSS
    _lowrank(w.d, w.V, w.r, w.Ms[0], w.dtype, mode, w.temperature, seed=w.seeds["weights"], offset=2,
             want_logits=False)


def test_runs_are_bit_identical():
    w = configs.LLAMA
    M = 48
    h = P.to_device(synth.hidden(M, w.d, "bf16", 3), "bf16")
    Wd, Wu = synth.lowrank_weights(w.V, w.d, w.r, "bf16", 3)
    Wd, Wu = P.to_device(Wd, "bf16"), P.to_device(Wu, "bf16")
    a = sh.draft_head_lowrank(h, Wd, Wu, mode="sample", seed=9, offset=4)
    b = sh.draft_head_lowrank(h, Wd, Wu, mode="sample", seed=9, offset=4)
    torch.cuda.synchronize()
    for k in ("token", "lse", "logprob"):
        assert torch.equal(a[k], b[k]), k


@pytest.mark.parametrize("case", [
    ("dense", 4096, 20000, 48),    # K-chunked pass with the side buffer
    ("dense", 4096, 20000, 6),     # K-chunked pass, one column block
    ("wide", 360, 30000, 192),     # wide pass (low-rank up-projection shape)
], ids=lambda c: "%s-K%d-V%d-M%d" % c)
def test_head_passes_are_bit_identical(case):
    kind, K, V, M = case
    if kind == "dense":
        h = P.to_device(synth.hidden(M, K, "bf16", 5), "bf16")
        W = P.to_device(synth.dense_weights(V, K, "bf16", 5), "bf16")
        run = lambda: sh.draft_head_dense(h, W, mode="sample", seed=3, offset=2)
    else:
        d = 2880
        h = P.to_device(synth.hidden(M, d, "bf16", 5), "bf16")
        Wd, Wu = synth.lowrank_weights(V, d, K, "bf16", 5)
        Wd, Wu = P.to_device(Wd, "bf16"), P.to_device(Wu, "bf16")
        run = lambda: sh.draft_head_lowrank(h, Wd, Wu, mode="sample", temperature=0.7, seed=3, offset=2)
    a = run()
    b = run()
    torch.cuda.synchronize()
    for k in ("token", "lse", "logprob"):
        assert torch.equal(a[k], b[k]), k
