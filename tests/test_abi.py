"""Host-side checks of the C ABI (no GPU needed, no compute call is made).

Validation must reject bad arguments before any HIP call, so these calls use fake device
addresses that are never dereferenced.  They are skipped where a GPU is visible: there a
validation bug could reach a launch with those addresses.
"""
import ctypes

import pytest
import torch

from drafter_lm_head_slimspec_amd import spechead as sh
from tests import libutil


@pytest.fixture(scope="module")
def lib():
    libutil.ensure_built()
    return sh.load()


def test_header_declares_the_four_entry_points():
    names = libutil.header_functions()
    for n in ("draft_head_dense", "draft_head_lowrank", "draft_head_specvocab", "spec_verify",
              "spec_verify_sparse", "spec_verify_tree", "draft_head_lowrank_adaptive", "draft_head_trimmed"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    raw = ctypes.CDLL(libutil.LIB)
    missing = [n for n in libutil.header_functions() if not hasattr(raw, n)]
    assert not missing, missing


def test_status_strings(lib):
    assert lib.sh_status_str(0) == b"ok"
    assert lib.sh_status_str(sh.SH_ERR_WORKSPACE).startswith(b"workspace")
    assert lib.sh_status_str(99) == b"unknown status"


def test_workspace_sizes(lib):
    a = lib.sh_head_workspace_bytes(sh.OP_LOWRANK, 6, 4096, 512, 128256, 0)
    b = lib.sh_head_workspace_bytes(sh.OP_LOWRANK, 48, 4096, 512, 128256, 0)
    assert 0 < a < b and a % 256 == 0
    assert lib.sh_head_workspace_bytes(sh.OP_DENSE, 0, 4096, 0, 128256, 0) == 0
    assert lib.sh_head_workspace_bytes(sh.OP_SPECVOCAB, 1, 4096, 256, 1000, 1001) == 0
    s = lib.sh_head_workspace_bytes(sh.OP_SPECVOCAB, 16, 4096, 256, 151936, 2048)
    assert s >= 16 * 151936 * 4
    assert lib.sh_verify_workspace_bytes(sh.SAMPLE, 64, 5, 151936) > 0
    assert lib.sh_verify_workspace_bytes(sh.GREEDY, 64, 0, 151936) == 0
    assert lib.sh_verify_workspace_bytes(7, 64, 5, 151936) == 0


def test_intermediate_offset(lib):
    SIZE_MAX = (1 << 64) - 1
    for op, r, k in ((sh.OP_LOWRANK, 512, 0), (sh.OP_SPECVOCAB, 256, 2048)):
        M, d, V = 48, 4096, 128256
        off = lib.sh_head_intermediate_offset(op, M, d, r, V, k)
        total = lib.sh_head_workspace_bytes(op, M, d, r, V, k)
        # the intermediate (f32-sized slot, so it fits either dtype) lies inside the workspace
        assert off % 256 == 0 and off + M * r * 4 <= total
    assert lib.sh_head_intermediate_offset(sh.OP_DENSE, 48, 4096, 0, 128256, 0) == SIZE_MAX
    assert lib.sh_head_intermediate_offset(sh.OP_LOWRANK, 0, 4096, 512, 128256, 0) == SIZE_MAX


# fake, 256-byte aligned device addresses; never dereferenced
A = ctypes.c_void_p(0x7f0000100000)
B = ctypes.c_void_p(0x7f0000200000)
C = ctypes.c_void_p(0x7f0000300000)
D = ctypes.c_void_p(0x7f0000400000)
WS = ctypes.c_void_p(0x7f0000500000)
MIS = ctypes.c_void_p(0x7f0000100008)

no_gpu = pytest.mark.skipif(torch.cuda.is_available(), reason="validation checks use fake addresses")


def _dense(lib, h=A, M=4, d=256, W=B, V=1024, dtype=sh.SH_F32, mode=sh.GREEDY, T=1.0, tok=C,
           ws=WS, wsb=1 << 30):
    return lib.draft_head_dense(h, M, d, W, V, dtype, mode, T, 0, 0, tok, None, None, None, ws, wsb, None)


@no_gpu
def test_dense_validation(lib):
    assert _dense(lib, h=None) == sh.SH_ERR_NULL
    assert _dense(lib, W=None) == sh.SH_ERR_NULL
    assert _dense(lib, tok=None) == sh.SH_ERR_NULL
    assert _dense(lib, h=MIS) == sh.SH_ERR_ALIGN
    assert _dense(lib, M=0) == sh.SH_ERR_SHAPE
    assert _dense(lib, V=0) == sh.SH_ERR_SHAPE
    assert _dense(lib, d=6, dtype=sh.SH_BF16) == sh.SH_ERR_SHAPE   # 12 bytes per row
    assert _dense(lib, d=16384, dtype=sh.SH_BF16) == sh.SH_ERR_UNSUPPORTED
    assert _dense(lib, dtype=5) == sh.SH_ERR_DTYPE
    assert _dense(lib, mode=3) == sh.SH_ERR_DTYPE
    assert _dense(lib, T=0.0) == sh.SH_ERR_PARAM
    assert _dense(lib, T=float("nan")) == sh.SH_ERR_PARAM
    assert _dense(lib, T=float("inf")) == sh.SH_ERR_PARAM
    assert _dense(lib, ws=None) == sh.SH_ERR_WORKSPACE
    assert _dense(lib, wsb=100) == sh.SH_ERR_WORKSPACE
    assert _dense(lib, ws=ctypes.c_void_p(0x7f0000500010)) == sh.SH_ERR_ALIGN
    assert b"workspace" in lib.sh_last_error()


@no_gpu
def test_lowrank_and_specvocab_validation(lib):
    r = lib.draft_head_lowrank(A, 4, 256, B, 3, C, 1024, sh.SH_F32, 0, 1.0, 0, 0, D, None, None, None, WS, 1 << 30, None)
    assert r == sh.SH_ERR_SHAPE                      # r * 4 bytes not a multiple of 16
    r = lib.draft_head_lowrank(A, 4, 256, None, 32, C, 1024, sh.SH_F32, 0, 1.0, 0, 0, D, None, None, None, WS, 1 << 30, None)
    assert r == sh.SH_ERR_NULL
    r = lib.draft_head_lowrank(A, 4, 256, B, 32, C, 1024, sh.SH_F32, 0, 1.0, 0, 0, D, None, None, None, WS, 16, None)
    assert r == sh.SH_ERR_WORKSPACE

    def sv(k=64, V=1024, dprime=16, idx=D, ws=WS, wsb=1 << 30):
        return lib.draft_head_specvocab(A, 4, 256, B, dprime, C, C, V, k, sh.SH_F32, 0, 1.0, 0, 0, idx, None,
                                        None, D, None, None, ws, wsb, None)
    assert sv(k=0) == sh.SH_ERR_PARAM
    assert sv(k=1025) == sh.SH_ERR_PARAM
    assert sv(k=20000, V=40000) == sh.SH_ERR_UNSUPPORTED
    assert sv(idx=None) == sh.SH_ERR_NULL
    assert sv(dprime=2) == sh.SH_ERR_SHAPE
    assert sv(wsb=1000) == sh.SH_ERR_WORKSPACE


@no_gpu
def test_verify_validation(lib):
    def v(mode=sh.SAMPLE, B=2, gamma=4, V=1024, tl=A, dl=B, tok=C, u=D, T=1.0, acc=C, out=D, wsb=1 << 30):
        return lib.spec_verify(mode, B, gamma, V, sh.SH_F32, tl, dl, tok, u, T, 0, 0, acc, out, WS, wsb, None)
    assert v(gamma=0) == sh.SH_ERR_SHAPE
    assert v(gamma=65) == sh.SH_ERR_SHAPE
    assert v(B=0) == sh.SH_ERR_SHAPE
    assert v(V=1023) == sh.SH_ERR_SHAPE
    assert v(dl=None) == sh.SH_ERR_NULL
    assert v(u=None) == sh.SH_ERR_NULL
    assert v(tl=None) == sh.SH_ERR_NULL
    assert v(tok=None) == sh.SH_ERR_NULL
    assert v(T=-1.0) == sh.SH_ERR_PARAM
    assert v(wsb=8) == sh.SH_ERR_WORKSPACE
    assert v(mode=sh.GREEDY, dl=None, u=None, wsb=8) == sh.SH_ERR_WORKSPACE   # greedy needs no draft
    assert v(mode=9) == sh.SH_ERR_DTYPE


@no_gpu
def test_verify_sparse_validation(lib):
    def v(B=2, gamma=4, V=1024, k=64, tl=A, idx=B, prob=C, tok=D, u=A, T=1.0, acc=C, out=D, wsb=1 << 30,
          dtype=sh.SH_F32):
        return lib.spec_verify_sparse(B, gamma, V, k, dtype, tl, idx, prob, tok, u, T, 0, 0, acc, out, WS, wsb,
                                      None)
    assert v(gamma=0) == sh.SH_ERR_SHAPE
    assert v(gamma=65) == sh.SH_ERR_SHAPE
    assert v(B=0) == sh.SH_ERR_SHAPE
    assert v(V=1023) == sh.SH_ERR_SHAPE
    assert v(k=0) == sh.SH_ERR_PARAM
    assert v(k=1025) == sh.SH_ERR_PARAM
    assert v(k=20000, V=40000) == sh.SH_ERR_UNSUPPORTED
    assert v(idx=None) == sh.SH_ERR_NULL
    assert v(prob=None) == sh.SH_ERR_NULL
    assert v(tok=None) == sh.SH_ERR_NULL
    assert v(u=None) == sh.SH_ERR_NULL
    assert v(tl=None) == sh.SH_ERR_NULL
    assert v(idx=ctypes.c_void_p(0x7f0000100002)) == sh.SH_ERR_ALIGN
    assert v(T=0.0) == sh.SH_ERR_PARAM
    assert v(dtype=5) == sh.SH_ERR_DTYPE
    assert v(wsb=8) == sh.SH_ERR_WORKSPACE
    assert lib.sh_verify_sparse_workspace_bytes(64, 5, 151936, 2048) > 0
    assert lib.sh_verify_sparse_workspace_bytes(64, 5, 151936, 0) == 0


@no_gpu
def test_verify_tree_validation(lib):
    def v(B=2, N=8, V=1024, tl=A, tok=B, par=C, acc=C, node=D, out=D, wsb=1 << 30, dtype=sh.SH_F32):
        return lib.spec_verify_tree(B, N, V, dtype, tl, tok, par, acc, node, out, WS, wsb, None)
    assert v(N=0) == sh.SH_ERR_SHAPE
    assert v(N=1025) == sh.SH_ERR_SHAPE
    assert v(B=0) == sh.SH_ERR_SHAPE
    assert v(V=1023) == sh.SH_ERR_SHAPE
    assert v(tl=None) == sh.SH_ERR_NULL
    assert v(tok=None) == sh.SH_ERR_NULL
    assert v(par=None) == sh.SH_ERR_NULL
    assert v(node=None) == sh.SH_ERR_NULL
    assert v(par=ctypes.c_void_p(0x7f0000100002)) == sh.SH_ERR_ALIGN
    assert v(dtype=3) == sh.SH_ERR_DTYPE
    assert v(wsb=8) == sh.SH_ERR_WORKSPACE
    assert lib.sh_verify_tree_workspace_bytes(64, 32, 151936) > 0
    assert lib.sh_verify_tree_workspace_bytes(64, 1025, 151936) == 0


@no_gpu
def test_lowrank_adaptive_validation(lib):
    ranks = (ctypes.c_int32 * 4)(128, 64, 32, 1)
    bad = (ctypes.c_int32 * 4)(128, 0, 32, 1)
    big = (ctypes.c_int32 * 4)(513, 64, 32, 1)

    def v(M=4, d=512, r=512, V=8200, rk=ranks, dtype=sh.SH_BF16, wsb=1 << 30):
        return lib.draft_head_lowrank_adaptive(A, M, d, B, r, C, V, rk, dtype, 0, 1.0, 0, 0, D, None, None, None,
                                               WS, wsb, None)
    assert v(rk=None) == sh.SH_ERR_NULL
    assert v(rk=bad) == sh.SH_ERR_PARAM
    assert v(rk=big) == sh.SH_ERR_PARAM
    assert v(dtype=sh.SH_F32) == sh.SH_ERR_UNSUPPORTED
    assert v(M=65) == sh.SH_ERR_UNSUPPORTED
    assert v(r=520, rk=big) == sh.SH_ERR_UNSUPPORTED   # 520 columns read: outside the tile pass
    assert v(wsb=16) == sh.SH_ERR_WORKSPACE


@no_gpu
def test_trimmed_validation(lib):
    def v(M=4, d=256, n=1024, ids=C, tok=D, wsb=1 << 30, mode=0):
        return lib.draft_head_trimmed(A, M, d, B, n, ids, sh.SH_F32, mode, 1.0, 0, 0, tok, None, None, None, WS, wsb,
                                      None)
    assert v(ids=None) == sh.SH_ERR_NULL
    assert v(ids=ctypes.c_void_p(0x7f0000100002)) == sh.SH_ERR_ALIGN
    assert v(tok=None) == sh.SH_ERR_NULL
    assert v(n=0) != sh.SH_OK
    assert v(M=0) == sh.SH_ERR_SHAPE
    assert v(mode=4) == sh.SH_ERR_DTYPE
    assert v(wsb=16) == sh.SH_ERR_WORKSPACE


@no_gpu
def test_topk_and_philox_validation(lib):
    assert lib.sh_topk(A, 2, 100, 0, C, None, 0, None) == sh.SH_ERR_PARAM
    assert lib.sh_topk(A, 2, 100, 101, C, None, 0, None) == sh.SH_ERR_PARAM
    assert lib.sh_topk(None, 2, 100, 5, C, None, 0, None) == sh.SH_ERR_NULL
    assert lib.sh_topk(A, 0, 100, 5, C, None, 0, None) == sh.SH_ERR_SHAPE
    assert lib.sh_philox_uniform(0, 0, 0, 0, 10, A, None) == sh.SH_ERR_SHAPE
    assert lib.sh_philox_uniform(0, 0, 0, 1, 10, None, None) == sh.SH_ERR_NULL


@no_gpu
def test_read_probe_validation(lib):
    assert lib.sh_read_probe(None, 1024, C, None) == sh.SH_ERR_NULL
    assert lib.sh_read_probe(A, 1024, None, None) == sh.SH_ERR_NULL
    assert lib.sh_read_probe(ctypes.c_void_p(A.value + 4), 1024, C, None) == sh.SH_ERR_ALIGN
    assert lib.sh_read_probe(A, 1024, ctypes.c_void_p(C.value + 2), None) == sh.SH_ERR_ALIGN
    for nbytes in (0, 1000, 0xFFFFFFF0 + 16):
        assert lib.sh_read_probe(A, nbytes, C, None) == sh.SH_ERR_SHAPE


def test_binding_fails_loudly_without_library(tmp_path):
    with pytest.raises(FileNotFoundError):
        sh.load(str(tmp_path / "missing.so"))
