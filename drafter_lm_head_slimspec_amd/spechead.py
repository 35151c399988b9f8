"""Thin ctypes binding of libspechead.so (C ABI in include/spechead.h).

Argument marshalling only: every step of the head and verification path runs in the HIP
kernels behind the C ABI.  PyTorch provides device memory and the current stream.  If the
library has not been built, ``load()`` raises; there is no fallback.
"""
import ctypes
import os
import threading

import numpy as np
import torch

# the built library next to this file; SPECHEAD_LIB names another build of the same sources
LIB_PATH = os.environ.get("SPECHEAD_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libspechead.so")

SH_OK, SH_ERR_NULL, SH_ERR_SHAPE, SH_ERR_DTYPE, SH_ERR_ALIGN = 0, 1, 2, 3, 4
SH_ERR_WORKSPACE, SH_ERR_PARAM, SH_ERR_UNSUPPORTED, SH_ERR_HIP = 5, 6, 7, 8
SH_F32, SH_BF16 = 0, 1
GREEDY, SAMPLE = 0, 1
OP_DENSE, OP_LOWRANK, OP_SPECVOCAB = 0, 1, 2

_lib = None
_lock = threading.Lock()

_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_u64 = ctypes.c_uint64
_f = ctypes.c_float
_i = ctypes.c_int
_sz = ctypes.c_size_t

_SIGS = {
    "sh_head_workspace_bytes": (_sz, [_i, _i64, _i64, _i64, _i64, _i64]),
    "sh_head_intermediate_offset": (_sz, [_i, _i64, _i64, _i64, _i64, _i64]),
    "sh_verify_workspace_bytes": (_sz, [_i, _i64, _i64, _i64]),
    "sh_topk_workspace_bytes": (_sz, [_i64, _i64, _i64]),
    "draft_head_dense": (_i, [_vp, _i64, _i64, _vp, _i64, _i, _i, _f, _u64, _u64, _vp, _vp, _vp, _vp,
                              _vp, _sz, _vp]),
    "draft_head_lowrank": (_i, [_vp, _i64, _i64, _vp, _i64, _vp, _i64, _i, _i, _f, _u64, _u64, _vp,
                                _vp, _vp, _vp, _vp, _sz, _vp]),
    "draft_head_lowrank_noalloc": (_i, [_vp, _i64, _i64, _vp, _i64, _vp, _i64, _i, _i, _f, _u64, _u64, _vp,
                                        _vp, _vp, _vp, _vp]),
    "draft_head_trimmed": (_i, [_vp, _i64, _i64, _vp, _i64, _vp, _i, _i, _f, _u64, _u64, _vp, _vp, _vp, _vp, _vp,
                                _sz, _vp]),
    "draft_head_lowrank_adaptive": (_i, [_vp, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i, _i, _f, _u64, _u64,
                                         _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "draft_head_specvocab": (_i, [_vp, _i64, _i64, _vp, _i64, _vp, _vp, _i64, _i64, _i, _i, _f, _u64,
                                  _u64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "spec_verify": (_i, [_i, _i64, _i64, _i64, _i, _vp, _vp, _vp, _vp, _f, _u64, _u64, _vp, _vp, _vp,
                         _sz, _vp]),
    "sh_verify_sparse_workspace_bytes": (_sz, [_i64, _i64, _i64, _i64]),
    "sh_verify_tree_workspace_bytes": (_sz, [_i64, _i64, _i64]),
    "spec_verify_tree": (_i, [_i64, _i64, _i64, _i, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "spec_verify_sparse": (_i, [_i64, _i64, _i64, _i64, _i, _vp, _vp, _vp, _vp, _vp, _f, _u64, _u64, _vp,
                                _vp, _vp, _sz, _vp]),
    "sh_topk": (_i, [_vp, _i64, _i64, _i64, _vp, _vp, _sz, _vp]),
    "sh_philox_uniform": (_i, [_u64, _u64, ctypes.c_uint32, _i64, _i64, _vp, _vp]),
    "sh_read_probe": (_i, [_vp, _u64, _vp, _vp]),
    "sh_trace_enable": (_i, [_i64]),
    "sh_trace_read": (_i, [ctypes.c_char_p, _sz]),
    "sh_status_str": (ctypes.c_char_p, [_i]),
    "sh_last_error": (ctypes.c_char_p, []),
}


class SpecHeadError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"spechead status {status}: {msg}")
        self.status = status


def load(path=None):
    """Load libspechead.so (once) and declare its signatures.  Raises if it is missing."""
    global _lib
    with _lock:
        if _lib is not None and path is None:
            return _lib
        p = path or LIB_PATH
        if not os.path.exists(p):
            raise FileNotFoundError(
                f"{p} not found: build it with `python -m drafter_lm_head_slimspec_amd.build`")
        lib = ctypes.CDLL(p)
        for name, (res, args) in _SIGS.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        if path is None:
            _lib = lib
        return lib


def _check(rc):
    if rc != SH_OK:
        lib = load()
        raise SpecHeadError(rc, lib.sh_last_error().decode(errors="replace"))


def _dt(t):
    if t.dtype == torch.bfloat16:
        return SH_BF16
    if t.dtype == torch.float32:
        return SH_F32
    raise TypeError(f"unsupported dtype {t.dtype}: use torch.bfloat16 or torch.float32")


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _mode(mode):
    if mode in ("greedy", GREEDY):
        return GREEDY
    if mode in ("sample", SAMPLE):
        return SAMPLE
    raise ValueError(mode)


_ws_cache = {}


def workspace(nbytes, device, kind="head"):
    """Device workspace of at least nbytes, cached per (device, stream, kind)."""
    key = (torch.device(device).index, torch.cuda.current_stream(device).cuda_stream, kind)
    buf = _ws_cache.get(key)
    if buf is None or buf.numel() < nbytes:
        buf = torch.zeros(max(int(nbytes), 256), dtype=torch.uint8, device=device)
        _ws_cache[key] = buf
    return buf


def _intermediate(lib, op, ws, M, d, r, V, k, dtype):
    """Copy of the rounded intermediate (h_r or h') a head call left in its workspace."""
    off = lib.sh_head_intermediate_offset(op, M, d, r, V, k)
    esz = 2 if dtype == torch.bfloat16 else 4
    raw = ws[off:off + M * r * esz].clone()
    return raw.view(dtype).view(M, r)


def _contig(*ts):
    for t in ts:
        if t is not None and not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def draft_head_dense(h, W, mode="greedy", temperature=1.0, seed=0, offset=0, want_logits=False,
                     want_lse=True):
    lib = load()
    _contig(h, W)
    M, d = h.shape
    V = W.shape[0]
    dev = h.device
    token = torch.empty(M, dtype=torch.int32, device=dev)
    lse = torch.empty(M, dtype=torch.float32, device=dev) if want_lse else None
    logprob = torch.empty(M, dtype=torch.float32, device=dev) if want_lse else None
    logits = torch.empty(M, V, dtype=torch.float32, device=dev) if want_logits else None
    need = lib.sh_head_workspace_bytes(OP_DENSE, M, d, 0, V, 0)
    ws = workspace(need, dev)
    _check(lib.draft_head_dense(_p(h), M, d, _p(W), V, _dt(h), _mode(mode), float(temperature),
                                int(seed), int(offset), _p(token), _p(lse), _p(logprob), _p(logits),
                                _p(ws), ws.numel(), _stream(dev)))
    return {"token": token, "lse": lse, "logprob": logprob, "logits": logits}


def draft_head_lowrank(h, W_down, W_up, mode="greedy", temperature=1.0, seed=0, offset=0,
                       want_logits=False, want_lse=True, want_intermediate=False):
    lib = load()
    _contig(h, W_down, W_up)
    M, d = h.shape
    r = W_down.shape[0]
    V = W_up.shape[0]
    dev = h.device
    token = torch.empty(M, dtype=torch.int32, device=dev)
    lse = torch.empty(M, dtype=torch.float32, device=dev) if want_lse else None
    logprob = torch.empty(M, dtype=torch.float32, device=dev) if want_lse else None
    logits = torch.empty(M, V, dtype=torch.float32, device=dev) if want_logits else None
    need = lib.sh_head_workspace_bytes(OP_LOWRANK, M, d, r, V, 0)
    ws = workspace(need, dev)
    _check(lib.draft_head_lowrank(_p(h), M, d, _p(W_down), r, _p(W_up), V, _dt(h), _mode(mode),
                                  float(temperature), int(seed), int(offset), _p(token), _p(lse),
                                  _p(logprob), _p(logits), _p(ws), ws.numel(), _stream(dev)))
    out = {"token": token, "lse": lse, "logprob": logprob, "logits": logits}
    if want_intermediate:
        out["h_r"] = _intermediate(lib, OP_LOWRANK, ws, M, d, r, V, 0, h.dtype)
    return out


def draft_head_lowrank_noalloc(h, W_down, W_up, token, lse=None, logprob=None, logits=None, mode="greedy",
                               temperature=1.0, seed=0, offset=0):
    """draft_head_lowrank on the library's static scratch: no workspace, and this wrapper
    allocates nothing either -- the caller passes the output tensors (token [M] int32; lse,
    logprob [M] and logits [M, V] float32 or None)."""
    lib = load()
    _contig(h, W_down, W_up, token, lse, logprob, logits)
    M, d = h.shape
    r = W_down.shape[0]
    V = W_up.shape[0]
    dev = h.device
    _check(lib.draft_head_lowrank_noalloc(_p(h), M, d, _p(W_down), r, _p(W_up), V, _dt(h), _mode(mode),
                                          float(temperature), int(seed), int(offset), _p(token), _p(lse),
                                          _p(logprob), _p(logits), _stream(dev)))


def draft_head_trimmed(h, W_S, ids, mode="greedy", temperature=1.0, seed=0, offset=0, want_logits=False):
    """Dense head over the kept rows W_S = W[ids]; the token is the vocabulary id ids[j]."""
    lib = load()
    _contig(h, W_S, ids)
    M, d = h.shape
    n = W_S.shape[0]
    if ids.dtype != torch.int32 or ids.shape != (n,):
        raise TypeError("ids must be int32 [n_S]")
    dev = h.device
    token = torch.empty(M, dtype=torch.int32, device=dev)
    lse = torch.empty(M, dtype=torch.float32, device=dev)
    logprob = torch.empty(M, dtype=torch.float32, device=dev)
    logits = torch.empty(M, n, dtype=torch.float32, device=dev) if want_logits else None
    need = lib.sh_head_workspace_bytes(OP_DENSE, M, d, 0, n, 0)
    ws = workspace(need, dev)
    _check(lib.draft_head_trimmed(_p(h), M, d, _p(W_S), n, _p(ids), _dt(h), _mode(mode), float(temperature),
                                  int(seed), int(offset), _p(token), _p(lse), _p(logprob), _p(logits), _p(ws),
                                  ws.numel(), _stream(dev)))
    return {"token": token, "lse": lse, "logprob": logprob, "logits": logits}


def draft_head_lowrank_adaptive(h, W_down, W_up, ranks, mode="greedy", temperature=1.0, seed=0, offset=0,
                                want_logits=False, want_intermediate=False):
    """Position-adaptive rank: row m uses the first ranks[m] rows of W_down / columns of W_up
    (ranks: host integers, one per row)."""
    lib = load()
    _contig(h, W_down, W_up)
    M, d = h.shape
    r = W_down.shape[0]
    V = W_up.shape[0]
    rk = np.ascontiguousarray(np.asarray(ranks, dtype=np.int32).reshape(-1))
    if rk.size != M:
        raise ValueError("one rank per row")
    dev = h.device
    token = torch.empty(M, dtype=torch.int32, device=dev)
    lse = torch.empty(M, dtype=torch.float32, device=dev)
    logprob = torch.empty(M, dtype=torch.float32, device=dev)
    logits = torch.empty(M, V, dtype=torch.float32, device=dev) if want_logits else None
    need = lib.sh_head_workspace_bytes(OP_LOWRANK, M, d, r, V, 0)
    ws = workspace(need, dev)
    _check(lib.draft_head_lowrank_adaptive(_p(h), M, d, _p(W_down), r, _p(W_up), V, rk.ctypes.data_as(_vp), _dt(h),
                                           _mode(mode), float(temperature), int(seed), int(offset), _p(token),
                                           _p(lse), _p(logprob), _p(logits), _p(ws), ws.numel(), _stream(dev)))
    out = {"token": token, "lse": lse, "logprob": logprob, "logits": logits}
    if want_intermediate:
        out["h_r"] = _intermediate(lib, OP_LOWRANK, ws, M, d, r, V, 0, h.dtype)
    return out


def draft_head_specvocab(h, W_down, W_vocab, U, k, mode="greedy", temperature=1.0, seed=0, offset=0,
                         want_lse=True, want_intermediate=False):
    lib = load()
    _contig(h, W_down, W_vocab, U)
    M, d = h.shape
    dprime = W_down.shape[0]
    V = W_vocab.shape[0]
    dev = h.device
    idx = torch.empty(M, k, dtype=torch.int32, device=dev)
    zl = torch.empty(M, k, dtype=torch.float32, device=dev)
    q = torch.empty(M, k, dtype=torch.float32, device=dev)
    token = torch.empty(M, dtype=torch.int32, device=dev)
    lse = torch.empty(M, dtype=torch.float32, device=dev) if want_lse else None
    logprob = torch.empty(M, dtype=torch.float32, device=dev) if want_lse else None
    need = lib.sh_head_workspace_bytes(OP_SPECVOCAB, M, d, dprime, V, k)
    ws = workspace(need, dev, "specvocab")
    _check(lib.draft_head_specvocab(_p(h), M, d, _p(W_down), dprime, _p(W_vocab), _p(U), V, int(k),
                                    _dt(h), _mode(mode), float(temperature), int(seed), int(offset),
                                    _p(idx), _p(zl), _p(q), _p(token), _p(lse), _p(logprob), _p(ws),
                                    ws.numel(), _stream(dev)))
    out = {"topk_idx": idx, "topk_logit": zl, "topk_prob": q, "token": token, "lse": lse,
           "logprob": logprob}
    if want_intermediate:
        out["h_prime"] = _intermediate(lib, OP_SPECVOCAB, ws, M, d, dprime, V, k, h.dtype)
    return out


def spec_verify(target, draft, tokens, u=None, mode="sample", temperature=1.0, seed=0, offset=0):
    lib = load()
    m = _mode(mode)
    _contig(target, draft, tokens, u)
    B, g1, V = target.shape
    gamma = g1 - 1
    dev = target.device
    if tokens.dtype != torch.int32:
        raise TypeError("draft tokens must be int32")
    if u is not None and u.dtype != torch.float32:
        raise TypeError("u must be float32")
    acc = torch.empty(B, dtype=torch.int32, device=dev)
    out = torch.empty(B, gamma + 1, dtype=torch.int32, device=dev)
    need = lib.sh_verify_workspace_bytes(m, B, gamma, V)
    ws = workspace(need, dev, "verify")
    _check(lib.spec_verify(m, B, gamma, V, _dt(target), _p(target), _p(draft) if m == SAMPLE else None,
                           _p(tokens), _p(u) if m == SAMPLE else None, float(temperature), int(seed),
                           int(offset), _p(acc), _p(out), _p(ws), ws.numel(), _stream(dev)))
    return acc, out


def spec_verify_sparse(target, draft_idx, draft_prob, tokens, u, temperature=1.0, seed=0, offset=0):
    """Sampling verification against a sparse draft distribution (draft_prob on draft_idx,
    zero elsewhere): the SpecVocab head's (topk_idx, topk_prob) per draft position."""
    lib = load()
    _contig(target, draft_idx, draft_prob, tokens, u)
    B, g1, V = target.shape
    gamma = g1 - 1
    k = draft_idx.shape[-1]
    dev = target.device
    if draft_idx.shape != (B, gamma, k) or draft_prob.shape != (B, gamma, k):
        raise ValueError("draft_idx / draft_prob must be [B, gamma, k]")
    if draft_idx.dtype != torch.int32 or tokens.dtype != torch.int32:
        raise TypeError("draft_idx and draft tokens must be int32")
    if draft_prob.dtype != torch.float32 or u.dtype != torch.float32:
        raise TypeError("draft_prob and u must be float32")
    acc = torch.empty(B, dtype=torch.int32, device=dev)
    out = torch.empty(B, gamma + 1, dtype=torch.int32, device=dev)
    need = lib.sh_verify_sparse_workspace_bytes(B, gamma, V, k)
    ws = workspace(need, dev, "verify")
    _check(lib.spec_verify_sparse(B, gamma, V, k, _dt(target), _p(target), _p(draft_idx), _p(draft_prob),
                                  _p(tokens), _p(u), float(temperature), int(seed), int(offset), _p(acc), _p(out),
                                  _p(ws), ws.numel(), _stream(dev)))
    return acc, out


def spec_verify_tree(target, node_token, parent):
    """Greedy verification of B candidate trees of N nodes: target [B, N, V], node_token and
    parent [B, N] int32 -> (accept_len [B], accept_node [B], out_tokens [B, N])."""
    lib = load()
    _contig(target, node_token, parent)
    B, N, V = target.shape
    dev = target.device
    if node_token.shape != (B, N) or parent.shape != (B, N):
        raise ValueError("node_token / parent must be [B, N]")
    if node_token.dtype != torch.int32 or parent.dtype != torch.int32:
        raise TypeError("node_token and parent must be int32")
    acc = torch.empty(B, dtype=torch.int32, device=dev)
    node = torch.empty(B, dtype=torch.int32, device=dev)
    out = torch.empty(B, N, dtype=torch.int32, device=dev)
    need = lib.sh_verify_tree_workspace_bytes(B, N, V)
    ws = workspace(need, dev, "verify")
    _check(lib.spec_verify_tree(B, N, V, _dt(target), _p(target), _p(node_token), _p(parent), _p(acc), _p(node),
                                _p(out), _p(ws), ws.numel(), _stream(dev)))
    return acc, node, out


def topk(scores, k):
    lib = load()
    _contig(scores)
    if scores.dtype != torch.float32:
        raise TypeError("scores must be float32")
    M, V = scores.shape
    dev = scores.device
    idx = torch.empty(M, k, dtype=torch.int32, device=dev)
    need = lib.sh_topk_workspace_bytes(M, V, k)
    ws = workspace(need, dev, "topk")
    _check(lib.sh_topk(_p(scores), M, V, int(k), _p(idx), _p(ws), ws.numel(), _stream(dev)))
    return idx


def philox_uniform(seed, offset, purpose, rows, n, device):
    lib = load()
    out = torch.empty(rows, n, dtype=torch.float32, device=device)
    _check(lib.sh_philox_uniform(int(seed), int(offset), int(purpose), rows, n, _p(out),
                                 _stream(device)))
    return out


def read_probe(buf, sink):
    """XOR of every 32-bit word of the device tensor `buf` into the int32 device word `sink`
    (a measurement helper: the flat read whose rate is the attainable HBM read bandwidth)."""
    lib = load()
    nbytes = buf.numel() * buf.element_size()
    _check(lib.sh_read_probe(_p(buf), nbytes, _p(sink), _stream(buf.device)))


def trace_enable(max_records=65536):
    """Start per-kernel event timing inside the library (0 disables)."""
    _check(load().sh_trace_enable(int(max_records)))


def trace_read():
    """Per-kernel timing since the last read: {name: {count, total_us, min_us, max_us}}."""
    import json
    buf = ctypes.create_string_buffer(1 << 16)
    _check(load().sh_trace_read(buf, len(buf)))
    return json.loads(buf.value.decode())


def prepared(fn_name, *args):
    """A zero-argument callable that invokes the C entry point `fn_name` with arguments
    converted once up front (tensors become device addresses).  For launch loops whose
    per-call Python cost must stay small; raises SpecHeadError on a non-zero status."""
    lib = load()
    fn = getattr(lib, fn_name)
    conv = []
    for a in args:
        if isinstance(a, torch.Tensor):
            conv.append(ctypes.c_void_p(a.data_ptr()))
        elif isinstance(a, np.ndarray):   # host array (kept alive by the closure below)
            conv.append(a.ctypes.data_as(_vp))
        else:
            conv.append(a)
    conv = tuple(conv)

    hold = args

    def call():
        assert hold is not None
        rc = fn(*conv)
        if rc != SH_OK:
            _check(rc)
    return call
