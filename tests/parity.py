"""Helpers for GPU-vs-oracle parity checks.

Expected values always come from the oracle on the same seeded inputs.  Decisions taken in
floating point (argmax, Gumbel draws, top-k boundary) may differ from the float64 oracle
only where the oracle itself puts the competing choices within the arithmetic's error;
every such excusal is counted and printed, and tests bound how many may occur.
"""
import sys

import numpy as np
import torch

from oracle import fp, philox, sampler

# logits tolerance (relative to |o| + rms of the row): bf16 inputs 1e-2, f32 inputs 1e-5
RTOL = {"bf16": 1e-2, "f32": 1e-5}
# decision tolerance for fp32 accumulation vs float64: 1e-5 * (1 + |score|)
DEC_TOL = 1e-5
# row log-sum-exp and log-probability against float64 on the same (exact) inputs: the GPU's
# fp32 accumulation and fp32 exp / log / sums move them by a few 1e-6 at the head shapes, so
# 1e-5 * (1 + |lse|) holds with margin while a dropped or doubled 64-row group (about
# 64 / V in lse: 5e-4 at V = 128256, 1e-2 at V = 8200) does not pass
LSE_RTOL = 1e-5


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_device(arr, dtype, device="cuda"):
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32))
    return t.to(device)


def assert_logits_close(got, want, dtype, what="logits"):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    rms = np.sqrt(np.mean(want ** 2, axis=-1, keepdims=True))
    tol = RTOL[dtype] * (np.abs(want) + rms)
    bad = np.abs(got - want) > tol
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {bad.sum()} elements outside tolerance, first at {tuple(i)}: "
                             f"got {got[tuple(i)]} want {want[tuple(i)]}")
    return float(np.max(np.abs(got - want) / tol))


def rounding_flip_bound(pre_exact, terms_abs_sum, dtype, W_next_abs):
    """Bound on how much a row of the next product can move because the fp32 accumulation
    of the rounded intermediate (h_r or h') lands on the other side of a bf16 rounding
    midpoint than the float64 value.  pre_exact: [M, r] float64 values before rounding;
    terms_abs_sum: [M, r] sum of |terms| of each dot product; W_next_abs: [V, r] |weights|.
    Returns [M, V] bounds (zero where no element of the row is ambiguous)."""
    if dtype != "bf16":
        delta = 2.0 ** -20 * terms_abs_sum
        lo = fp.round_to_dtype(pre_exact - delta, "f32")
        hi = fp.round_to_dtype(pre_exact + delta, "f32")
    else:
        delta = 2.0 ** -16 * terms_abs_sum
        lo = fp.round_to_dtype(pre_exact - delta, "bf16")
        hi = fp.round_to_dtype(pre_exact + delta, "bf16")
    amb = np.abs(hi - lo)                        # 0 where the rounding is unambiguous
    if not amb.any():
        return np.zeros((pre_exact.shape[0], W_next_abs.shape[0]))
    return amb @ W_next_abs.T


def check_lse_logprob(lse_gpu, lp_gpu, lse_o, y_tok, what):
    """lse and logprob (y_tok - lse) of the GPU against the oracle's values on the same
    inputs; y_tok is the oracle's y = z / T at the GPU's own token.  Returns the largest
    error / tolerance ratios (lse, logprob)."""
    lse_o = np.asarray(lse_o, np.float64)
    tol = LSE_RTOL * (1 + np.abs(lse_o))
    r1 = 0.0
    if lse_gpu is not None:
        e = np.abs(np.asarray(lse_gpu, np.float64) - lse_o)
        bad = e > tol
        assert not bad.any(), f"{what} lse: rows {np.flatnonzero(bad)[:5]} err {e[bad][:5]} tol {tol[bad][:5]}"
        r1 = float(np.max(e / tol))
    r2 = 0.0
    if lp_gpu is not None:
        want = np.asarray(y_tok, np.float64) - lse_o
        tol2 = LSE_RTOL * (1 + np.abs(lse_o) + np.abs(y_tok))
        e = np.abs(np.asarray(lp_gpu, np.float64) - want)
        bad = e > tol2
        assert not bad.any(), f"{what} logprob: rows {np.flatnonzero(bad)[:5]} err {e[bad][:5]} tol {tol2[bad][:5]}"
        r2 = float(np.max(e / tol2))
    log(f"  {what}: lse err/tol {r1:.3g}, logprob err/tol {r2:.3g}")
    return r1, r2


def check_intermediate(got, exact, terms_abs_sum, dtype, what, max_frac=0.01):
    """The GPU's rounded intermediate (h_r or h') against the oracle's: float32 values from
    fp32 accumulation rounded once to `dtype`.  bf16: each element is the oracle's rounding
    of the exact product, or -- only where the exact value lies within the fp32 accumulation
    error (2^-16 * sum |terms|) of a rounding midpoint -- a bf16 value within that error
    band around it.  f32: within 2^-20 * sum |terms| of the exact value.  Returns the number of
    flipped elements (bf16)."""
    got = np.asarray(got, np.float64)
    exact = np.asarray(exact, np.float64)
    if dtype != "bf16":
        e = np.abs(got - exact)
        tol = 2.0 ** -20 * terms_abs_sum + 1e-30
        assert np.all(e <= tol), f"{what}: max err/tol {np.max(e / tol)}"
        return 0
    want = fp.round_to_dtype(exact, "bf16")
    diff = got != want
    if not diff.any():
        return 0
    delta = 2.0 ** -16 * terms_abs_sum
    lo = fp.round_to_dtype(exact - delta, "bf16")
    hi = fp.round_to_dtype(exact + delta, "bf16")
    ok = diff & (got >= lo) & (got <= hi) & (lo != hi)
    bad = diff & ~ok
    assert not bad.any(), f"{what}: {bad.sum()} elements off the oracle's rounding, first {np.argwhere(bad)[0]}"
    n = int(diff.sum())
    log(f"  {what}: {n} of {got.size} elements rounded the other way at a midpoint")
    assert n <= max(2, max_frac * got.size), n
    return n


class Excusals:
    def __init__(self, name):
        self.name = name
        self.items = []

    def add(self, why):
        self.items.append(why)

    def report(self, total, max_frac=0.02, max_abs=1):
        log(f"[{self.name}] excused {len(self.items)} of {total}: {self.items[:5]}")
        assert len(self.items) <= max(max_abs, int(max_frac * total)), self.items


def check_greedy_tokens(got, z_oracle, ex, bound=None):
    """got: [M] tokens; z_oracle: [M, V] float64 logits; bound: optional [M, V] extra error."""
    for m in range(z_oracle.shape[0]):
        z = z_oracle[m]
        to = int(np.argmax(z))
        tg = int(got[m])
        if tg == to:
            continue
        assert 0 <= tg < z.size, (m, tg)
        tol = DEC_TOL * (1 + abs(z[to]))
        if bound is not None:
            tol += bound[m, to] + bound[m, tg]
        margin = z[to] - z[tg]
        assert margin <= tol, f"row {m}: gpu {tg} oracle {to} margin {margin} > tol {tol}"
        ex.add(("argmax", m, tg, to, float(margin)))


def check_sampled_token(tg, to, ell, group_u, elem_u, diag, tol_fn, ex, tag):
    """Two-level Gumbel decision check on one row.
    ell: float64 log-weights the oracle used; diag: oracle's sampler diagnostics;
    tol_fn(i, j): allowed score error between candidates i and j (same units as ell)."""
    if tg == to:
        return
    G = sampler.GROUP
    assert 0 <= tg < ell.size and np.isfinite(ell[tg]), (tag, tg)
    go, gg = to // G, tg // G
    if go == gg:
        es = diag["elem_scores"]
        lo = go * G
        margin = es[to - lo] - es[tg - lo]
        tol = DEC_TOL * (1 + abs(es[to - lo])) + tol_fn(to, tg)
        assert margin <= tol, f"{tag}: element {tg} vs {to}: margin {margin} > {tol}"
        ex.add(("element", tag, tg, to, float(margin)))
        return
    gs = diag["group_scores"]
    margin = gs[go] - gs[gg]
    # a group score moves with the error of its members' weights
    lo_o, lo_g = go * G, gg * G
    tol = DEC_TOL * (1 + abs(gs[go])) + tol_fn(slice(lo_o, lo_o + G), slice(lo_g, lo_g + G))
    assert margin <= tol, f"{tag}: group {gg} vs {go}: margin {margin} > {tol}"
    # inside the GPU's group the element must be the oracle's pick there (or a near-tie)
    pick, es = sampler.pick_in_group(ell, gg, elem_u)
    if pick != tg:
        m2 = es[pick - lo_g] - es[tg - lo_g]
        assert m2 <= DEC_TOL * (1 + abs(es[pick - lo_g])) + tol_fn(pick, tg), (tag, pick, tg, m2)
    ex.add(("group", tag, gg, go, float(margin)))


def head_sample_check(tok_gpu, out_oracle, seed, offset, temperature, ex, bound=None):
    """Check GPU sampled tokens of a head call against the oracle's draws."""
    Z = out_oracle["logits"]
    for m in range(Z.shape[0]):
        y = Z[m] / temperature
        dg = out_oracle["diag"][m]

        def tol_fn(i, j, m=m):
            if bound is None:
                return 0.0
            bi = np.max(bound[m, i]) if isinstance(i, slice) else bound[m, i]
            bj = np.max(bound[m, j]) if isinstance(j, slice) else bound[m, j]
            return (bi + bj) / temperature

        check_sampled_token(int(tok_gpu[m]), int(out_oracle["token"][m]), y,
                            lambda g, m=m: philox.uniforms(seed, offset, 0, m, g),
                            lambda i, m=m: philox.uniforms(seed, offset, 1, m, i),
                            dg, tol_fn, ex, f"row{m}")
