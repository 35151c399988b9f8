"""Seeded synthetic inputs shared by the tests, the benchmark and the CPU baseline.

This module only draws random numbers and stores them in the input formats; it holds none
of the method's arithmetic (no head product, no softmax of the method, no verification).
Recipe (per workload; see ``configs``):
* hidden states h ~ N(0, 1);
* weights ~ N(0, std = 1/sqrt(fan_in)), fan_in = d for W, W_down, W_down', U;
  r for W_up; d' for W_vocab  (so logits are roughly N(0, 1));
* target logits ~ N(0, 3^2); draft logits = target + N(0, sigma^2), both stored in the
  workload dtype;
* draft tokens: x ~ categorical(softmax(draft / T)) drawn by NumPy's own Gumbel draws
  (sampling) or x = argmax(draft) (greedy);
* accept uniforms u = (n + 0.5) * 2^-23 with n uniform in [0, 2^23), drawn by NumPy's
  Philox bit generator, so u is exact in float32 and strictly inside (0, 1);
* a sparse draft distribution (input data of the sparse verification, in the layout of the
  SpecVocab head's output): per position the k ids of largest draft logit, with weights
  exp(draft / T) normalised over those ids, and a token drawn from them;
* candidate trees: parent[n] uniform in [0, n) (a random recursive tree) or, with probability
  `chain`, n - 1; the c-th child of a node proposes the c-th largest id of a noisy copy
  (target + N(0, sigma^2)) of that node's target row, as a tree drafter's top-c branches.
bf16 values are produced by PyTorch's float32 -> bfloat16 conversion (round to nearest
even) and kept as uint16 bit patterns on the host.
"""
import numpy as np


def _bf16_bits(x_f32):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x_f32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _bits_to_f32(bits):
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def store(x_f32, dtype):
    """float32 array -> storage format: uint16 bf16 bits, or float32."""
    if dtype == "bf16":
        return _bf16_bits(x_f32)
    if dtype == "f32":
        return np.ascontiguousarray(x_f32, dtype=np.float32)
    raise ValueError(dtype)


def as_f32(arr, dtype):
    """Storage format -> float32 (exact)."""
    if dtype == "bf16":
        return _bits_to_f32(np.asarray(arr, dtype=np.uint16))
    return np.asarray(arr, dtype=np.float32)


def normal(rng, shape, std, dtype, chunk_rows=16384):
    """N(0, std^2) array in the storage dtype, generated in row chunks to bound memory."""
    shape = tuple(int(s) for s in shape)
    out = np.empty(shape, dtype=np.uint16 if dtype == "bf16" else np.float32)
    rows = shape[0]
    for lo in range(0, rows, chunk_rows):
        hi = min(rows, lo + chunk_rows)
        x = rng.standard_normal((hi - lo,) + shape[1:], dtype=np.float32)
        if std != 1.0:
            x *= np.float32(std)
        out[lo:hi] = store(x, dtype)
    return out


def hidden(M, d, dtype, seed):
    return normal(np.random.default_rng(seed), (M, d), 1.0, dtype)


def dense_weights(V, d, dtype, seed):
    rng = np.random.default_rng([seed, 1])
    return normal(rng, (V, d), 1.0 / np.sqrt(d), dtype)


def lowrank_weights(V, d, r, dtype, seed):
    rng = np.random.default_rng([seed, 2])
    W_down = normal(rng, (r, d), 1.0 / np.sqrt(d), dtype)
    W_up = normal(rng, (V, r), 1.0 / np.sqrt(r), dtype)
    return W_down, W_up


def specvocab_weights(V, d, dprime, dtype, seed, with_U=True):
    rng = np.random.default_rng([seed, 3])
    W_down = normal(rng, (dprime, d), 1.0 / np.sqrt(d), dtype)
    W_vocab = normal(rng, (V, dprime), 1.0 / np.sqrt(dprime), dtype)
    U = dense_weights(V, d, dtype, seed) if with_U else None
    return W_down, W_vocab, U


def uniforms_open(n_shape, seed):
    """float32 uniforms strictly inside (0,1), centred on a 2^-23 grid (exact in float32),
    from NumPy's Philox bit generator."""
    g = np.random.Generator(np.random.Philox(seed))
    n = g.integers(0, 1 << 23, size=n_shape, dtype=np.int64)
    return ((n.astype(np.float64) + 0.5) * 2.0 ** -23).astype(np.float32)


def verify_inputs(B, gamma, V, sigma, dtype, seeds, mode="sample", temperature=1.0,
                  target_std=3.0):
    """Target/draft logits, draft tokens and accept uniforms for one verification call."""
    rng = np.random.default_rng([seeds["logits"], int(round(sigma * 1000))])
    target = normal(rng, (B, gamma + 1, V), target_std, dtype, chunk_rows=4)
    noise_rng = np.random.default_rng([seeds["logits"], int(round(sigma * 1000)), 7])
    draft = np.empty((B, gamma, V), dtype=target.dtype)
    for b in range(B):
        t32 = as_f32(target[b, :gamma], dtype)
        n32 = noise_rng.standard_normal(t32.shape, dtype=np.float32) * np.float32(sigma)
        draft[b] = store(t32 + n32, dtype)
    tok_rng = np.random.default_rng([seeds["tokens"], int(round(sigma * 1000))])
    tokens = np.empty((B, gamma), dtype=np.int32)
    for b in range(B):
        d32 = as_f32(draft[b], dtype)
        if mode == "greedy":
            tokens[b] = np.argmax(d32, axis=-1)
        else:
            g = tok_rng.gumbel(size=d32.shape).astype(np.float32)
            tokens[b] = np.argmax(d32 / np.float32(temperature) + g, axis=-1)
    u = uniforms_open((B, gamma), seeds["uniforms"] + int(round(sigma * 1000)))
    return {"target": target, "draft": draft, "tokens": tokens, "u": u}


def verify_sparse_inputs(B, gamma, V, k, sigma, dtype, seeds, temperature=1.0, target_std=3.0):
    """verify_inputs' target logits and uniforms with a sparse draft distribution in place of
    the draft logits: per position the k ids with the largest draft logits (ascending ids) and
    q = softmax(draft / T) over those ids alone (the shape of the SpecVocab head's topk_idx /
    topk_prob); draft tokens are drawn from q."""
    base = verify_inputs(B, gamma, V, sigma, dtype, seeds, mode="greedy", temperature=temperature,
                         target_std=target_std)
    tok_rng = np.random.default_rng([seeds["tokens"], int(round(sigma * 1000)), k])
    idx = np.empty((B, gamma, k), dtype=np.int32)
    prob = np.empty((B, gamma, k), dtype=np.float32)
    tokens = np.empty((B, gamma), dtype=np.int32)
    for b in range(B):
        d = as_f32(base["draft"][b], dtype).astype(np.float64) / temperature
        for t in range(gamma):
            top = np.sort(np.argpartition(-d[t], k - 1)[:k]) if k < V else np.arange(V)
            y = d[t, top]
            w = np.exp(y - y.max())
            q = (w / w.sum()).astype(np.float32)
            idx[b, t] = top
            prob[b, t] = q
            qq = q.astype(np.float64)
            tokens[b, t] = top[tok_rng.choice(k, p=qq / qq.sum())]
    return {"target": base["target"], "idx": idx, "prob": prob, "tokens": tokens, "u": base["u"]}


def tree_inputs(B, N, V, sigma, dtype, seeds, chain=0.5, target_std=3.0):
    """Target logits [B, N, V] (row n scores the token after node n's prefix), node tokens and
    parent links [B, N] of B candidate trees of N nodes (node 0 the root, parent -1)."""
    rng = np.random.default_rng([seeds["logits"], int(round(sigma * 1000)), N])
    target = normal(rng, (B, N, V), target_std, dtype, chunk_rows=4)
    shape_rng = np.random.default_rng([seeds["tokens"], N, 11])
    noise_rng = np.random.default_rng([seeds["logits"], int(round(sigma * 1000)), N, 13])
    parent = np.full((B, N), -1, dtype=np.int32)
    tokens = np.zeros((B, N), dtype=np.int32)
    for b in range(B):
        for n in range(1, N):
            parent[b, n] = n - 1 if shape_rng.random() < chain else shape_rng.integers(0, n)
        tokens[b, 0] = shape_rng.integers(0, V)
        children = {}
        for n in range(1, N):
            children.setdefault(int(parent[b, n]), []).append(n)
        for p, kids in children.items():
            noisy = as_f32(target[b, p], dtype) + noise_rng.standard_normal(V, dtype=np.float32) * np.float32(sigma)
            order = np.argsort(-noisy, kind="stable")[:len(kids)]
            for c, n in enumerate(kids):
                tokens[b, n] = order[c]
    return {"target": target, "tokens": tokens, "parent": parent}
