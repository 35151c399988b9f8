/*
 * spechead.h -- C ABI of the MI355X (gfx950) drafter LM-head and speculative-verification
 * library (libspechead.so).
 *
 * What the calls compute (sources: the pages this library is built from):
 *   - draft_head_dense:     z = W h over the whole vocabulary (SlimSpec write-up, mhpn.cn,
 *                           section 三: a V x d matrix projects the d-dim hidden state).
 *   - draft_head_lowrank:   SlimSpec, same section and Q&A Q1: h_r = W_down h (d -> r),
 *                           z = W_up h_r (r -> V), all V scores kept.
 *   - draft_head_specvocab: SpecVocab write-up (2kiu.com), sections 2.2.1-2.2.3:
 *                           h' = W_down h (d' = d/16), s = W_vocab h', K = top-k(s),
 *                           z' = U[K,:] h, q = softmax(z') over the k candidates.
 *   - spec_verify:          speculative-decoding explainer (liuchunshan.com), sections
 *                           "小模型起草，大模型批改" and "为什么答案不会变": greedy
 *                           longest-prefix match, or rejection sampling accepting with
 *                           min(1, p/q), residual draw from norm(max(0, p - q)) at the first
 *                           rejection, bonus draw from the target when all drafts pass.
 *   Each head is fused with selection: greedy argmax (ties -> lowest id) or sampling from
 *   softmax(z / T), and returns the row's log-sum-exp and the chosen token's log-probability.
 *
 * Conventions (all calls):
 *   - Buffers are DEVICE pointers owned by the caller, packed row-major, 16-byte aligned
 *     (the workspace 256-byte aligned).  `stream` is a hipStream_t (NULL = null stream).
 *   - dtype: SH_F32 (float32) or SH_BF16 (bfloat16 stored as 16-bit patterns) for hidden
 *     states, weights and logits inputs.  Row lengths must be a multiple of 16 bytes
 *     (bf16: multiple of 8 elements; f32: multiple of 4).  Outputs are int32 / float32.
 *   - Return value: SH_OK (0) means all work was enqueued on `stream`; the call never
 *     synchronises.  Any other value below SH_ERR_HIP means validation failed BEFORE any
 *     HIP call: nothing was enqueued and no output was touched.  SH_ERR_HIP means a HIP
 *     runtime call or launch failed; sh_last_error() holds a thread-local message.
 *   - No allocation: the caller passes a workspace of at least sh_*_workspace_bytes(...)
 *     bytes; its contents on entry do not matter (each call clears what it counts into).
 *     Calls that may overlap in time must use distinct workspaces.
 *   - Threads: calls from several host threads are safe when their workspaces are distinct
 *     (the per-device attribute cache is filled under a lock).  Tracing (sh_trace_*) is a
 *     process-wide switch meant for one measuring thread.
 *   - Determinism: identical inputs, seed and offset give bit-identical outputs.
 *   - Sampling randomness: Philox4x64-10 (Salmon et al., SC'11) with key (seed, 0) and
 *     counter (index / 4, row, purpose, offset); the draw is output word index % 4 mapped to
 *     u = ((word >> 41) + 0.5) * 2^-23 in (0,1).  Purposes: 0 draft group, 1 draft element,
 *     2 verify accept (caller-side), 3 residual group, 4 residual element, 5 bonus group,
 *     6 bonus element.  A draw from softmax(l) is a two-level Gumbel-max: groups of 64
 *     consecutive candidates compete with log-sum-exp + Gumbel(u_group) (ties -> lowest
 *     group), then the members of the winning group with l_i + Gumbel(u_i) (ties -> lowest
 *     index), which is an exact draw from softmax(l).  Callers advance `offset` per call.
 */
#ifndef SPECHEAD_H
#define SPECHEAD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum sh_status {
  SH_OK = 0,
  SH_ERR_NULL = 1,        /* a required pointer is NULL                               */
  SH_ERR_SHAPE = 2,       /* a size is out of range or inconsistent                   */
  SH_ERR_DTYPE = 3,       /* unknown dtype or mode                                    */
  SH_ERR_ALIGN = 4,       /* a pointer is not 16-byte (workspace: 256-byte) aligned    */
  SH_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than required                  */
  SH_ERR_PARAM = 6,       /* temperature <= 0 or not finite, k outside [1, V], ...    */
  SH_ERR_UNSUPPORTED = 7, /* valid request outside what the library implements        */
  SH_ERR_HIP = 8          /* a HIP call or kernel launch failed                       */
};

enum sh_dtype { SH_F32 = 0, SH_BF16 = 1 };
enum sh_mode { SH_GREEDY = 0, SH_SAMPLE = 1 };
enum sh_op { SH_OP_DENSE = 0, SH_OP_LOWRANK = 1, SH_OP_SPECVOCAB = 2 };

/* Workspace size for a head call.  op = SH_OP_*; r is the low-rank width (lowrank) or the
 * reduced width d' (specvocab) and is ignored for dense; k is ignored except for specvocab.
 * Pure host arithmetic, no HIP call.  Returns 0 for invalid arguments. */
size_t sh_head_workspace_bytes(int op, int64_t M, int64_t d, int64_t r, int64_t V, int64_t k);

/* Where a completed low-rank or SpecVocab head call leaves its rounded intermediate in the
 * workspace: the byte offset of h_r = round(W_down h) [M, r] (SH_OP_LOWRANK; also the
 * position-adaptive call, with r = r_max, rows zero past their rank) or h' [M, d'] (SH_OP_SPECVOCAB,
 * r = d'), row-major in the call's dtype.  The value is the one the oracle of the SlimSpec
 * write-up, section 三, rounds once to the storage dtype; callers may read it back after the
 * call has completed on its stream (e.g. to check the up-projection on the exact h_r the
 * kernels used).  Same arguments as sh_head_workspace_bytes; pure host arithmetic.  Returns
 * SIZE_MAX for SH_OP_DENSE or invalid arguments. */
size_t sh_head_intermediate_offset(int op, int64_t M, int64_t d, int64_t r, int64_t V, int64_t k);

/* Workspace size for spec_verify.  Pure host arithmetic, no HIP call. */
size_t sh_verify_workspace_bytes(int mode, int64_t B, int64_t gamma, int64_t V);

/* Workspace size for spec_verify_tree (0 for invalid sizes).  Pure host arithmetic. */
size_t sh_verify_tree_workspace_bytes(int64_t B, int64_t N, int64_t V);

/* Workspace size for spec_verify_sparse (0 for invalid sizes).  Pure host arithmetic. */
size_t sh_verify_sparse_workspace_bytes(int64_t B, int64_t gamma, int64_t V, int64_t k);

/*
 * Dense head (SlimSpec write-up, section 三).
 *   h       [M, d]   hidden states, dtype
 *   W       [V, d]   head matrix, dtype
 *   mode, temperature: SH_GREEDY picks argmax_i z_i (ties -> lowest i); SH_SAMPLE draws from
 *           softmax(z / T).  temperature must be > 0 and finite in both modes: lse and
 *           logprob are those of y = z / T.
 *   seed, offset: Philox key / counter word (sampling; ignored when greedy).  Row index of
 *           the draw = row of h.
 *   token   [M] int32 (required)   chosen vocabulary id
 *   lse     [M] float (nullable)   log sum_i exp(y_i)
 *   logprob [M] float (nullable)   y_token - lse
 *   logits  [M, V] float (nullable) raw z, written only when non-NULL (extra M*V*4 bytes)
 */
int draft_head_dense(const void* h, int64_t M, int64_t d, const void* W, int64_t V, int dtype,
                     int mode, float temperature, uint64_t seed, uint64_t offset,
                     int32_t* token, float* lse, float* logprob, float* logits,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * Static trimmed-vocabulary head (SlimSpec write-up, section 二: static trimming scores only a
 * fixed reduced vocabulary, and a trimmed-away token can never be proposed, which caps the
 * acceptance rate at the target's mass on the kept ids).  The dense head over n_S kept rows:
 *   W_S [n_S, d] device: the kept rows W[ids], gathered once by the caller
 *   ids [n_S] int32 device: their vocabulary ids
 *   token [M]: ids[j] for the chosen kept position j; lse / logprob (of y = z / T) over the
 *   kept rows;
 *   logits (nullable) [M, n_S] float: the raw scores z = W_S h in kept-row order (not divided
 *   by T, as for draft_head_dense).
 *   Sampling groups are the 64-position groups of the kept-row order (Philox purposes 0/1,
 *   row m).  Shapes, dtypes and errors as draft_head_dense with V = n_S.
 *   Workspace: sh_head_workspace_bytes(SH_OP_DENSE, M, d, 0, n_S, 0).
 */
int draft_head_trimmed(const void* h, int64_t M, int64_t d, const void* W_S, int64_t n_S, const int32_t* ids,
                       int dtype, int mode, float temperature, uint64_t seed, uint64_t offset, int32_t* token,
                       float* lse, float* logprob, float* logits, void* workspace, size_t workspace_bytes,
                       void* stream);

/*
 * SlimSpec low-rank head (SlimSpec write-up, section 三 and Q&A Q1).
 *   W_down  [r, d]   (the d -> r map stored row per output), dtype
 *   W_up    [V, r]   dtype
 *   h_r = W_down h is accumulated in float32 and rounded once (nearest-even) to dtype, then
 *   z = W_up h_r.  Other arguments and outputs as draft_head_dense.
 */
int draft_head_lowrank(const void* h, int64_t M, int64_t d, const void* W_down, int64_t r,
                       const void* W_up, int64_t V, int dtype, int mode, float temperature,
                       uint64_t seed, uint64_t offset, int32_t* token, float* lse,
                       float* logprob, float* logits, void* workspace, size_t workspace_bytes,
                       void* stream);

/*
 * draft_head_lowrank without a workspace argument, for callers that cannot allocate device
 * memory or do not own a workspace: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  Same arguments (minus workspace / workspace_bytes),
 * kernels, outputs and error codes as draft_head_lowrank; the scratch is a static device
 * array of 8 MiB (one per GPU the library runs on, held until the process ends), so calls
 * whose sh_head_workspace_bytes(SH_OP_LOWRANK, M, d, r, V, 0) exceeds 8 MiB return
 * SH_ERR_UNSUPPORTED before any HIP call (M <= 64 rows at r = 512 fits up to V = 2^19).  The
 * call allocates nothing.  Every call on one GPU shares that GPU's array: calls that may
 * overlap in time on one GPU (different streams, or different host threads) race and must
 * be serialised by the caller.  The first call on a device looks up the array's device
 * address (a HIP symbol query, no allocation).
 */
int draft_head_lowrank_noalloc(const void* h, int64_t M, int64_t d, const void* W_down, int64_t r,
                               const void* W_up, int64_t V, int dtype, int mode, float temperature,
                               uint64_t seed, uint64_t offset, int32_t* token, float* lse,
                               float* logprob, float* logits, void* stream);

/*
 * Position-adaptive rank (SlimSpec write-up, section 七, second future direction: earlier
 * draft positions get a larger rank, later ones a smaller one).  One factor pair of rank
 * r_max serves every row through nested prefixes: row m uses the first ranks[m] rows of
 * W_down and the first ranks[m] columns of W_up,
 *   z_m = W_up[:, :r_m] round(W_down[:r_m] h_m),
 * with the selection, outputs and Philox uniforms of draft_head_lowrank.
 *   h [M, d], W_down [r_max, d], W_up [V, r_max]: device, bf16 only, 1 <= M <= 64
 *   ranks [M] int32: a HOST array, each in [1, r_max] (read during the call)
 *   Only the first max(ranks) columns of W_up are read, rounded up to 128 (or r_max): a call
 *   whose rows all have small ranks streams fewer bytes.  Shapes outside the bf16 tile pass
 *   (r_max a multiple of 8, columns read in {128, 256, 384, 512}) return SH_ERR_UNSUPPORTED.
 *   Workspace: sh_head_workspace_bytes(SH_OP_LOWRANK, M, d, r_max, V, 0).
 */
int draft_head_lowrank_adaptive(const void* h, int64_t M, int64_t d, const void* W_down, int64_t r_max,
                                const void* W_up, int64_t V, const int32_t* ranks, int dtype, int mode,
                                float temperature, uint64_t seed, uint64_t offset, int32_t* token,
                                float* lse, float* logprob, float* logits, void* workspace,
                                size_t workspace_bytes, void* stream);

/*
 * SpecVocab dynamic-vocabulary head (SpecVocab write-up, sections 2.2.1-2.2.3 and 5.1).
 *   W_down  [d', d]  reduced-state map, dtype;  h' = W_down h rounded once to dtype
 *   W_vocab [V, d']  approximate scorer, dtype;  s = W_vocab h' (float32)
 *   U       [V, d]   exact head, dtype; only the k gathered rows are read
 *   k       1 <= k <= min(V, 16384): K = the k largest s (ties -> lowest id), ascending ids;
 *           V <= 2^19, M <= 65535
 *   topk_idx   [M, k] int32 (required)  K
 *   topk_logit [M, k] float (nullable)  z'_j = U[K_j,:] . h   (full-precision h)
 *   topk_prob  [M, k] float (nullable)  softmax(z' / T) over the k candidates
 *   token      [M] int32 (required)     chosen vocabulary id (an element of K); sampling
 *              groups are formed over candidate positions 0..k-1 (ascending ids)
 *   lse, logprob [M] (nullable)          over the k candidates
 */
int draft_head_specvocab(const void* h, int64_t M, int64_t d, const void* W_down, int64_t dprime,
                         const void* W_vocab, const void* U, int64_t V, int64_t k, int dtype,
                         int mode, float temperature, uint64_t seed, uint64_t offset,
                         int32_t* topk_idx, float* topk_logit, float* topk_prob, int32_t* token,
                         float* lse, float* logprob, void* workspace, size_t workspace_bytes,
                         void* stream);

/*
 * Batched verification (explainer sections "小模型起草，大模型批改", "为什么答案不会变";
 * SpecTr-GBV write-up: the first rejection ends the block, residual next token, bonus token).
 *   target_logits [B, gamma+1, V] dtype: target scores at the gamma+1 positions
 *   draft_logits  [B, gamma,   V] dtype: draft scores (SH_SAMPLE only; NULL for greedy)
 *                 Scores may be -inf (a token of zero probability, e.g. outside a drafter's
 *                 trimmed vocabulary); every row needs one finite score; NaN and +inf are
 *                 not allowed.
 *   B <= 65535, 1 <= gamma <= 64, V <= 2^28
 *   draft_tokens  [B, gamma] int32: proposed ids; an id outside [0, V) is never accepted
 *   u_accept      [B, gamma] float in (0,1): accept uniforms (SH_SAMPLE only; else NULL)
 *   temperature > 0: p = softmax(target / T), q = softmax(draft / T) (sampling)
 *   SH_GREEDY: a = first t with draft_tokens[t] != argmax target[t] (ties -> lowest id),
 *              else gamma; emitted = drafts[0..a-1], argmax target[a].
 *   SH_SAMPLE: accept t iff u_t < p_t(x_t) / q_t(x_t); a = leading accepts; if a < gamma the
 *              last token is drawn from norm(max(0, p_a - q_a)) (purposes 3/4, row b; if that
 *              mass is 0, from p_a), else from p_gamma (purposes 5/6, row b).
 *   accept_len [B] int32: a
 *   out_tokens [B, gamma+1] int32: emitted tokens, -1 after the last one
 *   Workspace: sh_verify_workspace_bytes(mode, B, gamma, V).
 */
int spec_verify(int mode, int64_t B, int64_t gamma, int64_t V, int dtype,
                const void* target_logits, const void* draft_logits, const int32_t* draft_tokens,
                const float* u_accept, float temperature, uint64_t seed, uint64_t offset,
                int32_t* accept_len, int32_t* out_tokens, void* workspace,
                size_t workspace_bytes, void* stream);

/*
 * Greedy verification of a tree of candidate continuations (phrase-level speculation page,
 * section "更换单元：从 token 到短语": the candidates of a round share prefixes, form a prefix
 * tree scored in one target pass, and a candidate survives only where it equals the target's
 * own argmax, so the output equals greedy decoding).
 *   target_logits [B, N, V] dtype (device): row n scores the token that follows node n's prefix
 *   node_token    [B, N] int32 (device): the token node n proposes (node 0 is the root, the
 *                 last accepted token; its entry is not verified)
 *   parent        [B, N] int32 (device): parent of node n; a node whose parent is not in
 *                 [0, n) is never accepted, nor is any node below it
 *   B <= 65535, 1 <= N <= 1024, V <= 2^28
 *   Node n is accepted when its parent is accepted and node_token[n] equals the argmax (ties ->
 *   lowest id) of its parent's row.  The deepest accepted node m (lowest index on ties) ends
 *   the accepted path; the argmax of row m follows it (correction or bonus token).
 *   accept_len  [B] int32: depth of m (tokens accepted)
 *   accept_node [B] int32: m
 *   out_tokens  [B, N] int32: the path's tokens root-side first, then argmax of row m, then -1
 *   Returns SH_ERR_* before any launch on invalid arguments; asynchronous on `stream`.
 *   Workspace: sh_verify_tree_workspace_bytes(B, N, V), 256-byte aligned, contents irrelevant.
 */
int spec_verify_tree(int64_t B, int64_t N, int64_t V, int dtype, const void* target_logits,
                     const int32_t* node_token, const int32_t* parent, int32_t* accept_len,
                     int32_t* accept_node, int32_t* out_tokens, void* workspace,
                     size_t workspace_bytes, void* stream);

/*
 * Sampling verification against a sparse draft distribution: the bridge from the SpecVocab
 * head (SpecVocab write-up, 2.2.3: the draft's probabilities live on its k candidates; 3.3:
 * verification keeps the full vocabulary) to speculative sampling (explainer, "为什么答案
 * 不会变").  q_t is draft_prob on draft_idx and zero elsewhere; p_t = softmax(target_t / T).
 *   target_logits [B, gamma+1, V] dtype (device)
 *   draft_idx     [B, gamma, k] int32 (device): candidate ids of each position, distinct,
 *                 in [0, V) (the SpecVocab head's topk_idx)
 *   draft_prob    [B, gamma, k] float (device): q on those ids (its topk_prob)
 *   draft_tokens  [B, gamma] int32, u_accept [B, gamma] float in (0,1) (device)
 *   B <= 65535, 1 <= gamma <= 64, V <= 2^28, 1 <= k <= min(V, 16384), temperature > 0
 *   Accept t iff u_t < p_t(x_t) / q_t(x_t); a draft id with q_t(x_t) = 0 is accepted when
 *   p_t(x_t) > 0 (the ratio is infinite); an id outside [0, V) is never accepted.  If a < gamma
 *   the last token is drawn from norm(max(0, p_a - q_a)), which is p_a outside the candidates
 *   (purposes 3/4, row b), else from p_gamma (purposes 5/6, row b), by the same two-level
 *   Gumbel rule as spec_verify.
 *   accept_len [B] int32, out_tokens [B, gamma+1] int32 (-1 after the last emitted token).
 *   Returns SH_ERR_* before any launch on invalid arguments; the call is asynchronous on
 *   `stream`.  Workspace: sh_verify_sparse_workspace_bytes(B, gamma, V, k), 256-byte aligned,
 *   contents irrelevant.
 */
int spec_verify_sparse(int64_t B, int64_t gamma, int64_t V, int64_t k, int dtype,
                       const void* target_logits, const int32_t* draft_idx, const float* draft_prob,
                       const int32_t* draft_tokens, const float* u_accept, float temperature,
                       uint64_t seed, uint64_t offset, int32_t* accept_len, int32_t* out_tokens,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * Top-k building block of draft_head_specvocab (SpecVocab write-up, section 2.2.2), exposed
 * so it can be checked on given scores: for each of M rows of float32 scores [M, V], the k
 * largest (ties -> lowest index), written as ascending ids to topk_idx [M, k].  Scores must
 * be finite; V <= 2^19.  Workspace: sh_topk_workspace_bytes(M, V, k).
 */
size_t sh_topk_workspace_bytes(int64_t M, int64_t V, int64_t k);
int sh_topk(const float* scores, int64_t M, int64_t V, int64_t k, int32_t* topk_idx,
            void* workspace, size_t workspace_bytes, void* stream);

/*
 * The library's in-kernel uniform stream, exported for checking: out[row, i] = the uniform
 * for (seed, offset, purpose, row, index i), rows x n floats.
 */
int sh_philox_uniform(uint64_t seed, uint64_t offset, uint32_t purpose, int64_t rows, int64_t n,
                      float* out, void* stream);

/*
 * Measurement helper, not a step of the method: reads the `bytes` bytes at device address buf
 * with 16-byte loads in the flat order (1024 workgroups of 256 threads striding over the
 * buffer, four loads in flight per thread) and XORs every 32-bit word into *sink (a device
 * word the caller zeroes first), so that no load can be skipped and the result does not depend
 * on order.  Timed on a buffer larger than the 256 MB Infinity Cache it gives the attainable
 * HBM read rate, the bench's second denominator beside the 8 TB/s peak.  bytes: a nonzero
 * multiple of 16, at most 0xFFFFFFF0; buf 16-byte aligned, sink 4-byte aligned.  Returns SH_ERR_*
 * before any launch on invalid arguments; asynchronous on `stream`.
 */
int sh_read_probe(const void* buf, uint64_t bytes, uint32_t* sink, void* stream);

/*
 * Opt-in kernel timing (tracing).  sh_trace_enable(n) creates 2n host-side event objects and,
 * from then on, brackets every kernel this library launches with two events recorded on the
 * launch stream (at most n launches until the next read); n = 0 disables and frees them.
 * sh_trace_read waits for the recorded events and writes a JSON object
 * {"kernel": {"count", "total_us", "min_us", "max_us"}, ...} into buf (NUL-terminated),
 * then clears the records.  SH_ERR_PARAM if buf is too small; SH_ERR_HIP on event errors.
 */
int sh_trace_enable(int64_t max_records);
int sh_trace_read(char* buf, size_t bytes);

/* Static description of a status code. */
const char* sh_status_str(int status);
/* Message of the last failed call on this host thread ("" if none). */
const char* sh_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SPECHEAD_H */
