// Internal launch interface between the C-ABI layer (api.hip) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sh {

struct Partial;

// One streaming pass z[m, v] = W[v, :] . x[m, :] for v < V, m < M (M rows of this chunk).
// Outputs, each optional: the raw logits (zout), the per-group log-sum-exp of y = z * invT
// (lg, one value per row and 64-row vocabulary group, consumed by the finalize for the row
// lse and the group draw), and per-workgroup argmax partials (greedy).
struct StreamArgs {
  const void* W;      // [V, K] dtype
  const void* x;      // [M, K] dtype
  int64_t V, K;
  int M;
  bool bf16;
  bool want_argmax;
  float invT;
  float* zout;           // nullable [M, zout_ld]
  int64_t zout_ld;
  float* lg;             // nullable [M, lg_ld], lg_ld >= ceil(V / 64)
  int64_t lg_ld;
  Partial* partials;     // [M, partials_ld] when want_argmax, one per producer workgroup
  int64_t partials_ld;
};

struct FinalizeArgs {
  const Partial* partials;  // [M, ld] argmax partials (greedy)
  int64_t partials_ld;
  int P;                    // producers per row
  const float* lg;          // [M, lg_ld] group log-sum-exp (lse and sampling)
  int64_t lg_ld;
  const void* W;            // [V, K] (sampling: recompute the winning group)
  const void* x;            // [M, K]
  int64_t V, K;
  int64_t ld;               // row stride of W and x in elements (0: K); K <= ld uses row prefixes
  int M;
  bool bf16;
  int mode;                 // 0 greedy, 1 sample
  float invT;
  uint64_t seed, offset;
  int32_t* token;
  float* lse;
  float* logprob;
  const int32_t* id_map;    // nullable [V]: the token written is id_map[row chosen]
  const float* gz;          // nullable [M, gz_ld, 64]: the winning group's logits as written by
  int64_t gz_ld;            // the pass (by its owner among the P producers), not recomputed
  int gz_map;               // owner of group g: 0 K-chunked (consecutive ranges), 1 tile (wave stride)
};

// Tile-streaming head pass (bf16, rows of 128, 256, 384 or 512 elements, at most kTileMaxRows
// activation rows):
// z[m, v] = W[v, :] . x[m, :]; optional raw logits; per-workgroup Partials of y = z * invT
// (lse, best group score with the Philox group draw, argmax).
constexpr int kTileMaxRows = 64;
struct TileArgs {
  const void* W;      // [V, K] bf16
  const void* x;      // [M, K] bf16
  int64_t V;
  int K;              // elements of each row used (the prefix of rows of `ld` elements)
  int ld;             // row stride of W and x in elements (0: K)
  int M;              // rows of this pass, <= kTileMaxRows
  int row0;           // absolute index of x's first row (Philox row of the group draws)
  float invT;
  int want_stats;     // row lse (and, with sample, the group draws)
  int want_argmax;
  int sample;
  uint64_t seed, offset;
  float* zout;        // nullable [M, zout_ld]
  int64_t zout_ld;
  Partial* partials;  // [M, partials_ld], one per workgroup; nullable when no stats are wanted
  int64_t partials_ld;
  uint32_t* hist;     // nullable (with zout, M <= kTileHistRows): [M, 4096] counts of the top 12
                      // bits of each score's order key, added to (cleared by the caller)
  float* gz;          // nullable, sampling mode of the K-chunked pass, and of the tile pass with at
  int64_t gz_ld;      // most kTileSideMaxRows rows: [M, gz_ld, 64] raw logits of each row's best
                      // group of each workgroup
};
constexpr int kTileSideMaxRows = 16;   // rows whose best-group logits the tile pass keeps
constexpr int kTileMaxGrid = 256;      // workgroups of a tile pass at most (the side buffer's gz_ld)
constexpr int kTileHistRows = 2;
bool head_tile_supported(int64_t M, int64_t K, int64_t V, bool bf16, int64_t ld = 0);

// workgroups of a tile pass over V rows for passes of up to M activation rows
int head_tile_grid(int64_t M, int64_t K, int64_t V);
hipError_t launch_head_tile(const TileArgs& a, int grid, hipStream_t st);

// Wide-batch pass (bf16 rows of at most 512 elements, kTileMaxRows < M <= kWideMaxRows): the
// same contract as the tile pass (Partials only, no raw scores)
constexpr int kWideMaxRows = 256;
bool head_wide_supported(int64_t M, int64_t K, int64_t V, bool bf16, int64_t ld = 0);
int head_wide_grid(int64_t V);
hipError_t launch_head_wide(const TileArgs& a, int grid, hipStream_t st);
// K-chunked pass (bf16 rows of more than 512 elements, M <= kTileMaxRows, no row stride): the
// same contract as the tile pass (Partials only, no raw scores).  Workgroup b owns groups
// [b NG / grid, (b + 1) NG / grid) and, in sampling mode, writes the logits of each row's best
// group among them to gz[m, b, :].
constexpr int kKcMaxGroups = 8;   // groups a workgroup owns at most
bool head_kchunk_supported(int64_t M, int64_t K, int64_t V, bool bf16);
int head_kchunk_grid(int64_t V);
// bytes of the side buffer gz for any grid head_kchunk_grid returns (0: the pass does not apply)
size_t head_kchunk_side_bytes(int64_t M, int64_t K, int64_t V);
hipError_t launch_head_kchunk(const TileArgs& a, int grid, hipStream_t st);
// per row: merge the Partials, greedy token or the two-level draw (recomputing the winning group)
hipError_t launch_head_fin(const FinalizeArgs& f, hipStream_t st);

struct DeviceInfo {
  int cus;
  int max_lds;   // bytes of dynamic LDS a workgroup may use
};
hipError_t device_info(DeviceInfo* out);

// h_out[m, j] = round_dtype(sum_k Wd[j, k] x[m, k]), j < R; also clears zero[0, zero_words).
// bf16 runs split over K on MFMA and needs rowdot_scratch_bytes(M, R, K) of fp32 scratch.
size_t rowdot_scratch_bytes(int64_t M, int64_t R, int64_t K);
hipError_t launch_rowdot(const void* Wd, const void* x, int64_t R, int64_t K, int64_t M, bool bf16,
                         void* out, float* scratch, hipStream_t st, uint32_t* zero = nullptr,
                         int64_t zero_words = 0);
// bf16, M <= kRowdotRanksMaxM: as launch_rowdot, but row m keeps only its first ranks[m]
// outputs (the rest are written as zero); ranks is a host array
constexpr int kRowdotRanksMaxM = 64;
hipError_t launch_rowdot_ranked(const void* Wd, const void* x, int64_t R, int64_t K, int64_t M,
                                const int32_t* ranks, void* out, hipStream_t st);
// Chooses the VALU (skinny) or MFMA path; returns the number of producer workgroups.
hipError_t launch_stream(const StreamArgs& a, bool use_mfma, int* producers, hipStream_t st);
hipError_t launch_head_finalize(const FinalizeArgs& f, hipStream_t st);

// SpecVocab pieces
// Top-k of [M, V] float scores.  hist, count and hist2 (contiguous, topk_counter_words(M)
// words from hist) must be zero when the top-k kernels start; cand and mask are scratch.
struct TopkArgs {
  const float* scores;  // [M, V]
  int64_t V;
  int k;
  int M;
  int chunks;           // topk_chunks(V) workgroups per row
  uint32_t* hist;       // [M, 4096] key bits 31..20 of every score
  uint32_t* count;      // [M, kTkCounterStride] (one 128-byte line per row)
  uint32_t* hist2;      // [M, 4096] key bits 19..8 of the scores in the threshold bin
  uint2* cand;          // [M, V]
  uint64_t* mask;       // [M, ceil(V / 64)]
  int32_t* out;         // [M, k] ascending ids
  bool hist_ready;      // the row histograms are already built (by the scorer)
};
constexpr int64_t kTopkMaxV = int64_t{1} << 19;  // finishing bitmasks live in LDS
int topk_chunks(int64_t V);
constexpr int kTkCounterStride = 32;
inline int64_t topk_counter_words(int64_t M) { return M * 4096 * 2 + M * kTkCounterStride; }
hipError_t launch_zero(uint32_t* p, int64_t words, hipStream_t st);
size_t topk_finish_lds(int64_t V);
hipError_t launch_topk(const TopkArgs& a, hipStream_t st);
// exact logits of the gathered candidates, then (by the workgroup finishing each row) the
// softmax over the k candidates and the token; counters [M, kTkCounterStride] zero on entry
hipError_t launch_gather_select(const void* U, const void* h, const int32_t* idx, int64_t M, int64_t d, int64_t V,
                                int64_t k, bool bf16, float* zbuf, int mode, float invT, uint64_t seed,
                                uint64_t offset, float* topk_logit, float* topk_prob, int32_t* token, float* lse,
                                float* logprob, uint32_t* counters, hipStream_t st);

// verification
// mode 0 greedy, 1 sampling against dense draft logits, 2 sampling against a sparse draft
// distribution (q given on a candidate set per position, zero elsewhere)
struct VerifyArgs {
  int mode;
  int64_t B, gamma, V;
  bool bf16;
  const void* target;
  const void* draft;
  const int32_t* tokens;
  const float* u;
  float invT;
  uint64_t seed, offset;
  int32_t* accept_len;
  int32_t* out_tokens;
  Partial* partials;   // [B, rows, S] row-segment partials
  int S;
  Partial* partials2;  // [B, S2 + 1]: residual-segment records, then the acceptance record (sampling)
  int S2;
  const int32_t* qidx;  // mode 2: [B, gamma, k] candidate ids (distinct)
  const float* qprob;   // mode 2: [B, gamma, k] their draft probabilities
  int64_t k;
  const int32_t* parent;  // tree verification: [B, gamma + 1] parent of each node
  int32_t* accept_node;   // tree verification: [B] deepest accepted node
};
// target rows + (mode 1) draft rows per sequence
__host__ __device__ inline int64_t verify_rows_per_seq(int mode, int64_t gamma) { return mode == 1 ? 2 * gamma + 1 : gamma + 1; }
int verify_segments(int64_t B, int64_t gamma, int64_t V, int mode);
int verify_resid_segments(int64_t B, int64_t V, int mode);
hipError_t launch_verify(const VerifyArgs& a, hipStream_t st);
// greedy verification of a candidate tree of gamma + 1 nodes per sequence (mode 0 rows)
constexpr int kMaxTreeNodes = 1024;
hipError_t launch_verify_tree(const VerifyArgs& a, hipStream_t st);

// measurement helper: XOR of every 32-bit word of buf[0, bytes) into *sink (bytes a multiple of 16,
// at most 0xFFFFFFF0), read in the flat grid-stride order
hipError_t launch_read_probe(const void* buf, uint64_t bytes, uint32_t* sink, hipStream_t st);
hipError_t launch_philox(uint64_t seed, uint64_t offset, uint32_t purpose, int64_t rows, int64_t n,
                         float* out, hipStream_t st);

}  // namespace sh
