// C ABI of libspechead: argument validation (host only, before any HIP call), workspace
// carving and the kernel sequence of each call.  Declarations and contracts: spechead.h.
#include <cmath>
#include <cstdint>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>
#include <utility>

#include "../../include/spechead.h"
#include "device_common.h"
#include "launch.h"

// Scratch of draft_head_lowrank_noalloc: one array per GPU, held until the process ends.
constexpr size_t kNoallocScratchBytes = size_t{8} << 20;
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int hip_fail(hipError_t e, const char* where) {
  return fail(SH_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

constexpr int64_t kMaxV = (int64_t{1} << 31) - 64;
constexpr int64_t kMaxRowBytes = 16 * 1024;     // d * esize for the row-dot and gather kernels
constexpr int64_t kMaxK = 16384;
constexpr int64_t kMaxGamma = 64;
constexpr int kValuMaxRows = 8;                 // skinny path up to this many rows
constexpr int kMfmaMaxRows = 192;               // rows per MFMA pass (6 column blocks, no spills)

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
size_t esize(int dtype) { return dtype == SH_BF16 ? 2 : 4; }

int check_dtype_mode(int dtype, int mode) {
  if (dtype != SH_F32 && dtype != SH_BF16) return fail(SH_ERR_DTYPE, "unknown dtype %d", dtype);
  if (mode != SH_GREEDY && mode != SH_SAMPLE) return fail(SH_ERR_DTYPE, "unknown mode %d", mode);
  return SH_OK;
}

int check_temperature(float T) {
  if (!(T > 0.f) || !std::isfinite(T)) return fail(SH_ERR_PARAM, "temperature must be > 0 and finite");
  return SH_OK;
}

int check_rowlen(const char* name, int64_t n, int dtype) {
  if (n < 1) return fail(SH_ERR_SHAPE, "%s must be >= 1", name);
  if ((n * static_cast<int64_t>(esize(dtype))) % 16 != 0)
    return fail(SH_ERR_SHAPE, "%s * element size must be a multiple of 16 bytes (got %lld)", name,
                static_cast<long long>(n));
  return SH_OK;
}

int check_ptr(const void* p, const char* name) {
  if (p == nullptr) return fail(SH_ERR_NULL, "%s is NULL", name);
  if (!aligned(p, 16)) return fail(SH_ERR_ALIGN, "%s is not 16-byte aligned", name);
  return SH_OK;
}
int check_out(const void* p, const char* name) {
  if (p == nullptr) return fail(SH_ERR_NULL, "%s is NULL", name);
  if (!aligned(p, 4)) return fail(SH_ERR_ALIGN, "%s is not 4-byte aligned", name);
  return SH_OK;
}
int check_opt_out(const void* p, const char* name) {
  if (p != nullptr && !aligned(p, 4)) return fail(SH_ERR_ALIGN, "%s is not 4-byte aligned", name);
  return SH_OK;
}

// Top-k scratch: the counter block (cleared at the start of each call) first, then the
// candidates and the bitmask.
struct TopkLayout {
  size_t hist_off, count_off, hist2_off, cand_off, mask_off, total;
};

TopkLayout topk_layout(int64_t M, int64_t V) {
  TopkLayout L{};
  size_t off = 0;
  L.hist_off = off;
  off += static_cast<size_t>(M) * 4096 * 4;
  L.count_off = off;
  off += static_cast<size_t>(M) * sh::kTkCounterStride * 4;
  L.hist2_off = off;   // (hist, count and hist2 are one block the call clears)
  off = align_up(off + static_cast<size_t>(M) * 4096 * 4, 256);
  L.cand_off = off;
  off = align_up(off + static_cast<size_t>(M * V) * 8, 256);
  L.mask_off = off;
  off = align_up(off + static_cast<size_t>(M) * static_cast<size_t>((V + 63) / 64) * 8, 256);
  L.total = off;
  return L;
}

sh::TopkArgs topk_args(void* ws, const TopkLayout& L, const float* scores, int64_t M, int64_t V,
                       int64_t k, int32_t* out) {
  char* b = static_cast<char*>(ws);
  sh::TopkArgs a{};
  a.scores = scores;
  a.V = V;
  a.k = static_cast<int>(k);
  a.M = static_cast<int>(M);
  a.chunks = sh::topk_chunks(V);
  a.hist = reinterpret_cast<uint32_t*>(b + L.hist_off);
  a.count = reinterpret_cast<uint32_t*>(b + L.count_off);
  a.hist2 = reinterpret_cast<uint32_t*>(b + L.hist2_off);
  a.cand = reinterpret_cast<uint2*>(b + L.cand_off);
  a.mask = reinterpret_cast<uint64_t*>(b + L.mask_off);
  a.out = out;
  return a;
}

// group log-sum-exp rows are padded to a multiple of 4 groups (16-byte aligned quads)
int64_t lg_stride(int64_t V) { return ((V + sh::kGroup - 1) / sh::kGroup + 3) / 4 * 4; }

struct HeadLayout {
  size_t tk_off, tk_bytes;   // SpecVocab: the top-k block, at offset 0
  size_t rd_off, rd_bytes;   // fp32 split-K partials of the down-projection
  size_t hr_off, hr_bytes;
  size_t part_off, part_bytes;
  size_t lg_off, lg_bytes;
  size_t gz_off, gz_bytes;     // dense: the K-chunked pass's best-group logits
  size_t score_off, score_bytes;
  size_t z_off, z_bytes;
  size_t total;
};

HeadLayout head_layout(int op, int64_t M, int64_t d, int64_t r, int64_t V, int64_t k, int dtype) {
  HeadLayout L{};
  size_t off = 0;
  L.tk_off = off;
  L.tk_bytes = (op == SH_OP_SPECVOCAB) ? topk_layout(M, V).total : 0;
  off += L.tk_bytes;
  L.rd_off = off;
  L.rd_bytes = (op == SH_OP_DENSE) ? 0 : align_up(sh::rowdot_scratch_bytes(M, r, d), 256);
  off += L.rd_bytes;
  L.hr_off = off;
  L.hr_bytes = (op == SH_OP_DENSE) ? 0 : align_up(static_cast<size_t>(M * r) * esize(dtype), 256);
  off += L.hr_bytes;
  L.part_off = off;
  L.part_bytes = (op == SH_OP_SPECVOCAB) ? 0 : align_up(static_cast<size_t>(M) * sh::kMaxPartials * sizeof(sh::Partial), 256);
  off += L.part_bytes;
  L.lg_off = off;
  L.lg_bytes = (op == SH_OP_SPECVOCAB) ? 0 : align_up(static_cast<size_t>(M) * static_cast<size_t>(lg_stride(V)) * 4, 256);
  off += L.lg_bytes;
  L.gz_off = off;
  // best-group logits: the dense head's K-chunked pass, or the low-rank head's tile pass with at
  // most kTileSideMaxRows rows (one slot per workgroup of at most kTileMaxGrid)
  L.gz_bytes = (op == SH_OP_DENSE) ? align_up(sh::head_kchunk_side_bytes(M, d, V), 256)
               : (op == SH_OP_LOWRANK && M <= sh::kTileSideMaxRows)
                   ? align_up(static_cast<size_t>(M) * sh::kTileMaxGrid * sh::kGroup * sizeof(float), 256)
                   : 0;
  off += L.gz_bytes;
  L.score_off = off;
  L.score_bytes = (op == SH_OP_SPECVOCAB) ? align_up(static_cast<size_t>(M * V) * 4, 256) : 0;
  off += L.score_bytes;
  L.z_off = off;
  L.z_bytes = (op == SH_OP_SPECVOCAB) ? align_up(static_cast<size_t>(M * k) * 4, 256) : 0;
  off += L.z_bytes;
  L.total = off;
  return L;
}

// Verification scratch: row-segment partials, then residual-segment partials.
struct VerifyLayout {
  size_t part_off, part2_off, total;
  int S, S2;
};

// kind: 0 greedy, 1 sampling against draft logits, 2 sampling against a sparse draft
VerifyLayout verify_layout(int kind, int64_t B, int64_t gamma, int64_t V) {
  VerifyLayout L{};
  const int mode = kind;
  const int64_t R = sh::verify_rows_per_seq(kind, gamma);
  L.S = sh::verify_segments(B, gamma, V, mode);
  L.S2 = sh::verify_resid_segments(B, V, mode);
  size_t off = 0;
  L.part_off = off;
  off = align_up(off + static_cast<size_t>(B * R * L.S) * sizeof(sh::Partial), 256);
  L.part2_off = off;
  // per sequence: S2 residual-segment records and one acceptance record
  off = align_up(off + static_cast<size_t>(B * (L.S2 + 1)) * sizeof(sh::Partial), 256);
  L.total = off;
  return L;
}

int check_workspace(void* ws, size_t have, size_t need) {
  if (need == 0) return SH_OK;
  if (ws == nullptr) return fail(SH_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
  if (!aligned(ws, 256)) return fail(SH_ERR_ALIGN, "workspace is not 256-byte aligned");
  if (have < need) return fail(SH_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", have, need);
  return SH_OK;
}

#define SH_TRY(expr)              \
  do {                            \
    const int _rc = (expr);       \
    if (_rc != SH_OK) return _rc; \
  } while (0)

#define SH_HIP(expr, where)                      \
  do {                                           \
    const hipError_t _e = (expr);                \
    if (_e != hipSuccess) return hip_fail(_e, where); \
  } while (0)

// Stream z = W x over V rows for M rows of x, then finalize selection.  Shared by the dense
// and low-rank heads.  lg: [M][ceil(V/64)] group log-sum-exps, partials: [M][kMaxPartials].
// ld: row stride of W and x in elements when only the first K elements of each row are used
// (0: rows of K elements); a stride other than K needs the tile path.
int run_head(const void* x, int64_t M, int64_t K, const void* W, int64_t V, int dtype, int mode,
             float temperature, uint64_t seed, uint64_t offset, int32_t* token, float* lse,
             float* logprob, float* logits, sh::Partial* partials, float* lg, hipStream_t st,
             int64_t ld = 0, const int32_t* id_map = nullptr, float* gz = nullptr) {
  const bool bf16 = dtype == SH_BF16;
  const float invT = 1.0f / temperature;
  const bool want_lg = mode == SH_SAMPLE || lse != nullptr || logprob != nullptr;
  if (ld != 0 && ld != K && !sh::head_tile_supported(M, K, V, bf16, ld))
    return fail(SH_ERR_UNSUPPORTED, "row prefixes need the tile path");
  if (sh::head_tile_supported(M, K, V, bf16, ld)) {
    // short bf16 rows, at most kTileMaxRows activation rows: one tile-streaming pass with
    // in-kernel group draws, then the finalize
    const int grid = sh::head_tile_grid(M, K, V);
    sh::TileArgs a{};
    a.W = W;
    a.x = x;
    a.V = V;
    a.K = static_cast<int>(K);
    a.ld = static_cast<int>(ld);
    a.M = static_cast<int>(M);
    a.row0 = 0;
    a.invT = invT;
    a.want_stats = want_lg ? 1 : 0;
    a.want_argmax = mode == SH_GREEDY ? 1 : 0;
    a.sample = mode == SH_SAMPLE ? 1 : 0;
    a.seed = seed;
    a.offset = offset;
    a.zout = logits;
    a.zout_ld = V;
    a.partials = partials;
    a.partials_ld = sh::kMaxPartials;
    // sampling without raw logits: the pass keeps each workgroup's best-group logits per row
    const bool side = gz != nullptr && mode == SH_SAMPLE && logits == nullptr && M <= sh::kTileSideMaxRows &&
                      grid <= sh::kTileMaxGrid;
    if (side) {
      a.gz = gz;
      a.gz_ld = sh::kTileMaxGrid;
    }
    SH_HIP(sh::launch_head_tile(a, grid, st), "head tile kernel");
    sh::FinalizeArgs f{};
    f.partials = partials;
    f.partials_ld = sh::kMaxPartials;
    f.P = grid;
    f.W = W;
    f.x = x;
    f.V = V;
    f.K = K;
    f.ld = ld;
    f.M = static_cast<int>(M);
    f.bf16 = true;
    f.mode = mode == SH_SAMPLE ? 1 : 0;
    f.invT = invT;
    f.seed = seed;
    f.offset = offset;
    f.token = token;
    f.lse = lse;
    f.logprob = logprob;
    f.id_map = id_map;
    if (side) {
      f.gz = gz;
      f.gz_ld = sh::kTileMaxGrid;
      f.gz_map = 1;
    }
    SH_HIP(sh::launch_head_fin(f, st), "head finalize kernel");
    return SH_OK;
  }
  const bool kchunk = logits == nullptr && (ld == 0 || ld == K) && sh::head_kchunk_supported(M, K, V, bf16);
  if (kchunk || (logits == nullptr && sh::head_wide_supported(M, K, V, bf16, ld))) {
    // long rows (K-chunked pass) or more rows than the tile pass holds (wide pass): one pass
    // with in-kernel group draws, then the finalize
    const int grid = kchunk ? sh::head_kchunk_grid(V) : sh::head_wide_grid(V);
    sh::TileArgs a{};
    a.W = W;
    a.x = x;
    a.V = V;
    a.K = static_cast<int>(K);
    a.ld = static_cast<int>(ld);
    a.M = static_cast<int>(M);
    a.row0 = 0;
    a.invT = invT;
    a.want_stats = want_lg ? 1 : 0;
    a.want_argmax = mode == SH_GREEDY ? 1 : 0;
    a.sample = mode == SH_SAMPLE ? 1 : 0;
    a.seed = seed;
    a.offset = offset;
    a.partials = partials;
    a.partials_ld = sh::kMaxPartials;
    if (kchunk) {
      a.ld = 0;
      a.gz = gz;
      a.gz_ld = grid;
      SH_HIP(sh::launch_head_kchunk(a, grid, st), "head K-chunked kernel");
    } else {
      SH_HIP(sh::launch_head_wide(a, grid, st), "head wide kernel");
    }
    sh::FinalizeArgs f{};
    f.partials = partials;
    f.partials_ld = sh::kMaxPartials;
    f.P = grid;
    f.W = W;
    f.x = x;
    f.V = V;
    f.K = K;
    f.ld = ld;
    f.M = static_cast<int>(M);
    f.bf16 = true;
    f.mode = mode == SH_SAMPLE ? 1 : 0;
    f.invT = invT;
    f.seed = seed;
    f.offset = offset;
    f.token = token;
    f.lse = lse;
    f.logprob = logprob;
    f.id_map = id_map;
    if (kchunk) {
      f.gz = gz;
      f.gz_ld = grid;
    }
    SH_HIP(sh::launch_head_fin(f, st), "head finalize kernel");
    return SH_OK;
  }
  const bool mfma = bf16 && M > kValuMaxRows;
  const int64_t chunk = mfma ? kMfmaMaxRows : kValuMaxRows;
  int producers = 0;
  for (int64_t m0 = 0; m0 < M; m0 += chunk) {
    const int64_t mc = (M - m0) < chunk ? (M - m0) : chunk;
    sh::StreamArgs a{};
    a.W = W;
    a.x = static_cast<const char*>(x) + static_cast<size_t>(m0 * K) * esize(dtype);
    a.V = V;
    a.K = K;
    a.M = static_cast<int>(mc);
    a.bf16 = bf16;
    a.want_argmax = mode == SH_GREEDY;
    a.invT = invT;
    a.zout = logits ? logits + m0 * V : nullptr;
    a.zout_ld = V;
    a.lg = want_lg ? lg + m0 * lg_stride(V) : nullptr;
    a.lg_ld = lg_stride(V);
    a.partials = partials + m0 * sh::kMaxPartials;
    a.partials_ld = sh::kMaxPartials;
    int p = 0;
    SH_HIP(sh::launch_stream(a, mfma, &p, st), "head stream kernel");
    producers = p;
  }
  sh::FinalizeArgs f{};
  f.partials = partials;
  f.partials_ld = sh::kMaxPartials;
  f.P = producers;
  f.lg = lg;
  f.lg_ld = lg_stride(V);
  f.W = W;
  f.x = x;
  f.V = V;
  f.K = K;
  f.M = static_cast<int>(M);
  f.bf16 = bf16;
  f.mode = mode == SH_SAMPLE ? 1 : 0;
  f.invT = invT;
  f.seed = seed;
  f.offset = offset;
  f.token = token;
  f.lse = lse;
  f.logprob = logprob;
  f.id_map = id_map;
  SH_HIP(sh::launch_head_finalize(f, st), "head finalize kernel");
  return SH_OK;
}

int check_common_head(const void* h, int64_t M, int64_t d, int64_t V, int dtype, int mode,
                      float temperature, int32_t* token, float* lse, float* logprob) {
  SH_TRY(check_dtype_mode(dtype, mode));
  SH_TRY(check_temperature(temperature));
  SH_TRY(check_ptr(h, "h"));
  if (M < 1 || M > (int64_t{1} << 20)) return fail(SH_ERR_SHAPE, "M must be in [1, 2^20]");
  SH_TRY(check_rowlen("d", d, dtype));
  if (d * static_cast<int64_t>(esize(dtype)) > kMaxRowBytes)
    return fail(SH_ERR_UNSUPPORTED, "d * element size above %lld bytes", static_cast<long long>(kMaxRowBytes));
  if (V < 1 || V > kMaxV) return fail(SH_ERR_SHAPE, "V must be in [1, 2^31 - 64]");
  SH_TRY(check_out(token, "token"));
  SH_TRY(check_opt_out(lse, "lse"));
  SH_TRY(check_opt_out(logprob, "logprob"));
  return SH_OK;
}

int check_lowrank_args(const void* h, int64_t M, int64_t d, const void* W_down, int64_t r, const void* W_up,
                       int64_t V, int dtype, int mode, float temperature, int32_t* token, float* lse,
                       float* logprob, float* logits) {
  SH_TRY(check_common_head(h, M, d, V, dtype, mode, temperature, token, lse, logprob));
  SH_TRY(check_ptr(W_down, "W_down"));
  SH_TRY(check_ptr(W_up, "W_up"));
  SH_TRY(check_rowlen("r", r, dtype));
  if (r * static_cast<int64_t>(esize(dtype)) > kMaxRowBytes)
    return fail(SH_ERR_UNSUPPORTED, "r * element size above %lld bytes", static_cast<long long>(kMaxRowBytes));
  SH_TRY(check_opt_out(logits, "logits"));
  return SH_OK;
}

// The low-rank call on a validated scratch area laid out as L (a caller workspace or the
// static scratch below): h_r = round(W_down h), then the head over W_up.
int run_lowrank(const void* h, int64_t M, int64_t d, const void* W_down, int64_t r, const void* W_up, int64_t V,
                int dtype, int mode, float temperature, uint64_t seed, uint64_t offset, int32_t* token, float* lse,
                float* logprob, float* logits, char* ws, const HeadLayout& L, hipStream_t st) {
  void* hr = ws + L.hr_off;
  auto* parts = reinterpret_cast<sh::Partial*>(ws + L.part_off);
  auto* lg = reinterpret_cast<float*>(ws + L.lg_off);
  SH_HIP(sh::launch_rowdot(W_down, h, r, d, M, dtype == SH_BF16, hr, reinterpret_cast<float*>(ws + L.rd_off), st),
         "down-projection kernels");
  auto* gz = L.gz_bytes ? reinterpret_cast<float*>(ws + L.gz_off) : nullptr;
  return run_head(hr, M, r, W_up, V, dtype, mode, temperature, seed, offset, token, lse, logprob,
                  logits, parts, lg, st, 0, nullptr, gz);
}

// Device address of the static scratch on the current device, looked up once per device
// with that device current.  In host code the array's name stands for a host-side shadow,
// never the device memory: kernels only ever receive the looked-up address.
std::mutex g_scratch_mu;
char* g_scratch_ptr[kMaxDevices] = {};

int noalloc_scratch(char** out) {
  int dev = 0;
  SH_HIP(hipGetDevice(&dev), "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(SH_ERR_UNSUPPORTED, "device index %d above %d", dev, kMaxDevices - 1);
  std::lock_guard<std::mutex> g(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    SH_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
    if (p == nullptr) return fail(SH_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = static_cast<char*>(p);
  }
  *out = g_scratch_ptr[dev];
  return SH_OK;
}

}  // namespace

extern "C" {

const char* sh_status_str(int status) {
  switch (status) {
    case SH_OK: return "ok";
    case SH_ERR_NULL: return "null pointer";
    case SH_ERR_SHAPE: return "bad shape";
    case SH_ERR_DTYPE: return "bad dtype or mode";
    case SH_ERR_ALIGN: return "misaligned pointer";
    case SH_ERR_WORKSPACE: return "workspace missing or too small";
    case SH_ERR_PARAM: return "bad parameter";
    case SH_ERR_UNSUPPORTED: return "unsupported";
    case SH_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

const char* sh_last_error(void) { return g_last_error.c_str(); }

size_t sh_head_workspace_bytes(int op, int64_t M, int64_t d, int64_t r, int64_t V, int64_t k) {
  if (M < 1 || d < 1 || V < 1) return 0;
  if (op == SH_OP_DENSE) r = 0;
  else if (r < 1) return 0;
  if (op == SH_OP_SPECVOCAB && (k < 1 || k > V)) return 0;
  if (op != SH_OP_DENSE && op != SH_OP_LOWRANK && op != SH_OP_SPECVOCAB) return 0;
  // sized for f32 intermediates so one workspace serves both dtypes
  return head_layout(op, M, d, r, V, k, SH_F32).total;
}

size_t sh_head_intermediate_offset(int op, int64_t M, int64_t d, int64_t r, int64_t V, int64_t k) {
  if (op != SH_OP_LOWRANK && op != SH_OP_SPECVOCAB) return SIZE_MAX;
  if (sh_head_workspace_bytes(op, M, d, r, V, k) == 0) return SIZE_MAX;
  return head_layout(op, M, d, r, V, k, SH_F32).hr_off;
}

size_t sh_verify_workspace_bytes(int mode, int64_t B, int64_t gamma, int64_t V) {
  if ((mode != SH_GREEDY && mode != SH_SAMPLE) || B < 1 || gamma < 1 || V < 1) return 0;
  return verify_layout(mode, B, gamma, V).total;
}

size_t sh_verify_tree_workspace_bytes(int64_t B, int64_t N, int64_t V) {
  if (B < 1 || N < 1 || N > sh::kMaxTreeNodes || V < 1) return 0;
  return verify_layout(0, B, N - 1, V).total;
}

size_t sh_verify_sparse_workspace_bytes(int64_t B, int64_t gamma, int64_t V, int64_t k) {
  if (B < 1 || gamma < 1 || V < 1 || k < 1 || k > V) return 0;
  return verify_layout(2, B, gamma, V).total;
}

size_t sh_topk_workspace_bytes(int64_t M, int64_t V, int64_t k) {
  if (M < 1 || V < 1 || k < 1 || k > V) return 0;
  return topk_layout(M, V).total;
}

int draft_head_dense(const void* h, int64_t M, int64_t d, const void* W, int64_t V, int dtype,
                     int mode, float temperature, uint64_t seed, uint64_t offset, int32_t* token,
                     float* lse, float* logprob, float* logits, void* workspace,
                     size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  SH_TRY(check_common_head(h, M, d, V, dtype, mode, temperature, token, lse, logprob));
  SH_TRY(check_ptr(W, "W"));
  SH_TRY(check_opt_out(logits, "logits"));
  const HeadLayout L = head_layout(SH_OP_DENSE, M, d, 0, V, 0, SH_F32);
  SH_TRY(check_workspace(workspace, workspace_bytes, L.total));
  hipStream_t st = static_cast<hipStream_t>(stream);
  auto* parts = reinterpret_cast<sh::Partial*>(static_cast<char*>(workspace) + L.part_off);
  auto* lg = reinterpret_cast<float*>(static_cast<char*>(workspace) + L.lg_off);
  auto* gz = L.gz_bytes ? reinterpret_cast<float*>(static_cast<char*>(workspace) + L.gz_off) : nullptr;
  return run_head(h, M, d, W, V, dtype, mode, temperature, seed, offset, token, lse, logprob,
                  logits, parts, lg, st, 0, nullptr, gz);
}

int draft_head_trimmed(const void* h, int64_t M, int64_t d, const void* W_S, int64_t n_S, const int32_t* ids,
                       int dtype, int mode, float temperature, uint64_t seed, uint64_t offset, int32_t* token,
                       float* lse, float* logprob, float* logits, void* workspace, size_t workspace_bytes,
                       void* stream) {
  g_last_error.clear();
  SH_TRY(check_common_head(h, M, d, n_S, dtype, mode, temperature, token, lse, logprob));
  SH_TRY(check_ptr(W_S, "W_S"));
  if (ids == nullptr) return fail(SH_ERR_NULL, "ids is NULL");
  if (!aligned(ids, 4)) return fail(SH_ERR_ALIGN, "ids is not 4-byte aligned");
  SH_TRY(check_opt_out(logits, "logits"));
  const HeadLayout L = head_layout(SH_OP_DENSE, M, d, 0, n_S, 0, SH_F32);
  SH_TRY(check_workspace(workspace, workspace_bytes, L.total));
  hipStream_t st = static_cast<hipStream_t>(stream);
  auto* parts = reinterpret_cast<sh::Partial*>(static_cast<char*>(workspace) + L.part_off);
  auto* lg = reinterpret_cast<float*>(static_cast<char*>(workspace) + L.lg_off);
  auto* gz = L.gz_bytes ? reinterpret_cast<float*>(static_cast<char*>(workspace) + L.gz_off) : nullptr;
  return run_head(h, M, d, W_S, n_S, dtype, mode, temperature, seed, offset, token, lse, logprob, logits, parts, lg,
                  st, 0, ids, gz);
}

int draft_head_lowrank(const void* h, int64_t M, int64_t d, const void* W_down, int64_t r,
                       const void* W_up, int64_t V, int dtype, int mode, float temperature,
                       uint64_t seed, uint64_t offset, int32_t* token, float* lse, float* logprob,
                       float* logits, void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  SH_TRY(check_lowrank_args(h, M, d, W_down, r, W_up, V, dtype, mode, temperature, token, lse, logprob, logits));
  const HeadLayout L = head_layout(SH_OP_LOWRANK, M, d, r, V, 0, SH_F32);
  SH_TRY(check_workspace(workspace, workspace_bytes, L.total));
  return run_lowrank(h, M, d, W_down, r, W_up, V, dtype, mode, temperature, seed, offset, token, lse, logprob,
                     logits, static_cast<char*>(workspace), L, static_cast<hipStream_t>(stream));
}

int draft_head_lowrank_noalloc(const void* h, int64_t M, int64_t d, const void* W_down, int64_t r,
                               const void* W_up, int64_t V, int dtype, int mode, float temperature,
                               uint64_t seed, uint64_t offset, int32_t* token, float* lse, float* logprob,
                               float* logits, void* stream) {
  g_last_error.clear();
  SH_TRY(check_lowrank_args(h, M, d, W_down, r, W_up, V, dtype, mode, temperature, token, lse, logprob, logits));
  const HeadLayout L = head_layout(SH_OP_LOWRANK, M, d, r, V, 0, SH_F32);
  if (L.total > kNoallocScratchBytes)
    return fail(SH_ERR_UNSUPPORTED, "the call needs %zu bytes of scratch, above the %zu-byte static scratch", L.total,
                kNoallocScratchBytes);
  char* ws = nullptr;
  SH_TRY(noalloc_scratch(&ws));
  return run_lowrank(h, M, d, W_down, r, W_up, V, dtype, mode, temperature, seed, offset, token, lse, logprob,
                     logits, ws, L, static_cast<hipStream_t>(stream));
}

int draft_head_lowrank_adaptive(const void* h, int64_t M, int64_t d, const void* W_down, int64_t r_max,
                                const void* W_up, int64_t V, const int32_t* ranks, int dtype, int mode,
                                float temperature, uint64_t seed, uint64_t offset, int32_t* token, float* lse,
                                float* logprob, float* logits, void* workspace, size_t workspace_bytes,
                                void* stream) {
  g_last_error.clear();
  SH_TRY(check_common_head(h, M, d, V, dtype, mode, temperature, token, lse, logprob));
  SH_TRY(check_ptr(W_down, "W_down"));
  SH_TRY(check_ptr(W_up, "W_up"));
  SH_TRY(check_rowlen("r_max", r_max, dtype));
  SH_TRY(check_opt_out(logits, "logits"));
  if (ranks == nullptr) return fail(SH_ERR_NULL, "ranks is NULL");
  if (dtype != SH_BF16) return fail(SH_ERR_UNSUPPORTED, "position-adaptive rank needs bf16");
  if (M > sh::kRowdotRanksMaxM) return fail(SH_ERR_UNSUPPORTED, "M above %d", sh::kRowdotRanksMaxM);
  int64_t rmax_used = 0;
  for (int64_t m = 0; m < M; ++m) {
    if (ranks[m] < 1 || ranks[m] > r_max) return fail(SH_ERR_PARAM, "ranks[%lld] not in [1, r_max]", static_cast<long long>(m));
    rmax_used = ranks[m] > rmax_used ? ranks[m] : rmax_used;
  }
  // columns read: the largest rank rounded up to 128 (the tile pass's row lengths), or r_max
  int64_t K = (rmax_used + 127) / 128 * 128;
  if (K > r_max) K = r_max;
  if (!sh::head_tile_supported(M, K, V, true, r_max))
    return fail(SH_ERR_UNSUPPORTED, "shape outside the tile pass (r_max %lld, columns %lld)",
                static_cast<long long>(r_max), static_cast<long long>(K));
  const HeadLayout L = head_layout(SH_OP_LOWRANK, M, d, r_max, V, 0, SH_F32);
  SH_TRY(check_workspace(workspace, workspace_bytes, L.total));
  hipStream_t st = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  void* hr = ws + L.hr_off;
  auto* parts = reinterpret_cast<sh::Partial*>(ws + L.part_off);
  auto* lg = reinterpret_cast<float*>(ws + L.lg_off);
  auto* gz = L.gz_bytes ? reinterpret_cast<float*>(ws + L.gz_off) : nullptr;
  SH_HIP(sh::launch_rowdot_ranked(W_down, h, r_max, d, M, ranks, hr, st), "down-projection kernel");
  return run_head(hr, M, K, W_up, V, dtype, mode, temperature, seed, offset, token, lse, logprob, logits, parts,
                  lg, st, r_max, nullptr, gz);
}

int draft_head_specvocab(const void* h, int64_t M, int64_t d, const void* W_down, int64_t dprime,
                         const void* W_vocab, const void* U, int64_t V, int64_t k, int dtype,
                         int mode, float temperature, uint64_t seed, uint64_t offset,
                         int32_t* topk_idx, float* topk_logit, float* topk_prob, int32_t* token,
                         float* lse, float* logprob, void* workspace, size_t workspace_bytes,
                         void* stream) {
  g_last_error.clear();
  SH_TRY(check_common_head(h, M, d, V, dtype, mode, temperature, token, lse, logprob));
  SH_TRY(check_ptr(W_down, "W_down"));
  SH_TRY(check_ptr(W_vocab, "W_vocab"));
  SH_TRY(check_ptr(U, "U"));
  SH_TRY(check_rowlen("dprime", dprime, dtype));
  if (dprime * static_cast<int64_t>(esize(dtype)) > kMaxRowBytes)
    return fail(SH_ERR_UNSUPPORTED, "dprime * element size above %lld bytes", static_cast<long long>(kMaxRowBytes));
  if (k < 1 || k > V) return fail(SH_ERR_PARAM, "k must be in [1, V]");
  if (k > kMaxK) return fail(SH_ERR_UNSUPPORTED, "k above %lld", static_cast<long long>(kMaxK));
  if (V > sh::kTopkMaxV) return fail(SH_ERR_UNSUPPORTED, "V above %lld", static_cast<long long>(sh::kTopkMaxV));
  if (M > 65535) return fail(SH_ERR_UNSUPPORTED, "M above 65535");
  SH_TRY(check_out(topk_idx, "topk_idx"));
  SH_TRY(check_opt_out(topk_logit, "topk_logit"));
  SH_TRY(check_opt_out(topk_prob, "topk_prob"));
  const HeadLayout L = head_layout(SH_OP_SPECVOCAB, M, d, dprime, V, k, SH_F32);
  SH_TRY(check_workspace(workspace, workspace_bytes, L.total));
  hipStream_t st = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  void* hp = ws + L.hr_off;
  float* scores = reinterpret_cast<float*>(ws + L.score_off);
  float* zbuf = reinterpret_cast<float*>(ws + L.z_off);
  const bool bf16 = dtype == SH_BF16;
  const TopkLayout TL = topk_layout(M, V);
  SH_HIP(sh::launch_rowdot(W_down, h, dprime, d, M, bf16, hp, reinterpret_cast<float*>(ws + L.rd_off), st,
                           reinterpret_cast<uint32_t*>(ws + L.tk_off + TL.hist_off), sh::topk_counter_words(M)),
         "reduced-state kernels");
  const bool tile = sh::head_tile_supported(M, dprime, V, bf16);
  const int tile_grid = tile ? sh::head_tile_grid(M, dprime, V) : 0;
  const bool mfma = bf16 && M > kValuMaxRows;
  const int64_t chunk = tile ? M : mfma ? kMfmaMaxRows : kValuMaxRows;
  for (int64_t m0 = 0; m0 < M; m0 += chunk) {
    const int64_t mc = (M - m0) < chunk ? (M - m0) : chunk;
    if (tile) {
      sh::TileArgs a{};
      a.W = W_vocab;
      a.x = static_cast<const char*>(hp) + static_cast<size_t>(m0 * dprime) * 2;
      a.V = V;
      a.K = static_cast<int>(dprime);
      a.M = static_cast<int>(mc);
      a.row0 = static_cast<int>(m0);
      a.invT = 1.f;
      a.zout = scores + m0 * V;
      a.zout_ld = V;
      // a few rows: the scorer also builds the top-k histograms (cleared by the d -> d' kernel)
      if (M <= sh::kTileHistRows) a.hist = reinterpret_cast<uint32_t*>(ws + L.tk_off + TL.hist_off);
      SH_HIP(sh::launch_head_tile(a, tile_grid, st), "approximate scorer kernel");
      continue;
    }
    sh::StreamArgs a{};
    a.W = W_vocab;
    a.x = static_cast<const char*>(hp) + static_cast<size_t>(m0 * dprime) * esize(dtype);
    a.V = V;
    a.K = dprime;
    a.M = static_cast<int>(mc);
    a.bf16 = bf16;
    a.want_argmax = false;
    a.invT = 1.f;
    a.zout = scores + m0 * V;
    a.zout_ld = V;
    a.lg = nullptr;
    a.lg_ld = 0;
    a.partials = nullptr;
    a.partials_ld = 0;
    int p = 0;
    SH_HIP(sh::launch_stream(a, mfma, &p, st), "approximate scorer kernel");
  }
  sh::TopkArgs ta = topk_args(ws + L.tk_off, TL, scores, M, V, k, topk_idx);
  ta.hist_ready = tile && M <= sh::kTileHistRows;
  SH_HIP(sh::launch_topk(ta, st), "top-k kernels");
  SH_HIP(sh::launch_gather_select(U, h, topk_idx, M, d, V, k, bf16, zbuf, mode == SH_SAMPLE ? 1 : 0, 1.0f / temperature,
                                  seed, offset, topk_logit, topk_prob, token, lse, logprob, ta.count, st),
         "gather and candidate softmax kernel");
  return SH_OK;
}

int spec_verify(int mode, int64_t B, int64_t gamma, int64_t V, int dtype, const void* target_logits,
                const void* draft_logits, const int32_t* draft_tokens, const float* u_accept,
                float temperature, uint64_t seed, uint64_t offset, int32_t* accept_len,
                int32_t* out_tokens, void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  SH_TRY(check_dtype_mode(dtype, mode));
  SH_TRY(check_temperature(temperature));
  if (B < 1 || B > (int64_t{1} << 20)) return fail(SH_ERR_SHAPE, "B must be in [1, 2^20]");
  if (gamma < 1 || gamma > kMaxGamma) return fail(SH_ERR_SHAPE, "gamma must be in [1, %lld]", static_cast<long long>(kMaxGamma));
  SH_TRY(check_rowlen("V", V, dtype));
  if (V > (int64_t{1} << 28)) return fail(SH_ERR_SHAPE, "V above 2^28");
  if (B > 65535) return fail(SH_ERR_UNSUPPORTED, "B above 65535");
  SH_TRY(check_ptr(target_logits, "target_logits"));
  if (draft_tokens == nullptr) return fail(SH_ERR_NULL, "draft_tokens is NULL");
  if (!aligned(draft_tokens, 4)) return fail(SH_ERR_ALIGN, "draft_tokens is not 4-byte aligned");
  if (mode == SH_SAMPLE) {
    SH_TRY(check_ptr(draft_logits, "draft_logits"));
    if (u_accept == nullptr) return fail(SH_ERR_NULL, "u_accept is NULL");
    if (!aligned(u_accept, 4)) return fail(SH_ERR_ALIGN, "u_accept is not 4-byte aligned");
  }
  SH_TRY(check_out(accept_len, "accept_len"));
  SH_TRY(check_out(out_tokens, "out_tokens"));
  const size_t need = sh_verify_workspace_bytes(mode, B, gamma, V);
  SH_TRY(check_workspace(workspace, workspace_bytes, need));
  sh::VerifyArgs a{};
  a.mode = mode == SH_SAMPLE ? 1 : 0;
  a.B = B;
  a.gamma = gamma;
  a.V = V;
  a.bf16 = dtype == SH_BF16;
  a.target = target_logits;
  a.draft = draft_logits;
  a.tokens = draft_tokens;
  a.u = u_accept;
  a.invT = 1.0f / temperature;
  a.seed = seed;
  a.offset = offset;
  a.accept_len = accept_len;
  a.out_tokens = out_tokens;
  const VerifyLayout L = verify_layout(mode, B, gamma, V);
  char* ws = static_cast<char*>(workspace);
  a.partials = reinterpret_cast<sh::Partial*>(ws + L.part_off);
  a.S = L.S;
  a.partials2 = reinterpret_cast<sh::Partial*>(ws + L.part2_off);
  a.S2 = L.S2;
  SH_HIP(sh::launch_verify(a, static_cast<hipStream_t>(stream)), "verify kernels");
  return SH_OK;
}

int spec_verify_sparse(int64_t B, int64_t gamma, int64_t V, int64_t k, int dtype, const void* target_logits,
                       const int32_t* draft_idx, const float* draft_prob, const int32_t* draft_tokens,
                       const float* u_accept, float temperature, uint64_t seed, uint64_t offset,
                       int32_t* accept_len, int32_t* out_tokens, void* workspace, size_t workspace_bytes,
                       void* stream) {
  g_last_error.clear();
  SH_TRY(check_dtype_mode(dtype, SH_SAMPLE));
  SH_TRY(check_temperature(temperature));
  if (B < 1 || B > 65535) return fail(SH_ERR_SHAPE, "B must be in [1, 65535]");
  if (gamma < 1 || gamma > kMaxGamma) return fail(SH_ERR_SHAPE, "gamma must be in [1, %lld]", static_cast<long long>(kMaxGamma));
  SH_TRY(check_rowlen("V", V, dtype));
  if (V > (int64_t{1} << 28)) return fail(SH_ERR_SHAPE, "V above 2^28");
  if (k < 1 || k > V) return fail(SH_ERR_PARAM, "k must be in [1, V]");
  if (k > kMaxK) return fail(SH_ERR_UNSUPPORTED, "k above %lld", static_cast<long long>(kMaxK));
  SH_TRY(check_ptr(target_logits, "target_logits"));
  const std::pair<const void*, const char*> small[] = {
      {draft_idx, "draft_idx"}, {draft_prob, "draft_prob"}, {draft_tokens, "draft_tokens"}, {u_accept, "u_accept"}};
  for (const auto& pn : small) {
    if (pn.first == nullptr) return fail(SH_ERR_NULL, "%s is NULL", pn.second);
    if (!aligned(pn.first, 4)) return fail(SH_ERR_ALIGN, "%s is not 4-byte aligned", pn.second);
  }
  SH_TRY(check_out(accept_len, "accept_len"));
  SH_TRY(check_out(out_tokens, "out_tokens"));
  const size_t need = sh_verify_sparse_workspace_bytes(B, gamma, V, k);
  SH_TRY(check_workspace(workspace, workspace_bytes, need));
  sh::VerifyArgs a{};
  a.mode = 2;
  a.B = B;
  a.gamma = gamma;
  a.V = V;
  a.bf16 = dtype == SH_BF16;
  a.target = target_logits;
  a.draft = nullptr;
  a.tokens = draft_tokens;
  a.u = u_accept;
  a.invT = 1.0f / temperature;
  a.seed = seed;
  a.offset = offset;
  a.accept_len = accept_len;
  a.out_tokens = out_tokens;
  a.qidx = draft_idx;
  a.qprob = draft_prob;
  a.k = k;
  const VerifyLayout L = verify_layout(2, B, gamma, V);
  char* ws = static_cast<char*>(workspace);
  a.partials = reinterpret_cast<sh::Partial*>(ws + L.part_off);
  a.S = L.S;
  a.partials2 = reinterpret_cast<sh::Partial*>(ws + L.part2_off);
  a.S2 = L.S2;
  SH_HIP(sh::launch_verify(a, static_cast<hipStream_t>(stream)), "verify kernels");
  return SH_OK;
}

int spec_verify_tree(int64_t B, int64_t N, int64_t V, int dtype, const void* target_logits,
                     const int32_t* node_token, const int32_t* parent, int32_t* accept_len,
                     int32_t* accept_node, int32_t* out_tokens, void* workspace, size_t workspace_bytes,
                     void* stream) {
  g_last_error.clear();
  SH_TRY(check_dtype_mode(dtype, SH_GREEDY));
  if (B < 1 || B > 65535) return fail(SH_ERR_SHAPE, "B must be in [1, 65535]");
  if (N < 1 || N > sh::kMaxTreeNodes) return fail(SH_ERR_SHAPE, "N must be in [1, %d]", sh::kMaxTreeNodes);
  SH_TRY(check_rowlen("V", V, dtype));
  if (V > (int64_t{1} << 28)) return fail(SH_ERR_SHAPE, "V above 2^28");
  SH_TRY(check_ptr(target_logits, "target_logits"));
  const std::pair<const void*, const char*> small[] = {{node_token, "node_token"}, {parent, "parent"}};
  for (const auto& pn : small) {
    if (pn.first == nullptr) return fail(SH_ERR_NULL, "%s is NULL", pn.second);
    if (!aligned(pn.first, 4)) return fail(SH_ERR_ALIGN, "%s is not 4-byte aligned", pn.second);
  }
  SH_TRY(check_out(accept_len, "accept_len"));
  SH_TRY(check_out(accept_node, "accept_node"));
  SH_TRY(check_out(out_tokens, "out_tokens"));
  const size_t need = sh_verify_tree_workspace_bytes(B, N, V);
  SH_TRY(check_workspace(workspace, workspace_bytes, need));
  sh::VerifyArgs a{};
  a.mode = 0;
  a.B = B;
  a.gamma = N - 1;
  a.V = V;
  a.bf16 = dtype == SH_BF16;
  a.target = target_logits;
  a.tokens = node_token;
  a.parent = parent;
  a.accept_len = accept_len;
  a.accept_node = accept_node;
  a.out_tokens = out_tokens;
  const VerifyLayout L = verify_layout(0, B, N - 1, V);
  a.partials = reinterpret_cast<sh::Partial*>(static_cast<char*>(workspace) + L.part_off);
  a.S = L.S;
  SH_HIP(sh::launch_verify_tree(a, static_cast<hipStream_t>(stream)), "tree verify kernels");
  return SH_OK;
}

int sh_topk(const float* scores, int64_t M, int64_t V, int64_t k, int32_t* topk_idx, void* workspace,
            size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  SH_TRY(check_ptr(scores, "scores"));
  SH_TRY(check_out(topk_idx, "topk_idx"));
  if (M < 1 || M > 65535) return fail(SH_ERR_SHAPE, "M must be in [1, 65535]");
  if (V < 1 || V > sh::kTopkMaxV) return fail(SH_ERR_SHAPE, "V must be in [1, 2^19]");
  if (k < 1 || k > V) return fail(SH_ERR_PARAM, "k must be in [1, V]");
  SH_TRY(check_workspace(workspace, workspace_bytes, sh_topk_workspace_bytes(M, V, k)));
  const TopkLayout TL = topk_layout(M, V);
  hipStream_t st = static_cast<hipStream_t>(stream);
  SH_HIP(sh::launch_zero(reinterpret_cast<uint32_t*>(static_cast<char*>(workspace) + TL.hist_off),
                         sh::topk_counter_words(M), st),
         "top-k counter clear");
  SH_HIP(sh::launch_topk(topk_args(workspace, TL, scores, M, V, k, topk_idx), st), "top-k kernels");
  return SH_OK;
}

int sh_philox_uniform(uint64_t seed, uint64_t offset, uint32_t purpose, int64_t rows, int64_t n,
                      float* out, void* stream) {
  g_last_error.clear();
  if (out == nullptr) return fail(SH_ERR_NULL, "out is NULL");
  if (!aligned(out, 4)) return fail(SH_ERR_ALIGN, "out is not 4-byte aligned");
  if (rows < 1 || n < 1 || rows * n > (int64_t{1} << 31))
    return fail(SH_ERR_SHAPE, "rows * n must be in [1, 2^31]");
  SH_HIP(sh::launch_philox(seed, offset, purpose, rows, n, out, static_cast<hipStream_t>(stream)),
         "philox kernel");
  return SH_OK;
}

int sh_read_probe(const void* buf, uint64_t bytes, uint32_t* sink, void* stream) {
  g_last_error.clear();
  SH_TRY(check_ptr(buf, "buf"));
  if (sink == nullptr) return fail(SH_ERR_NULL, "sink is NULL");
  if (!aligned(buf, 16)) return fail(SH_ERR_ALIGN, "buf is not 16-byte aligned");
  if (!aligned(sink, 4)) return fail(SH_ERR_ALIGN, "sink is not 4-byte aligned");
  if (bytes == 0 || bytes % 16 != 0 || bytes > 0xFFFFFFF0ull)
    return fail(SH_ERR_SHAPE, "bytes must be a nonzero multiple of 16, at most 0xFFFFFFF0");
  SH_HIP(sh::launch_read_probe(buf, bytes, sink, static_cast<hipStream_t>(stream)), "read probe kernel");
  return SH_OK;
}

}  // extern "C"
