// SpecVocab dynamic-vocabulary pieces (SpecVocab write-up, sections 2.2.2, 2.2.3 and 2.3):
//   k_topk            per-row exact radix select of the k largest approximate scores,
//                     ties -> lowest id, compacted in ascending id order
//   k_gather_exact    z'_j = U[K_j, :] . h read straight from the gathered rows (no slice copy),
//                     the hidden state held in registers
//   k_gather_finalize softmax over the k candidates, argmax or two-level Gumbel draw
#include "device_common.h"
#include "launch.h"
#include "trace.h"

namespace sh {

// order-preserving map float -> uint32 (larger float -> larger key); -0 is treated as +0
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u << 1) == 0u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / kWave;

__global__ __launch_bounds__(kTopkThreads) void k_topk(const float* __restrict__ scores, int V, int k,
                                                       int32_t* __restrict__ out) {
  __shared__ uint32_t hist[kTopkWaves][256];
  __shared__ uint32_t total[256];
  __shared__ uint32_t sh_prefix, sh_mask, sh_rem;
  __shared__ uint32_t wcnt[kTopkWaves], wcnt2[kTopkWaves];
  const int m = blockIdx.x;
  const float* s = scores + static_cast<size_t>(m) * V;
  const int tid = threadIdx.x, l = lane_id(), w = wave_id();
  uint32_t prefix = 0u, mask = 0u, rem = static_cast<uint32_t>(k);
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int i = tid; i < kTopkWaves * 256; i += kTopkThreads) (&hist[0][0])[i] = 0u;
    __syncthreads();
    for (int i = tid; i < V; i += kTopkThreads) {
      const uint32_t key = order_key(s[i]);
      if ((key & mask) == prefix) atomicAdd(&hist[w][(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid < 256) {
      uint32_t c = 0;
      for (int ww = 0; ww < kTopkWaves; ++ww) c += hist[ww][tid];
      total[tid] = c;
    }
    __syncthreads();
    if (tid == 0) {
      uint32_t cum = 0;
      int d = 255;
      for (; d > 0; --d) {
        if (cum + total[d] >= rem) break;
        cum += total[d];
      }
      rem -= cum;
      prefix |= static_cast<uint32_t>(d) << shift;
      mask |= 255u << shift;
      sh_prefix = prefix;
      sh_mask = mask;
      sh_rem = rem;
    }
    __syncthreads();
    prefix = sh_prefix;
    mask = sh_mask;
    rem = sh_rem;
  }
  // threshold key T = prefix; take every key > T and the first `rem` keys == T (by index)
  const uint32_t T = prefix, need = rem;
  const uint64_t lt = (l == 0) ? 0ull : ((~0ull) >> (64 - l));
  uint32_t base = 0, eq_before = 0;
  for (int start = 0; start < V; start += kTopkThreads) {
    const int i = start + tid;
    const bool in = i < V;
    const uint32_t key = in ? order_key(s[i]) : 0u;
    const bool gt = in && key > T;
    const bool eq = in && key == T;
    const uint64_t be = __ballot(eq);
    if (l == 0) wcnt[w] = static_cast<uint32_t>(__popcll(be));
    __syncthreads();
    uint32_t eq_wave = 0, eq_total = 0;
    for (int ww = 0; ww < kTopkWaves; ++ww) {
      if (ww < w) eq_wave += wcnt[ww];
      eq_total += wcnt[ww];
    }
    const uint32_t eq_rank = eq_before + eq_wave + static_cast<uint32_t>(__popcll(be & lt));
    const bool sel = gt || (eq && eq_rank < need);
    const uint64_t bsel = __ballot(sel);
    if (l == 0) wcnt2[w] = static_cast<uint32_t>(__popcll(bsel));
    __syncthreads();
    uint32_t sel_wave = 0, sel_total = 0;
    for (int ww = 0; ww < kTopkWaves; ++ww) {
      if (ww < w) sel_wave += wcnt2[ww];
      sel_total += wcnt2[ww];
    }
    if (sel) {
      const uint32_t pos = base + sel_wave + static_cast<uint32_t>(__popcll(bsel & lt));
      if (pos < static_cast<uint32_t>(k)) out[static_cast<size_t>(m) * k + pos] = i;
    }
    base += sel_total;
    eq_before += eq_total;
    __syncthreads();
  }
}

hipError_t launch_topk(const float* scores, int64_t M, int64_t V, int64_t k, int32_t* idx,
                       hipStream_t st) {
  TraceScope ts("topk", st);
  hipLaunchKernelGGL(k_topk, dim3(static_cast<unsigned>(M)), dim3(kTopkThreads), 0, st, scores,
                     static_cast<int>(V), static_cast<int>(k), idx);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------------------
// gather + exact logits: grid (ceil(k / 16), M); each wave computes 4 candidates of row m.
// ----------------------------------------------------------------------------------------
constexpr int kGatherPerWave = 4;
constexpr int kGatherMaxCPL = 16;

template <bool BF16>
__global__ __launch_bounds__(256) void k_gather_exact(const void* __restrict__ U,
                                                      const void* __restrict__ h,
                                                      const int32_t* __restrict__ idx, int C,
                                                      int k, int V, float* __restrict__ zbuf) {
  const int m = blockIdx.y;
  const int l = lane_id(), w = wave_id();
  const int CPL = (C + kWave - 1) / kWave;
  const size_t rowbytes = static_cast<size_t>(C) * 16;
  const char* hrow = static_cast<const char*>(h) + static_cast<size_t>(m) * rowbytes;
  uint4 hr[kGatherMaxCPL];
#pragma unroll
  for (int q = 0; q < kGatherMaxCPL; ++q) {
    const int c = q * kWave + l;
    hr[q] = (q < CPL && c < C) ? load16(hrow + static_cast<size_t>(c) * 16) : zero16();
  }
  const int j0 = (blockIdx.x * (blockDim.x / kWave) + w) * kGatherPerWave;
  int64_t rows[kGatherPerWave];
#pragma unroll
  for (int jj = 0; jj < kGatherPerWave; ++jj) {
    const int j = j0 + jj;
    const int64_t id = (j < k) ? idx[static_cast<size_t>(m) * k + j] : -1;
    rows[jj] = (id >= 0 && id < V) ? id : -1;   // ids come from k_topk; guard anyway
  }
  float z[kGatherPerWave];
#pragma unroll
  for (int jj = 0; jj < kGatherPerWave; ++jj) z[jj] = 0.f;
#pragma unroll
  for (int q = 0; q < kGatherMaxCPL; ++q) {
    const int c = q * kWave + l;
    if (q < CPL && c < C) {
      uint4 wv[kGatherPerWave];
#pragma unroll
      for (int jj = 0; jj < kGatherPerWave; ++jj)
        wv[jj] = rows[jj] >= 0 ? load16(static_cast<const char*>(U) + static_cast<size_t>(rows[jj]) * rowbytes +
                                        static_cast<size_t>(c) * 16)
                               : zero16();
#pragma unroll
      for (int jj = 0; jj < kGatherPerWave; ++jj) z[jj] = chunk_dot<BF16>(wv[jj], hr[q], z[jj]);
    }
  }
#pragma unroll
  for (int jj = 0; jj < kGatherPerWave; ++jj) {
    const float t = wave_sum(z[jj]);
    if (l == 0 && j0 + jj < k) zbuf[static_cast<size_t>(m) * k + j0 + jj] = t;
  }
}

hipError_t launch_gather_exact(const void* U, const void* h, const int32_t* idx, int64_t M,
                               int64_t d, int64_t V, int64_t k, bool bf16, float* zbuf,
                               hipStream_t st) {
  const int C = static_cast<int>(d * (bf16 ? 2 : 4) / 16);
  const int per_wg = 4 * kGatherPerWave;
  const dim3 grid(static_cast<unsigned>((k + per_wg - 1) / per_wg), static_cast<unsigned>(M));
  TraceScope ts("gather_exact", st);
  if (bf16)
    hipLaunchKernelGGL(k_gather_exact<true>, grid, dim3(256), 0, st, U, h, idx, C,
                       static_cast<int>(k), static_cast<int>(V), zbuf);
  else
    hipLaunchKernelGGL(k_gather_exact<false>, grid, dim3(256), 0, st, U, h, idx, C,
                       static_cast<int>(k), static_cast<int>(V), zbuf);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------------------
// softmax over the k candidates + selection; one workgroup (4 waves) per row
// ----------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_gather_finalize(const float* __restrict__ zbuf,
                                                         const int32_t* __restrict__ idx, int k,
                                                         int mode, float invT, uint64_t seed,
                                                         uint64_t offset, float* topk_logit,
                                                         float* topk_prob, int32_t* token,
                                                         float* lse_out, float* logprob) {
  __shared__ float red_f[4];
  __shared__ int32_t red_i[4];
  __shared__ float sh_lse;
  const int m = blockIdx.x;
  const int l = lane_id(), w = wave_id();
  const float* z = zbuf + static_cast<size_t>(m) * k;
  // max of y
  float mx = -INFINITY;
  for (int j = threadIdx.x; j < k; j += blockDim.x) mx = fmaxf(mx, z[j] * invT);
  mx = wave_max(mx);
  if (l == 0) red_f[w] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(red_f[0], red_f[1]), fmaxf(red_f[2], red_f[3]));
  __syncthreads();
  float sm = 0.f;
  for (int j = threadIdx.x; j < k; j += blockDim.x) sm += __expf(z[j] * invT - mx);
  sm = wave_sum(sm);
  if (l == 0) red_f[w] = sm;
  __syncthreads();
  if (threadIdx.x == 0) sh_lse = mx + logf((red_f[0] + red_f[1]) + (red_f[2] + red_f[3]));
  __syncthreads();
  const float lse = sh_lse;
  for (int j = threadIdx.x; j < k; j += blockDim.x) {
    const float zj = z[j];
    if (topk_prob) topk_prob[static_cast<size_t>(m) * k + j] = __expf(zj * invT - lse);
    if (topk_logit) topk_logit[static_cast<size_t>(m) * k + j] = zj;
  }
  __syncthreads();
  int32_t jstar;
  if (mode == 0) {
    float v = -INFINITY;
    int32_t vi = 0x7fffffff;
    for (int j = threadIdx.x; j < k; j += blockDim.x) argmax_merge(v, vi, z[j], j);
    wave_argmax(v, vi);
    if (l == 0) {
      red_f[w] = v;
      red_i[w] = vi;
    }
    __syncthreads();
    v = red_f[0];
    vi = red_i[0];
    for (int i = 1; i < 4; ++i) argmax_merge(v, vi, red_f[i], red_i[i]);
    jstar = vi;
  } else {
    const int ng = (k + kGroup - 1) / kGroup;
    float best = -INFINITY;
    int32_t bg = 0x7fffffff;
    for (int g = w; g < ng; g += 4) {
      const int j = g * kGroup + l;
      const bool valid = j < k;
      const float y = valid ? z[j] * invT : -INFINITY;
      const float gm = wave_max(y);
      const float gs = wave_sum(valid ? __expf(y - gm) : 0.f);
      const float L = gm + logf(gs);
      const float sc = L + gumbel(philox_uniform(seed, offset, kDraftGroup, m, g));
      argmax_merge(best, bg, sc, g);
    }
    if (l == 0) {
      red_f[w] = best;
      red_i[w] = bg;
    }
    __syncthreads();
    best = red_f[0];
    bg = red_i[0];
    for (int i = 1; i < 4; ++i) argmax_merge(best, bg, red_f[i], red_i[i]);
    const int j = bg * kGroup + l;
    const bool valid = j < k;
    float e = valid ? z[j] * invT + gumbel(philox_uniform(seed, offset, kDraftElem, m, j)) : -INFINITY;
    int32_t ei = valid ? j : 0x7fffffff;
    wave_argmax(e, ei);
    jstar = ei;
  }
  if (jstar < 0 || jstar >= k) jstar = 0;   // only if every candidate score were -inf
  if (threadIdx.x == 0) {
    token[m] = idx[static_cast<size_t>(m) * k + jstar];
    if (lse_out) lse_out[m] = lse;
    if (logprob) logprob[m] = z[jstar] * invT - lse;
  }
}

hipError_t launch_gather_finalize(const float* zbuf, const int32_t* idx, int64_t M, int64_t k,
                                  int mode, float invT, uint64_t seed, uint64_t offset,
                                  float* topk_logit, float* topk_prob, int32_t* token, float* lse,
                                  float* logprob, hipStream_t st) {
  TraceScope ts("gather_finalize", st);
  hipLaunchKernelGGL(k_gather_finalize, dim3(static_cast<unsigned>(M)), dim3(256), 0, st, zbuf, idx,
                     static_cast<int>(k), mode, invT, seed, offset, topk_logit, topk_prob, token,
                     lse, logprob);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------------------
// exported uniform stream
// ----------------------------------------------------------------------------------------
__global__ void k_philox(uint64_t seed, uint64_t offset, uint32_t purpose, int64_t rows, int64_t n,
                         float* out) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= rows * n) return;
  const int64_t row = i / n, idx = i - row * n;
  out[i] = philox_uniform(seed, offset, purpose, static_cast<uint64_t>(row), static_cast<uint64_t>(idx));
}

hipError_t launch_philox(uint64_t seed, uint64_t offset, uint32_t purpose, int64_t rows, int64_t n,
                         float* out, hipStream_t st) {
  const int64_t total = rows * n;
  const int64_t blocks = (total + 255) / 256;
  hipLaunchKernelGGL(k_philox, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st, seed, offset,
                     purpose, rows, n, out);
  return hipGetLastError();
}

}  // namespace sh
