// SpecVocab dynamic-vocabulary pieces (SpecVocab write-up, sections 2.2.2, 2.2.3 and 2.3):
//   k_topk_*          exact top-k of the approximate scores (ties -> lowest id), as a
//                     threshold search over order-preserving keys, ascending ids out
//   k_gather_exact    z'_j = U[K_j, :] . h read straight from the gathered rows (no slice copy),
//                     the hidden state held in registers; the workgroup that completes a row
//                     then runs its softmax over the k candidates and the argmax or two-level
//                     Gumbel draw (a last-arriver hand-off, no second launch)
#include "device_common.h"
#include "launch.h"
#include "trace.h"

namespace sh {


// ----------------------------------------------------------------------------------------
// Top-k as a threshold search over the order keys, spread over many workgroups per row:
//   k_topk_hist    grid (V / 4096, M): histogram of the top 12 key bits of each 4096-score
//                  chunk in LDS, added into the row histogram [M, 4096] in the workspace.
//   k_topk_select  grid (chunks, M): every workgroup finds the threshold bin b* (the bin
//                  where the count of larger keys reaches k) from the row histogram, marks
//                  its chunk's keys above b* in the row's selection bitmask (one 64-bit word
//                  per 64 scores), appends the keys inside b* to the row's candidate list
//                  (one counter update per workgroup) and adds them to the row's histogram of
//                  key bits 19..8; the row's first workgroup records b* and the count above.
//   k_topk_finish  one workgroup per row: finds the bin of key bits 19..8 from the second
//                  histogram, resolves the remaining 8 bits over the candidates in one
//                  histogram pass, takes the lowest ids among keys equal to the final
//                  threshold and compacts the bitmask into ascending ids.
//   The histograms and the candidate counter are cleared by an earlier kernel of the call.
//   Kernel boundaries order the phases: an in-kernel hand-off between workgroups would need
//   a device-scope release per workgroup, which writes back the issuing XCD's L2.
// ----------------------------------------------------------------------------------------
constexpr int kTkThreads = 256;
constexpr int kTkPerThread = 8;
constexpr int kTkChunk = kTkThreads * kTkPerThread;
constexpr int kTkWaves = kTkThreads / kWave;
constexpr int kTkShift2 = 8;         // second level: key bits 19..8
constexpr uint32_t kTkDirect = 512;  // in-bin keys of a workgroup added to the second histogram one by one
// the histogram pass takes twice the select's chunk: half the workgroups, each adding its bins
// to the row's histogram once (measured at 16 rows: 7.6 -> 6.8 us; the select at 16 scores per
// thread slowed more than that at one row, so it keeps 8)
constexpr int kTkHistPerThread = 2 * kTkPerThread;
constexpr int kTkHistChunk = kTkThreads * kTkHistPerThread;

__global__ __launch_bounds__(kTkThreads) void k_topk_hist(TopkArgs a) {
  __shared__ uint32_t h[kTkBins];
  const int m = blockIdx.y;
  const int64_t c0 = static_cast<int64_t>(blockIdx.x) * kTkHistChunk;
  const int tid = threadIdx.x;
  const rsrc_t rs = make_rsrc(a.scores + static_cast<size_t>(m) * a.V, static_cast<uint32_t>(a.V) * 4u);
  uint32_t raw[kTkHistPerThread];
#pragma unroll
  for (int j = 0; j < kTkHistPerThread; ++j) {
    const int64_t e = c0 + j * kTkThreads + tid;
    raw[j] = buffer_load4(rs, e < a.V ? static_cast<uint32_t>(e) * 4u : kOutOfRange);
  }
  for (int i = tid; i < kTkBins; i += kTkThreads) h[i] = 0u;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kTkHistPerThread; ++j) {
    const int64_t e = c0 + j * kTkThreads + tid;
    if (e < a.V) atomicAdd(&h[order_key(__uint_as_float(raw[j])) >> kTkShift], 1u);
  }
  __syncthreads();
  uint32_t* hg = a.hist + static_cast<size_t>(m) * kTkBins;
  for (int i = tid; i < kTkBins; i += kTkThreads) {
    const uint32_t c = h[i];
    if (c != 0u) atomicAdd(&hg[i], c);
  }
}

// Inclusive prefix sum over the lanes of a wave: shifts of 1, 2, 4 and 8 lanes within each
// 16-lane row (DPP row_shr; a lane without a source adds 0), then the totals of the rows
// below (lanes 15, 31, 47) from scalar reads.
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t x) {
  x += __builtin_amdgcn_update_dpp(0u, x, 0x111, 0xF, 0xF, false);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0u, x, 0x112, 0xF, 0xF, false);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0u, x, 0x114, 0xF, 0xF, false);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0u, x, 0x118, 0xF, 0xF, false);   // row_shr:8
  const uint32_t r0 = __builtin_amdgcn_readlane(x, 15);
  const uint32_t r1 = __builtin_amdgcn_readlane(x, 31);
  const uint32_t r2 = __builtin_amdgcn_readlane(x, 47);
  const int row = lane_id() >> 4;
  return x + (row >= 1 ? r0 : 0u) + (row >= 2 ? r1 : 0u) + (row >= 3 ? r2 : 0u);
}

// Exclusive prefix sum over the threads of the workgroup (thread order); also the total.
__device__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* wsum, uint32_t* total) {
  const int l = lane_id(), w = wave_id(), nw = blockDim.x / kWave;
  const uint32_t x = wave_inclusive_scan(v);
  if (l == kWave - 1) wsum[w] = x;
  __syncthreads();
  uint32_t before = 0u, all = 0u;
  for (int i = 0; i < nw; ++i) {
    const uint32_t t = wsum[i];
    if (i < w) before += t;
    all += t;
  }
  __syncthreads();
  *total = all;
  return before + x - v;
}

// Bins [N*tid, N*tid + N) of a histogram are in c[]; find the bin b where the count of
// larger bins is below `target` and the count including b reaches it.  The thread owning b
// writes b and the count above it to out[0], out[1].
template <int N>
__device__ void find_crossing(const uint32_t (&c)[N], uint32_t target, uint32_t* wsum, uint32_t* out) {
  uint32_t mine = 0u;
#pragma unroll
  for (int i = 0; i < N; ++i) mine += c[i];
  uint32_t total;
  const uint32_t before = block_exclusive_scan(mine, wsum, &total);
  uint32_t cum = total - before - mine;  // count in bins above this thread's range
#pragma unroll
  for (int i = N - 1; i >= 0; --i) {
    if (cum < target && cum + c[i] >= target) {
      out[0] = static_cast<uint32_t>(N * threadIdx.x + i);
      out[1] = cum;
    }
    cum += c[i];
  }
  __syncthreads();
}

__global__ __launch_bounds__(kTkThreads) void k_topk_select(TopkArgs a) {
  __shared__ uint32_t wsum[kTkWaves];
  __shared__ uint32_t wcnt[kTkWaves];
  __shared__ uint32_t res[2];
  __shared__ uint32_t wbase;
  __shared__ uint32_t h2l[kTkBins];   // second-level counts when a chunk holds many in-bin keys
  const int m = blockIdx.y;
  const int tid = threadIdx.x, l = lane_id(), w = wave_id();
  const int64_t V = a.V;
  const uint32_t k = static_cast<uint32_t>(a.k);
  const int64_t c0 = static_cast<int64_t>(blockIdx.x) * kTkChunk;
  const rsrc_t rs = make_rsrc(a.scores + static_cast<size_t>(m) * V, static_cast<uint32_t>(V) * 4u);
  // the chunk's scores: wave w takes 64-score segments w, w + 4, ... (issued first)
  uint32_t raw[kTkPerThread];
#pragma unroll
  for (int j = 0; j < kTkPerThread; ++j) {
    const int64_t e = c0 + static_cast<int64_t>(w + kTkWaves * j) * kWave + l;
    raw[j] = buffer_load4(rs, e < V ? static_cast<uint32_t>(e) * 4u : kOutOfRange);
  }
  // 1. threshold bin from the row histogram (16 bins per thread)
  {
    const uint4* hg = reinterpret_cast<const uint4*>(a.hist + static_cast<size_t>(m) * kTkBins) + tid * 4;
    uint32_t c[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint4 t = hg[q];
      c[4 * q] = t.x;
      c[4 * q + 1] = t.y;
      c[4 * q + 2] = t.z;
      c[4 * q + 3] = t.w;
    }
    find_crossing<16>(c, k, wsum, res);
  }
  const uint32_t bstar = res[0], above = res[1];
  // 2. mark keys above b*, collect keys inside b*; one counter update per workgroup
  const int64_t mw = (V + kWave - 1) / kWave;
  uint64_t* mask = a.mask + static_cast<size_t>(m) * mw;
  uint2* cand = a.cand + static_cast<size_t>(m) * V;
  uint32_t* count = a.count + static_cast<size_t>(m) * kTkCounterStride;
  if (blockIdx.x == 0 && tid == 0) {   // for the finish: b* and the count above it
    count[4] = bstar;
    count[5] = above;
  }
  uint64_t bcs[kTkPerThread];
  uint32_t keys[kTkPerThread];
  uint32_t mine = 0u;
#pragma unroll
  for (int j = 0; j < kTkPerThread; ++j) {
    const int64_t sb = c0 + static_cast<int64_t>(w + kTkWaves * j) * kWave;
    const int64_t e = sb + l;
    keys[j] = order_key(__uint_as_float(raw[j]));
    const uint32_t bin = keys[j] >> kTkShift;
    const bool in = e < V;
    const uint64_t bs = __ballot(in && bin > bstar);
    bcs[j] = __ballot(in && bin == bstar);
    if (l == 0 && sb < V) mask[sb / kWave] = bs;
    mine += static_cast<uint32_t>(__popcll(bcs[j]));
  }
  if (l == 0) wcnt[w] = mine;
  __syncthreads();
  uint32_t tot = 0u;
  for (int i = 0; i < kTkWaves; ++i) tot += wcnt[i];
  if (tid == 0) wbase = tot != 0u ? atomicAdd(count, tot) : 0u;
  // the in-bin keys' bits 19..8 into the row's second histogram: one device atomic per key,
  // or through LDS counts when the chunk holds many (a row of equal scores)
  uint32_t* h2 = a.hist2 + static_cast<size_t>(m) * kTkBins;
  if (tot <= kTkDirect) {
#pragma unroll
    for (int j = 0; j < kTkPerThread; ++j)
      if ((bcs[j] >> l) & 1ull) atomicAdd(&h2[(keys[j] >> kTkShift2) & (kTkBins - 1)], 1u);
  } else {   // uniform over the workgroup
    for (int i = tid; i < kTkBins; i += kTkThreads) h2l[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kTkPerThread; ++j)
      if ((bcs[j] >> l) & 1ull) atomicAdd(&h2l[(keys[j] >> kTkShift2) & (kTkBins - 1)], 1u);
    __syncthreads();
    for (int i = tid; i < kTkBins; i += kTkThreads)
      if (h2l[i] != 0u) atomicAdd(&h2[i], h2l[i]);
  }
  __syncthreads();
  uint32_t base = wbase;
  for (int i = 0; i < w; ++i) base += wcnt[i];
#pragma unroll
  for (int j = 0; j < kTkPerThread; ++j) {
    const uint64_t bc = bcs[j];
    const int64_t e = c0 + static_cast<int64_t>(w + kTkWaves * j) * kWave + l;
    const uint32_t rank = __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(bc >> 32),
                                                    __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(bc), 0u));
    // base + rank < V whenever the counter started at zero; the guard keeps a corrupted
    // counter from writing out of bounds
    if (((bc >> l) & 1ull) && base + rank < static_cast<uint64_t>(V))
      cand[base + rank] = make_uint2(keys[j], static_cast<uint32_t>(e));
    base += static_cast<uint32_t>(__popcll(bc));
  }
}

// One workgroup per row: resolve the threshold bin's candidates and compact the row.
// Candidates are staged in LDS when they fit (cand_cap entries), the selection bitmask is
// loaded into LDS at the start; equal-key ties at the final threshold are resolved by id only
// when more of them exist than are needed.
constexpr int kTfThreads = 1024;
constexpr int kTfWaves = kTfThreads / kWave;
constexpr int kTfBatch = 8;   // words (candidates) each thread loads per round trip
constexpr int kTfSpec = 2;    // candidates per thread loaded before their count is known
typedef uint32_t tf_u32x2_t __attribute__((ext_vector_type(2)));

// Finish of row m by the NT threads of a workgroup.  LDS: fin = sel[nw], tie[nw],
// hist[1024], cand[cand_cap] (uint2); wsum[NT / 64], res[2], nties.
template <int NT>
__device__ void topk_finish_row(const TopkArgs& a, int m, int cand_cap, uint32_t* fin, uint32_t* wsum, uint32_t* res,
                                uint32_t* nties_p) {
  constexpr int HB = kTkBins / NT;    // second-histogram bins per thread
  static_assert(HB >= 4 && HB % 4 == 0, "second-histogram bins per thread");
  constexpr int aux = 0;
  uint32_t& nties = *nties_p;
  const int tid = threadIdx.x;
  const int64_t V = a.V;
  const uint32_t k = static_cast<uint32_t>(a.k);
  const int64_t mw = (V + kWave - 1) / kWave;
  const int nw = static_cast<int>(2 * mw);  // 32-bit words of the bitmask
  uint32_t* sel = fin;
  uint32_t* tie = fin + nw;
  uint32_t* h1 = fin + 2 * nw;
  uint2* cl = reinterpret_cast<uint2*>(fin + 2 * nw + 1024);
  // loads that depend on nothing, issued together: the first candidates (before their count is
  // known; the row's list has room for V), the second histogram, the count line (candidate
  // count, threshold bin b*, count above b*) and the bitmask (kTfBatch words per thread per
  // round trip)
  const uint2* cg = a.cand + static_cast<size_t>(m) * V;
  const rsrc_t crow = make_rsrc(cg, static_cast<uint32_t>(V) * 8u);
  tf_u32x2_t sv[kTfSpec];
#pragma unroll
  for (int q = 0; q < kTfSpec; ++q) {
    const int64_t i = static_cast<int64_t>(q) * NT + tid;
    sv[q] = __builtin_amdgcn_raw_buffer_load_b64(crow, i < V ? static_cast<uint32_t>(i) * 8u : kOutOfRange, 0, aux);
  }
  uint32_t hb[HB];
  {
    const uint4* hq = reinterpret_cast<const uint4*>(a.hist2 + static_cast<size_t>(m) * kTkBins) + tid * (HB / 4);
#pragma unroll
    for (int q = 0; q < HB / 4; ++q) {
      const uint4 t = hq[q];
      hb[4 * q] = t.x;
      hb[4 * q + 1] = t.y;
      hb[4 * q + 2] = t.z;
      hb[4 * q + 3] = t.w;
    }
  }
  const uint32_t* line = a.count + static_cast<size_t>(m) * kTkCounterStride;
  uint32_t C = line[0];
  const uint32_t bstar = line[4], above = line[5];
  {
    const rsrc_t mr = make_rsrc(a.mask + static_cast<size_t>(m) * mw, static_cast<uint32_t>(nw) * 4u);
    auto batch = [&](int i0) {
      uint32_t v[kTfBatch];
#pragma unroll
      for (int q = 0; q < kTfBatch; ++q) {
        const int i = i0 + q * NT + tid;
        v[q] = __builtin_amdgcn_raw_buffer_load_b32(mr, i < nw ? static_cast<uint32_t>(i) * 4u : kOutOfRange, 0, aux);
      }
#pragma unroll
      for (int q = 0; q < kTfBatch; ++q) {
        const int i = i0 + q * NT + tid;
        if (i < nw) {
          sel[i] = v[q];
          tie[i] = 0u;
        }
      }
    };
    batch(0);   // (the first batch outside the loop: its loads go out with the ones above)
    for (int i0 = kTfBatch * NT; i0 < nw; i0 += kTfBatch * NT) batch(i0);
  }
  if (C > static_cast<uint64_t>(V)) C = static_cast<uint32_t>(V);
  const rsrc_t cr = make_rsrc(cg, C * 8u);
  const bool in_lds = C <= static_cast<uint32_t>(cand_cap);
  if (in_lds) {
    // the candidates into LDS: the first ones are in registers already, the rest kTfBatch per
    // thread per round trip
#pragma unroll
    for (int q = 0; q < kTfSpec; ++q) {
      const uint32_t i = static_cast<uint32_t>(q * NT + tid);
      if (i < C) cl[i] = make_uint2(sv[q].x, sv[q].y);
    }
    auto batch = [&](uint32_t i0) {
      tf_u32x2_t v[kTfBatch];
#pragma unroll
      for (int q = 0; q < kTfBatch; ++q) {
        const uint32_t i = i0 + q * NT + tid;
        v[q] = __builtin_amdgcn_raw_buffer_load_b64(cr, i < C ? i * 8u : kOutOfRange, 0, aux);
      }
#pragma unroll
      for (int q = 0; q < kTfBatch; ++q) {
        const uint32_t i = i0 + q * NT + tid;
        if (i < C) cl[i] = make_uint2(v[q].x, v[q].y);
      }
    };
    for (uint32_t i0 = kTfSpec * NT; i0 < C; i0 += kTfBatch * NT) batch(i0);
  }
  // a candidate from LDS, or from the global list when it did not fit (uniform branch: LDS
  // reads stay LDS reads)
  auto cand_at = [&](uint32_t i) -> uint2 {
    if (in_lds) return cl[i];
    const tf_u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(cr, i * 8u, 0, aux);
    return make_uint2(v.x, v.y);
  };
  if (tid == 0) nties = 0u;
  // key bits 19..8 from the second histogram (the select kernel's counts of the b* keys)
  uint32_t need = k - above;
  uint32_t thr = bstar << kTkShift;
  find_crossing<HB>(hb, need, wsum, res);   // includes a barrier: LDS stores above are visible
  thr |= res[0] << kTkShift2;
  need -= res[1];
  // key bits 7..0: one histogram pass over the candidates in that bin
  if (tid < 256) h1[tid] = 0u;
  __syncthreads();
  for (uint32_t i = tid; i < C; i += NT) {
    const uint32_t key = cand_at(i).x;
    if ((key >> kTkShift2) == (thr >> kTkShift2)) atomicAdd(&h1[key & 255u], 1u);
  }
  __syncthreads();
  {
    const uint32_t c1[1] = {tid < 256 ? h1[tid] : 0u};
    find_crossing<1>(c1, need, wsum, res);
    thr |= res[0];
    need -= res[1];
  }
  // keys above the threshold are in; keys equal to it are in if all are needed, else they
  // compete by id
  for (uint32_t i = tid; i < C; i += NT) {
    const uint2 ce = cand_at(i);
    if (ce.y >= static_cast<uint64_t>(V)) continue;
    if (ce.x > thr) {
      atomicOr(&sel[ce.y >> 5], 1u << (ce.y & 31u));
    } else if (ce.x == thr) {
      atomicOr(&tie[ce.y >> 5], 1u << (ce.y & 31u));
      atomicAdd(&nties, 1u);
    }
  }
  __syncthreads();
  const int per = (nw + NT - 1) / NT;
  const int w0 = tid * per < nw ? tid * per : nw;
  const int w1 = w0 + per < nw ? w0 + per : nw;
  if (nties <= need) {
    for (int i = w0; i < w1; ++i) sel[i] |= tie[i];
  } else {
    uint32_t cnt = 0u, total;
    for (int i = w0; i < w1; ++i) cnt += __popc(tie[i]);
    uint32_t rank = block_exclusive_scan(cnt, wsum, &total);
    for (int i = w0; i < w1 && rank < need; ++i) {
      uint32_t bits = tie[i];
      while (bits != 0u && rank < need) {
        const uint32_t b = __builtin_ctz(bits);
        sel[i] |= 1u << b;
        bits &= bits - 1u;
        ++rank;
      }
    }
  }
  // ascending ids (each thread compacts its own words)
  uint32_t cnt = 0u, total;
  for (int i = w0; i < w1; ++i) cnt += __popc(sel[i]);
  uint32_t pos = block_exclusive_scan(cnt, wsum, &total);
  int32_t* out = a.out + static_cast<size_t>(m) * k;
  for (int i = w0; i < w1; ++i) {
    uint32_t bits = sel[i];
    while (bits != 0u) {
      const uint32_t b = __builtin_ctz(bits);
      if (pos < k) out[pos] = static_cast<int32_t>(32 * i + b);
      ++pos;
      bits &= bits - 1u;
    }
  }
}

__global__ __launch_bounds__(kTfThreads) void k_topk_finish(TopkArgs a, int cand_cap) {
  extern __shared__ uint32_t fin[];  // sel[nw], tie[nw], hist[1024], cand[cand_cap] (uint2)
  __shared__ uint32_t wsum[kTfWaves];
  __shared__ uint32_t res[2];
  __shared__ uint32_t nties;
  topk_finish_row<kTfThreads>(a, static_cast<int>(blockIdx.x), cand_cap, fin, wsum, res, &nties);
}

__global__ void k_zero(uint32_t* p, int64_t words) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < words;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x)
    p[i] = 0u;
}

hipError_t launch_zero(uint32_t* p, int64_t words, hipStream_t st) {
  int64_t blocks = (words + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  if (blocks < 1) blocks = 1;
  TraceScope ts("zero", st);
  hipLaunchKernelGGL(k_zero, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st, p, words);
  return hipGetLastError();
}

int topk_chunks(int64_t V) { return static_cast<int>((V + kTkChunk - 1) / kTkChunk); }

size_t topk_finish_lds(int64_t V) {
  const int64_t nw = 2 * ((V + kWave - 1) / kWave);
  return static_cast<size_t>(2 * nw + 1024) * 4;
}

hipError_t launch_topk(const TopkArgs& a, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(a.chunks), static_cast<unsigned>(a.M));
  hipError_t e;
  if (!a.hist_ready) {   // else the scorer built the row histograms while writing the scores
    const dim3 hgrid(static_cast<unsigned>((a.V + kTkHistChunk - 1) / kTkHistChunk), static_cast<unsigned>(a.M));
    TraceScope ts("topk_hist", st);
    hipLaunchKernelGGL(k_topk_hist, hgrid, dim3(kTkThreads), 0, st, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // LDS of a finishing workgroup: the two bitmasks and the 1024-bin histogram, then as many
  // candidates as fit
  const size_t base = topk_finish_lds(a.V);
  {
    TraceScope ts("topk_select", st);
    hipLaunchKernelGGL(k_topk_select, grid, dim3(kTkThreads), 0, st, a);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t limit = 160 * 1024 - 1024;   // leave room for the static arrays
  int cap = base < limit ? static_cast<int>((limit - base) / 8) : 0;
  if (cap > 8192) cap = 8192;
  const size_t lds = base + static_cast<size_t>(cap) * 8;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(k_topk_finish),
                          hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
  if (e != hipSuccess) return e;
  TraceScope ts("topk_finish", st);
  hipLaunchKernelGGL(k_topk_finish, dim3(static_cast<unsigned>(a.M)), dim3(kTfThreads), lds, st, a, cap);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------------------
// softmax over the k candidates + selection of one row, by the 4 waves of one workgroup (the
// gather workgroup that completes the row).  The row's logits are staged in LDS once; the
// group draw computes all group uniforms in one pass.
// ----------------------------------------------------------------------------------------
constexpr int kGfThreads = 256;
constexpr int kGfWaves = kGfThreads / kWave;
constexpr int kGfBatch = 8;   // logits each thread loads per round trip

struct GatherOut {
  int k;
  int mode;
  float invT;
  uint64_t seed, offset;
  float* topk_logit;
  float* topk_prob;
  int32_t* token;
  float* lse;
  float* logprob;
  uint32_t* counters;   // [M, kTkCounterStride]: word 2 counts the row's finished workgroups
};

// Sums over the wave of 8 values per lane, transposed: three exchanges that each halve the
// values a lane holds, then three full ones, leave lane L with the total of value (L >> 3) mod 8
// (10 exchanges instead of 8 x 6).
__device__ __forceinline__ float wave_sum8(const float (&v)[8]) {
  const int l = lane_id();
  float b[4], c[2];
  const bool h5 = (l & 32) != 0, h4 = (l & 16) != 0, h3 = (l & 8) != 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) b[i] = (h5 ? v[i + 4] : v[i]) + xor_lane(h5 ? v[i] : v[i + 4], 32);
#pragma unroll
  for (int i = 0; i < 2; ++i) c[i] = (h4 ? b[i + 2] : b[i]) + xor_lane(h4 ? b[i] : b[i + 2], 16);
  float d = (h3 ? c[1] : c[0]) + xor_lane(h3 ? c[0] : c[1], 8);
  d += xor_lane(d, 4);
  d += xor_lane(d, 2);
  d += xor_lane(d, 1);
  return d;
}

// zl: LDS [k] logits then [ceil(k / 64)] group sums; the logits are read with device-coherent
// loads (other workgroups of this kernel wrote them)
__device__ void gather_finalize_row(const float* __restrict__ zbuf, const int32_t* __restrict__ idx,
                                    const GatherOut& o, int m, float* zl, float* red_f) {
  const int k = o.k;
  const int l = lane_id(), w = wave_id();
  const float* z = zbuf + static_cast<size_t>(m) * k;
  const int ng = (k + kGroup - 1) / kGroup;
  float* Lg = zl + k;
  float mx = -INFINITY;
  // sampling with at most 64 groups: the group Gumbels depend on nothing loaded, so wave 0
  // computes them (lane g, group g) while the logits are in flight
  const bool early = o.mode != 0 && ng <= kWave && w == 0;
  float gu_early = 0.f;
  {
    // kGfBatch loads per thread issued together (one memory round trip per batch)
    const rsrc_t zr = make_rsrc(z, static_cast<uint32_t>(k) * 4u);
    for (int j0 = 0; j0 < k; j0 += kGfBatch * kGfThreads) {
      uint32_t v[kGfBatch];
#pragma unroll
      for (int q = 0; q < kGfBatch; ++q) {
        const int j = j0 + q * kGfThreads + static_cast<int>(threadIdx.x);
        v[q] = __builtin_amdgcn_raw_buffer_load_b32(zr, j < k ? static_cast<uint32_t>(j) * 4u : kOutOfRange, 0,
                                                    kCoherent);
      }
      if (j0 == 0 && early && l < ng) gu_early = gumbel(philox_uniform(o.seed, o.offset, kDraftGroup, m, l));
#pragma unroll
      for (int q = 0; q < kGfBatch; ++q) {
        const int j = j0 + q * kGfThreads + static_cast<int>(threadIdx.x);
        if (j < k) {
          const float f = __uint_as_float(v[q]);
          zl[j] = f;
          mx = fmaxf(mx, f);
        }
      }
    }
  }
  mx = wave_max(mx);
  if (l == 0) red_f[w] = mx;
  __syncthreads();
  mx = red_f[0];
  for (int i = 1; i < kGfWaves; ++i) mx = fmaxf(mx, red_f[i]);
  const float c = o.invT * kLog2e;
  const float mxc = mx * c;
  // group sums (base 2, shifted by the row max) and the row sum from them
  for (int g0 = w * 8; g0 < ng; g0 += kGfWaves * 8) {   // eight consecutive groups per wave
    float t[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int j = (g0 + q) * kGroup + l;
      t[q] = (g0 + q < ng && j < k) ? fast_exp2(fmaf(zl[j], c, -mxc)) : 0.f;
    }
    const float gs = wave_sum8(t);   // lane L: group g0 + (L >> 3) mod 8
    if ((l & 7) == 0 && g0 + (l >> 3) < ng) Lg[g0 + (l >> 3)] = gs;
  }
  __syncthreads();
  float sm = 0.f;
  for (int g = threadIdx.x; g < ng; g += blockDim.x) sm += Lg[g];
  sm = wave_sum(sm);
  __syncthreads();
  if (l == 0) red_f[w] = sm;
  __syncthreads();
  sm = red_f[0];
  for (int i = 1; i < kGfWaves; ++i) sm += red_f[i];
  const float lse = mx * o.invT + logf(sm);          // natural-log units of y = z / T
  const float lse2 = mxc + log2f(sm);                // base-2 units of z * c
  for (int j = threadIdx.x; j < k; j += blockDim.x) {
    const float zj = zl[j];
    if (o.topk_prob) o.topk_prob[static_cast<size_t>(m) * k + j] = fast_exp2(fmaf(zj, c, -lse2));
    if (o.topk_logit) o.topk_logit[static_cast<size_t>(m) * k + j] = zj;
  }
  int32_t jstar = 0;
  if (w == 0) {
    if (o.mode == 0) {
      float v = -INFINITY;
      int32_t vi = 0x7fffffff;
      for (int j = l; j < k; j += kWave) argmax_merge(v, vi, zl[j], j);
      wave_argmax(v, vi);
      jstar = vi;
    } else {
      // group scores: log of the group sum (natural units) + Gumbel(u_g), all groups at once
      float best = -INFINITY;
      int32_t bg = 0x7fffffff;
      for (int g = l; g < ng; g += kWave) {
        const float gs = Lg[g];
        if (gs > 0.f) {
          const float L = (mxc + log2f(gs)) * kLn2;
          const float gu = early ? gu_early : gumbel(philox_uniform(o.seed, o.offset, kDraftGroup, m, g));
          argmax_merge(best, bg, L + gu, g);
        }
      }
      wave_argmax(best, bg);
      const int j = bg * kGroup + l;
      const bool valid = bg != 0x7fffffff && j < k;
      float e = valid ? zl[j] * o.invT + gumbel(philox_uniform(o.seed, o.offset, kDraftElem, m, j)) : -INFINITY;
      int32_t ei = valid ? j : 0x7fffffff;
      wave_argmax(e, ei);
      jstar = ei;
    }
    if (jstar < 0 || jstar >= k) jstar = 0;   // only if every candidate score were -inf
    if (l == 0) {
      o.token[m] = idx[static_cast<size_t>(m) * k + jstar];
      if (o.lse) o.lse[m] = lse;
      if (o.logprob) o.logprob[m] = zl[jstar] * o.invT - lse;
    }
  }
}

// ----------------------------------------------------------------------------------------
// gather + exact logits, then the row's softmax: grid (ceil(k / (4 RPW)), M); each wave
// computes RPW candidates of row m; the workgroup that finishes row m last runs its softmax and
// selection (gather_finalize_row), so the call needs no separate finalize launch.  RPW = 4 for
// one or two rows (fewer workgroups to count in: measured at M = 1, 15.8 -> 15.0 us), else 2
// (at M = 16, 4 measured 52.7 against 53.0 us, 1 slower everywhere).
// ----------------------------------------------------------------------------------------

// z'[m, j] = U[K[m, j], :] . h[m, :].  Each wave takes RPW candidates, all loads in flight
// together; a candidate's row is one buffer descriptor (an invalid id gets an empty range, so
// its loads read zero).
template <bool BF16, int CPL, int RPW>
__global__ __launch_bounds__(kGfThreads) void k_gather_exact(const void* __restrict__ U,
                                                             const void* __restrict__ h,
                                                             const int32_t* __restrict__ idx, int C,
                                                             int V, float* __restrict__ zbuf, GatherOut o) {
  extern __shared__ float zl[];   // the finishing workgroup's logits and group sums
  __shared__ float red_f[kGfWaves];
  __shared__ uint32_t last;
  const int m = blockIdx.y;
  const int k = o.k;
  const int l = lane_id(), w = wave_id();
  const uint32_t rowbytes = static_cast<uint32_t>(C) * 16;
  const int j0 = (blockIdx.x * (blockDim.x / kWave) + w) * RPW;
  uint4 wv[RPW][CPL];
#pragma unroll
  for (int jj = 0; jj < RPW; ++jj) {
    const int j = j0 + jj;
    const int id = j < k ? idx[static_cast<size_t>(m) * k + j] : -1;
    const bool ok = id >= 0 && id < V;   // ids come from the top-k; guarded anyway
    const rsrc_t rs = make_rsrc(static_cast<const char*>(U) + static_cast<size_t>(ok ? id : 0) * rowbytes,
                                ok ? rowbytes : 0u);
#pragma unroll
    for (int q = 0; q < CPL; ++q) {
      const int c = q * kWave + l;
      wv[jj][q] = buffer_load16(rs, c < C ? static_cast<uint32_t>(c) * 16 : kOutOfRange);
    }
  }
  const rsrc_t hrs = make_rsrc(static_cast<const char*>(h) + static_cast<size_t>(m) * rowbytes, rowbytes);
  uint4 hr[CPL];
#pragma unroll
  for (int q = 0; q < CPL; ++q) {
    const int c = q * kWave + l;
    hr[q] = buffer_load16(hrs, c < C ? static_cast<uint32_t>(c) * 16 : kOutOfRange);
  }
#pragma unroll
  for (int jj = 0; jj < RPW; ++jj) {
    float z = 0.f;
#pragma unroll
    for (int q = 0; q < CPL; ++q) z = chunk_dot<BF16>(wv[jj][q], hr[q], z);
    z = wave_sum(z);
    if (l == 0 && j0 + jj < k) coherent_store(&zbuf[static_cast<size_t>(m) * k + j0 + jj], z);
  }
  if (arrive_last(&o.counters[static_cast<size_t>(m) * kTkCounterStride + 2], gridDim.x, &last))
    gather_finalize_row(zbuf, idx, o, m, zl, red_f);
}

template <bool BF16, int CPL, int RPW>
static hipError_t run_gather_rpw(const void* U, const void* h, const int32_t* idx, int C, int64_t M,
                                 int64_t V, float* zbuf, const GatherOut& o, hipStream_t st) {
  const int per_wg = kGfWaves * RPW;
  const dim3 grid(static_cast<unsigned>((o.k + per_wg - 1) / per_wg), static_cast<unsigned>(M));
  const int lds = static_cast<int>((o.k + (o.k + kGroup - 1) / kGroup) * 4);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k_gather_exact<BF16, CPL, RPW>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_gather_exact<BF16, CPL, RPW>), grid, dim3(kGfThreads), lds, st, U, h, idx, C,
                     static_cast<int>(V), zbuf, o);
  return hipGetLastError();
}

template <bool BF16, int CPL>
static hipError_t run_gather(const void* U, const void* h, const int32_t* idx, int C, int64_t M,
                             int64_t V, float* zbuf, const GatherOut& o, hipStream_t st) {
  if constexpr (CPL <= 8)
    if (M <= 2) return run_gather_rpw<BF16, CPL, 4>(U, h, idx, C, M, V, zbuf, o, st);
  return run_gather_rpw<BF16, CPL, 2>(U, h, idx, C, M, V, zbuf, o, st);
}

template <bool BF16>
static hipError_t gather_dispatch(const void* U, const void* h, const int32_t* idx, int C, int64_t M,
                                  int64_t V, float* zbuf, const GatherOut& o, hipStream_t st) {
  const int cpl = (C + kWave - 1) / kWave;
  if (cpl <= 1) return run_gather<BF16, 1>(U, h, idx, C, M, V, zbuf, o, st);
  if (cpl <= 2) return run_gather<BF16, 2>(U, h, idx, C, M, V, zbuf, o, st);
  if (cpl <= 4) return run_gather<BF16, 4>(U, h, idx, C, M, V, zbuf, o, st);
  if (cpl <= 8) return run_gather<BF16, 8>(U, h, idx, C, M, V, zbuf, o, st);
  return run_gather<BF16, 16>(U, h, idx, C, M, V, zbuf, o, st);
}

hipError_t launch_gather_select(const void* U, const void* h, const int32_t* idx, int64_t M, int64_t d, int64_t V,
                                int64_t k, bool bf16, float* zbuf, int mode, float invT, uint64_t seed,
                                uint64_t offset, float* topk_logit, float* topk_prob, int32_t* token, float* lse,
                                float* logprob, uint32_t* counters, hipStream_t st) {
  const int C = static_cast<int>(d * (bf16 ? 2 : 4) / 16);
  GatherOut o{};
  o.k = static_cast<int>(k);
  o.mode = mode;
  o.invT = invT;
  o.seed = seed;
  o.offset = offset;
  o.topk_logit = topk_logit;
  o.topk_prob = topk_prob;
  o.token = token;
  o.lse = lse;
  o.logprob = logprob;
  o.counters = counters;
  TraceScope ts("gather_select", st);
  return bf16 ? gather_dispatch<true>(U, h, idx, C, M, V, zbuf, o, st)
              : gather_dispatch<false>(U, h, idx, C, M, V, zbuf, o, st);
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
