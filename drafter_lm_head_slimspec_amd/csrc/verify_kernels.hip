// Batched speculative verification (explainer sections "小模型起草，大模型批改" and
// "为什么答案不会变"; SpecTr-GBV write-up, "第三步").
//   k_verify_rows   one pass over the target / draft logit rows, split in S segments:
//                   greedy: argmax of z; sampling: online log-sum-exp of y = z/T
//   k_verify_resid  (sampling) grid (S2 segments, B sequences): every workgroup merges its
//                   sequence's row partials, decides acceptance (u < p/q) and the
//                   leading-accept count a; its segment of the residual
//                   norm(max(0, p_a - q_a)) (a < gamma) or of p_gamma (a = gamma, the bonus
//                   draw) is folded into the group scores of the two-level draw
//                   With a sparse draft distribution (q given on a candidate set per position,
//                   the SpecVocab head's top-k probabilities; zero elsewhere) the row pass
//                   skips the draft rows and looks q_t(x_t) up in the candidate list, and the
//                   residual is max(0, p - q) with q scattered from that list (equal to p
//                   outside it; SpecVocab write-up 3.3: verification keeps the full vocabulary).
//   k_verify_finish one workgroup per sequence: the same acceptance, then the last token
//                   (greedy: argmax of p_a; sampling: the element draw inside the winning
//                   residual group, or inside the bonus group of p_gamma) and the outputs
#include "device_common.h"
#include "launch.h"
#include "trace.h"

namespace sh {

template <bool BF16>
__device__ __forceinline__ void unpack(const uint4& v, float* out) {
  if constexpr (BF16) {
    out[0] = bf16_lo(v.x);
    out[1] = bf16_hi(v.x);
    out[2] = bf16_lo(v.y);
    out[3] = bf16_hi(v.y);
    out[4] = bf16_lo(v.z);
    out[5] = bf16_hi(v.z);
    out[6] = bf16_lo(v.w);
    out[7] = bf16_hi(v.w);
  } else {
    out[0] = __uint_as_float(v.x);
    out[1] = __uint_as_float(v.y);
    out[2] = __uint_as_float(v.z);
    out[3] = __uint_as_float(v.w);
  }
}

template <bool BF16>
__device__ __forceinline__ float load_logit(const void* row, int64_t i) {
  if constexpr (BF16)
    return bf16_to_f32(static_cast<const uint16_t*>(row)[i]);
  else
    return static_cast<const float*>(row)[i];
}

__device__ __forceinline__ int rows_per_seq(int mode, int64_t gamma) {
  return static_cast<int>(verify_rows_per_seq(mode, gamma));
}

template <bool BF16>
__device__ __forceinline__ const void* row_ptr(const VerifyArgs& a, int64_t b, int r) {
  const size_t es = BF16 ? 2 : 4;
  if (r <= a.gamma)
    return static_cast<const char*>(a.target) + static_cast<size_t>((b * (a.gamma + 1) + r) * a.V) * es;
  const int64_t t = r - (a.gamma + 1);
  return static_cast<const char*>(a.draft) + static_cast<size_t>((b * a.gamma + t) * a.V) * es;
}

// block-wide fixed-order merge of one Partial per thread; result valid in thread 0.  Each wave
// reduces the fields separately (the largest m by a max butterfly, each lane's s rescaled to it
// once and summed, the group score and the argmax by compare butterflies: no exponential inside
// a butterfly), then the waves' records merge through LDS
__device__ __forceinline__ Partial block_merge(Partial p, Partial* red4) {
  float mw = p.m;
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) mw = fmaxf(mw, xor_lane(mw, s));
  float sw = p.m == -INFINITY ? 0.f : p.s * __expf(p.m - mw);
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) {
    sw += xor_lane(sw, s);
    argmax_merge(p.gscore, p.g, xor_lane(p.gscore, s), xor_lane(p.g, s));
    argmax_merge(p.zmax, p.zid, xor_lane(p.zmax, s), xor_lane(p.zid, s));
  }
  p.m = mw;
  p.s = sw;
  const int w = wave_id(), nw = blockDim.x / kWave;
  if (lane_id() == 0) red4[w] = p;
  __syncthreads();
  Partial r = red4[0];
  for (int i = 1; i < nw; ++i) partial_merge(r, red4[i]);
  __syncthreads();
  return r;
}

// block-wide argmax of one (score, id) per thread, lowest id on ties; result valid in thread 0
__device__ __forceinline__ void block_argmax(float& v, int32_t& i, Partial* red4) {
  wave_argmax(v, i);
  const int w = wave_id(), nw = blockDim.x / kWave;
  if (lane_id() == 0) {
    red4[w].gscore = v;
    red4[w].g = i;
  }
  __syncthreads();
  v = red4[0].gscore;
  i = red4[0].g;
  for (int k = 1; k < nw; ++k) argmax_merge(v, i, red4[k].gscore, red4[k].g);
  __syncthreads();
}

// Software-pipelined walk over [0, n) in spans of UNR chunks: the next span's loads are in
// flight while the current one is processed (ping-pong buffers; past n the loads are
// out-of-range, which costs no memory traffic, and proc sees chunks with e >= n).
template <int UNR, typename Load, typename Proc, typename Pre>
__device__ __forceinline__ void pipelined(uint32_t n, uint32_t span, Load load, Proc proc, Pre pre) {
  uint4 A[UNR], B[UNR];
  load(A, 0u);
  pre();   // work that needs none of the data, done while the first loads are in flight
  for (uint32_t base = 0; base < n; base += 2 * span) {
    load(B, base + span);
    proc(A, base);
    load(A, base + 2 * span);
    proc(B, base + span);
  }
}
template <int UNR, typename Load, typename Proc>
__device__ __forceinline__ void pipelined(uint32_t n, uint32_t span, Load load, Proc proc) {
  pipelined<UNR>(n, span, load, proc, [] {});
}

// Max of the EPT values of one 16-byte chunk.
template <int EPT>
__device__ __forceinline__ float chunk_max(const float* v) {
  float m = v[0];
#pragma unroll
  for (int i = 1; i < EPT; ++i) m = fmaxf(m, v[i]);
  return m;
}

// Row pass.  The per-element work is kept to what the mode needs (VALU issue, not HBM, bounds
// a naive version): greedy rows track only the largest chunk maximum and the chunk holding
// it (the position inside that chunk is found once at the end); sampling rows keep only the
// running log-sum-exp, in base-2 units.
// Visit the k candidate ids of one draft position (sparse draft): f(j, id) for every entry,
// the ids read kScanBatch per thread per round trip (one memory latency per batch rather than
// one per id).
constexpr int kScanBatch = 8;
template <typename F>
__device__ __forceinline__ void scan_candidates(const int32_t* ids, int64_t k, F&& f) {
  const rsrc_t ri = make_rsrc(ids, static_cast<uint32_t>(k) * 4u);
  const int64_t nt = blockDim.x;
  for (int64_t j0 = 0; j0 < k; j0 += kScanBatch * nt) {
    uint32_t v[kScanBatch];
#pragma unroll
    for (int q = 0; q < kScanBatch; ++q) {
      const int64_t j = j0 + q * nt + threadIdx.x;
      v[q] = buffer_load4(ri, j < k ? static_cast<uint32_t>(j) * 4u : kOutOfRange);
    }
#pragma unroll
    for (int q = 0; q < kScanBatch; ++q) {
      const int64_t j = j0 + q * nt + threadIdx.x;
      if (j < k) f(j, static_cast<int32_t>(v[q]));
    }
  }
}

// UNR: 16-byte loads per thread per pipeline step (measured on one machine: two for the dense
// sampling rows, 41.0 -> 40.2 us, and the greedy target rows, 25.4 -> 24.9; four for the sparse
// draft's target rows, 24.0 against 25.9 with two, and for the tree's rows, 58.7 against 59.9)
template <bool BF16, bool GREEDY, int UNR>
__global__ __launch_bounds__(256) void k_verify_rows(VerifyArgs a) {
  constexpr int EPT = BF16 ? 8 : 4;   // elements per 16-byte load
  constexpr uint32_t ES = BF16 ? 2 : 4;
  __shared__ Partial red4[4];
  const int s = blockIdx.x, r = blockIdx.y;
  const int64_t b = blockIdx.z;
  const int R = rows_per_seq(a.mode, a.gamma);
  // sampling never needs the normaliser of p_gamma: its bonus draw (only when every draft
  // is accepted) is formed by the residual kernel
  if (!GREEDY && r == a.gamma) return;
  const char* row = static_cast<const char*>(row_ptr<BF16>(a, b, r));
  const int64_t NG = (a.V + kGroup - 1) / kGroup;
  const int64_t GPS = (NG + a.S - 1) / a.S;
  const int64_t g0 = s * GPS;
  const int64_t g1 = min(NG, g0 + GPS);
  const int64_t e_begin = g0 * kGroup;
  const int64_t e_end = min(a.V, g1 * kGroup);
  const uint32_t n = e_end > e_begin ? static_cast<uint32_t>(e_end - e_begin) : 0u;
  const rsrc_t rs = make_rsrc(row + static_cast<size_t>(e_begin) * ES, n * ES);
  const uint32_t tid = threadIdx.x;
  const uint32_t step = blockDim.x * EPT;
  Partial p = partial_empty();
  auto load = [&](uint4 (&buf)[UNR], uint32_t base) {
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const uint32_t e = base + u * step + tid * EPT;
      buf[u] = buffer_load16(rs, e < n ? e * ES : kOutOfRange);
    }
  };
  if constexpr (GREEDY) {
    float best = -INFINITY;
    uint32_t bchunk = 0xffffffffu;
    pipelined<UNR>(n, step * UNR, load, [&](uint4 (&buf)[UNR], uint32_t base) {
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const uint32_t e = base + u * step + tid * EPT;
        float v[EPT];
        unpack<BF16>(buf[u], v);
        const float cm = e < n ? chunk_max<EPT>(v) : -INFINITY;
        if (cm > best) {   // chunks of a thread rise in index: strict > keeps the first
          best = cm;
          bchunk = e;
        }
      }
    });
    int32_t bid = 0x7fffffff;
    if (bchunk != 0xffffffffu) {
      float v[EPT];
      unpack<BF16>(buffer_load16(rs, bchunk * ES), v);
      int j = EPT - 1;
#pragma unroll
      for (int i = EPT - 1; i >= 0; --i)
        if (v[i] == best) j = i;
      bid = static_cast<int32_t>(e_begin + bchunk + j);
    }
    p.zmax = best;
    p.zid = bid;
  } else {
    const float c = a.invT * kLog2e;   // y * log2(e) = z * c
    float M = -INFINITY, S = 0.f;      // sum of exp2(z c - M)
    pipelined<UNR>(n, step * UNR, load, [&](uint4 (&buf)[UNR], uint32_t base) {
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const uint32_t e = base + u * step + tid * EPT;
        float v[EPT];
        unpack<BF16>(buf[u], v);
        if (e < n) {
          // The chunk's exponentials against the running reference M, kept unless their
          // sum is not below 2^64: a value more than 64 (log2 units) above M, M still -inf
          // (before the first finite value, or -inf - -inf = NaN).  Only then is the chunk
          // redone against a raised reference (its maximum) and the sum rescaled, so most
          // chunks pay no maximum and no rescaling exponential; S stays below 2^64 per term
          // and far from overflow.  Logits of -inf (tokens a distribution excludes, e.g.
          // outside a trimmed vocabulary) weigh zero, and an all -inf prefix leaves S at 0.
          float cs = fast_exp2(fmaf(v[0], c, -M));
#pragma unroll
          for (int i = 1; i < EPT; ++i) cs += fast_exp2(fmaf(v[i], c, -M));
          if (!(cs < 0x1p64f)) {
            const float Mn = fmaxf(M, chunk_max<EPT>(v) * c);
            const float off = Mn == -INFINITY ? 0.f : Mn;
            cs = 0.f;
#pragma unroll
            for (int i = 0; i < EPT; ++i) cs += fast_exp2(fmaf(v[i], c, -off));
            S = M == Mn ? S : S * fast_exp2(M - Mn);
            M = Mn;
          }
          S += cs;
        }
      }
    });
    // (m, s) with lse = m + log(s): m = M ln 2, s = S
    p.m = M == -INFINITY ? -INFINITY : M * kLn2;
    p.s = S;
  }
  // sparse draft (segment 0 only): q_t(x_t) from the candidate list, into pad1 (-1: absent)
  float qx = -1.f;
  if (!GREEDY && a.mode == 2 && s == 0) {
    __shared__ float sh_q;
    if (threadIdx.x == 0) sh_q = 0.f;
    __syncthreads();
    const int32_t x = a.tokens[b * a.gamma + r];
    const int64_t base = (b * a.gamma + r) * a.k;
    scan_candidates(a.qidx + base, a.k, [&](int64_t j, int32_t id) {
      if (id == x) sh_q = a.qprob[base + j];
    });
    __syncthreads();
    qx = sh_q;
  }
  Partial out = block_merge(p, red4);
  if (threadIdx.x == 0) {
    out.pad1 = qx;
    // sampling: the raw logit at this row's draft token if it lies in the segment, so that
    // acceptance finds it among the partials instead of in the logit row
    out.xz = -INFINITY;
    if constexpr (!GREEDY) {
      const int t = r < a.gamma ? r : r - static_cast<int>(a.gamma) - 1;
      const int32_t x = a.tokens[b * a.gamma + t];
      if (x >= e_begin && x < e_end) out.xz = load_logit<BF16>(row, x);
    }
    a.partials[(b * R + r) * a.S + s] = out;
  }
}

// Element draw of a two-level Gumbel-max inside 64-element group g (wave 0): returns the
// winning index, or 0x7fffffff if no element has finite weight.
template <bool BF16, typename Ell>
__device__ __forceinline__ int32_t draw_in_group(int32_t g, int64_t V, uint64_t seed, uint64_t offset,
                                                 uint32_t purpose, int64_t row, Ell ell_of) {
  const int l = lane_id();
  const int64_t i = static_cast<int64_t>(g) * kGroup + l;
  const bool valid = g != 0x7fffffff && i < V;
  const float ell = valid ? ell_of(i) : -INFINITY;
  float e = ell != -INFINITY ? ell + gumbel(philox_uniform(seed, offset, purpose, row, i)) : -INFINITY;
  int32_t ei = ell != -INFINITY ? static_cast<int32_t>(i) : 0x7fffffff;
  wave_argmax(e, ei);
  return ei;
}

// Merges the row partials of sequence b into rowp (lane i of a wave loads segment partial i,
// S <= 64, merged by a fixed butterfly over the first S lanes rounded up to a power of two:
// every kernel that calls this computes the same values) and returns the leading-accept
// count (acceptance of all positions at once, lane t).
// The draft token's logits come from the partials' xz fields, so no logit row is read here.
template <bool BF16>
__device__ int seq_accept(const VerifyArgs& a, int64_t b, Partial* rowp, int* sh_a) {
  const int l = lane_id(), w = wave_id();
  const int R = rows_per_seq(a.mode, a.gamma);
  const int gamma = static_cast<int>(a.gamma);
  const int nw = blockDim.x / kWave;
  // wave 0, lanes < gamma: the draft token and its uniform, issued first (they depend on
  // nothing); then every partial of the sequence this wave merges, all through one buffer
  // descriptor with out-of-range lanes, so no load waits behind a branch
  int32_t x = -1;
  float uu = 0.f;
  if (w == 0 && l < gamma) {
    x = a.tokens[b * a.gamma + l];
    if (a.mode != 0) uu = a.u[b * a.gamma + l];
  }
  const rsrc_t prs = make_rsrc(a.partials + b * R * a.S, static_cast<uint32_t>(R * a.S) * sizeof(Partial));
  int span = 1;
  while (span < a.S) span <<= 1;
  constexpr int kAccBatch = 4;
  for (int r0 = w; r0 < R; r0 += nw * kAccBatch) {
    uint4 raw[kAccBatch][2];
#pragma unroll
    for (int j = 0; j < kAccBatch; ++j) {
      const int r = r0 + j * nw;
      const uint32_t off = (r < R && l < a.S) ? static_cast<uint32_t>(r * a.S + l) * sizeof(Partial) : kOutOfRange;
      raw[j][0] = buffer_load16(prs, off);
      raw[j][1] = buffer_load16(prs, off == kOutOfRange ? kOutOfRange : off + 16);
    }
#pragma unroll
    for (int j = 0; j < kAccBatch; ++j) {
      const int r = r0 + j * nw;
      Partial p = partial_empty();
      if (r < R && l < a.S) {   // selects on loaded values, not a guard of the loads
        p.m = __uint_as_float(raw[j][0].x);
        p.s = __uint_as_float(raw[j][0].y);
        p.gscore = __uint_as_float(raw[j][0].z);
        p.g = static_cast<int32_t>(raw[j][0].w);
        p.zmax = __uint_as_float(raw[j][1].x);
        p.zid = static_cast<int32_t>(raw[j][1].y);
        p.xz = __uint_as_float(raw[j][1].z);
        p.pad1 = __uint_as_float(raw[j][1].w);
      }
      // butterfly over the first `span` lanes only (span = S rounded up to a power of two):
      // lanes past S hold empty records, and every kernel merges in this same order
      float xz = p.xz;   // one segment at most holds a finite value
      float qx = l < a.S ? p.pad1 : -1.f;   // sparse draft: segment 0 holds it
#pragma unroll
      for (int sh = 32; sh >= 1; sh >>= 1) {
        if (sh >= span) continue;
        xz = fmaxf(xz, xor_lane(xz, sh));
        qx = fmaxf(qx, xor_lane(qx, sh));
        Partial o;
        o.m = xor_lane(p.m, sh);
        o.s = xor_lane(p.s, sh);
        o.gscore = xor_lane(p.gscore, sh);
        o.g = xor_lane(p.g, sh);
        o.zmax = xor_lane(p.zmax, sh);
        o.zid = xor_lane(p.zid, sh);
        partial_merge(p, o);
      }
      if (l == 0 && r < R) {
        p.xz = xz;
        p.pad1 = qx;
        rowp[r] = p;
      }
    }
  }
  __syncthreads();
  if (w == 0) {
    bool acc = false;
    if (l < gamma) {
      const bool valid = x >= 0 && x < a.V;
      if (a.mode == 0) {
        acc = valid && x == rowp[l].zid;
      } else if (a.mode == 2) {
        // q_t(x) = 0 makes p/q infinite: accepted whenever p_t(x) > 0 (in double precision:
        // log p above the logarithm of the smallest subnormal)
        const float lp = rowp[l].xz * a.invT - (rowp[l].m + logf(rowp[l].s));
        const float qx = rowp[l].pad1;
        acc = valid && (qx > 0.f ? uu < expf(lp - logf(qx)) : lp > -745.13f);
      } else if (valid) {
        const float yp = rowp[l].xz * a.invT;
        const float yq = rowp[gamma + 1 + l].xz * a.invT;
        const float lp = yp - (rowp[l].m + logf(rowp[l].s));
        const float lq = yq - (rowp[gamma + 1 + l].m + logf(rowp[gamma + 1 + l].s));
        acc = uu < expf(lp - lq);
      }
    }
    const uint64_t rej = __ballot(!acc);   // lanes >= gamma count as rejections
    const int first = rej == 0ull ? kWave : static_cast<int>(__builtin_ctzll(rej));
    if (l == 0) *sh_a = first < gamma ? first : gamma;
  }
  __syncthreads();
  return *sh_a;
}

constexpr int kMaxVerifyRows = 2 * 64 + 1;
constexpr int kResidGroups = 1024;   // groups of a residual segment handled per round
constexpr int kSparseRoundGroups = 128;   // the same with a sparse draft (q of the span in LDS)

// Residual group scores of one vocabulary segment of the rejected position (sampling only):
// per group log2 of sum max(0, p - q), with p = exp2(z_p c - lse_p log2 e) and q likewise
// (dense draft), or q from the candidate list, scattered into LDS one round at a time
// (sparse draft: zero outside the candidates).
template <bool BF16, bool SPARSE>
__global__ __launch_bounds__(256) void k_verify_resid(VerifyArgs a) {
  constexpr int EPT = BF16 ? 8 : 4;
  constexpr int LPG = kGroup / EPT;
  constexpr uint32_t ES = BF16 ? 2 : 4;
  // chunks of each row per thread per pipeline step: one for dense rows (five steps over a
  // Qwen-sized segment; two chunks per step measured 15.3 against 14.4 us, five 20.6)
  constexpr int UNR = SPARSE ? 2 : 1;
  constexpr int RG = SPARSE ? kSparseRoundGroups : kResidGroups;   // groups per round
  __shared__ Partial rowp[kMaxVerifyRows];
  __shared__ Partial red4[4];
  __shared__ int sh_a;
  __shared__ float gw[RG];                             // log2 weight of each group of the round
  __shared__ float gg[RG];                             // Gumbel of each group of the round
  __shared__ float qs[SPARSE ? RG * kGroup : 1];       // sparse draft: q over the round's span
  const int s2 = blockIdx.x;
  const int64_t b = blockIdx.y;
  const int l = lane_id();
  const uint32_t tid = threadIdx.x;
  const int gamma = static_cast<int>(a.gamma);
  const int acc_len = seq_accept<BF16>(a, b, rowp, &sh_a);
  // rejected at a: residual max(0, p_a - q_a); all accepted: the bonus draw from p_gamma
  const bool bonus = acc_len == gamma;
  const char* prow = static_cast<const char*>(row_ptr<BF16>(a, b, acc_len));
  const char* qrow = (bonus || SPARSE) ? prow : static_cast<const char*>(row_ptr<BF16>(a, b, gamma + 1 + acc_len));
  const bool qdense = !bonus && !SPARSE;
  const float c = a.invT * kLog2e;
  const float Lp = bonus ? 0.f : (rowp[acc_len].m + logf(rowp[acc_len].s)) * kLog2e;
  const float Lq = qdense ? (rowp[gamma + 1 + acc_len].m + logf(rowp[gamma + 1 + acc_len].s)) * kLog2e : 0.f;
  const uint32_t purpose = bonus ? kBonusGroup : kResidGroup;
  const int64_t NG = (a.V + kGroup - 1) / kGroup;
  const int64_t GPS = (NG + a.S2 - 1) / a.S2;
  const int64_t e_begin = s2 * GPS * kGroup;
  const int64_t e_end = min(a.V, (s2 + 1) * GPS * kGroup);
  const uint32_t n = e_end > e_begin ? static_cast<uint32_t>(e_end - e_begin) : 0u;
  const rsrc_t rp = make_rsrc(prow + static_cast<size_t>(e_begin) * ES, n * ES);
  const rsrc_t rq = make_rsrc(qrow + static_cast<size_t>(e_begin) * ES, n * ES);
  Partial best = partial_empty();
  const uint32_t step = blockDim.x * EPT;
  // p and q chunks interleaved in one buffer: [2u] from p, [2u + 1] from q
  auto load = [&](uint4 (&buf)[2 * UNR], uint32_t base) {
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const uint32_t e = base + u * step + tid * EPT;
      buf[2 * u] = buffer_load16(rp, e < n ? e * ES : kOutOfRange);
      buf[2 * u + 1] = buffer_load16(rq, (e < n && qdense) ? e * ES : kOutOfRange);
    }
  };
  // sparse draft: the candidate list of position acc_len, read once into registers when it
  // has at most kQReg entries per thread (one round trip; the rounds below only scatter)
  constexpr int kQReg = 8;
  int32_t qid[kQReg];
  float qpr[kQReg];
  const bool qreg = SPARSE && !bonus && a.k <= static_cast<int64_t>(kQReg) * blockDim.x;
  if constexpr (SPARSE) {
    if (qreg) {
      const int64_t base = (b * a.gamma + acc_len) * a.k;
      const rsrc_t ri = make_rsrc(a.qidx + base, static_cast<uint32_t>(a.k) * 4u);
      const rsrc_t rpq = make_rsrc(a.qprob + base, static_cast<uint32_t>(a.k) * 4u);
#pragma unroll
      for (int j = 0; j < kQReg; ++j) {
        const uint32_t idx = j * blockDim.x + tid;
        const bool ok = idx < static_cast<uint64_t>(a.k);
        const uint32_t rid = buffer_load4(ri, ok ? idx * 4u : kOutOfRange);
        const uint32_t rpr = buffer_load4(rpq, ok ? idx * 4u : kOutOfRange);
        qid[j] = ok ? static_cast<int32_t>(rid) : -1;
        qpr[j] = __uint_as_float(rpr);
      }
    }
  }
  // the segment's groups in rounds of kResidGroups: first their log2 weights into LDS ...
  const int64_t g_first = e_begin / kGroup;
  for (uint32_t r0 = 0; r0 < n; r0 += RG * kGroup) {
    const uint32_t rn = n - r0 < RG * kGroup ? n - r0 : RG * kGroup;
    if constexpr (SPARSE) {
      if (!bonus) {
        for (uint32_t i = tid; i < rn; i += blockDim.x) qs[i] = 0.f;
        __syncthreads();
        const int64_t lo = e_begin + r0, hi = lo + rn;
        if (qreg) {
#pragma unroll
          for (int j = 0; j < kQReg; ++j)
            if (qid[j] >= lo && qid[j] < hi) qs[qid[j] - lo] = qpr[j];
        } else {
          const int64_t base = (b * a.gamma + acc_len) * a.k;
          for (int64_t j = tid; j < a.k; j += blockDim.x) {
            const int32_t id = a.qidx[base + j];
            if (id >= lo && id < hi) qs[id - lo] = a.qprob[base + j];
          }
        }
        __syncthreads();
      }
    }
    const int64_t ga = g_first + r0 / kGroup;                 // first group of the round
    const int64_t gb = ga + (rn + kGroup - 1) / kGroup;       // one past the last
    // the round's group Gumbels depend only on (seed, offset, purpose, b, group): one Philox
    // block per four consecutive groups, computed while the round's first loads are in flight
    auto gumbels = [&] {
      for (int64_t q = ga / 4 + tid; q * 4 < gb; q += blockDim.x) {
        uint64_t words[4];
        philox_block(a.seed, a.offset, purpose, static_cast<uint64_t>(b), static_cast<uint64_t>(q) * 4, words);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int64_t gi = q * 4 + j;
          if (gi >= ga && gi < gb) gg[gi - ga] = gumbel(word_to_uniform(words[j]));
        }
      }
    };
    pipelined<2 * UNR>(rn, step * UNR, [&](uint4 (&buf)[2 * UNR], uint32_t base) { load(buf, r0 + base); },
                       [&](uint4 (&buf)[2 * UNR], uint32_t base) {
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const uint32_t e = base + u * step + tid * EPT;   // relative to r0
        const bool in = e < rn;
        float vp[EPT], vq[EPT];
        unpack<BF16>(buf[2 * u], vp);
        unpack<BF16>(buf[2 * u + 1], vq);
        float gr = 0.f, gm = 0.f;   // group weight = 2^gm * gr
        if (bonus) {
          // log-sum-exp of the group's y values (base 2), max-shifted over its LPG lanes
          gm = in ? chunk_max<EPT>(vp) * c : -INFINITY;
#pragma unroll
          for (int o = 1; o < LPG; o <<= 1) gm = fmaxf(gm, xor_lane(gm, o));
          if (in) {
#pragma unroll
            for (int i = 0; i < EPT; ++i) gr += fast_exp2(fmaf(vp[i], c, -gm));
          }
        } else if (in) {
          if constexpr (SPARSE) {
#pragma unroll
            for (int i = 0; i < EPT; ++i) vq[i] = qs[e + i];
#pragma unroll
            for (int i = 0; i < EPT; ++i) gr += fmaxf(fast_exp2(fmaf(vp[i], c, -Lp)) - vq[i], 0.f);
          } else {
#pragma unroll
            for (int i = 0; i < EPT; ++i)
              gr += fmaxf(fast_exp2(fmaf(vp[i], c, -Lp)) - fast_exp2(fmaf(vq[i], c, -Lq)), 0.f);
          }
        }
#pragma unroll
        for (int o = 1; o < LPG; o <<= 1) gr += xor_lane(gr, o);
        if (in && (l % LPG) == 0) gw[e / kGroup] = gr > 0.f ? gm + log2f(gr) : -INFINITY;
      }
    }, gumbels);
    __syncthreads();
    // ... then the group scores L_g + Gumbel(u_g), all threads at once
    for (int64_t gi = ga + tid; gi < gb; gi += blockDim.x) {
      const float lw = gw[gi - ga];
      if (lw != -INFINITY) argmax_merge(best.gscore, best.g, lw * kLn2 + gg[gi - ga], static_cast<int32_t>(gi));
    }
    __syncthreads();   // gw and gg are rewritten by the next round
  }
  block_argmax(best.gscore, best.g, red4);   // only the group draw is carried
  if (threadIdx.x == 0) {
    a.partials2[b * (a.S2 + 1) + s2] = best;
    if (s2 == 0) {
      // the sequence's acceptance for the finish kernel: accept count and the two lse
      Partial rec = partial_empty();
      rec.g = acc_len;
      rec.m = Lp;
      rec.s = Lq;
      a.partials2[b * (a.S2 + 1) + a.S2] = rec;
    }
  }
}

// One workgroup per sequence: the accepted prefix, the last token, the outputs.
template <bool BF16>
__global__ __launch_bounds__(256) void k_verify_finish(VerifyArgs a) {
  constexpr int EPT = BF16 ? 8 : 4;
  constexpr uint32_t ES = BF16 ? 2 : 4;
  __shared__ Partial rowp[kMaxVerifyRows];
  __shared__ Partial red4[4];
  __shared__ int sh_a;
  const int64_t b = blockIdx.x;
  const int l = lane_id(), w = wave_id();
  const int gamma = static_cast<int>(a.gamma);
  __shared__ float qg[kGroup];   // sparse draft: q over the winning residual group
  // sampling: the residual kernel recorded the acceptance (count, lse of p_a and q_a);
  // greedy: merge the row partials here
  int acc_len;
  float Lp = 0.f, Lq = 0.f;
  Partial best = partial_empty();
  if (a.mode != 0) {
    const Partial rec = a.partials2[b * (a.S2 + 1) + a.S2];
    acc_len = rec.g;
    Lp = rec.m;
    Lq = rec.s;
    // residual or bonus group winner from the residual kernel's segments
    best = l < a.S2 ? a.partials2[b * (a.S2 + 1) + l] : partial_empty();
    wave_argmax(best.gscore, best.g);   // argmax merges: exact in any order
  } else {
    acc_len = seq_accept<BF16>(a, b, rowp, &sh_a);
  }
  const bool resid = a.mode != 0 && acc_len < gamma;
  const bool qdense = resid && a.mode == 1;
  const char* prow = static_cast<const char*>(row_ptr<BF16>(a, b, acc_len));
  const char* qrow = qdense ? static_cast<const char*>(row_ptr<BF16>(a, b, gamma + 1 + acc_len)) : nullptr;
  const float c = a.invT * kLog2e;
  if (a.mode == 2 && resid) {
    // the candidates that fall in the winning group (every wave merged the same winner)
    if (threadIdx.x < kGroup) qg[threadIdx.x] = 0.f;
    __syncthreads();
    if (best.g != 0x7fffffff) {
      const int64_t lo = static_cast<int64_t>(best.g) * kGroup;
      const int64_t base = (b * a.gamma + acc_len) * a.k;
      scan_candidates(a.qidx + base, a.k, [&](int64_t j, int32_t id) {
        if (id >= lo && id < lo + kGroup) qg[id - lo] = a.qprob[base + j];
      });
    }
    __syncthreads();
  }
  const bool fallback = resid && best.gscore == -INFINITY;
  if (fallback) {
    // no residual mass anywhere (p <= q everywhere): draw from p at this position, scanning
    // the whole row here (a degenerate case, never on the common path)
    const int64_t NG = (a.V + kGroup - 1) / kGroup;
    const rsrc_t rp = make_rsrc(prow, static_cast<uint32_t>(a.V) * ES);
    Partial f = partial_empty();
    for (int64_t g = threadIdx.x; g < NG; g += blockDim.x) {
      float gm = -INFINITY, gs = 0.f;
      for (int q = 0; q < kGroup / EPT; ++q) {
        const int64_t e = g * kGroup + q * EPT;
        if (e >= a.V) break;
        float v[EPT];
        unpack<BF16>(buffer_load16(rp, static_cast<uint32_t>(e) * ES), v);
        const float cm = chunk_max<EPT>(v) * c;
        const float mn = fmaxf(gm, cm);
        float cs = 0.f;
#pragma unroll
        for (int i = 0; i < EPT; ++i) cs += exp2f(fmaf(v[i], c, -mn));
        gs = gs * exp2f(gm - mn) + cs;
        gm = mn;
      }
      const float sc = (gm + log2f(gs)) * kLn2 + gumbel(philox_uniform(a.seed, a.offset, kResidGroup, b, g));
      argmax_merge(f.gscore, f.g, sc, static_cast<int32_t>(g));
    }
    f = block_merge(f, red4);
    best.zmax = f.gscore;
    best.zid = f.g;
  }
  if (w != 0) return;
  int32_t tok;
  if (a.mode == 0) {
    tok = rowp[acc_len].zid;
  } else if (!resid) {
    tok = draw_in_group<BF16>(best.g, a.V, a.seed, a.offset, kBonusElem, b,
                              [&](int64_t i) { return load_logit<BF16>(prow, i) * a.invT; });
  } else if (!fallback) {
    tok = draw_in_group<BF16>(best.g, a.V, a.seed, a.offset, kResidElem, b, [&](int64_t i) {
      const float qi = qdense ? fast_exp2(fmaf(load_logit<BF16>(qrow, i), c, -Lq))
                              : qg[i - static_cast<int64_t>(best.g) * kGroup];
      const float rr = fmaxf(fast_exp2(fmaf(load_logit<BF16>(prow, i), c, -Lp)) - qi, 0.f);
      return rr > 0.f ? logf(rr) : -INFINITY;
    });
  } else {
    tok = draw_in_group<BF16>(best.zid, a.V, a.seed, a.offset, kResidElem, b,
                              [&](int64_t i) { return load_logit<BF16>(prow, i) * a.invT; });
  }
  for (int t = l; t <= gamma; t += kWave) {
    int32_t o = -1;
    if (t < acc_len)
      o = a.tokens[b * a.gamma + t];
    else if (t == acc_len)
      o = tok;
    a.out_tokens[b * (a.gamma + 1) + t] = o;
  }
  if (l == 0) a.accept_len[b] = acc_len;
}

// Greedy verification of a candidate tree (phrase-level speculation page, "更换单元：从
// token 到短语": the candidates of a round form a prefix tree scored in one target pass, and a
// node survives only where it equals the target's own argmax).  One workgroup per tree of
// N = gamma + 1 nodes, one thread per node: node n is accepted when its parent p (in [0, n))
// is accepted and its token equals the argmax of p's target row; pointer jumping over the
// parent links gives every node "all links to the root match" and its depth in log2 N rounds;
// the deepest accepted node (lowest index on ties) ends the path, followed by its argmax.
__global__ __launch_bounds__(kMaxTreeNodes) void k_tree_finish(VerifyArgs a) {
  __shared__ int32_t g[kMaxTreeNodes];     // argmax of each node's target row
  __shared__ int32_t anc[kMaxTreeNodes];   // current jump target (0 = the root)
  __shared__ int32_t dep[kMaxTreeNodes];   // links summed so far
  __shared__ int32_t okf[kMaxTreeNodes];   // every link summed so far matches
  __shared__ int32_t red_k[kMaxTreeNodes / kWave], red_n[kMaxTreeNodes / kWave];
  const int64_t b = blockIdx.x;
  const int N = static_cast<int>(a.gamma + 1);
  const int l = lane_id(), w = wave_id(), nw = blockDim.x / kWave;
  const int n = threadIdx.x;
  for (int r = w; r < N; r += nw) {
    Partial p = l < a.S ? a.partials[(b * N + r) * a.S + l] : partial_empty();
    wave_argmax(p.zmax, p.zid);   // greedy rows: only the argmax is needed
    if (l == 0) g[r] = p.zid;
  }
  int32_t par = 0, tok = 0;
  if (n < N) {
    par = a.parent[b * N + n];
    tok = a.tokens[b * N + n];
  }
  __syncthreads();
  if (n < N) {
    const bool valid = n > 0 && par >= 0 && par < n;
    anc[n] = valid ? par : 0;
    dep[n] = n > 0 ? 1 : 0;
    okf[n] = n == 0 ? 1 : (valid && tok == g[par] ? 1 : 0);
  }
  __syncthreads();
  for (int span = 1; span < N; span <<= 1) {
    int32_t a2 = 0, d2 = 0, o2 = 1;
    if (n < N) {
      const int32_t up = anc[n];
      a2 = anc[up];
      d2 = dep[n] + dep[up];
      o2 = okf[n] & okf[up];
    }
    __syncthreads();
    if (n < N) {
      anc[n] = a2;
      dep[n] = d2;
      okf[n] = o2;
    }
    __syncthreads();
  }
  // deepest accepted node, lowest index on ties (the root, depth 0, is always accepted)
  int32_t key = (n < N && okf[n]) ? dep[n] : -1, id = n;
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) {
    const int32_t k2 = __shfl_xor(key, s), i2 = __shfl_xor(id, s);
    if (k2 > key || (k2 == key && i2 < id)) {
      key = k2;
      id = i2;
    }
  }
  if (l == 0) {
    red_k[w] = key;
    red_n[w] = id;
  }
  __syncthreads();
  int32_t best = red_n[0], bdep = red_k[0];
  for (int i = 1; i < nw; ++i)
    if (red_k[i] > bdep || (red_k[i] == bdep && red_n[i] < best)) {
      bdep = red_k[i];
      best = red_n[i];
    }
  int32_t* out = a.out_tokens + b * N;
  if (n < N && n > bdep) out[n] = -1;
  if (n == 0) {
    // the path, leaf to root: node m sits at position depth(m) - 1
    int32_t m = best;
    for (int t = bdep - 1; t >= 0; --t) {
      out[t] = a.tokens[b * N + m];
      m = a.parent[b * N + m];
    }
    out[bdep] = g[best];
    a.accept_len[b] = bdep;
    a.accept_node[b] = best;
  }
}

hipError_t launch_verify_tree(const VerifyArgs& a, hipStream_t st) {
  const int N = static_cast<int>(a.gamma + 1);
  if (N < 1 || N > kMaxTreeNodes || a.mode != 0) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(a.S), static_cast<unsigned>(N), static_cast<unsigned>(a.B));
  {
    TraceScope ts("verify_rows", st);
    if (a.bf16)
      hipLaunchKernelGGL((k_verify_rows<true, true, 4>), grid, dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL((k_verify_rows<false, true, 4>), grid, dim3(256), 0, st, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  TraceScope ts("tree_finish", st);
  hipLaunchKernelGGL(k_tree_finish, dim3(static_cast<unsigned>(a.B)), dim3(kMaxTreeNodes), 0, st, a);
  return hipGetLastError();
}

int verify_segments(int64_t B, int64_t gamma, int64_t V, int mode) {
  const int64_t R = verify_rows_per_seq(mode, gamma);
  const int64_t NG = (V + kGroup - 1) / kGroup;
  int64_t S = (256 + B * R - 1) / (B * R);
  if (S > 64) S = 64;
  if (S > NG) S = NG;
  if (S < 1) S = 1;
  return static_cast<int>(S);
}

int verify_resid_segments(int64_t B, int64_t V, int mode) {
  if (mode == 0) return 1;
  const int64_t NG = (V + kGroup - 1) / kGroup;
  int64_t S = (1024 + B - 1) / B;
  if (S > 64) S = 64;
  if (S > NG) S = NG;
  if (S < 1) S = 1;
  return static_cast<int>(S);
}

hipError_t launch_verify(const VerifyArgs& a, hipStream_t st) {
  const int R = static_cast<int>(verify_rows_per_seq(a.mode, a.gamma));
  const dim3 grid(static_cast<unsigned>(a.S), static_cast<unsigned>(R), static_cast<unsigned>(a.B));
  {
    TraceScope ts("verify_rows", st);
    if (a.mode == 0) {
      if (a.bf16)
        hipLaunchKernelGGL((k_verify_rows<true, true, 2>), grid, dim3(256), 0, st, a);
      else
        hipLaunchKernelGGL((k_verify_rows<false, true, 2>), grid, dim3(256), 0, st, a);
    } else if (a.mode == 1) {
      if (a.bf16)
        hipLaunchKernelGGL((k_verify_rows<true, false, 2>), grid, dim3(256), 0, st, a);
      else
        hipLaunchKernelGGL((k_verify_rows<false, false, 2>), grid, dim3(256), 0, st, a);
    } else {
      if (a.bf16)
        hipLaunchKernelGGL((k_verify_rows<true, false, 4>), grid, dim3(256), 0, st, a);
      else
        hipLaunchKernelGGL((k_verify_rows<false, false, 4>), grid, dim3(256), 0, st, a);
    }
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.mode != 0) {
    const dim3 grid2(static_cast<unsigned>(a.S2), static_cast<unsigned>(a.B));
    TraceScope ts("verify_resid", st);
    if (a.mode == 2) {
      if (a.bf16)
        hipLaunchKernelGGL((k_verify_resid<true, true>), grid2, dim3(256), 0, st, a);
      else
        hipLaunchKernelGGL((k_verify_resid<false, true>), grid2, dim3(256), 0, st, a);
    } else {
      if (a.bf16)
        hipLaunchKernelGGL((k_verify_resid<true, false>), grid2, dim3(256), 0, st, a);
      else
        hipLaunchKernelGGL((k_verify_resid<false, false>), grid2, dim3(256), 0, st, a);
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  TraceScope ts("verify_finish", st);
  if (a.bf16)
    hipLaunchKernelGGL(k_verify_finish<true>, dim3(static_cast<unsigned>(a.B)), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(k_verify_finish<false>, dim3(static_cast<unsigned>(a.B)), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace sh
