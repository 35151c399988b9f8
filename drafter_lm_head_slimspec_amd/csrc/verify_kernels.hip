// Batched speculative verification (explainer sections "小模型起草，大模型批改" and
// "为什么答案不会变"; SpecTr-GBV write-up, "第三步").
//   k_verify_rows      one pass over every target / draft logit row, split in S segments:
//                      online log-sum-exp of y = z/T, argmax of z, and for the bonus row the
//                      group-Gumbel scores of the two-level draw
//   k_verify_finalize  one workgroup per sequence: acceptance (u < p/q or x == argmax),
//                      leading-accept count, residual draw norm(max(0, p - q)) at the first
//                      rejection or the bonus draw, output assembly
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
  return mode == 0 ? static_cast<int>(gamma + 1) : static_cast<int>(2 * gamma + 1);
}

template <bool BF16>
__device__ __forceinline__ const void* row_ptr(const VerifyArgs& a, int64_t b, int r) {
  const size_t es = BF16 ? 2 : 4;
  if (r <= a.gamma)
    return static_cast<const char*>(a.target) + static_cast<size_t>((b * (a.gamma + 1) + r) * a.V) * es;
  const int64_t t = r - (a.gamma + 1);
  return static_cast<const char*>(a.draft) + static_cast<size_t>((b * a.gamma + t) * a.V) * es;
}

// block-wide fixed-order merge of one Partial per thread; result valid in thread 0
__device__ __forceinline__ Partial block_merge(Partial p, Partial* red4) {
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) {
    Partial q;
    q.m = xor_lane(p.m, s);
    q.s = xor_lane(p.s, s);
    q.gscore = xor_lane(p.gscore, s);
    q.g = xor_lane(p.g, s);
    q.zmax = xor_lane(p.zmax, s);
    q.zid = xor_lane(p.zid, s);
    partial_merge(p, q);
  }
  const int w = wave_id(), nw = blockDim.x / kWave;
  if (lane_id() == 0) red4[w] = p;
  __syncthreads();
  Partial r = red4[0];
  for (int i = 1; i < nw; ++i) partial_merge(r, red4[i]);
  __syncthreads();
  return r;
}

template <bool BF16>
__global__ __launch_bounds__(256) void k_verify_rows(VerifyArgs a) {
  constexpr int EPT = BF16 ? 8 : 4;
  constexpr int LPG = kGroup / EPT;
  __shared__ Partial red4[4];
  const int s = blockIdx.x, r = blockIdx.y;
  const int64_t b = blockIdx.z;
  const int R = rows_per_seq(a.mode, a.gamma);
  const void* row = row_ptr<BF16>(a, b, r);
  const int64_t NG = (a.V + kGroup - 1) / kGroup;
  const int64_t GPS = (NG + a.S - 1) / a.S;
  const int64_t g0 = s * GPS;
  const int64_t g1 = min(NG, g0 + GPS);
  const int64_t e_begin = g0 * kGroup;
  const int64_t e_end = min(a.V, g1 * kGroup);
  const bool bonus = (a.mode == 1) && (r == a.gamma);
  const int l = lane_id();
  Partial p = partial_empty();
  const int64_t span = static_cast<int64_t>(blockDim.x) * EPT;
  const int64_t iters = e_end > e_begin ? (e_end - e_begin + span - 1) / span : 0;
  for (int64_t it = 0; it < iters; ++it) {
    const int64_t e0 = e_begin + it * span + static_cast<int64_t>(threadIdx.x) * EPT;
    const bool in = e0 < e_end;
    float v[EPT];
    if (in) {
      unpack<BF16>(load16(static_cast<const char*>(row) + static_cast<size_t>(e0) * (BF16 ? 2 : 4)), v);
    }
    float lmax = -INFINITY, lsum = 0.f;
    if (in) {
#pragma unroll
      for (int i = 0; i < EPT; ++i) {
        argmax_merge(p.zmax, p.zid, v[i], static_cast<int32_t>(e0 + i));
        lmax = fmaxf(lmax, v[i] * a.invT);
      }
#pragma unroll
      for (int i = 0; i < EPT; ++i) lsum += __expf(v[i] * a.invT - lmax);
      lse_merge(p.m, p.s, lmax, lsum);
    }
    if (bonus) {
      // group = LPG consecutive lanes; reduce (max, sum) inside the group
      float gm = lmax;
#pragma unroll
      for (int o = 1; o < LPG; o <<= 1) gm = fmaxf(gm, xor_lane(gm, o));
      float gs = (in && gm != -INFINITY) ? lsum * __expf(lmax - gm) : 0.f;
#pragma unroll
      for (int o = 1; o < LPG; o <<= 1) gs += xor_lane(gs, o);
      if (in && (l % LPG) == 0) {
        const int64_t gi = e0 / kGroup;
        const float L = gm + logf(gs);
        const float sc = L + gumbel(philox_uniform(a.seed, a.offset, kBonusGroup, b, gi));
        argmax_merge(p.gscore, p.g, sc, static_cast<int32_t>(gi));
      }
    }
  }
  Partial out = block_merge(p, red4);
  if (threadIdx.x == 0) a.partials[(b * R + r) * a.S + s] = out;
}

template <bool BF16>
__global__ __launch_bounds__(256) void k_verify_finalize(VerifyArgs a) {
  constexpr int EPT = BF16 ? 8 : 4;
  constexpr int LPG = kGroup / EPT;
  constexpr int kMaxRows = 2 * 64 + 1;
  __shared__ Partial rowp[kMaxRows];
  __shared__ Partial red4[4];
  __shared__ int sh_a;
  __shared__ int32_t sh_tok;
  const int64_t b = blockIdx.x;
  const int l = lane_id(), w = wave_id();
  const int R = rows_per_seq(a.mode, a.gamma);
  const int gamma = static_cast<int>(a.gamma);
  // 1. per-row totals from the segment partials (fixed order)
  for (int r = w; r < R; r += blockDim.x / kWave) {
    if (l == 0) {
      Partial p = a.partials[(b * R + r) * a.S];
      for (int i = 1; i < a.S; ++i) partial_merge(p, a.partials[(b * R + r) * a.S + i]);
      rowp[r] = p;
    }
  }
  __syncthreads();
  // 2. acceptance and leading-accept count
  if (threadIdx.x == 0) {
    int acc_len = gamma;
    for (int t = 0; t < gamma; ++t) {
      const int32_t x = a.tokens[b * a.gamma + t];
      const bool valid = x >= 0 && x < a.V;
      bool acc;
      if (a.mode == 0) {
        acc = valid && x == rowp[t].zid;
      } else if (!valid) {
        acc = false;
      } else {
        const float yp = load_logit<BF16>(row_ptr<BF16>(a, b, t), x) * a.invT;
        const float yq = load_logit<BF16>(row_ptr<BF16>(a, b, gamma + 1 + t), x) * a.invT;
        const float lp = yp - (rowp[t].m + logf(rowp[t].s));
        const float lq = yq - (rowp[gamma + 1 + t].m + logf(rowp[gamma + 1 + t].s));
        const float ratio = expf(lp - lq);
        acc = a.u[b * a.gamma + t] < ratio;
      }
      if (!acc) {
        acc_len = t;
        break;
      }
    }
    sh_a = acc_len;
  }
  __syncthreads();
  const int acc_len = sh_a;
  int32_t tok = 0;
  if (a.mode == 0) {
    tok = rowp[acc_len].zid;
  } else if (acc_len == gamma) {
    // bonus: draw inside the winning group of p_gamma
    if (w == 0) {
      const void* row = row_ptr<BF16>(a, b, gamma);
      const int64_t i = static_cast<int64_t>(rowp[gamma].g) * kGroup + l;
      const bool valid = i < a.V;
      float e = valid ? load_logit<BF16>(row, i) * a.invT +
                            gumbel(philox_uniform(a.seed, a.offset, kBonusElem, b, i))
                      : -INFINITY;
      int32_t ei = valid ? static_cast<int32_t>(i) : 0x7fffffff;
      wave_argmax(e, ei);
      if (l == 0) sh_tok = ei;
    }
    __syncthreads();
    tok = sh_tok;
  } else {
    // residual norm(max(0, p_a - q_a)) at the rejected position
    const void* prow = row_ptr<BF16>(a, b, acc_len);
    const void* qrow = row_ptr<BF16>(a, b, gamma + 1 + acc_len);
    const float lse_p = rowp[acc_len].m + logf(rowp[acc_len].s);
    const float lse_q = rowp[gamma + 1 + acc_len].m + logf(rowp[gamma + 1 + acc_len].s);
    const int64_t span = static_cast<int64_t>(blockDim.x) * EPT;
    const int64_t iters = (a.V + span - 1) / span;
    Partial best = partial_empty();
    bool fallback = false;
    for (int pass = 0; pass < 2; ++pass) {   // pass 1 only if the residual mass is zero
      fallback = pass == 1;
      best = partial_empty();
      for (int64_t it = 0; it < iters; ++it) {
        const int64_t e0 = it * span + static_cast<int64_t>(threadIdx.x) * EPT;
        const bool in = e0 < a.V;
        float vp[EPT], vq[EPT];
        float lsum = 0.f, lmax = -INFINITY;
        if (in) {
          unpack<BF16>(load16(static_cast<const char*>(prow) + static_cast<size_t>(e0) * (BF16 ? 2 : 4)), vp);
          if (!fallback) {
            unpack<BF16>(load16(static_cast<const char*>(qrow) + static_cast<size_t>(e0) * (BF16 ? 2 : 4)), vq);
#pragma unroll
            for (int i = 0; i < EPT; ++i)
              lsum += fmaxf(expf(vp[i] * a.invT - lse_p) - expf(vq[i] * a.invT - lse_q), 0.f);
          } else {
#pragma unroll
            for (int i = 0; i < EPT; ++i) lmax = fmaxf(lmax, vp[i] * a.invT);
#pragma unroll
            for (int i = 0; i < EPT; ++i) lsum += __expf(vp[i] * a.invT - lmax);
          }
        }
        float L;
        if (!fallback) {
          float gs = lsum;
#pragma unroll
          for (int o = 1; o < LPG; o <<= 1) gs += xor_lane(gs, o);
          L = gs > 0.f ? logf(gs) : -INFINITY;
        } else {
          float gm = lmax;
#pragma unroll
          for (int o = 1; o < LPG; o <<= 1) gm = fmaxf(gm, xor_lane(gm, o));
          float gs = (in && gm != -INFINITY) ? lsum * __expf(lmax - gm) : 0.f;
#pragma unroll
          for (int o = 1; o < LPG; o <<= 1) gs += xor_lane(gs, o);
          L = gm + logf(gs);
        }
        if (in && (l % LPG) == 0 && L != -INFINITY) {
          const int64_t gi = e0 / kGroup;
          const float sc = L + gumbel(philox_uniform(a.seed, a.offset, kResidGroup, b, gi));
          argmax_merge(best.gscore, best.g, sc, static_cast<int32_t>(gi));
        }
      }
      best = block_merge(best, red4);
      if (best.gscore != -INFINITY) break;
    }
    if (w == 0) {
      // element draw inside the winning group; same arithmetic as the group pass
      const int64_t i = static_cast<int64_t>(best.g) * kGroup + l;
      const bool valid = best.g != 0x7fffffff && i < a.V;
      float ell = -INFINITY;
      if (valid) {
        const float yp = load_logit<BF16>(prow, i) * a.invT;
        if (fallback) {
          ell = yp;
        } else {
          const float yq = load_logit<BF16>(qrow, i) * a.invT;
          const float rr = fmaxf(expf(yp - lse_p) - expf(yq - lse_q), 0.f);
          ell = rr > 0.f ? logf(rr) : -INFINITY;
        }
      }
      float e = ell != -INFINITY ? ell + gumbel(philox_uniform(a.seed, a.offset, kResidElem, b, i)) : -INFINITY;
      int32_t ei = (valid && ell != -INFINITY) ? static_cast<int32_t>(i) : 0x7fffffff;
      wave_argmax(e, ei);
      if (l == 0) sh_tok = ei;
    }
    __syncthreads();
    tok = sh_tok;
  }
  if (threadIdx.x == 0) {
    a.accept_len[b] = acc_len;
    for (int t = 0; t <= gamma; ++t) {
      int32_t o = -1;
      if (t < acc_len)
        o = a.tokens[b * a.gamma + t];
      else if (t == acc_len)
        o = tok;
      a.out_tokens[b * (a.gamma + 1) + t] = o;
    }
  }
}

int verify_segments(int64_t B, int64_t gamma, int64_t V, int mode) {
  const int64_t R = mode == 0 ? gamma + 1 : 2 * gamma + 1;
  const int64_t NG = (V + kGroup - 1) / kGroup;
  int64_t S = (2048 + B * R - 1) / (B * R);
  if (S > 64) S = 64;
  if (S > NG) S = NG;
  if (S < 1) S = 1;
  return static_cast<int>(S);
}

hipError_t launch_verify(const VerifyArgs& a, hipStream_t st) {
  const int R = a.mode == 0 ? static_cast<int>(a.gamma + 1) : static_cast<int>(2 * a.gamma + 1);
  const dim3 grid(static_cast<unsigned>(a.S), static_cast<unsigned>(R), static_cast<unsigned>(a.B));
  {
    TraceScope ts("verify_rows", st);
    if (a.bf16) {
      hipLaunchKernelGGL(k_verify_rows<true>, grid, dim3(256), 0, st, a);
    } else {
      hipLaunchKernelGGL(k_verify_rows<false>, grid, dim3(256), 0, st, a);
    }
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  TraceScope ts("verify_finalize", st);
  if (a.bf16)
    hipLaunchKernelGGL(k_verify_finalize<true>, dim3(static_cast<unsigned>(a.B)), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(k_verify_finalize<false>, dim3(static_cast<unsigned>(a.B)), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace sh
