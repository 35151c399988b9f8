// Drafter LM-head kernels for gfx950.
//
//   k_rowdot        h_r = round(W_down h): the SlimSpec d -> r map (SlimSpec write-up,
//                   section 三) and the SpecVocab d -> d' map (SpecVocab write-up, 2.2.1).
//   k_stream_valu   skinny head product (M <= 8 rows): coalesced 16-byte weight streaming,
//                   one 64-row vocabulary group per wave, fused softmax / argmax /
//                   group-Gumbel statistics.
//   k_stream_mfma   the same contract once the rows make the product dense (M > 8):
//                   v_mfma_f32_32x32x16_bf16, weights HBM -> VGPR, activations in LDS.
//   k_head_finalize fixed-order combine of the per-workgroup partials, row lse, token
//                   (argmax, or the winning group's element draw when sampling).
#include "device_common.h"
#include "launch.h"

namespace sh {

// ----------------------------------------------------------------------------------------
// k_rowdot: workgroup = 4 waves, 8 output rows (2 per wave) x 8 input rows.  The 8 input
// rows are staged in LDS, the weight rows live in registers.
// ----------------------------------------------------------------------------------------
constexpr int kRowdotRows = 8;
constexpr int kRowdotM = 8;
constexpr int kRowdotMaxCPL = 16;   // row bytes <= 16 KB

template <bool BF16>
__global__ __launch_bounds__(256) void k_rowdot(const void* __restrict__ Wd,
                                                const void* __restrict__ x, int R, int C, int M,
                                                void* __restrict__ out) {
  extern __shared__ uint4 xs[];  // [kRowdotM][C]
  const int m0 = blockIdx.y * kRowdotM;
  for (int i = threadIdx.x; i < kRowdotM * C; i += blockDim.x) {
    const int mm = i / C, c = i - mm * C;
    const int m = m0 + mm;
    xs[i] = (m < M) ? load16(static_cast<const char*>(x) + (static_cast<size_t>(m) * C + c) * 16)
                    : zero16();
  }
  __syncthreads();
  const int l = lane_id(), w = wave_id();
  const int j0 = blockIdx.x * kRowdotRows + w * 2;
  const int CPL = (C + kWave - 1) / kWave;
  uint4 wr0[kRowdotMaxCPL], wr1[kRowdotMaxCPL];
#pragma unroll
  for (int q = 0; q < kRowdotMaxCPL; ++q) {
    const int c = q * kWave + l;
    const bool ok = q < CPL && c < C;
    wr0[q] = (ok && j0 < R) ? load16(static_cast<const char*>(Wd) + (static_cast<size_t>(j0) * C + c) * 16)
                            : zero16();
    wr1[q] = (ok && j0 + 1 < R)
                 ? load16(static_cast<const char*>(Wd) + (static_cast<size_t>(j0 + 1) * C + c) * 16)
                 : zero16();
  }
  for (int mm = 0; mm < kRowdotM; ++mm) {
    const int m = m0 + mm;
    if (m >= M) break;
    float a0 = 0.f, a1 = 0.f;
#pragma unroll
    for (int q = 0; q < kRowdotMaxCPL; ++q) {
      const int c = q * kWave + l;
      if (q < CPL && c < C) {
        const uint4 xv = xs[mm * C + c];
        a0 = chunk_dot<BF16>(wr0[q], xv, a0);
        a1 = chunk_dot<BF16>(wr1[q], xv, a1);
      }
    }
    a0 = wave_sum(a0);
    a1 = wave_sum(a1);
    if (l == 0) {
      if constexpr (BF16) {
        uint16_t* o = static_cast<uint16_t*>(out) + static_cast<size_t>(m) * R;
        if (j0 < R) o[j0] = f32_to_bf16_rne(a0);
        if (j0 + 1 < R) o[j0 + 1] = f32_to_bf16_rne(a1);
      } else {
        float* o = static_cast<float*>(out) + static_cast<size_t>(m) * R;
        if (j0 < R) o[j0] = a0;
        if (j0 + 1 < R) o[j0 + 1] = a1;
      }
    }
  }
}

// ----------------------------------------------------------------------------------------
// Workgroup-level combine of per-wave running states into one Partial per row.
// rec: LDS scratch of nwaves * M Partials.  Every wave calls with its lane-m state.
// ----------------------------------------------------------------------------------------
__device__ __forceinline__ void wg_combine_store(Partial* rec, const Partial& mine, bool holds,
                                                 int m_of_lane, int M, Partial* partials,
                                                 int64_t ld) {
  const int w = wave_id(), nw = blockDim.x / kWave;
  if (holds) rec[w * M + m_of_lane] = mine;
  __syncthreads();
  for (int m = threadIdx.x; m < M; m += blockDim.x) {
    Partial p = rec[m];
    for (int i = 1; i < nw; ++i) partial_merge(p, rec[i * M + m]);
    partials[static_cast<int64_t>(m) * ld + blockIdx.x] = p;
  }
}

// ----------------------------------------------------------------------------------------
// k_stream_valu: M <= MB <= 8 rows.
//   A row of the weight matrix is C = K*esize/16 chunks of 16 bytes.  LPR lanes share a row
//   (LPR = 64 when C >= 64, else the next power of two >= C), so one load instruction reads
//   RPI = 64/LPR rows.  A row-block is 8 load-instructions deep; its per-lane partial sums
//   acc[8][MB] are reduced with a halving butterfly so that afterwards each lane holds one
//   finished row (the row-slot given by its top 3 lane bits inside the LPR segment).
// ----------------------------------------------------------------------------------------
template <bool BF16, int MB, int LPR>
__global__ __launch_bounds__(256) void k_stream_valu(StreamArgs a) {
  constexpr int RB = 8;
  constexpr int RPI = kWave / LPR;
  constexpr int ROWS_RB = RB * RPI;
  constexpr int NRB = kGroup / ROWS_RB;
  constexpr int DUP = LPR / RB;
  extern __shared__ uint4 xs[];  // [MB][C] then (after the loop) Partial records
  const int C = static_cast<int>(a.K * (BF16 ? 2 : 4) / 16);
  const int CPL = (C + LPR - 1) / LPR;
  for (int i = threadIdx.x; i < MB * C; i += blockDim.x) {
    const int m = i / C, c = i - m * C;
    xs[i] = (m < a.M) ? load16(static_cast<const char*>(a.x) + (static_cast<size_t>(m) * C + c) * 16)
                      : zero16();
  }
  __syncthreads();

  const int l = lane_id(), w = wave_id();
  const int lr = l % LPR;
  const int ri = l / LPR;
  const int jslot = lr / DUP;
  const bool leader = (lr % DUP) == 0;
  const int64_t NG = (a.V + kGroup - 1) / kGroup;
  const int64_t nwt = static_cast<int64_t>(gridDim.x) * (blockDim.x / kWave);
  const size_t rowbytes = static_cast<size_t>(C) * 16;
  const char* Wb = static_cast<const char*>(a.W);

  uint4 xr[MB];
  if (CPL == 1) {
#pragma unroll
    for (int m = 0; m < MB; ++m) xr[m] = (lr < C) ? xs[m * C + lr] : zero16();
  }

  Partial run = partial_empty();  // lane m holds row m's running state

  for (int64_t g = static_cast<int64_t>(blockIdx.x) * (blockDim.x / kWave) + w; g < NG; g += nwt) {
    float gm[MB], gs[MB], gz[MB];
    int32_t gi[MB];
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      gm[m] = -INFINITY;
      gs[m] = 0.f;
      gz[m] = -INFINITY;
      gi[m] = 0x7fffffff;
    }
#pragma unroll 1
    for (int rb = 0; rb < NRB; ++rb) {
      const int64_t rbase = g * kGroup + rb * ROWS_RB;
      float acc[RB][MB];
#pragma unroll
      for (int j = 0; j < RB; ++j)
#pragma unroll
        for (int m = 0; m < MB; ++m) acc[j][m] = 0.f;
      for (int q = 0; q < CPL; ++q) {
        const int c = q * LPR + lr;
        const bool cok = c < C;
        uint4 xq[MB];
        if (CPL == 1) {
#pragma unroll
          for (int m = 0; m < MB; ++m) xq[m] = xr[m];
        } else {
#pragma unroll
          for (int m = 0; m < MB; ++m) xq[m] = cok ? xs[m * C + c] : zero16();
        }
        uint4 wv[RB];
#pragma unroll
        for (int j = 0; j < RB; ++j) {
          const int64_t row = rbase + j * RPI + ri;
          wv[j] = (cok && row < a.V) ? load16(Wb + static_cast<size_t>(row) * rowbytes + static_cast<size_t>(c) * 16)
                                     : zero16();
        }
#pragma unroll
        for (int j = 0; j < RB; ++j)
#pragma unroll
          for (int m = 0; m < MB; ++m) acc[j][m] = chunk_dot<BF16>(wv[j], xq[m], acc[j][m]);
      }
      // halving butterfly over the top 3 bits of the LPR segment
#pragma unroll
      for (int step = 0; step < 3; ++step) {
        const int n = RB >> step;
        const int s = LPR >> (step + 1);
        const bool upper = (lr & s) != 0;
#pragma unroll
        for (int i = 0; i < (RB >> (step + 1)); ++i) {
#pragma unroll
          for (int m = 0; m < MB; ++m) {
            const float lo = acc[i][m], hi = acc[i + n / 2][m];
            const float send = upper ? lo : hi;
            const float keep = upper ? hi : lo;
            acc[i][m] = keep + __shfl_xor(send, s);
          }
        }
      }
#pragma unroll
      for (int s = LPR >> 4; s >= 1; s >>= 1)
#pragma unroll
        for (int m = 0; m < MB; ++m) acc[0][m] += __shfl_xor(acc[0][m], s);

      const int64_t row = rbase + jslot * RPI + ri;
      const bool valid = row < a.V;
      if (a.zout != nullptr && leader && valid) {
#pragma unroll
        for (int m = 0; m < MB; ++m)
          if (m < a.M) a.zout[static_cast<int64_t>(m) * a.zout_ld + row] = acc[0][m];
      }
      if (a.stats != kStatsNone && valid) {
#pragma unroll
        for (int m = 0; m < MB; ++m) {
          const float z = acc[0][m];
          argmax_merge(gz[m], gi[m], z, static_cast<int32_t>(row));
          if (a.stats >= kStatsLse) lse_merge(gm[m], gs[m], z * a.invT, 1.f);
        }
      }
    }
    if (a.stats != kStatsNone) {
      // combine the distinct rows of the group (lanes differing in bits >= DUP)
#pragma unroll
      for (int s = DUP; s < kWave; s <<= 1) {
#pragma unroll
        for (int m = 0; m < MB; ++m) {
          const float m2 = __shfl_xor(gm[m], s), s2 = __shfl_xor(gs[m], s);
          const float z2 = __shfl_xor(gz[m], s);
          const int32_t i2 = __shfl_xor(gi[m], s);
          lse_merge(gm[m], gs[m], m2, s2);
          argmax_merge(gz[m], gi[m], z2, i2);
        }
      }
      float my_m = -INFINITY, my_s = 0.f, my_z = -INFINITY;
      int32_t my_i = 0x7fffffff;
#pragma unroll
      for (int m = 0; m < MB; ++m)
        if (l == m) {
          my_m = gm[m];
          my_s = gs[m];
          my_z = gz[m];
          my_i = gi[m];
        }
      if (l < a.M) {
        if (a.stats == kStatsSample) {
          const float L = my_m + logf(my_s);
          const float u = philox_uniform(a.seed, a.offset, kDraftGroup, a.row0 + l, g);
          argmax_merge(run.gscore, run.g, L + gumbel(u), static_cast<int32_t>(g));
        }
        lse_merge(run.m, run.s, my_m, my_s);
        argmax_merge(run.zmax, run.zid, my_z, my_i);
      }
    }
  }
  if (a.stats == kStatsNone) return;
  __syncthreads();
  Partial* rec = reinterpret_cast<Partial*>(xs);
  wg_combine_store(rec, run, l < a.M, l, a.M, a.partials, a.partials_ld);
}

// ----------------------------------------------------------------------------------------
// k_stream_mfma: bf16, M <= 32*NCB rows.  Each wave owns one 64-row vocabulary group per
// round, computed as two 32-row tiles with v_mfma_f32_32x32x16_bf16 (A = weight tile from
// HBM straight into registers, B = activations from LDS, pre-swizzled into B-fragment order
// [k-step][column block][lane] so each lane reads one conflict-free 16-byte word).
// Output layout of the 32x32 tile: lane l holds column l%32 and rows
// 8*(v/4) + 4*(l/32) + v%4 for its 16 accumulators v.
// ----------------------------------------------------------------------------------------
template <int NCB>
__global__ __launch_bounds__(256) void k_stream_mfma(StreamArgs a, int KSC) {
  extern __shared__ uint4 bs[];  // [KSC][NCB][64] 16-byte B fragments, later Partial records
  const int l = lane_id(), w = wave_id();
  const int NW = blockDim.x / kWave;
  const int n = l & 31, hf = l >> 5;
  const int K = static_cast<int>(a.K);
  const int KS = (K + 15) / 16;
  const int NKC = (KS + KSC - 1) / KSC;
  const size_t rowbytes = static_cast<size_t>(K) * 2;
  const int64_t NG = (a.V + kGroup - 1) / kGroup;
  const char* xb = static_cast<const char*>(a.x);
  const char* Wb = static_cast<const char*>(a.W);

  auto stage = [&](int kc) {
    const int items = KSC * NCB * kWave;
    for (int it = threadIdx.x; it < items; it += blockDim.x) {
      const int ks = it / (NCB * kWave);
      const int cb = (it / kWave) % NCB;
      const int ll = it & (kWave - 1);
      const int m = cb * 32 + (ll & 31);
      const int k = (kc * KSC + ks) * 16 + (ll >> 5) * 8;
      bs[it] = (m < a.M && k < K) ? load16(xb + (static_cast<size_t>(m) * K + k) * 2) : zero16();
    }
  };

  Partial run[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) run[cb] = partial_empty();

  if (NKC == 1) {
    stage(0);
    __syncthreads();
  }
  for (int64_t round = blockIdx.x; round * NW < NG; round += gridDim.x) {
    const int64_t g = round * NW + w;
    const bool gvalid = g < NG;
    float hm[NCB], hs[NCB], hz[NCB];
    int32_t hi[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      hm[cb] = -INFINITY;
      hs[cb] = 0.f;
      hz[cb] = -INFINITY;
      hi[cb] = 0x7fffffff;
    }
    for (int t = 0; t < 2; ++t) {
      const int64_t tbase = g * kGroup + t * 32;
      f32x16_t acc[NCB];
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[cb][v] = 0.f;
      const int64_t arow = tbase + n;
      const bool arow_ok = gvalid && arow < a.V;
      const char* wrow = Wb + static_cast<size_t>(arow_ok ? arow : 0) * rowbytes;
      for (int kc = 0; kc < NKC; ++kc) {
        if (NKC > 1) {
          __syncthreads();
          stage(kc);
          __syncthreads();
        }
        if (gvalid) {
          const int ks_n = min(KSC, KS - kc * KSC);
#pragma unroll 8
          for (int ks = 0; ks < ks_n; ++ks) {
            const int k = (kc * KSC + ks) * 16 + hf * 8;
            const uint4 av = (arow_ok && k < K) ? load16(wrow + static_cast<size_t>(k) * 2) : zero16();
            const bf16x8_t af = __builtin_bit_cast(bf16x8_t, av);
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
              const bf16x8_t bf = __builtin_bit_cast(bf16x8_t, bs[(ks * NCB + cb) * kWave + l]);
              acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bf, acc[cb], 0, 0, 0);
            }
          }
        }
      }
      if (!gvalid) continue;
      // epilogue: per column (= row m of the call) over this tile's 32 vocabulary rows
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        const int m = cb * 32 + n;
        float zb = -INFINITY, ym = -INFINITY, ss = 0.f;
        int32_t ib = 0x7fffffff;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int64_t row = tbase + 8 * (v >> 2) + 4 * hf + (v & 3);
          if (row < a.V) {
            const float z = acc[cb][v];
            argmax_merge(zb, ib, z, static_cast<int32_t>(row));
            ym = fmaxf(ym, z * a.invT);
            if (a.zout != nullptr && m < a.M) a.zout[static_cast<int64_t>(m) * a.zout_ld + row] = z;
          }
        }
        if (a.stats >= kStatsLse && ym != -INFINITY) {
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int64_t row = tbase + 8 * (v >> 2) + 4 * hf + (v & 3);
            if (row < a.V) ss += __expf(acc[cb][v] * a.invT - ym);
          }
        }
        const float zb2 = __shfl_xor(zb, 32);
        const int32_t ib2 = __shfl_xor(ib, 32);
        const float ym2 = __shfl_xor(ym, 32), ss2 = __shfl_xor(ss, 32);
        argmax_merge(zb, ib, zb2, ib2);
        lse_merge(ym, ss, ym2, ss2);
        lse_merge(hm[cb], hs[cb], ym, ss);
        argmax_merge(hz[cb], hi[cb], zb, ib);
      }
    }
    if (gvalid && a.stats != kStatsNone) {
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        const int m = cb * 32 + n;
        if (m < a.M) {
          if (a.stats == kStatsSample) {
            const float L = hm[cb] + logf(hs[cb]);
            const float u = philox_uniform(a.seed, a.offset, kDraftGroup, a.row0 + m, g);
            argmax_merge(run[cb].gscore, run[cb].g, L + gumbel(u), static_cast<int32_t>(g));
          }
          lse_merge(run[cb].m, run[cb].s, hm[cb], hs[cb]);
          argmax_merge(run[cb].zmax, run[cb].zid, hz[cb], hi[cb]);
        }
      }
    }
  }
  if (a.stats == kStatsNone) return;
  __syncthreads();
  Partial* rec = reinterpret_cast<Partial*>(bs);
  if (hf == 0) {
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      const int m = cb * 32 + n;
      if (m < a.M) rec[w * a.M + m] = run[cb];
    }
  }
  __syncthreads();
  for (int m = threadIdx.x; m < a.M; m += blockDim.x) {
    Partial p = rec[m];
    for (int i = 1; i < NW; ++i) partial_merge(p, rec[i * a.M + m]);
    a.partials[static_cast<int64_t>(m) * a.partials_ld + blockIdx.x] = p;
  }
}

// ----------------------------------------------------------------------------------------
// k_head_finalize: one workgroup per row.
// ----------------------------------------------------------------------------------------
template <bool BF16>
__global__ __launch_bounds__(256) void k_head_finalize(FinalizeArgs f) {
  __shared__ Partial red[256];
  __shared__ float zs[kGroup];
  const int m = blockIdx.x;
  const int l = lane_id(), w = wave_id();
  Partial p = partial_empty();
  for (int i = threadIdx.x; i < f.P; i += blockDim.x) partial_merge(p, f.partials[static_cast<int64_t>(m) * f.partials_ld + i]);
  red[threadIdx.x] = p;
  __syncthreads();
  for (int s = blockDim.x / 2; s >= 1; s >>= 1) {
    if (static_cast<int>(threadIdx.x) < s) {
      Partial q = red[threadIdx.x];
      partial_merge(q, red[threadIdx.x + s]);
      red[threadIdx.x] = q;
    }
    __syncthreads();
  }
  p = red[0];
  const float lse = p.m + logf(p.s);
  int32_t tok;
  float ytok;
  if (f.mode == 0) {
    tok = p.zid;
    ytok = p.zmax * f.invT;
  } else {
    // recompute the 64 logits of the winning group and draw inside it
    const int C = static_cast<int>(f.K * (BF16 ? 2 : 4) / 16);
    const size_t rowbytes = static_cast<size_t>(C) * 16;
    const char* xr = static_cast<const char*>(f.x) + static_cast<size_t>(m) * rowbytes;
    const int64_t gbase = static_cast<int64_t>(p.g) * kGroup;
    for (int j = 0; j < 16; ++j) {
      const int64_t row = gbase + w * 16 + j;
      float z = 0.f;
      if (row < f.V) {
        const char* wr = static_cast<const char*>(f.W) + static_cast<size_t>(row) * rowbytes;
        for (int c = l; c < C; c += kWave) z = chunk_dot<BF16>(load16(wr + c * 16), load16(xr + c * 16), z);
      }
      z = wave_sum(z);
      if (l == 0) zs[w * 16 + j] = z;
    }
    __syncthreads();
    const int64_t row = gbase + l;
    const bool valid = row < f.V;
    const float y = zs[l] * f.invT;
    float e = valid ? y + gumbel(philox_uniform(f.seed, f.offset, kDraftElem, f.row0 + m, row)) : -INFINITY;
    int32_t ei = valid ? l : 0x7fffffff;
    wave_argmax(e, ei);
    tok = static_cast<int32_t>(gbase + ei);
    ytok = __shfl(y, ei);
  }
  if (threadIdx.x == 0) {
    f.token[m] = tok;
    if (f.lse) f.lse[m] = lse;
    if (f.logprob) f.logprob[m] = ytok - lse;
  }
}

// ----------------------------------------------------------------------------------------
// host launchers
// ----------------------------------------------------------------------------------------
hipError_t device_info(DeviceInfo* out) {
  static DeviceInfo cache[64];
  static bool have[64] = {false};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev >= 0 && dev < 64 && have[dev]) {
    *out = cache[dev];
    return hipSuccess;
  }
  DeviceInfo di;
  e = hipDeviceGetAttribute(&di.cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  int lds = 0;
  e = hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
  if (e != hipSuccess) return e;
  di.max_lds = lds;
  if (dev >= 0 && dev < 64) {
    cache[dev] = di;
    have[dev] = true;
  }
  *out = di;
  return hipSuccess;
}

template <typename F>
static hipError_t allow_lds(F kernel, int bytes) {
  if (bytes <= 64 * 1024) return hipSuccess;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                             hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
}

hipError_t launch_rowdot(const void* Wd, const void* x, int64_t R, int64_t K, int64_t M, bool bf16,
                         void* out, hipStream_t st) {
  const int C = static_cast<int>(K * (bf16 ? 2 : 4) / 16);
  const dim3 grid(static_cast<unsigned>((R + kRowdotRows - 1) / kRowdotRows),
                  static_cast<unsigned>((M + kRowdotM - 1) / kRowdotM));
  const int lds = kRowdotM * C * 16;
  hipError_t e;
  if (bf16) {
    e = allow_lds(k_rowdot<true>, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_rowdot<true>, grid, dim3(256), lds, st, Wd, x, static_cast<int>(R), C,
                       static_cast<int>(M), out);
  } else {
    e = allow_lds(k_rowdot<false>, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_rowdot<false>, grid, dim3(256), lds, st, Wd, x, static_cast<int>(R), C,
                       static_cast<int>(M), out);
  }
  return hipGetLastError();
}

template <bool BF16, int MB, int LPR>
static hipError_t run_valu(const StreamArgs& a, int grid, int lds, hipStream_t st) {
  const int rec = 4 * MB * static_cast<int>(sizeof(Partial));
  const int bytes = lds > rec ? lds : rec;
  hipError_t e = allow_lds(k_stream_valu<BF16, MB, LPR>, bytes);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_stream_valu<BF16, MB, LPR>), dim3(grid), dim3(256), bytes, st, a);
  return hipGetLastError();
}

template <bool BF16, int MB>
static hipError_t dispatch_lpr(const StreamArgs& a, int lpr, int grid, int lds, hipStream_t st) {
  switch (lpr) {
    case 8: return run_valu<BF16, MB, 8>(a, grid, lds, st);
    case 16: return run_valu<BF16, MB, 16>(a, grid, lds, st);
    case 32: return run_valu<BF16, MB, 32>(a, grid, lds, st);
    default: return run_valu<BF16, MB, 64>(a, grid, lds, st);
  }
}

template <bool BF16>
static hipError_t dispatch_mb(const StreamArgs& a, int lpr, int grid, int lds, hipStream_t st) {
  if (a.M <= 1) return dispatch_lpr<BF16, 1>(a, lpr, grid, lds, st);
  if (a.M <= 2) return dispatch_lpr<BF16, 2>(a, lpr, grid, lds, st);
  if (a.M <= 4) return dispatch_lpr<BF16, 4>(a, lpr, grid, lds, st);
  if (a.M <= 6) return dispatch_lpr<BF16, 6>(a, lpr, grid, lds, st);
  return dispatch_lpr<BF16, 8>(a, lpr, grid, lds, st);
}

template <int NCB>
static hipError_t run_mfma(const StreamArgs& a, int grid, int KSC, hipStream_t st) {
  const int nw = 4;
  const int rec = nw * a.M * static_cast<int>(sizeof(Partial));
  const int frag = KSC * NCB * 1024;
  const int bytes = frag > rec ? frag : rec;
  hipError_t e = allow_lds(k_stream_mfma<NCB>, bytes);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_stream_mfma<NCB>, dim3(grid), dim3(nw * kWave), bytes, st, a, KSC);
  return hipGetLastError();
}

hipError_t launch_stream(const StreamArgs& a, bool use_mfma, int* producers, hipStream_t st) {
  DeviceInfo di;
  hipError_t e = device_info(&di);
  if (e != hipSuccess) return e;
  const int64_t NG = (a.V + kGroup - 1) / kGroup;
  int64_t grid = (NG + 3) / 4;  // one group per wave, 4 waves per workgroup
  if (grid > kMaxPartials) grid = kMaxPartials;
  if (grid < 1) grid = 1;
  *producers = static_cast<int>(grid);
  if (!use_mfma) {
    const int C = static_cast<int>(a.K * (a.bf16 ? 2 : 4) / 16);
    int lpr = 64;
    if (C < 64) {
      lpr = 8;
      while (lpr < C) lpr <<= 1;
    }
    const int MB = a.M <= 1 ? 1 : a.M <= 2 ? 2 : a.M <= 4 ? 4 : a.M <= 6 ? 6 : 8;
    const int lds = MB * C * 16;
    return a.bf16 ? dispatch_mb<true>(a, lpr, static_cast<int>(grid), lds, st)
                  : dispatch_mb<false>(a, lpr, static_cast<int>(grid), lds, st);
  }
  const int ncb = (a.M + 31) / 32;
  const int KS = static_cast<int>((a.K + 15) / 16);
  const int budget = di.max_lds;
  int KSC = budget / (ncb * 1024);
  if (KSC >= KS) KSC = KS;
  if (KSC < 1) return hipErrorInvalidValue;
  switch (ncb) {
    case 1: return run_mfma<1>(a, static_cast<int>(grid), KSC, st);
    case 2: return run_mfma<2>(a, static_cast<int>(grid), KSC, st);
    case 3: return run_mfma<3>(a, static_cast<int>(grid), KSC, st);
    case 4: return run_mfma<4>(a, static_cast<int>(grid), KSC, st);
    case 5: return run_mfma<5>(a, static_cast<int>(grid), KSC, st);
    case 6: return run_mfma<6>(a, static_cast<int>(grid), KSC, st);
    case 7: return run_mfma<7>(a, static_cast<int>(grid), KSC, st);
    case 8: return run_mfma<8>(a, static_cast<int>(grid), KSC, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_head_finalize(const FinalizeArgs& f, hipStream_t st) {
  if (f.bf16)
    hipLaunchKernelGGL(k_head_finalize<true>, dim3(f.M), dim3(256), 0, st, f);
  else
    hipLaunchKernelGGL(k_head_finalize<false>, dim3(f.M), dim3(256), 0, st, f);
  return hipGetLastError();
}

}  // namespace sh
