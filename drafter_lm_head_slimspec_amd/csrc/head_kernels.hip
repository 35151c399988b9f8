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
//
// Memory-level parallelism is explicit everywhere: global loads of a batch are issued into
// registers before any of them is consumed (and, in the streaming loops, one batch ahead of
// the compute), because a load followed by an LDS store, a lane shuffle or an atomic in the
// same loop iteration is otherwise waited for before the next iteration's load is issued.
#include "device_common.h"
#include "launch.h"
#include "trace.h"

namespace sh {

// Copy `items` 16-byte words fetch(i) -> lds[i] with BATCH loads in flight per thread.
template <int BATCH, typename F>
__device__ __forceinline__ void stage16(uint4* lds, int items, F fetch) {
  for (int base = threadIdx.x; base < items; base += blockDim.x * BATCH) {
    uint4 v[BATCH];
#pragma unroll
    for (int b = 0; b < BATCH; ++b) {
      const int i = base + b * static_cast<int>(blockDim.x);
      v[b] = i < items ? fetch(i) : zero16();
    }
#pragma unroll
    for (int b = 0; b < BATCH; ++b) {
      const int i = base + b * static_cast<int>(blockDim.x);
      if (i < items) lds[i] = v[b];
    }
  }
}

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
  const int l = lane_id(), w = wave_id();
  const int j0 = blockIdx.x * kRowdotRows + w * 2;
  const int CPL = (C + kWave - 1) / kWave;
  // weight rows first (their loads overlap the staging below)
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
  const char* xb = static_cast<const char*>(x);
  stage16<8>(xs, kRowdotM * C, [&](int i) {
    const int mm = i / C, c = i - mm * C;
    const int m = m0 + mm;
    return (m < M) ? load16(xb + (static_cast<size_t>(m) * C + c) * 16) : zero16();
  });
  __syncthreads();
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
//   ONE (each lane owns one chunk of every row, C <= LPR): the next row-block's weights are
//   loaded before the current one is reduced, across group boundaries.
// ----------------------------------------------------------------------------------------
template <bool BF16, int MB, int LPR, bool ONE>
__global__ __launch_bounds__(256) void k_stream_valu(StreamArgs a) {
  constexpr int RB = 8;
  constexpr int RPI = kWave / LPR;
  constexpr int ROWS_RB = RB * RPI;
  constexpr int NRB = kGroup / ROWS_RB;
  constexpr int DUP = LPR / RB;
  extern __shared__ uint4 xs[];  // [MB][C] then (after the loop) Partial records
  const int C = static_cast<int>(a.K * (BF16 ? 2 : 4) / 16);
  const int CPL = (C + LPR - 1) / LPR;
  const char* xg = static_cast<const char*>(a.x);
  const int Mx = a.M;
  stage16<4>(xs, MB * C, [&](int i) {
    const int m = i / C, c = i - m * C;
    return (m < Mx) ? load16(xg + (static_cast<size_t>(m) * C + c) * 16) : zero16();
  });
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
#pragma unroll
  for (int m = 0; m < MB; ++m) xr[m] = (ONE && lr < C) ? xs[m * C + lr] : zero16();

  Partial run = partial_empty();  // lane m holds row m's running state
  float gm[MB], gs[MB], gz[MB];
  int32_t gi[MB];

  auto group_reset = [&]() {
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      gm[m] = -INFINITY;
      gs[m] = 0.f;
      gz[m] = -INFINITY;
      gi[m] = 0x7fffffff;
    }
  };

  // reduce acc over the row's lanes, then fold the finished row into the group state
  auto finish_rb = [&](float (&acc)[RB][MB], int64_t rbase) {
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
          acc[i][m] = keep + xor_lane(send, s);
        }
      }
    }
#pragma unroll
    for (int s = LPR >> 4; s >= 1; s >>= 1)
#pragma unroll
      for (int m = 0; m < MB; ++m) acc[0][m] += xor_lane(acc[0][m], s);
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
  };

  auto group_end = [&](int64_t g) {
    if (a.stats == kStatsNone) return;
#pragma unroll
    for (int s = DUP; s < kWave; s <<= 1) {
#pragma unroll
      for (int m = 0; m < MB; ++m) {
        const float m2 = xor_lane(gm[m], s), s2 = xor_lane(gs[m], s);
        const float z2 = xor_lane(gz[m], s);
        const int32_t i2 = xor_lane(gi[m], s);
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
  };

  const int64_t gw = static_cast<int64_t>(blockIdx.x) * (blockDim.x / kWave) + w;
  if constexpr (ONE) {
    auto load_rb = [&](int64_t g, int rb, uint4 (&wv)[RB]) {
      // descriptor over this group's rows: rows past V read as zero
      const int64_t g0 = g * kGroup;
      const int64_t rows = a.V - g0 < kGroup ? a.V - g0 : kGroup;
      const rsrc_t rs = make_rsrc(Wb + static_cast<size_t>(g0) * rowbytes, static_cast<uint32_t>(rows * rowbytes));
#pragma unroll
      for (int j = 0; j < RB; ++j) {
        const int rin = rb * ROWS_RB + j * RPI + ri;
        const uint32_t off = lr < C ? static_cast<uint32_t>(rin * rowbytes + lr * 16) : kOutOfRange;
        wv[j] = buffer_load16(rs, off);
      }
    };
    // one pipeline step: prefetch the next row-block into `fill`, consume `use`
    int64_t g = gw;
    int rb = 0;
    auto step = [&](uint4 (&use)[RB], uint4 (&fill)[RB]) -> bool {
      int64_t g2 = g;
      int rb2 = rb + 1;
      if (rb2 == NRB) {
        rb2 = 0;
        g2 += nwt;
      }
      // unconditional prefetch (at the end of the wave's work it re-reads the current,
      // cache-resident block) so the wait below can leave exactly these loads in flight
      if (g2 < NG)
        load_rb(g2, rb2, fill);
      else
        load_rb(g, rb, fill);
      if (rb == 0) group_reset();
      float acc[RB][MB];
#pragma unroll
      for (int j = 0; j < RB; ++j)
#pragma unroll
        for (int m = 0; m < MB; ++m) acc[j][m] = chunk_dot<BF16>(use[j], xr[m], 0.f);
      finish_rb(acc, g * kGroup + rb * ROWS_RB);
      if (rb == NRB - 1) group_end(g);
      g = g2;
      rb = rb2;
      return g < NG;
    };
    uint4 bufA[RB], bufB[RB];
    if (g < NG) {
      load_rb(g, 0, bufA);
      for (;;) {
        if (!step(bufA, bufB)) break;
        if (!step(bufB, bufA)) break;
      }
    }
  } else {
    for (int64_t g = gw; g < NG; g += nwt) {
      group_reset();
      const int64_t g0 = g * kGroup;
      const int64_t grows = a.V - g0 < kGroup ? a.V - g0 : kGroup;
      const rsrc_t rs = make_rsrc(Wb + static_cast<size_t>(g0) * rowbytes, static_cast<uint32_t>(grows * rowbytes));
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
          uint4 wv[RB];
#pragma unroll
          for (int j = 0; j < RB; ++j) {
            const int rin = rb * ROWS_RB + j * RPI + ri;
            wv[j] = buffer_load16(rs, cok ? static_cast<uint32_t>(rin * rowbytes + c * 16) : kOutOfRange);
          }
          uint4 xq[MB];
#pragma unroll
          for (int m = 0; m < MB; ++m) xq[m] = cok ? xs[m * C + c] : zero16();
#pragma unroll
          for (int j = 0; j < RB; ++j)
#pragma unroll
            for (int m = 0; m < MB; ++m) acc[j][m] = chunk_dot<BF16>(wv[j], xq[m], acc[j][m]);
        }
        finish_rb(acc, rbase);
      }
      group_end(g);
    }
  }
  if (a.stats == kStatsNone) return;
  __syncthreads();
  Partial* rec = reinterpret_cast<Partial*>(xs);
  wg_combine_store(rec, run, l < a.M, l, a.M, a.partials, a.partials_ld);
}

// ----------------------------------------------------------------------------------------
// k_stream_mfma: bf16, M <= 32*NCB rows.  Each wave walks its 64-row vocabulary groups as
// 32-row tiles computed with v_mfma_f32_32x32x16_bf16: A = weight tile from HBM straight
// into registers, B = activations.  The weight fragments are loaded KB k-steps at a time,
// one batch ahead, the prefetch running across tile and group boundaries so the next loads
// are in flight while a tile's statistics are folded.
//   BG = false: B comes from LDS, staged once per workgroup and pre-swizzled into fragment
//               order [k-step][column block][lane] (one conflict-free 16-byte read per lane).
//   BG = true:  the activations do not fit in LDS (large K): each lane loads its B fragment
//               directly from the (L2-resident) activation rows.
// Output layout of the 32x32 tile: lane l holds column l%32 and rows
// 8*(v/4) + 4*(l/32) + v%4 for its 16 accumulators v.
// ----------------------------------------------------------------------------------------
template <int NCB, bool BG>
__global__ __launch_bounds__(256) void k_stream_mfma(StreamArgs a) {
  constexpr int KB = BG ? 4 : 8;
  extern __shared__ uint4 bs[];  // [KS][NCB][64] 16-byte B fragments, later Partial records
  const int l = lane_id(), w = wave_id();
  const int NW = blockDim.x / kWave;
  const int n = l & 31, hf = l >> 5;
  const int K = static_cast<int>(a.K);
  const int KS = (K + 15) / 16;
  const int nb = (KS + KB - 1) / KB;
  const size_t rowbytes = static_cast<size_t>(K) * 2;
  const int64_t NG = (a.V + kGroup - 1) / kGroup;
  const int64_t nwt = static_cast<int64_t>(gridDim.x) * NW;
  const char* xb = static_cast<const char*>(a.x);
  const char* Wb = static_cast<const char*>(a.W);
  const int Mx = a.M;

  if constexpr (!BG) {
    stage16<8>(bs, KS * NCB * kWave, [&](int it) {
      const int ks = it / (NCB * kWave);
      const int cb = (it / kWave) % NCB;
      const int ll = it & (kWave - 1);
      const int m = cb * 32 + (ll & 31);
      const int k = ks * 16 + (ll >> 5) * 8;
      return (m < Mx && k < K) ? load16(xb + (static_cast<size_t>(m) * K + k) * 2) : zero16();
    });
    __syncthreads();
  }

  Partial run[NCB];
  float hm[NCB], hs[NCB], hz[NCB];
  int32_t hi[NCB];
  f32x16_t acc[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) run[cb] = partial_empty();

  // B fragment addresses of this lane (BG): column m = cb*32 + n, k-half hf
  const rsrc_t xrs = make_rsrc(xb, static_cast<uint32_t>(static_cast<size_t>(Mx) * K * 2));
  auto load_batch = [&](int64_t g, int t, int b, uint4 (&X)[KB], uint4 (&Y)[KB][NCB]) {
    // descriptor over this group's rows: rows past V read as zero
    const int64_t g0 = g * kGroup;
    const int64_t rows = a.V - g0 < kGroup ? a.V - g0 : kGroup;
    const rsrc_t rs = make_rsrc(Wb + static_cast<size_t>(g0) * rowbytes, static_cast<uint32_t>(rows * rowbytes));
    const uint32_t rbase = static_cast<uint32_t>((t * 32 + n) * rowbytes);
#pragma unroll
    for (int j = 0; j < KB; ++j) {
      const int ks = b * KB + j;
      const int k = ks * 16 + hf * 8;
      const bool kok = ks < KS && k < K;
      X[j] = buffer_load16(rs, kok ? rbase + static_cast<uint32_t>(k * 2) : kOutOfRange);
      if constexpr (BG) {
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
          const int m = cb * 32 + n;
          Y[j][cb] = buffer_load16(xrs, (kok && m < Mx) ? static_cast<uint32_t>((m * K + k) * 2) : kOutOfRange);
        }
      }
    }
  };

  auto epilogue_tile = [&](int64_t g, int t) {
    const int64_t tbase = g * kGroup + t * 32;
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
      if (a.stats == kStatsNone) continue;
      if (a.stats >= kStatsLse && ym != -INFINITY) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int64_t row = tbase + 8 * (v >> 2) + 4 * hf + (v & 3);
          if (row < a.V) ss += __expf(acc[cb][v] * a.invT - ym);
        }
      }
      const float zb2 = xor_lane(zb, 32);
      const int32_t ib2 = xor_lane(ib, 32);
      const float ym2 = xor_lane(ym, 32), ss2 = xor_lane(ss, 32);
      argmax_merge(zb, ib, zb2, ib2);
      lse_merge(ym, ss, ym2, ss2);
      if (t == 0) {
        hm[cb] = ym;
        hs[cb] = ss;
        hz[cb] = zb;
        hi[cb] = ib;
        continue;
      }
      lse_merge(ym, ss, hm[cb], hs[cb]);
      argmax_merge(zb, ib, hz[cb], hi[cb]);
      if (m < a.M) {
        if (a.stats == kStatsSample) {
          const float L = ym + logf(ss);
          const float u = philox_uniform(a.seed, a.offset, kDraftGroup, a.row0 + m, g);
          argmax_merge(run[cb].gscore, run[cb].g, L + gumbel(u), static_cast<int32_t>(g));
        }
        lse_merge(run[cb].m, run[cb].s, ym, ss);
        argmax_merge(run[cb].zmax, run[cb].zid, zb, ib);
      }
    }
  };

  int64_t g = static_cast<int64_t>(blockIdx.x) * NW + w;
  int t = 0, b = 0;
  // one pipeline step: prefetch the next batch into (FX, FY), consume (UX, UY)
  auto step = [&](uint4 (&UX)[KB], uint4 (&UY)[KB][NCB], uint4 (&FX)[KB], uint4 (&FY)[KB][NCB]) -> bool {
    int64_t g2 = g;
    int t2 = t, b2 = b + 1;
    if (b2 == nb) {
      b2 = 0;
      t2 = t + 1;
      if (t2 == 2) {
        t2 = 0;
        g2 = g + nwt;
      }
    }
    // unconditional prefetch (re-reads the current, cache-resident batch at the very end)
    if (g2 < NG)
      load_batch(g2, t2, b2, FX, FY);
    else
      load_batch(g, t, b, FX, FY);
    if (b == 0) {
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[cb][v] = 0.f;
    }
#pragma unroll
    for (int j = 0; j < KB; ++j) {
      const int ks = b * KB + j;
      if (ks < KS) {
        const bf16x8_t af = __builtin_bit_cast(bf16x8_t, UX[j]);
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
          const uint4 bv = BG ? UY[j][cb] : bs[(ks * NCB + cb) * kWave + l];
          acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, __builtin_bit_cast(bf16x8_t, bv), acc[cb], 0, 0, 0);
        }
      }
    }
    if (b == nb - 1) epilogue_tile(g, t);
    g = g2;
    t = t2;
    b = b2;
    return g < NG;
  };
  uint4 XA[KB], XB[KB];
  uint4 YA[KB][NCB], YB[KB][NCB];
  if (g < NG) {
    load_batch(g, 0, 0, XA, YA);
    for (;;) {
      if (!step(XA, YA, XB, YB)) break;
      if (!step(XB, YB, XA, YA)) break;
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
// k_head_finalize: one workgroup (16 waves) per row.
// ----------------------------------------------------------------------------------------
constexpr int kFinThreads = 1024;
constexpr int kFinPerThread = (kMaxPartials + kFinThreads - 1) / kFinThreads;
constexpr int kFinRowsPerWave = kGroup / (kFinThreads / kWave);   // 4
constexpr int kFinMaxCPL = 16;

template <bool BF16>
__global__ __launch_bounds__(kFinThreads) void k_head_finalize(FinalizeArgs f) {
  __shared__ Partial red[kFinThreads / kWave];
  __shared__ float zs[kGroup];
  const int m = blockIdx.x;
  const int l = lane_id(), w = wave_id();
  const Partial* pp = f.partials + static_cast<int64_t>(m) * f.partials_ld;
  Partial loaded[kFinPerThread];
#pragma unroll
  for (int i = 0; i < kFinPerThread; ++i) {
    const int idx = threadIdx.x + i * kFinThreads;
    loaded[i] = idx < f.P ? pp[idx] : partial_empty();
  }
  Partial p = loaded[0];
#pragma unroll
  for (int i = 1; i < kFinPerThread; ++i) partial_merge(p, loaded[i]);
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
  if (l == 0) red[w] = p;
  __syncthreads();
  p = red[0];
  for (int i = 1; i < kFinThreads / kWave; ++i) partial_merge(p, red[i]);
  const float lse = p.m + logf(p.s);
  int32_t tok;
  float ytok;
  if (f.mode == 0) {
    tok = p.zid;
    ytok = p.zmax * f.invT;
  } else {
    // recompute the 64 logits of the winning group (4 rows per wave, loads issued together)
    const int C = static_cast<int>(f.K * (BF16 ? 2 : 4) / 16);
    const int CPL = (C + kWave - 1) / kWave;
    const size_t rowbytes = static_cast<size_t>(C) * 16;
    const char* xr = static_cast<const char*>(f.x) + static_cast<size_t>(m) * rowbytes;
    const int64_t gbase = static_cast<int64_t>(p.g) * kGroup;
    float z[kFinRowsPerWave];
#pragma unroll
    for (int j = 0; j < kFinRowsPerWave; ++j) z[j] = 0.f;
    for (int q0 = 0; q0 < CPL; q0 += 4) {
      uint4 xv[4], wv[4][kFinRowsPerWave];
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const int c = (q0 + qq) * kWave + l;
        const bool cok = q0 + qq < CPL && c < C;
        xv[qq] = cok ? load16(xr + static_cast<size_t>(c) * 16) : zero16();
#pragma unroll
        for (int j = 0; j < kFinRowsPerWave; ++j) {
          const int64_t row = gbase + w * kFinRowsPerWave + j;
          wv[qq][j] = (cok && row < f.V)
                          ? load16(static_cast<const char*>(f.W) + static_cast<size_t>(row) * rowbytes + static_cast<size_t>(c) * 16)
                          : zero16();
        }
      }
#pragma unroll
      for (int qq = 0; qq < 4; ++qq)
#pragma unroll
        for (int j = 0; j < kFinRowsPerWave; ++j) z[j] = chunk_dot<BF16>(wv[qq][j], xv[qq], z[j]);
    }
#pragma unroll
    for (int j = 0; j < kFinRowsPerWave; ++j) {
      const float t = wave_sum(z[j]);
      if (l == 0) zs[w * kFinRowsPerWave + j] = t;
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
  TraceScope ts("rowdot", st);
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

template <bool BF16, int MB, int LPR, bool ONE>
static hipError_t run_valu(const StreamArgs& a, int grid, int lds, hipStream_t st) {
  const int rec = 4 * MB * static_cast<int>(sizeof(Partial));
  const int bytes = lds > rec ? lds : rec;
  hipError_t e = allow_lds(k_stream_valu<BF16, MB, LPR, ONE>, bytes);
  if (e != hipSuccess) return e;
  TraceScope ts("stream_valu", st);
  hipLaunchKernelGGL((k_stream_valu<BF16, MB, LPR, ONE>), dim3(grid), dim3(256), bytes, st, a);
  return hipGetLastError();
}

template <bool BF16, int MB>
static hipError_t dispatch_lpr(const StreamArgs& a, int lpr, bool one, int grid, int lds, hipStream_t st) {
  switch (lpr) {
    case 8: return run_valu<BF16, MB, 8, true>(a, grid, lds, st);
    case 16: return run_valu<BF16, MB, 16, true>(a, grid, lds, st);
    case 32: return run_valu<BF16, MB, 32, true>(a, grid, lds, st);
    default:
      return one ? run_valu<BF16, MB, 64, true>(a, grid, lds, st) : run_valu<BF16, MB, 64, false>(a, grid, lds, st);
  }
}

template <bool BF16>
static hipError_t dispatch_mb(const StreamArgs& a, int lpr, bool one, int grid, int lds, hipStream_t st) {
  if (a.M <= 1) return dispatch_lpr<BF16, 1>(a, lpr, one, grid, lds, st);
  if (a.M <= 2) return dispatch_lpr<BF16, 2>(a, lpr, one, grid, lds, st);
  if (a.M <= 4) return dispatch_lpr<BF16, 4>(a, lpr, one, grid, lds, st);
  if (a.M <= 6) return dispatch_lpr<BF16, 6>(a, lpr, one, grid, lds, st);
  return dispatch_lpr<BF16, 8>(a, lpr, one, grid, lds, st);
}

template <int NCB>
static hipError_t run_mfma(const StreamArgs& a, int grid, bool bg, hipStream_t st) {
  const int nw = 4;
  const int rec = nw * a.M * static_cast<int>(sizeof(Partial));
  const int KS = static_cast<int>((a.K + 15) / 16);
  const int frag = bg ? 0 : KS * NCB * 1024;
  const int bytes = frag > rec ? frag : rec;
  hipError_t e = bg ? allow_lds(k_stream_mfma<NCB, true>, bytes) : allow_lds(k_stream_mfma<NCB, false>, bytes);
  if (e != hipSuccess) return e;
  TraceScope ts("stream_mfma", st);
  if (bg)
    hipLaunchKernelGGL((k_stream_mfma<NCB, true>), dim3(grid), dim3(nw * kWave), bytes, st, a);
  else
    hipLaunchKernelGGL((k_stream_mfma<NCB, false>), dim3(grid), dim3(nw * kWave), bytes, st, a);
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
    const bool one = C <= lpr;
    const int MB = a.M <= 1 ? 1 : a.M <= 2 ? 2 : a.M <= 4 ? 4 : a.M <= 6 ? 6 : 8;
    const int lds = MB * C * 16;
    return a.bf16 ? dispatch_mb<true>(a, lpr, one, static_cast<int>(grid), lds, st)
                  : dispatch_mb<false>(a, lpr, one, static_cast<int>(grid), lds, st);
  }
  const int ncb = (a.M + 31) / 32;
  const int KS = static_cast<int>((a.K + 15) / 16);
  const bool bg = static_cast<int64_t>(KS) * ncb * 1024 > di.max_lds;
  switch (ncb) {
    case 1: return run_mfma<1>(a, static_cast<int>(grid), bg, st);
    case 2: return run_mfma<2>(a, static_cast<int>(grid), bg, st);
    case 3: return run_mfma<3>(a, static_cast<int>(grid), bg, st);
    case 4: return run_mfma<4>(a, static_cast<int>(grid), bg, st);
    case 5: return run_mfma<5>(a, static_cast<int>(grid), bg, st);
    case 6: return run_mfma<6>(a, static_cast<int>(grid), bg, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_head_finalize(const FinalizeArgs& f, hipStream_t st) {
  TraceScope ts("head_finalize", st);
  if (f.bf16)
    hipLaunchKernelGGL(k_head_finalize<true>, dim3(f.M), dim3(kFinThreads), 0, st, f);
  else
    hipLaunchKernelGGL(k_head_finalize<false>, dim3(f.M), dim3(kFinThreads), 0, st, f);
  return hipGetLastError();
}

}  // namespace sh
