// Wide-batch head kernel for gfx950: bf16 rows of at most 512 elements and 65..256 activation
// rows (the GPT-OSS-shaped SlimSpec head: r = 360, 32 sequences x 6 draft positions).
//
//   k_head_wide   z = W x over all V rows with per-workgroup Partials (lse, best group score
//                 with the Philox group draw, argmax), as k_head_tile, for more activation
//                 rows than fit one wave's registers.  A workgroup of eight waves (two per
//                 SIMD) walks a consecutive range of 64-row vocabulary groups in pairs; each
//                 group is read once by the whole workgroup with whole-row loads (full cache
//                 lines) into an LDS tile while the next pair's rows are in flight in
//                 registers.  The activation rows form 16-row column blocks dealt round-robin
//                 to the waves (block b to wave b mod 8, at most two per wave), so the two
//                 waves of a SIMD (waves w and w + 4: the SIMD field of HW_ID, read on this
//                 GPU) together hold a quarter of the blocks and one wave's VALU epilogue can
//                 issue while the other's MFMAs run.  The group Gumbels of the workgroup's
//                 whole range are drawn into LDS while its first loads are in flight.  Each wave multiplies the
//                 tile by its blocks (B fragments in registers for the whole pass) on
//                 v_mfma_f32_16x16x32_bf16, reading the A fragments from LDS, and folds each
//                 group into the running state of its rows exactly as the tile kernel does:
//                 per group one in-lane and two cross-lane reductions give the group
//                 log-sum-exp, the group draw L_g + Gumbel(u_g) and the argmax.
//   The per-row merge of the workgroups' Partials is k_head_fin (head_tile.hip).
#include <hip/hip_ext.h>

#include <type_traits>

#include "device_common.h"
#include "launch.h"
#include "trace.h"

namespace sh {

namespace {

typedef float wf32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWideThreads = 512;   // eight waves, two per SIMD
constexpr int kWideWaves = kWideThreads / kWave;
constexpr int kWideStats = 1, kWideArgmax = 2;
// LDS bytes of the pair's tile and its spare chunks, and the blocks [TB][kWideMaxRows][4] floats
// of the Gumbel table behind them: as many as fit in 160 KB, at most 8 (a workgroup's range at
// the GPT-OSS shape spans at most 5; a longer range falls back to a rolling table of 2)
constexpr int wide_lds_base(int ks) { return (2 * kGroup * (ks * 4 + 2) + kWave) * 16; }
constexpr int wide_gtab_blocks(int ks) {
  return (160 * 1024 - wide_lds_base(ks)) / (kWideMaxRows * 16) < 8 ? (160 * 1024 - wide_lds_base(ks)) / (kWideMaxRows * 16)
                                                                   : 8;
}

}  // namespace

// The pass of one wave holding NCBW column blocks (0, 1 or 2): blocks w and w + 8 of the
// ceil(M / 16) blocks.  Every wave runs the same loads, stores and barriers.
template <int NCBW, int KS, int EPI>
__device__ __forceinline__ void wide_wave(const TileArgs& a, uint4* tile) {
  constexpr bool STATS = (EPI & kWideStats) != 0, AMAX = (EPI & kWideArgmax) != 0;
  constexpr int CPR = KS * 4;            // 16-byte chunks per row covered by the k-steps
  // LDS row stride in chunks: 2 mod 4 (measured on gfx950: the 16-row fragment reads run at
  // ~170 B/clk per CU with such strides, ~110 with odd ones, far less with multiples of 8)
  constexpr int RS = CPR + 2;
  constexpr int PER = CPR * kGroup / kWideThreads;   // row chunks each thread loads per group
  const int l = lane_id(), w = wave_id();
  const int col = l & 15, qd = l >> 4;
  const int tid = static_cast<int>(threadIdx.x);
  const int K = a.K;
  const uint32_t rowbytes = static_cast<uint32_t>(a.ld > 0 ? a.ld : a.K) * 2;
  const int kc = K / 8;                  // chunks of a row that hold elements (K % 8 == 0)
  const int V32 = static_cast<int>(a.V);
  const int NG = (V32 + kGroup - 1) / kGroup;
  const uint32_t vbytes = static_cast<uint32_t>(V32) * rowbytes;
  const int Mx = a.M;
  // activation row of block cb of this wave, lane column col
  auto row_of = [&](int cb) { return (w + cb * kWideWaves) * 16 + col; };
  const float c2 = a.invT * kLog2e;

  // this wave's activation fragments: Bf[s][cb] = x[row_of(cb)][32 s + 8 qd .. +8]
  uint4 Bf[KS][NCBW > 0 ? NCBW : 1];
  if constexpr (NCBW > 0) {
    const rsrc_t xrs = make_rsrc(a.x, static_cast<uint32_t>(Mx) * rowbytes);
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
      for (int cb = 0; cb < NCBW; ++cb) {
        const int m = row_of(cb), c = 4 * s + qd;
        Bf[s][cb] = buffer_load16(xrs, (m < Mx && c < kc) ? static_cast<uint32_t>(m) * rowbytes + c * 16u : kOutOfRange);
      }
  }
  // chunks past K read zero from LDS: cleared once, never overwritten
  for (int i = tid; i < 2 * kGroup * (CPR - kc); i += kWideThreads) {
    const int r = i / (CPR - kc), c = kc + i % (CPR - kc);
    tile[r * RS + c] = zero16();
  }
  // this thread's row chunks of a group: slot tid + 256 j = (row, chunk), fixed for every group
  uint32_t goff[PER];
  int lidx[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int i = tid + kWideThreads * j;
    const int r = i / kc, c = i - r * kc;
    const bool ok = i < kGroup * kc;
    goff[j] = ok ? static_cast<uint32_t>(r) * rowbytes + c * 16u : kOutOfRange;
    lidx[j] = ok ? r * RS + c : 2 * kGroup * RS + (tid & 63);   // spare chunk: stores stay unconditional
  }
  auto gload = [&](int g, uint4 (&R)[PER]) {
    const int r0 = g * kGroup;
    const uint32_t b0 = r0 < V32 ? static_cast<uint32_t>(r0) * rowbytes : vbytes;
    const rsrc_t rs = make_rsrc(static_cast<const char*>(a.W) + b0, vbytes - b0);
#pragma unroll
    for (int j = 0; j < PER; ++j) R[j] = buffer_load16(rs, goff[j]);
  };
  auto gstore = [&](const uint4 (&R)[PER], int half) {
#pragma unroll
    for (int j = 0; j < PER; ++j) tile[lidx[j] + (lidx[j] < 2 * kGroup * RS ? half * kGroup * RS : 0)] = R[j];
  };

  // running state of activation row row_of(qd) (lanes with qd < NCBW)
  float rm = -INFINITY, rsum = 0.f, gbest = -INFINITY, bz = -INFINITY;
  int32_t gid = 0x7fffffff, bi = 0x7fffffff;

  // the workgroup's groups are the consecutive range [gs, ge), taken in pairs (g, g + 1):
  // while a pair is multiplied out of the LDS tile, the next pair's rows are in flight in
  // registers; storing a pair waits for every outstanding load, which is exactly that pair.
  // Past the range the loads go to group NG, an empty buffer range: they return zeros and
  // touch no memory (re-reading a group of the range would miss the cache by then: a range
  // is ~0.5 MB and 32 workgroups share one XCD's L2)
  const int G = static_cast<int>(gridDim.x);
  const int gs = static_cast<int>((static_cast<int64_t>(blockIdx.x) * NG) / G);
  const int ge = static_cast<int>((static_cast<int64_t>(blockIdx.x + 1) * NG) / G);
  auto clampg = [&](int g) { return g < ge ? g : NG; };
  uint4 RA[PER], RB[PER];
  gload(clampg(gs), RA);
  gload(clampg(gs + 1), RB);

  // Gumbel(u) of activation row m for group g: one Philox block holds groups 4 q .. 4 q + 3.
  // Every block of the range [q0, q0 + nq) is computed once per workgroup into gtab[q - q0][m]
  // while the first pair's loads are in flight (`whole`); a range with more blocks than the
  // table holds computes them as the walk reaches them (gumbel_blocks) into gtab[q mod 2][m].
  // Read by the wave owning row m.  (Measured at the GPT-OSS shape against computing every
  // block between the barriers: the pass 46.0 -> 43.9 us; with the split load issue below, 41.5.)
  float* gtab = reinterpret_cast<float*>(tile + 2 * kGroup * RS + kWave);   // [TB][kWideMaxRows][4]
  const int q0 = gs >> 2, nq = ge > gs ? ((ge - 1) >> 2) - q0 + 1 : 0;
  const bool whole = STATS && a.sample != 0 && nq <= wide_gtab_blocks(KS);
  if (whole) {
    for (int i = tid; i < nq * Mx; i += kWideThreads) {
      const int qq = i / Mx, m = i - qq * Mx;
      uint64_t wd[4];
      philox_block(a.seed, a.offset, kDraftGroup, static_cast<uint64_t>(a.row0 + m), static_cast<uint64_t>(q0 + qq) * 4, wd);
#pragma unroll
      for (int j = 0; j < 4; ++j) gtab[qq * kWideMaxRows * 4 + m * 4 + j] = gumbel(word_to_uniform(wd[j]));
    }
  }
  auto draw = [&](int g) -> float {
    float gu = 0.f;
    if constexpr (STATS) {
      const int m = row_of(qd);
      if (a.sample != 0 && qd < NCBW && m < Mx)
        gu = gtab[(whole ? (g >> 2) - q0 : ((g >> 2) & 1)) * kWideMaxRows * 4 + m * 4 + (g & 3)];
    }
    return gu;
  };
  // the blocks of groups g and g + 1 not computed yet (q_done: the last block computed)
  int q_done = -1;
  auto gumbel_blocks = [&](int g) {
    if constexpr (STATS) {
      if (a.sample != 0 && !whole) {
        for (int q = g >> 2; q <= ((g + 1) >> 2); ++q) {   // uniform over the workgroup
          if (q <= q_done) continue;
          q_done = q;
          if (tid < Mx) {
            uint64_t wd[4];
            philox_block(a.seed, a.offset, kDraftGroup, static_cast<uint64_t>(a.row0 + tid),
                         static_cast<uint64_t>(q) * 4, wd);
#pragma unroll
            for (int i = 0; i < 4; ++i) gtab[(q & 1) * kWideMaxRows * 4 + tid * 4 + i] = gumbel(word_to_uniform(wd[i]));
          }
        }
      }
    }
  };
  // z = tile half x this wave's activation fragments.  Per k-step the four tiles' A fragments
  // are one batch of LDS reads, issued a k-step ahead of the 4 * NCBW MFMAs that use them
  // (with `pin`, scheduling barriers keep the reads in front)
  auto mma = [&](int half, wf32x4_t (&acc)[4][NCBW > 0 ? NCBW : 1], auto pin) {
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int cb = 0; cb < NCBW; ++cb) acc[t][cb] = wf32x4_t{0.f, 0.f, 0.f, 0.f};
    const uint4* trow = tile + (half * kGroup + col) * RS + qd;
    auto aread = [&](uint4 (&af)[4], int s) {
#pragma unroll
      for (int t = 0; t < 4; ++t) af[t] = trow[t * 16 * RS + 4 * s];
    };
    auto amma = [&](const uint4 (&af)[4], int s) {
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int cb = 0; cb < NCBW; ++cb)
          acc[t][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, af[t]),
                                                               __builtin_bit_cast(bf16x8_t, Bf[s][cb]), acc[t][cb], 0, 0, 0);
    };
    static_assert(KS % 2 == 0, "k-steps in pairs");
    uint4 afA[4], afB[4];
    aread(afA, 0);
#pragma unroll
    for (int s = 0; s < KS; s += 2) {
      aread(afB, s + 1);
      if constexpr (decltype(pin)::value) __builtin_amdgcn_sched_barrier(0);
      amma(afA, s);
      if (s + 2 < KS) aread(afA, s + 2);
      if constexpr (decltype(pin)::value) __builtin_amdgcn_sched_barrier(0);
      amma(afB, s + 1);
    }
  };
  // fold group g into the running state of this lane's row (MASK: the vocabulary's last,
  // partial group, whose rows past V are -inf)
  auto epi_body = [&](int g, float gu, const wf32x4_t (&acc)[4][NCBW > 0 ? NCBW : 1], auto mask) {
    constexpr bool MASK = decltype(mask)::value;
    const int gb = g * kGroup;
    // per column block: the group's max, sum of exp and first argmax of activation row
    // row_of(cb); the four lanes col, col + 16, col + 32, col + 48 hold its 64 rows and
    // end with the same values (the max is taken first, so the sum needs no rescaling)
    float bm[NCBW > 0 ? NCBW : 1], bs[NCBW > 0 ? NCBW : 1];
    int32_t bx[NCBW > 0 ? NCBW : 1];
#pragma unroll
    for (int cb = 0; cb < NCBW; ++cb) {
      float z[16];
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          if constexpr (MASK) {
            const int row = gb + t * 16 + qd * 4 + v;
            z[t * 4 + v] = row < V32 ? acc[t][cb][v] : -INFINITY;
          } else {
            z[t * 4 + v] = acc[t][cb][v];
          }
        }
      float zm = z[0];
#pragma unroll
      for (int i = 1; i < 16; ++i) zm = fmaxf(zm, z[i]);
      zm = fmaxf(zm, xor_lane(zm, 16));
      zm = fmaxf(zm, xor_lane(zm, 32));
      float ss = 0.f;
      if constexpr (STATS) {
        const float off = zm * c2;
#pragma unroll
        for (int i = 0; i < 16; ++i) ss += fast_exp2(fmaf(z[i], c2, -off));
        ss += xor_lane(ss, 16);
        ss += xor_lane(ss, 32);
        ss = zm == -INFINITY ? 0.f : ss;
      }
      int32_t zi = 0x7fffffff;
      if constexpr (AMAX) {
#pragma unroll
        for (int i = 15; i >= 0; --i)   // the lane's rows rise with i: keep the lowest
          if (z[i] == zm) zi = gb + (i >> 2) * 16 + qd * 4 + (i & 3);
        zi = zm == -INFINITY ? 0x7fffffff : zi;
        zi = min(zi, xor_lane(zi, 16));
        zi = min(zi, xor_lane(zi, 32));
      }
      bm[cb] = zm;
      bs[cb] = ss;
      bx[cb] = zi;
    }
    // lane (col, qd) finishes activation row row_of(qd): one fold per lane
    float zm = bm[0], ss = bs[0];
    int32_t zi = bx[0];
#pragma unroll
    for (int cb = 1; cb < NCBW; ++cb)
      if (qd == cb) {
        zm = bm[cb];
        ss = bs[cb];
        zi = bx[cb];
      }
    if (qd < NCBW && row_of(qd) < Mx) {
      if constexpr (STATS) {
        const float L = zm * a.invT + log2f(ss) * kLn2;   // group log-sum-exp of y = z / T
        const float mn = fmaxf(rm, L);
        rsum = rsum * fast_exp2((rm - mn) * kLog2e) + fast_exp2((L - mn) * kLog2e);
        rm = mn;
        const float sc = L + gu;
        if (a.sample != 0 && sc > gbest) {   // groups rise: strict > keeps the lowest on ties
          gbest = sc;
          gid = g;
        }
      }
      if constexpr (AMAX) argmax_merge(bz, bi, zm, zi);
    }
  };
  auto epi = [&](int g, float gu, const wf32x4_t (&acc)[4][NCBW > 0 ? NCBW : 1]) {
    if (g * kGroup + kGroup <= V32) epi_body(g, gu, acc, std::false_type{});   // uniform
    else epi_body(g, gu, acc, std::true_type{});
  };
  wf32x4_t accA[4][NCBW > 0 ? NCBW : 1];

  // The next pair's loads go out in two halves: the first group's before the multiplications,
  // the second's after the first group's epilogue.  Issued together, the waves issuing last
  // stalled on them (back-pressure of the whole chip's burst) before their own MFMAs; measured
  // at the GPT-OSS shape (same machine, Gumbel table as above): 43.9 -> 41.5 us, and 38.0-39.0
  // against 39.2-39.8 with the second half after the second group's MFMAs or both halves
  // after the first group's.
  for (int g = gs; g < ge; g += 2) {
    __syncthreads();   // every wave is done with the previous pair's tile (and Gumbels)
    gstore(RA, 0);
    gstore(RB, 1);
    gumbel_blocks(g);   // a block is overwritten only two blocks later, after its last group
    __syncthreads();
    gload(clampg(g + 2), RA);
    if constexpr (NCBW > 0) {
      mma(0, accA, std::true_type{});
      epi(g, draw(g), accA);
      gload(clampg(g + 3), RB);
      if (g + 1 < ge) {
        mma(1, accA, std::true_type{});
        epi(g + 1, draw(g + 1), accA);
      }
    } else {
      gload(clampg(g + 3), RB);
    }
  }
  // one Partial per activation row per workgroup (each row belongs to one lane)
  const int m = row_of(qd);
  if (qd < NCBW && m < Mx) {
    Partial p;
    p.m = rm;
    p.s = rsum;
    p.gscore = gbest;
    p.g = gid;
    p.zmax = bz;
    p.zid = bi;
    p.xz = -INFINITY;
    p.pad1 = 0.f;
    a.partials[static_cast<int64_t>(m) * a.partials_ld + blockIdx.x] = p;
  }
}

template <int KS, int EPI>
__global__ __launch_bounds__(kWideThreads, 1) void k_head_wide(TileArgs a) {
  // [2][64][RS] the current pair of groups, 64 spare chunks, then the Gumbel table
  // [TB][kWideMaxRows][4] floats
  extern __shared__ uint4 tile[];
  const int w = wave_id();
  const int nb = (a.M + 15) / 16;   // column blocks, at most 2 * kWideWaves
  if constexpr (KS < 16) {   // rows of 512 elements: at most 128 activation rows, one block per wave
    if (w + kWideWaves < nb) {
      wide_wave<2, KS, EPI>(a, tile);
      return;
    }
  }
  if (w < nb) wide_wave<1, KS, EPI>(a, tile);
  else wide_wave<0, KS, EPI>(a, tile);
}

// ----------------------------------------------------------------------------------------
// host side
// ----------------------------------------------------------------------------------------
namespace {

int wide_ks(int64_t K) { return static_cast<int>((K + 127) / 128) * 4; }   // 4, 8, 12 or 16
int wide_lds(int ks) { return wide_lds_base(ks) + wide_gtab_blocks(ks) * kWideMaxRows * 4 * 4; }
// VGPRs per lane of a two-block wave: activation fragments, two row buffers (eight waves share
// each group's loads), accumulators, offsets and state
int wide_regs(int ncbw, int ks) { return ks * ncbw * 4 + 2 * (ks / 2) * 4 + 16 * ncbw + ks + 64; }

template <int KS, int EPI>
hipError_t run_wide(const TileArgs& a, int grid, hipStream_t st) {
  const int lds = wide_lds(KS);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k_head_wide<KS, EPI>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  TraceScope ts("head_wide", st, true);
  hipExtLaunchKernelGGL((k_head_wide<KS, EPI>), dim3(static_cast<unsigned>(grid)), dim3(kWideThreads), lds, st,
                        ts.start(), ts.stop(), 0, a);
  return hipGetLastError();
}

template <int KS>
hipError_t run_wide_mode(const TileArgs& a, int grid, hipStream_t st) {
  const int epi = (a.want_stats ? kWideStats : 0) | (a.want_argmax ? kWideArgmax : 0);
  switch (epi) {
    case kWideStats: return run_wide<KS, kWideStats>(a, grid, st);
    case kWideArgmax: return run_wide<KS, kWideArgmax>(a, grid, st);
    case kWideStats | kWideArgmax: return run_wide<KS, kWideStats | kWideArgmax>(a, grid, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool head_wide_supported(int64_t M, int64_t K, int64_t V, bool bf16, int64_t ld) {
  if (ld <= 0) ld = K;
  if (!bf16 || M <= kTileMaxRows || M > kWideMaxRows || K < 8 || K % 8 != 0 || K > 512) return false;
  if (ld < K || ld % 8 != 0 || V < 1 || V * ld * 2 > int64_t{0xFFFFFFF0}) return false;
  const int ks = wide_ks(K);
  const int ncbw = static_cast<int>((M + 16 * kWideWaves - 1) / (16 * kWideWaves));   // blocks per wave at most
  // two waves per SIMD: at most 256 registers per lane
  return wide_regs(ncbw, ks) <= 256 && wide_lds(ks) <= 160 * 1024;
}

int head_wide_grid(int64_t V) {
  DeviceInfo di;
  if (device_info(&di) != hipSuccess) di.cus = 256;
  const int64_t NG = (V + kGroup - 1) / kGroup;
  int64_t grid = NG < di.cus ? NG : di.cus;   // one workgroup per CU
  if (grid > kMaxPartials) grid = kMaxPartials;
  return static_cast<int>(grid < 1 ? 1 : grid);
}

hipError_t launch_head_wide(const TileArgs& a, int grid, hipStream_t st) {
  if (!head_wide_supported(a.M, a.K, a.V, true, a.ld) || a.zout != nullptr || a.hist != nullptr)
    return hipErrorInvalidValue;
  switch (wide_ks(a.K)) {
    case 4: return run_wide_mode<4>(a, grid, st);
    case 8: return run_wide_mode<8>(a, grid, st);
    case 12: return run_wide_mode<12>(a, grid, st);
    default: return run_wide_mode<16>(a, grid, st);
  }
}

}  // namespace sh
