// Tile-streaming head kernel for gfx950: bf16 weights with rows of at most 1 KB (the SlimSpec
// r -> V map at r <= 512, the SpecVocab approximate scorer at d' <= 512).
//
//   k_head_tile  four waves per workgroup, one workgroup per CU; each wave owns whole 64-row
//                vocabulary groups (g = its wave index + i * waves in the grid).  A group is
//                four 16-row tiles; tile t + 1 is loaded while tile t is multiplied on
//                v_mfma_f32_16x16x32_bf16 (weights as the A operand straight from HBM, one
//                16-byte load per lane per 32-wide k-step; the activations' B fragments stay in
//                registers for the whole pass).  After the fourth tile the group's 64 logits of
//                every activation row are reduced once: in-lane over 16 rows, then across the
//                four lanes holding the rest; lane (col, qd) then folds the group into the
//                running lse, the best group score L_g + Gumbel(u_g) (sampling) and the argmax of
//                activation row 16 qd + col.  Each workgroup writes one Partial per row.
//   k_head_fin   per row: merges the workgroups' Partials into lse, argmax and the winning
//                group; sampling recomputes that group's 64 logits and draws the element.
//
// The sampler is the two-level Gumbel-max over groups of 64 consecutive candidates; the group
// draws use Philox purpose 0 (draft group), the element draw purpose 1 (draft element).
#include "device_common.h"
#include "launch.h"
#include "trace.h"

namespace sh {

namespace {

typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kTileThreads = 256;   // 4 waves: the four 16-row tiles of a group

}  // namespace

// EPI bits: kEpiStats (row lse; with sampling, the group draws), kEpiArgmax (greedy argmax)
constexpr int kEpiStats = 1, kEpiArgmax = 2;

template <int NCB, int KS, bool ZOUT, int EPI>
__global__ __launch_bounds__(kTileThreads, 1) void k_head_tile(TileArgs a) {
  constexpr int NC = NCB * 16;           // activation rows (columns of the output tiles) per pass
  constexpr int RPL = (NCB + 3) / 4;     // activation rows finished by each lane
  constexpr bool STATS = (EPI & kEpiStats) != 0, AMAX = (EPI & kEpiArgmax) != 0;
  constexpr int CPRP = KS * 4;           // 16-byte chunks per activation row in LDS (K padded)
  constexpr int RS = CPRP + 4;           // LDS row stride in chunks
  extern __shared__ uint4 smem[];        // staged activations [NC][RS], later Partial records [4][NC]
  const int l = lane_id(), w = wave_id();
  const int col = l & 15, qd = l >> 4;
  const uint32_t rowbytes = static_cast<uint32_t>(a.K) * 2;
  const int CPR = static_cast<int>(rowbytes / 16);
  const int V32 = static_cast<int>(a.V);
  const int NG = (V32 + kGroup - 1) / kGroup;
  const int Mx = a.M;
  const int NW = static_cast<int>(gridDim.x) * (kTileThreads / kWave);
  const int gw = static_cast<int>(blockIdx.x) * (kTileThreads / kWave) + w;
  const int iters = gw < NG ? (NG - gw + NW - 1) / NW : 0;   // this wave's groups gw, gw + NW, ...
  const float c2 = a.invT * kLog2e;
  const char* Wb = static_cast<const char*>(a.W);

  // ---- weight tiles: tile t of group g is 16 rows; lane (col, qd) of load j holds row col,
  // bytes 64 j + 16 qd .. +16 (the A operand of v_mfma_f32_16x16x32_bf16).  The descriptor
  // starts at the tile's first row (or at V past the last row) and reaches to the end of the
  // matrix: rows past V read zero.  Scalar arithmetic only (the host admits matrices of at most
  // 0xFFFFFFF0 bytes, and rows of exactly KS 32-wide k-steps).
  const uint32_t vbytes = static_cast<uint32_t>(V32) * rowbytes;
  const uint32_t lane_off = static_cast<uint32_t>(col) * rowbytes + static_cast<uint32_t>(qd) * 16;
  auto tile_load = [&](int g, int t, uint4 (&X)[KS]) {
    const int r0 = g * kGroup + t * 16;
    const uint32_t b0 = r0 < V32 ? static_cast<uint32_t>(r0) * rowbytes : vbytes;
    const rsrc_t rs = make_rsrc(Wb + b0, vbytes - b0);
#pragma unroll
    for (int j = 0; j < KS; ++j) X[j] = buffer_load16(rs, lane_off + static_cast<uint32_t>(j) * 64);
  };

  // ---- activations: staged contiguously through LDS, then each wave keeps its B fragments in
  // registers: Bf[j][cb] holds x[cb * 16 + col][32 j + 8 qd ..+8], zero past M and K
  uint4 XA[KS], XB[KS];
  uint4 Bf[KS][NCB];
  {
    const rsrc_t xrs = make_rsrc(a.x, static_cast<uint32_t>(Mx) * rowbytes);
    constexpr int XPER = (NC * CPRP + kTileThreads - 1) / kTileThreads;
    uint4 xv[XPER];
#pragma unroll
    for (int q = 0; q < XPER; ++q) {
      const int f = q * kTileThreads + static_cast<int>(threadIdx.x);
      xv[q] = buffer_load16(xrs, f < Mx * CPR ? static_cast<uint32_t>(f) * 16 : kOutOfRange);
    }
    tile_load(iters > 0 ? gw : 0, 0, XA);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 0; q < XPER; ++q) {
      const int f = q * kTileThreads + static_cast<int>(threadIdx.x);
      const int m = f / CPR, c = f - m * CPR;
      if (f < Mx * CPR) smem[m * RS + c] = xv[q];
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < KS; ++j)
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        const int m = cb * 16 + col, c = 4 * j + qd;
        Bf[j][cb] = (m < Mx && c < CPR) ? smem[m * RS + c] : zero16();
      }
  }

  // ---- running state of the rows this lane finishes: row cb * 16 + col for cb = qd + 4 k
  float rm[RPL], rsum[RPL], gbest[RPL], bz[RPL];
  int32_t gid[RPL], bi[RPL];
#pragma unroll
  for (int k = 0; k < RPL; ++k) {
    rm[k] = -INFINITY;
    rsum[k] = 0.f;
    gbest[k] = -INFINITY;
    bz[k] = -INFINITY;
    gid[k] = 0x7fffffff;
    bi[k] = 0x7fffffff;
  }
  const bool sample = a.sample != 0;
  // Gumbel(u) of this lane's rows for group g (independent of the MFMAs: overlaps them)
  auto draw = [&](int g, float (&gu)[RPL]) {
#pragma unroll
    for (int k = 0; k < RPL; ++k) {
      const int m = (qd + 4 * k) * 16 + col;
      gu[k] = 0.f;
      if (STATS && sample && qd + 4 * k < NCB && m < Mx)
        gu[k] = gumbel(philox_uniform(a.seed, a.offset, kDraftGroup, static_cast<uint64_t>(a.row0 + m),
                                      static_cast<uint64_t>(g)));
    }
  };

  f32x4_t acc[4][NCB];
  auto mma = [&](const uint4 (&X)[KS], auto tc) {
    constexpr int t = decltype(tc)::value;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) acc[t][cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < KS; ++j) {
      const bf16x8_t af = __builtin_bit_cast(bf16x8_t, X[j]);
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
        acc[t][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, __builtin_bit_cast(bf16x8_t, Bf[j][cb]), acc[t][cb], 0, 0, 0);
    }
  };
  // raw logits of tile t: lane (col, qd) holds rows 16 t + 4 qd .. +3 of activation row cb * 16 + col
  auto store_z = [&](int g, int t) {
    if constexpr (ZOUT) {
      const int r0 = g * kGroup + t * 16 + qd * 4;
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        const int m = cb * 16 + col;
        if (m < Mx) {
          float* zo = a.zout + static_cast<int64_t>(m) * a.zout_ld;
#pragma unroll
          for (int v = 0; v < 4; ++v)
            if (r0 + v < V32) zo[r0 + v] = acc[t][cb][v];
        }
      }
    }
  };
  // fold group g (the four tiles' accumulators) into the running state
  auto group_end = [&](int g, const float (&gu)[RPL]) {
    if constexpr (EPI != 0) {
      const int gb = g * kGroup;
      const bool full = gb + kGroup <= V32;
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        float z[16];
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int row = gb + t * 16 + qd * 4 + v;
            z[t * 4 + v] = (full || row < V32) ? acc[t][cb][v] : -INFINITY;
          }
        float zm = z[0];
#pragma unroll
        for (int i = 1; i < 16; ++i) zm = fmaxf(zm, z[i]);
        float ss = 0.f;
        if constexpr (STATS) {
          // (a lane whose 16 rows all lie past V has zm = -inf and keeps ss = 0)
          const float off = zm * c2;
#pragma unroll
          for (int i = 0; i < 16; ++i) ss += fast_exp2(fmaf(z[i], c2, -off));
          ss = zm == -INFINITY ? 0.f : ss;
        }
        int32_t zi = 0x7fffffff;
        if constexpr (AMAX) {
          int bsel = 15;
#pragma unroll
          for (int i = 15; i >= 0; --i)   // the lane's rows rise with i: keep the lowest
            if (z[i] == zm) bsel = i;
          zi = gb + (bsel >> 2) * 16 + qd * 4 + (bsel & 3);
        }
        // the four lanes col, col + 16, col + 32, col + 48 hold the group's 64 rows
#pragma unroll
        for (int o = 16; o <= 32; o <<= 1) {
          const float zm2 = xor_lane(zm, o);
          if constexpr (STATS) {
            const float ss2 = xor_lane(ss, o);
            const float mx = fmaxf(zm, zm2);
            ss = mx == -INFINITY ? 0.f : ss * fast_exp2((zm - mx) * c2) + ss2 * fast_exp2((zm2 - mx) * c2);
          }
          if constexpr (AMAX) {
            const int32_t zi2 = xor_lane(zi, o);
            argmax_merge(zm, zi, zm2, zi2);
          } else {
            zm = fmaxf(zm, zm2);
          }
        }
        // lane (col, qd) finishes activation row cb * 16 + col when cb = qd + 4 k
#pragma unroll
        for (int k = 0; k < RPL; ++k) {
          if (cb == qd + 4 * k && cb * 16 + col < Mx) {
            if constexpr (STATS) {
              const float L = zm * a.invT + log2f(ss) * kLn2;   // group log-sum-exp of y = z / T
              const float mn = fmaxf(rm[k], L);
              rsum[k] = rsum[k] * fast_exp2((rm[k] - mn) * kLog2e) + fast_exp2((L - mn) * kLog2e);
              rm[k] = mn;
              const float sc = L + gu[k];
              if (sample && sc > gbest[k]) {   // groups rise: strict > keeps the lowest on ties
                gbest[k] = sc;
                gid[k] = g;
              }
            }
            if constexpr (AMAX) argmax_merge(bz[k], bi[k], zm, zi);
          }
        }
      }
    }
  };

  // Pipeline: tile t + 1 (or the next group's tile 0) is loaded while tile t is multiplied.
  // Loads are straight-line (past the last group the current tile is re-read, cache-resident)
  // and pinned above the MFMAs by scheduling barriers, so the wait before each MFMA leaves
  // exactly the next tile in flight.
  for (int i = 0; i < iters; ++i) {
    const int g = gw + i * NW;
    const int gn = i + 1 < iters ? g + NW : g;
    float gu[RPL];
    tile_load(g, 1, XB);
    __builtin_amdgcn_sched_barrier(0);
    draw(g, gu);
    mma(XA, std::integral_constant<int, 0>{});
    store_z(g, 0);
    tile_load(g, 2, XA);
    __builtin_amdgcn_sched_barrier(0);
    mma(XB, std::integral_constant<int, 1>{});
    store_z(g, 1);
    tile_load(g, 3, XB);
    __builtin_amdgcn_sched_barrier(0);
    mma(XA, std::integral_constant<int, 2>{});
    store_z(g, 2);
    tile_load(gn, i + 1 < iters ? 0 : 3, XA);
    __builtin_amdgcn_sched_barrier(0);
    mma(XB, std::integral_constant<int, 3>{});
    store_z(g, 3);
    group_end(g, gu);
  }
  if constexpr (EPI != 0) {
    // merge the four waves' states per activation row, one Partial per row per workgroup
    __syncthreads();   // the staged activations are no longer read
    Partial* rec = reinterpret_cast<Partial*>(smem);
#pragma unroll
    for (int k = 0; k < RPL; ++k) {
      const int cb = qd + 4 * k, m = cb * 16 + col;
      if (cb < NCB && m < Mx) {
        Partial p;
        p.m = rm[k];
        p.s = rsum[k];
        p.gscore = gbest[k];
        p.g = gid[k];
        p.zmax = bz[k];
        p.zid = bi[k];
        p.pad0 = p.pad1 = 0.f;
        rec[w * NC + m] = p;
      }
    }
    __syncthreads();
    for (int m = threadIdx.x; m < Mx; m += kTileThreads) {
      Partial p = rec[m];
#pragma unroll
      for (int ww = 1; ww < kTileThreads / kWave; ++ww) partial_merge(p, rec[ww * NC + m]);
      a.partials[static_cast<int64_t>(m) * a.partials_ld + blockIdx.x] = p;
    }
  }
}

// ----------------------------------------------------------------------------------------
// k_head_fin: one workgroup (16 waves) per row.
// ----------------------------------------------------------------------------------------
constexpr int kHfThreads = 1024;
constexpr int kHfWaves = kHfThreads / kWave;
constexpr int kHfRowsPerWave = kGroup / kHfWaves;   // 4

template <bool BF16>
__global__ __launch_bounds__(kHfThreads) void k_head_fin(FinalizeArgs f) {
  __shared__ Partial rec[kHfWaves];
  __shared__ float zs[kGroup];
  const int m = blockIdx.x;
  const int l = lane_id(), w = wave_id();
  Partial acc = partial_empty();
  const Partial* pp = f.partials + static_cast<int64_t>(m) * f.partials_ld;
  for (int p = threadIdx.x; p < f.P; p += kHfThreads) partial_merge(acc, pp[p]);
  wave_partial_merge(acc);
  if (l == 0) rec[w] = acc;
  __syncthreads();
  acc = l < kHfWaves ? rec[l] : partial_empty();
  wave_partial_merge(acc);   // the same result in every wave
  const float lse = acc.m + logf(acc.s);

  int32_t tok;
  float ytok;
  if (f.mode == 0) {
    tok = acc.zid;
    ytok = acc.zmax * f.invT;
  } else {
    // recompute the 64 logits of the winning group, 4 rows per wave, loads issued together
    const int C = static_cast<int>(f.K * (BF16 ? 2 : 4) / 16);
    const int CPL = (C + kWave - 1) / kWave;
    const uint32_t rowbytes = static_cast<uint32_t>(C) * 16;
    const int64_t gbase = static_cast<int64_t>(acc.g == 0x7fffffff ? 0 : acc.g) * kGroup;
    const int64_t r0 = gbase + w * kHfRowsPerWave;
    const int nrows = f.V - r0 >= kHfRowsPerWave ? kHfRowsPerWave : (f.V - r0 > 0 ? static_cast<int>(f.V - r0) : 0);
    const rsrc_t wrs = make_rsrc(static_cast<const char*>(f.W) + static_cast<size_t>(nrows > 0 ? r0 : 0) * rowbytes,
                                 static_cast<uint32_t>(nrows) * rowbytes);
    const rsrc_t xrs = make_rsrc(static_cast<const char*>(f.x) + static_cast<size_t>(m) * rowbytes, rowbytes);
    float z[kHfRowsPerWave];
#pragma unroll
    for (int j = 0; j < kHfRowsPerWave; ++j) z[j] = 0.f;
    for (int q0 = 0; q0 < CPL; q0 += 4) {
      uint4 xv[4], wv[4][kHfRowsPerWave];
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const int c = (q0 + qq) * kWave + l;
        const bool cok = q0 + qq < CPL && c < C;
        xv[qq] = buffer_load16(xrs, cok ? static_cast<uint32_t>(c) * 16 : kOutOfRange);
#pragma unroll
        for (int j = 0; j < kHfRowsPerWave; ++j)
          wv[qq][j] = buffer_load16(wrs, cok ? static_cast<uint32_t>(j) * rowbytes + static_cast<uint32_t>(c) * 16 : kOutOfRange);
      }
#pragma unroll
      for (int qq = 0; qq < 4; ++qq)
#pragma unroll
        for (int j = 0; j < kHfRowsPerWave; ++j) z[j] = chunk_dot<BF16>(wv[qq][j], xv[qq], z[j]);
    }
#pragma unroll
    for (int j = 0; j < kHfRowsPerWave; ++j) {
      const float s = wave_sum(z[j]);
      if (l == 0) zs[w * kHfRowsPerWave + j] = s;
    }
    __syncthreads();
    if (w != 0) return;   // the element draw is one wave's work
    const int64_t row = gbase + l;
    const bool valid = row < f.V;
    const float y = zs[l] * f.invT;
    float e = valid ? y + gumbel(philox_uniform(f.seed, f.offset, kDraftElem, static_cast<uint64_t>(m), row)) : -INFINITY;
    int32_t ei = valid ? l : 0x7fffffff;
    wave_argmax(e, ei);
    const int el = ei == 0x7fffffff ? 0 : ei;
    tok = static_cast<int32_t>(gbase + el);
    ytok = __shfl(y, el);
  }
  if (threadIdx.x == 0) {
    f.token[m] = tok;
    if (f.lse) f.lse[m] = lse;
    if (f.logprob) f.logprob[m] = ytok - lse;
  }
}

// ----------------------------------------------------------------------------------------
// host side
// ----------------------------------------------------------------------------------------
namespace {

template <typename F>
hipError_t allow_lds_tile(F kernel, int bytes) {
  if (bytes <= 64 * 1024) return hipSuccess;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                             bytes);
}

constexpr int kLdsPerCu = 160 * 1024;
// activation fragments live in registers: at most this many 16-byte fragments per lane
constexpr int kMaxBFrags = 64;

int tile_ks(int64_t K) {
  const int64_t ks = (K * 2 + 63) / 64;
  return ks <= 4 ? 4 : ks <= 8 ? 8 : ks <= 12 ? 12 : 16;
}
int tile_ncb(int64_t M) { return static_cast<int>((M + 15) / 16); }
int tile_lds(int ncb, int ks) {
  const int stage = ncb * 16 * (ks * 4 + 4) * 16;
  const int rec = 4 * ncb * 16 * static_cast<int>(sizeof(Partial));
  return stage > rec ? stage : rec;
}

template <int NCB, int KS, bool ZOUT, int EPI>
hipError_t run_tile(const TileArgs& a, int grid, hipStream_t st) {
  if constexpr (NCB * KS > kMaxBFrags) {
    return hipErrorInvalidValue;   // excluded by head_tile_supported
  } else {
    const int lds = tile_lds(NCB, KS);
    hipError_t e = allow_lds_tile(k_head_tile<NCB, KS, ZOUT, EPI>, lds);
    if (e != hipSuccess) return e;
    TraceScope ts("head_tile", st);
    hipLaunchKernelGGL((k_head_tile<NCB, KS, ZOUT, EPI>), dim3(static_cast<unsigned>(grid)), dim3(kTileThreads), lds,
                       st, a);
    return hipGetLastError();
  }
}

template <int NCB, int KS>
hipError_t run_tile_mode(const TileArgs& a, int grid, hipStream_t st) {
  const int epi = (a.want_stats ? kEpiStats : 0) | (a.want_argmax ? kEpiArgmax : 0);
  if (a.zout != nullptr) {
    switch (epi) {
      case 0: return run_tile<NCB, KS, true, 0>(a, grid, st);
      case kEpiStats: return run_tile<NCB, KS, true, kEpiStats>(a, grid, st);
      case kEpiArgmax: return run_tile<NCB, KS, true, kEpiArgmax>(a, grid, st);
      default: return run_tile<NCB, KS, true, kEpiStats | kEpiArgmax>(a, grid, st);
    }
  }
  switch (epi) {
    case kEpiStats: return run_tile<NCB, KS, false, kEpiStats>(a, grid, st);
    case kEpiArgmax: return run_tile<NCB, KS, false, kEpiArgmax>(a, grid, st);
    case kEpiStats | kEpiArgmax: return run_tile<NCB, KS, false, kEpiStats | kEpiArgmax>(a, grid, st);
    default: return hipErrorInvalidValue;   // nothing to compute
  }
}

template <int NCB>
hipError_t run_tile_ks(const TileArgs& a, int grid, hipStream_t st) {
  switch (tile_ks(a.K)) {
    case 4: return run_tile_mode<NCB, 4>(a, grid, st);
    case 8: return run_tile_mode<NCB, 8>(a, grid, st);
    case 12: return run_tile_mode<NCB, 12>(a, grid, st);
    default: return run_tile_mode<NCB, 16>(a, grid, st);
  }
}

}  // namespace

bool head_tile_supported(int64_t M, int64_t K, int64_t V, bool bf16) {
  if (!bf16 || M < 1 || M > kTileMaxRows || K < 1 || K * 2 > 1024) return false;
  if (K % 32 != 0 || tile_ks(K) * 32 != K) return false;   // rows of exactly KS 32-wide k-steps
  if (V < 1 || V * K * 2 > int64_t{0xFFFFFFF0}) return false;   // 32-bit buffer ranges
  const int ncb = tile_ncb(M), ks = tile_ks(K);
  return ks * ncb <= kMaxBFrags && tile_lds(ncb, ks) <= kLdsPerCu;
}

int head_tile_grid(int64_t M, int64_t K, int64_t V) {
  (void)M;
  (void)K;
  DeviceInfo di;
  if (device_info(&di) != hipSuccess) di.cus = 256;
  // one workgroup (four waves) per CU: the activation fragments take most of the register file
  const int64_t NG = (V + kGroup - 1) / kGroup;
  int64_t grid = (NG + 3) / 4;
  if (grid > di.cus) grid = di.cus;
  if (grid > kMaxPartials) grid = kMaxPartials;
  return static_cast<int>(grid < 1 ? 1 : grid);
}

hipError_t launch_head_tile(const TileArgs& a, int grid, hipStream_t st) {
  if (!head_tile_supported(a.M, a.K, a.V, true)) return hipErrorInvalidValue;
  switch (tile_ncb(a.M)) {
    case 1: return run_tile_ks<1>(a, grid, st);
    case 2: return run_tile_ks<2>(a, grid, st);
    case 3: return run_tile_ks<3>(a, grid, st);
    default: return run_tile_ks<4>(a, grid, st);
  }
}

hipError_t launch_head_fin(const FinalizeArgs& f, hipStream_t st) {
  TraceScope ts("head_fin", st);
  if (f.bf16)
    hipLaunchKernelGGL(k_head_fin<true>, dim3(f.M), dim3(kHfThreads), 0, st, f);
  else
    hipLaunchKernelGGL(k_head_fin<false>, dim3(f.M), dim3(kHfThreads), 0, st, f);
  return hipGetLastError();
}

}  // namespace sh
