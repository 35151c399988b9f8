// K-chunked head kernel for gfx950: bf16 rows of more than 512 elements (the dense V x d head
// at d = 4096, SlimSpec write-up section 三, and the trimmed head of its rows) and at most 64
// activation rows.
//
//   k_head_kchunk  z = W x over all V rows with per-workgroup Partials (lse, best group score
//                  with the Philox group draw, argmax), the contract of k_head_tile.  A
//                  workgroup owns a consecutive range of at most kKcMaxGroups 64-row
//                  vocabulary groups and walks K in chunks of 512 elements.  Per chunk each
//                  wave loads its B fragments of the chunk once, then every owned group's
//                  64 x 512 weight chunk is read with whole 1 KB row segments into a
//                  double-buffered LDS tile (the next group chunk's loads in flight in
//                  registers while the current one is multiplied) and multiplied on
//                  v_mfma_f32_16x16x32_bf16 into that group's accumulators, which stay in
//                  registers across chunks.  With NCB = ceil(M / 16) >= 2 column blocks, wave w
//                  multiplies all four 16-row tiles of a group for activation rows 16 w ..
//                  16 w + 15; with one column block the four waves split the group's tiles.
//                  After the last chunk every owned group is folded into the running state of
//                  its rows (group log-sum-exp, group draw, argmax), as in the tile kernel, and
//                  in sampling mode the 64 logits of each row's best group of the workgroup go
//                  to a side buffer, so that the finalize reads them instead of recomputing
//                  that group from W.  W is read once; x once per workgroup.
//   The per-row merge of the workgroups' Partials is k_head_fin (head_tile.hip).
#include <hip/hip_ext.h>

#include "device_common.h"
#include "launch.h"
#include "trace.h"

namespace sh {

namespace {

typedef float kf32x4_t __attribute__((ext_vector_type(4)));

constexpr int kKcChunk = 512;                    // elements of K per chunk
constexpr int kKcSteps = kKcChunk / 32;          // k-steps per chunk (16)
constexpr int kKcCpr = kKcChunk * 2 / 16;        // 16-byte pieces per row per chunk (64)
constexpr int kKcRS = kKcCpr + 1;                // LDS row stride in pieces (odd: conflict-free)
constexpr int kKcStats = 1, kKcArgmax = 2;

// per-group statistics of one activation row: max logit, sum of exp((z - max) / T), and the
// lowest row holding the max
struct KcStat {
  float zm, ss;
  int32_t zi;
};

}  // namespace

template <int NCB, int EPI>
__global__ __launch_bounds__((NCB == 1 ? 4 : NCB) * 64, 1) void k_head_kchunk(TileArgs a) {
  constexpr bool STATS = (EPI & kKcStats) != 0, AMAX = (EPI & kKcArgmax) != 0;
  constexpr int NW = NCB == 1 ? 4 : NCB;         // waves
  constexpr int TPW = NCB == 1 ? 1 : 4;          // 16-row tiles of a group each wave multiplies
  constexpr int PER = (kGroup + NW - 1) / NW;    // group rows each wave loads per chunk
  constexpr int TILE = kGroup * kKcRS;           // LDS pieces of one buffer
  constexpr int MG = kKcMaxGroups;
  extern __shared__ uint4 tile[];                // [2][64][kKcRS]
  const int l = lane_id(), w = wave_id();
  const int col = l & 15, qd = l >> 4;
  const int K = a.K;
  const uint32_t rowbytes = static_cast<uint32_t>(a.K) * 2;
  const int V32 = static_cast<int>(a.V);
  const int NG = (V32 + kGroup - 1) / kGroup;
  const uint32_t vbytes = static_cast<uint32_t>(V32) * rowbytes;
  const int Mx = a.M;
  const float c2 = a.invT * kLog2e;
  const int nch = (K + kKcChunk - 1) / kKcChunk;
  const int G = static_cast<int>(gridDim.x);
  const int gs = static_cast<int>((static_cast<int64_t>(blockIdx.x) * NG) / G);
  const int ge = static_cast<int>((static_cast<int64_t>(blockIdx.x + 1) * NG) / G);
  const int ng = ge - gs;                        // 1..kKcMaxGroups (the host sizes the grid)
  const int cb = NCB == 1 ? 0 : w;               // this wave's column block
  const int t0 = NCB == 1 ? w : 0;               // this wave's first tile
  const int mcol = cb * 16 + col;                // this lane's activation row in the B operand

  // This thread's pieces of a group chunk: wave w loads rows w, w + NW, ... of the group,
  // lane l the 16 bytes at element 8 l of the chunk (a whole 1 KB row segment per wave).
  const int prow = w, pc = l;
  const uint32_t pbase = static_cast<uint32_t>(prow) * rowbytes + static_cast<uint32_t>(pc) * 16u;
  const uint32_t pstep = static_cast<uint32_t>(NW) * rowbytes;
  // loads of (chunk ch, group g): rows of the group, elements [512 ch, 512 ch + 512) below K
  auto cload = [&](int ch, int g, uint4 (&R)[PER]) {
    const uint32_t b0 = static_cast<uint32_t>(g) * kGroup * rowbytes;   // g < NG: below vbytes
    const rsrc_t rs = make_rsrc(static_cast<const char*>(a.W) + b0, vbytes - b0);
    const bool kok = ch * kKcChunk + pc * 8 < K;
    const uint32_t o0 = pbase + static_cast<uint32_t>(ch) * (kKcChunk * 2);
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const bool ok = kok && prow + NW * j < kGroup;
      R[j] = buffer_load16(rs, ok ? o0 + pstep * static_cast<uint32_t>(j) : kOutOfRange);
    }
  };
  // row prow + NW j at LDS piece (prow + NW j) * kKcRS + pc (only the last row of a wave
  // can lie past the group; the test is uniform over the wave)
  auto cstore = [&](const uint4 (&R)[PER], int buf) {
    uint4* t = tile + buf * TILE + prow * kKcRS + pc;
#pragma unroll
    for (int j = 0; j < PER; ++j)
      if (j + 1 < PER || prow + NW * j < kGroup) t[NW * j * kKcRS] = R[j];
  };

  kf32x4_t acc[MG][TPW];
#pragma unroll
  for (int gi = 0; gi < MG; ++gi)
#pragma unroll
    for (int t = 0; t < TPW; ++t) acc[gi][t] = kf32x4_t{0.f, 0.f, 0.f, 0.f};

  const rsrc_t xrs = make_rsrc(a.x, static_cast<uint32_t>(Mx) * rowbytes);
  uint4 R[PER];
  cload(0, gs, R);
  int buf = 0;
  for (int ch = 0; ch < nch; ++ch) {
    // this wave's B fragments of the chunk: Bf[s] = x[mcol][512 ch + 32 s + 8 qd ..+8]
    uint4 Bf[kKcSteps];
#pragma unroll
    for (int s = 0; s < kKcSteps; ++s) {
      const int k = ch * kKcChunk + s * 32 + qd * 8;
      Bf[s] = buffer_load16(xrs, (mcol < Mx && k < K) ? static_cast<uint32_t>(mcol) * rowbytes + static_cast<uint32_t>(k) * 2u
                                                      : kOutOfRange);
    }
#pragma unroll
    for (int gi = 0; gi < MG; ++gi) {
      if (gi < ng) {   // uniform over the workgroup
        __syncthreads();   // every wave is done with this buffer's previous contents
        cstore(R, buf);    // waits for the outstanding loads: exactly this group chunk's
        __syncthreads();
        // the next group chunk (next group, or the first group of the next chunk; past the
        // end the current one is re-read, cache-resident) is in flight while this one is
        // multiplied
        {
          const bool last_g = gi + 1 >= ng;
          const bool more = !last_g || ch + 1 < nch;
          cload(more ? (last_g ? ch + 1 : ch) : ch, more ? (last_g ? gs : gs + gi + 1) : gs + gi, R);
        }
        __builtin_amdgcn_sched_barrier(0);
        const uint4* trow = tile + buf * TILE + (t0 * 16 + col) * kKcRS + qd;
        uint4 af[2][TPW];
#pragma unroll
        for (int t = 0; t < TPW; ++t) af[0][t] = trow[t * 16 * kKcRS];
#pragma unroll
        for (int s = 0; s < kKcSteps; ++s) {
          // the A fragments of k-step s + 1 are read while those of s are multiplied
          if (s + 1 < kKcSteps) {
#pragma unroll
            for (int t = 0; t < TPW; ++t) af[(s + 1) & 1][t] = trow[t * 16 * kKcRS + 4 * (s + 1)];
          }
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int t = 0; t < TPW; ++t)
            acc[gi][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, af[s & 1][t]),
                                                                 __builtin_bit_cast(bf16x8_t, Bf[s]), acc[gi][t], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
        buf ^= 1;
      }
    }
  }

  // ---- per-group statistics of this wave's rows of each group ----
  // lane (col, qd) holds rows gb + 16 (t0 + t) + 4 qd + v of activation row mcol
  auto zval = [&](int gi, int i) {
    const int row = (gs + gi) * kGroup + (t0 + (i >> 2)) * 16 + qd * 4 + (i & 3);
    return row < V32 ? acc[gi][i >> 2][i & 3] : -INFINITY;
  };
  KcStat st[MG];
#pragma unroll
  for (int gi = 0; gi < MG; ++gi) {
    st[gi] = KcStat{-INFINITY, 0.f, 0x7fffffff};
    if (gi < ng) {
      const int gb = (gs + gi) * kGroup;
      float z[TPW * 4];
#pragma unroll
      for (int i = 0; i < TPW * 4; ++i) z[i] = zval(gi, i);
      float zm = z[0];
#pragma unroll
      for (int i = 1; i < TPW * 4; ++i) zm = fmaxf(zm, z[i]);
      // the four lanes col, col + 16, col + 32, col + 48 hold the wave's rows of the group
      // and end with the same values (the max is taken first, so the sum needs no rescaling)
      zm = fmaxf(zm, xor_lane(zm, 16));
      zm = fmaxf(zm, xor_lane(zm, 32));
      float ss = 0.f;
      if constexpr (STATS) {
        const float off = zm * c2;
#pragma unroll
        for (int i = 0; i < TPW * 4; ++i) ss += fast_exp2(fmaf(z[i], c2, -off));
        ss += xor_lane(ss, 16);
        ss += xor_lane(ss, 32);
        ss = zm == -INFINITY ? 0.f : ss;
      }
      int32_t zi = 0x7fffffff;
      if constexpr (AMAX) {
#pragma unroll
        for (int i = TPW * 4 - 1; i >= 0; --i)   // the lane's rows rise with i: keep the lowest
          if (z[i] == zm) zi = gb + (t0 + (i >> 2)) * 16 + qd * 4 + (i & 3);
        zi = zm == -INFINITY ? 0x7fffffff : zi;
        zi = min(zi, xor_lane(zi, 16));
        zi = min(zi, xor_lane(zi, 32));
      }
      st[gi] = KcStat{zm, ss, zi};
    }
  }
  if constexpr (NCB == 1) {
    // the four waves hold the four tiles of each group: merge them, in tile order, through
    // LDS (the same result in every wave)
    KcStat* xs = reinterpret_cast<KcStat*>(tile);   // [MG][4 waves][16 cols]
    __syncthreads();                                // the tiles are no longer read
    if (qd == 0) {
#pragma unroll
      for (int gi = 0; gi < MG; ++gi) xs[(gi * 4 + w) * 16 + col] = st[gi];
    }
    __syncthreads();
#pragma unroll
    for (int gi = 0; gi < MG; ++gi) {
      if (gi < ng) {
        KcStat s = xs[(gi * 4) * 16 + col];
#pragma unroll
        for (int ww = 1; ww < 4; ++ww) {
          const KcStat o = xs[(gi * 4 + ww) * 16 + col];
          if constexpr (STATS) {
            const float mx = fmaxf(s.zm, o.zm);
            s.ss = mx == -INFINITY ? 0.f : s.ss * fast_exp2((s.zm - mx) * c2) + o.ss * fast_exp2((o.zm - mx) * c2);
          }
          if constexpr (AMAX) argmax_merge(s.zm, s.zi, o.zm, o.zi);
          else s.zm = fmaxf(s.zm, o.zm);
        }
        st[gi] = s;
      }
    }
  }

  // ---- fold the groups, in order, into the running state of row mcol ----
  // (every lane of the row does the same arithmetic; lanes keep their own logits of the best
  // group for the side buffer)
  const bool live = mcol < Mx;
  float rm = -INFINITY, rsum = 0.f, gbest = -INFINITY, bz = -INFINITY;
  int32_t gid = 0x7fffffff, bi = 0x7fffffff;
  float zb[TPW * 4];
#pragma unroll
  for (int i = 0; i < TPW * 4; ++i) zb[i] = -INFINITY;
  float gc[4] = {0.f, 0.f, 0.f, 0.f};
  int gq = -1;
#pragma unroll
  for (int gi = 0; gi < MG; ++gi) {
    if (gi < ng) {
      const int g = gs + gi;
      if constexpr (STATS) {
        float gu = 0.f;
        if (a.sample != 0) {
          if ((g >> 2) != gq) {   // one Philox block serves four consecutive groups
            gq = g >> 2;
            if (live) {
              uint64_t wd[4];
              philox_block(a.seed, a.offset, kDraftGroup, static_cast<uint64_t>(a.row0 + mcol),
                           static_cast<uint64_t>(gq) * 4, wd);
#pragma unroll
              for (int i = 0; i < 4; ++i) gc[i] = gumbel(word_to_uniform(wd[i]));
            }
          }
          const int q = g & 3;
          gu = q == 0 ? gc[0] : q == 1 ? gc[1] : q == 2 ? gc[2] : gc[3];
        }
        const float L = st[gi].zm * a.invT + log2f(st[gi].ss) * kLn2;   // group log-sum-exp of y = z / T
        const float mn = fmaxf(rm, L);
        rsum = rsum * fast_exp2((rm - mn) * kLog2e) + fast_exp2((L - mn) * kLog2e);
        rm = mn;
        const float sc = L + gu;
        if (a.sample != 0 && sc > gbest) {   // groups rise: strict > keeps the lowest on ties
          gbest = sc;
          gid = g;
#pragma unroll
          for (int i = 0; i < TPW * 4; ++i) zb[i] = zval(gi, i);
        }
      }
      if constexpr (AMAX) argmax_merge(bz, bi, st[gi].zm, st[gi].zi);
    }
  }
  if (live && w == cb && qd == 0) {   // one lane per activation row
    Partial p;
    p.m = rm;
    p.s = rsum;
    p.gscore = gbest;
    p.g = gid;
    p.zmax = bz;
    p.zid = bi;
    p.xz = -INFINITY;
    p.pad1 = 0.f;
    a.partials[static_cast<int64_t>(mcol) * a.partials_ld + blockIdx.x] = p;
  }
  if constexpr (STATS) {
    if (a.sample != 0 && a.gz != nullptr && live) {
      float* gz = a.gz + (static_cast<int64_t>(mcol) * a.gz_ld + blockIdx.x) * kGroup;
#pragma unroll
      for (int t = 0; t < TPW; ++t)
        *reinterpret_cast<float4*>(gz + (t0 + t) * 16 + qd * 4) =
            make_float4(zb[t * 4], zb[t * 4 + 1], zb[t * 4 + 2], zb[t * 4 + 3]);
    }
  }
}

// ----------------------------------------------------------------------------------------
// host side
// ----------------------------------------------------------------------------------------
namespace {

template <int NCB, int EPI>
hipError_t run_kchunk(const TileArgs& a, int grid, hipStream_t st) {
  constexpr int NW = NCB == 1 ? 4 : NCB;
  const int lds = 2 * kGroup * kKcRS * 16;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k_head_kchunk<NCB, EPI>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  TraceScope ts("head_kchunk", st, true);
  hipExtLaunchKernelGGL((k_head_kchunk<NCB, EPI>), dim3(static_cast<unsigned>(grid)), dim3(NW * kWave), lds, st,
                        ts.start(), ts.stop(), 0, a);
  return hipGetLastError();
}

template <int NCB>
hipError_t run_kchunk_mode(const TileArgs& a, int grid, hipStream_t st) {
  const int epi = (a.want_stats ? kKcStats : 0) | (a.want_argmax ? kKcArgmax : 0);
  switch (epi) {
    case kKcStats: return run_kchunk<NCB, kKcStats>(a, grid, st);
    case kKcArgmax: return run_kchunk<NCB, kKcArgmax>(a, grid, st);
    case kKcStats | kKcArgmax: return run_kchunk<NCB, kKcStats | kKcArgmax>(a, grid, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool head_kchunk_supported(int64_t M, int64_t K, int64_t V, bool bf16) {
  return bf16 && M >= 1 && M <= kTileMaxRows && K > 512 && K % 8 == 0 && V >= 1 &&
         V * K * 2 <= int64_t{0xFFFFFFF0};
}

int head_kchunk_grid(int64_t V) {
  DeviceInfo di;
  if (device_info(&di) != hipSuccess) di.cus = 256;
  const int64_t NG = (V + kGroup - 1) / kGroup;
  int64_t grid = di.cus;
  const int64_t need = (NG + kKcMaxGroups - 1) / kKcMaxGroups;   // at most kKcMaxGroups each
  if (grid < need) grid = need;
  if (grid > NG) grid = NG;
  if (grid > kMaxPartials) grid = kMaxPartials;
  return static_cast<int>(grid < 1 ? 1 : grid);
}

size_t head_kchunk_side_bytes(int64_t M, int64_t K, int64_t V) {
  if (!head_kchunk_supported(M, K, V, true)) return 0;
  const int64_t NG = (V + kGroup - 1) / kGroup;
  const int64_t P = NG < kMaxPartials ? NG : kMaxPartials;   // bounds the grid
  return static_cast<size_t>(M * P * kGroup) * sizeof(float);
}

hipError_t launch_head_kchunk(const TileArgs& a, int grid, hipStream_t st) {
  if (!head_kchunk_supported(a.M, a.K, a.V, true) || a.zout != nullptr || a.hist != nullptr || a.ld != 0)
    return hipErrorInvalidValue;
  const int64_t NG = (a.V + kGroup - 1) / kGroup;
  if (grid < 1 || grid > NG || (NG + grid - 1) / grid > kKcMaxGroups) return hipErrorInvalidValue;
  if (a.gz != nullptr && a.gz_ld < grid) return hipErrorInvalidValue;
  switch ((a.M + 15) / 16) {
    case 1: return run_kchunk_mode<1>(a, grid, st);
    case 2: return run_kchunk_mode<2>(a, grid, st);
    case 3: return run_kchunk_mode<3>(a, grid, st);
    default: return run_kchunk_mode<4>(a, grid, st);
  }
}

}  // namespace sh
