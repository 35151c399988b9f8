// Tile-streaming head kernels for gfx950: bf16 weights with rows of 128, 256, 384 or 512
// elements and at most 64 activation rows (the SlimSpec r -> V map at r = d/8, the SpecVocab
// approximate scorer at d' = d/16).
//
//   k_head_tile     z = W x over all V rows with per-workgroup Partials (lse, best group
//                   score, argmax) and/or raw scores.  Four waves per workgroup, one
//                   workgroup per CU; each wave owns whole 64-row vocabulary groups.  A group
//                   is four 16-row tiles; tile t + 1 (and t + 2 for rows of at most 256
//                   elements) is loaded while tile t is multiplied on v_mfma_f32_16x16x32_bf16:
//                   every tile is loaded in row layout (each load instruction reads whole rows,
//                   1 KB contiguous), written to the wave's LDS slot and read back as the A
//                   fragments; the activations' B fragments stay in registers for the whole
//                   pass.  After the fourth tile the group's 64
//                   logits of every activation row are reduced once: in-lane over 16 rows, then
//                   across the four lanes holding the rest; lane (col, qd) folds the group into
//                   the running lse, the best group score L_g + Gumbel(u_g) (sampling) and the
//                   argmax of activation row 16 qd + col.
//   k_head_fin      per row: merges the workgroups' Partials into lse, argmax and the winning
//                   group; sampling reads that group's 64 logits from the side buffer its owner
//                   wrote (at most 48 rows), or recomputes them, and draws the element.
//
// The sampler is the two-level Gumbel-max over groups of 64 consecutive candidates; the group
// draws use Philox purpose 0 (draft group), the element draw purpose 1 (draft element).
#include <hip/hip_ext.h>

#include "device_common.h"
#include "launch.h"
#include "trace.h"

namespace sh {

namespace {

typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kTileThreads = 256;   // four waves
constexpr int kTileWaves = kTileThreads / kWave;
// EPI bits: kEpiStats (row lse; with sampling, the group draws), kEpiArgmax (greedy argmax),
// kEpiHist (with raw scores: the top-k histogram of each row's order keys, in LDS, added to
// the caller's [M, 4096] counts at the end), kEpiSide (sampling: each wave copies the 64 logits
// of its best group so far per row into its own LDS area whenever that group changes; the
// workgroup's best of them go to a side buffer, so the finalize reads them instead of
// recomputing the winning group)
constexpr int kEpiStats = 1, kEpiArgmax = 2, kEpiHist = 4, kEpiSide = 8;
// the side copies pay for themselves at one column block (measured: at three blocks the
// tile pass grows by about what the finalize saves, 27.6 -> 29.4 against 9.7 -> 7.8 us)
constexpr int kTileSideMaxNcb = 1;

}  // namespace

// ----------------------------------------------------------------------------------------
// One tile pass of a workgroup: geometry, the activation fragments, the pipelined group loop
// and the per-workgroup Partial of every activation row.
// ----------------------------------------------------------------------------------------
template <int NCB, int KS, bool ZOUT, int EPI>
struct TilePass {
  static constexpr int NC = NCB * 16;   // activation rows (columns of the output tiles)
  static constexpr bool STATS = (EPI & kEpiStats) != 0, AMAX = (EPI & kEpiArgmax) != 0;
  static constexpr bool HIST = (EPI & kEpiHist) != 0;
  static constexpr bool SIDE = (EPI & kEpiSide) != 0;
  static_assert(!HIST || (ZOUT && NCB == 1), "the histogram rides on the raw scores of a few rows");
  static_assert(!SIDE || (STATS && !ZOUT && NCB <= kTileSideMaxNcb), "side copy: sampling stats, few rows");
  static constexpr int CPRP = KS * 4;   // 16-byte chunks per activation row
  static constexpr int RS = CPRP + 4;   // LDS row stride of the staged activations, in chunks
  static constexpr int XPER = (NC * CPRP + kTileThreads - 1) / kTileThreads;
  // LDS bytes: staged activations [NC][RS], later the Partial records [4][NC] and the winning
  // wave of each row [NC] (SIDE); then the side copies [4][NC][68] floats (SIDE: past the staged
  // activations, which other waves may still read when a wave's first group ends) or the
  // histograms [kTileHistRows][4096] (HIST)
  static constexpr int kLdsRec = kTileWaves * NC * 32 + NC * 4;
  // each wave's current weight tile, 16 rows of CPRP chunks at a row stride of CPRP + 1 chunks
  // (the 16 rows of one fragment read then fall on distinct banks); it shares its space with
  // the staged activations (a barrier separates them)
  static constexpr int kSW = CPRP + 1;
  // two tiles in flight (XA and XB) for rows of at most 256 elements, else one (XA).  Measured
  // on one machine: the SpecVocab scorer (256-element rows) 18.6 us with one tile in flight,
  // 17.9 with two; the Llama-shaped W_up pass (512) 27.5 with one, 28.4 with two
  static constexpr bool DUAL = KS <= 8;
  static constexpr int kLdsSlots = kTileWaves * 16 * kSW * 16;
  static constexpr int kLdsMain0 = (NC * RS * 16 > kLdsRec) ? NC * RS * 16 : kLdsRec;
  static constexpr int kLdsMain = kLdsMain0 > kLdsSlots ? kLdsMain0 : kLdsSlots;
  // side copies: a row stride of 68 floats keeps the 16 rows of one write on distinct banks
  static constexpr int kSideStride = kGroup + 4;
  static constexpr int kLds = kLdsMain + (HIST ? kTileHistRows * kTkBins * 4 : 0) +
                              (SIDE ? kTileWaves * NC * kSideStride * 4 : 0);

  const TileArgs& a;
  uint4* smem;
  uint4* slot;   // this wave's weight tile
  int l, w, col, qd;
  uint32_t rowbytes, vbytes;
  // a tile's loads repeat their row pattern every LP loads (64 LP chunks = LROWS whole rows):
  // this lane's offsets in the first LP loads, from the tile's first row
  static constexpr int LP = CPRP == 48 ? 3 : 1;
  static constexpr int LROWS = LP * kWave / CPRP;
  uint32_t loff[LP];
  int soff[LP];   // slot index of this lane's chunk of the first LP loads
  int foff;       // slot index of this lane's A fragment at k-step 0: row col, chunk qd
  int V32, NG, Mx;
  float c2;
  uint4 Bf[KS][NCB];
  f32x4_t acc[4][NCB];
  // running state of activation row 16 qd + col (lanes with qd < NCB)
  float rm = -INFINITY, rsum = 0.f, gbest = -INFINITY, bz = -INFINITY;
  int32_t gid = 0x7fffffff, bi = 0x7fffffff;

  __device__ __forceinline__ TilePass(const TileArgs& args, uint4* lds) : a(args), smem(lds) {
    l = lane_id();
    w = wave_id();
    col = l & 15;
    qd = l >> 4;
    rowbytes = static_cast<uint32_t>(a.ld > 0 ? a.ld : a.K) * 2;   // row stride
    V32 = static_cast<int>(a.V);
    NG = (V32 + kGroup - 1) / kGroup;
    Mx = a.M;
    c2 = a.invT * kLog2e;
    // (the host admits matrices of at most 0xFFFFFFF0 bytes and rows of exactly KS k-steps)
    vbytes = static_cast<uint32_t>(V32) * rowbytes;
    slot = lds + w * 16 * kSW;
#pragma unroll
    for (int j = 0; j < LP; ++j) {
      const int f = j * kWave + l, row = f / CPRP, ch = f - row * CPRP;
      loff[j] = static_cast<uint32_t>(row) * rowbytes + static_cast<uint32_t>(ch) * 16;
      soff[j] = row * kSW + ch;
    }
    foff = col * kSW + qd;
  }

  // Tile t of group g in row layout: load j brings the tile's chunks 64 j .. 64 j + 63 in row
  // order (whole rows, full cache lines per instruction), lane l chunk 64 j + l.  The descriptor
  // starts at the tile's first row (or at V past the last row: group NG is an empty range that
  // reads zeros without touching memory) and reaches to the end of the matrix, so rows past V
  // read zero.  Scalar arithmetic only besides the loads.
  __device__ __forceinline__ void tile_load(int g, int t, uint4 (&X)[KS]) const {
    const int r0 = g * kGroup + t * 16;
    const uint32_t b0 = r0 < V32 ? static_cast<uint32_t>(r0) * rowbytes : vbytes;
    const rsrc_t rs = make_rsrc(static_cast<const char*>(a.W) + b0, vbytes - b0);
#pragma unroll
    for (int j = 0; j < KS; ++j)
      X[j] = buffer_load16(rs, loff[j % LP] + static_cast<uint32_t>(j / LP * LROWS) * rowbytes);
  }
  // the tile into this wave's LDS slot: chunk ch of row r at r * kSW + ch
  __device__ __forceinline__ void stage_tile(const uint4 (&X)[KS]) const {
#pragma unroll
    for (int j = 0; j < KS; ++j) slot[soff[j % LP] + (j / LP) * LROWS * kSW] = X[j];
  }

  // Activations (16-byte chunks of the first K elements of each row of x), then through LDS into the
  // register B fragments: Bf[j][cb] = x[cb * 16 + col][32 j + 8 qd ..+8], zero past M.
  __device__ __forceinline__ void stage_issue(uint4 (&xv)[XPER]) const {
    const rsrc_t xrs = make_rsrc(a.x, static_cast<uint32_t>(Mx) * rowbytes);
#pragma unroll
    for (int q = 0; q < XPER; ++q) {
      const int f = q * kTileThreads + static_cast<int>(threadIdx.x);
      const int m = f / CPRP, c = f - m * CPRP;
      xv[q] = buffer_load16(xrs, f < Mx * CPRP ? static_cast<uint32_t>(m) * rowbytes + static_cast<uint32_t>(c) * 16
                                               : kOutOfRange);
    }
  }
  __device__ __forceinline__ void stage_finish(const uint4 (&xv)[XPER]) {
#pragma unroll
    for (int q = 0; q < XPER; ++q) {
      const int f = q * kTileThreads + static_cast<int>(threadIdx.x);
      const int m = f / CPRP, c = f - m * CPRP;
      if (f < Mx * CPRP) smem[m * RS + c] = xv[q];
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < KS; ++j)
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        const int m = cb * 16 + col;
        Bf[j][cb] = m < Mx ? smem[m * RS + 4 * j + qd] : zero16();
      }
  }

  // Gumbel(u) of this lane's row for group g (independent of the MFMAs, so it overlaps them)
  __device__ __forceinline__ float draw(int g) const {
    const int m = qd * 16 + col;
    if (STATS && a.sample != 0 && qd < NCB && m < Mx)
      return gumbel(philox_uniform(a.seed, a.offset, kDraftGroup, static_cast<uint64_t>(a.row0 + m),
                                   static_cast<uint64_t>(g)));
    return 0.f;
  }

  // tile T of the group from the LDS slot: the A fragment of k-step j is row col, chunk 4 j + qd
  template <int T>
  __device__ __forceinline__ void mma() {
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) acc[T][cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < KS; ++j) {
      const bf16x8_t af = __builtin_bit_cast(bf16x8_t, slot[foff + 4 * j]);
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
        acc[T][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, __builtin_bit_cast(bf16x8_t, Bf[j][cb]), acc[T][cb], 0, 0, 0);
    }
    // one fragment read ahead of its MFMAs at a time (the registers hold the tiles in flight)
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
    for (int j = 1; j < KS; ++j) {
      __builtin_amdgcn_sched_group_barrier(0x008, NCB, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, NCB, 0);
  }

  // raw logits of tile T: lane (col, qd) holds rows 16 T + 4 qd .. +3 of activation row cb*16+col
  template <int T>
  __device__ __forceinline__ void store_z(int g) const {
    if constexpr (ZOUT) {
      const int r0 = g * kGroup + T * 16 + qd * 4;
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        const int m = cb * 16 + col;
        if (m < Mx) {
          float* zo = a.zout + static_cast<int64_t>(m) * a.zout_ld;
#pragma unroll
          for (int v = 0; v < 4; ++v)
            if (r0 + v < V32) {
              zo[r0 + v] = acc[T][cb][v];
              if constexpr (HIST) atomicAdd(&hist()[m * kTkBins + (order_key(acc[T][cb][v]) >> kTkShift)], 1u);
            }
        }
      }
    }
  }
  __device__ __forceinline__ uint32_t* hist() const {
    return reinterpret_cast<uint32_t*>(reinterpret_cast<char*>(smem) + kLdsMain);
  }
  __device__ __forceinline__ void hist_clear() const {
    if constexpr (HIST)
      for (int i = threadIdx.x; i < kTileHistRows * kTkBins; i += kTileThreads) hist()[i] = 0u;
  }
  // add this workgroup's nonzero bins to the rows' histograms
  __device__ __forceinline__ void hist_flush() const {
    if constexpr (HIST) {
      __syncthreads();
      for (int i = threadIdx.x; i < Mx * kTkBins; i += kTileThreads) {
        const uint32_t c = hist()[i];
        if (c != 0u) atomicAdd(&a.hist[i], c);
      }
    }
  }

  // fold group g (the four tiles' accumulators) into the running state (MASK: the
  // vocabulary's last, partial group, whose rows past V are -inf)
  template <bool MASK>
  __device__ __forceinline__ void group_end_body(int g, float gu) {
    const int gb = g * kGroup;
    // per column block: the group's max, sum of exp and first argmax of activation row
    // 16 cb + col; the four lanes col, col + 16, col + 32, col + 48 hold its 64 rows and end
    // with the same values (the max is taken first, so the sum needs no rescaling)
    float bm[NCB], bs[NCB];
    int32_t bx[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
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
    // lane (col, qd) finishes activation row 16 qd + col: one fold per lane
    float zm = bm[0], ss = bs[0];
    int32_t zi = bx[0];
#pragma unroll
    for (int cb = 1; cb < NCB; ++cb)
      if (qd == cb) {
        zm = bm[cb];
        ss = bs[cb];
        zi = bx[cb];
      }
    bool better = false;
    if (qd < NCB && qd * 16 + col < Mx) {
      if constexpr (STATS) {
        const float L = zm * a.invT + log2f(ss) * kLn2;   // group log-sum-exp of y = z / T
        const float mn = fmaxf(rm, L);
        rsum = rsum * fast_exp2((rm - mn) * kLog2e) + fast_exp2((L - mn) * kLog2e);
        rm = mn;
        const float sc = L + gu;
        if (a.sample != 0 && sc > gbest) {   // groups rise: strict > keeps the lowest on ties
          gbest = sc;
          gid = g;
          better = true;
        }
      }
      if constexpr (AMAX) argmax_merge(bz, bi, zm, zi);
    }
    if constexpr (SIDE) {
      // lane (col, cb) decided for activation row 16 cb + col; lanes (col, 0..3) hold its 64
      // logits (tile t, value v: vocabulary row 16 t + 4 qd + v of the group)
      const uint64_t won = __builtin_amdgcn_ballot_w64(better);
      if (won != 0ull) {   // uniform; rare after the first groups
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
          if (((won >> (16 * cb)) & 0xFFFFull) == 0ull) continue;   // uniform
          if ((won >> (col + 16 * cb)) & 1ull) {
            float4* dst = side_copy(w, cb * 16 + col);
#pragma unroll
            for (int t = 0; t < 4; ++t) dst[t * 4 + qd] = make_float4(acc[t][cb][0], acc[t][cb][1], acc[t][cb][2], acc[t][cb][3]);
          }
        }
      }
    }
  }
  // wave w's copy of the best group's 64 logits of activation row m
  __device__ __forceinline__ float4* side_copy(int ww, int m) const {
    return reinterpret_cast<float4*>(reinterpret_cast<char*>(smem) + kLdsMain) + (ww * NC + m) * (kSideStride / 4);
  }
  __device__ __forceinline__ void group_end(int g, float gu) {
    if constexpr (STATS || AMAX) {
      if (g * kGroup + kGroup <= V32) group_end_body<false>(g, gu);   // uniform
      else group_end_body<true>(g, gu);
    }
  }

  // Groups gw, gw + nw, ... of this wave; XA and XB hold tiles 0 and 1 of the first (already
  // issued).  Each tile goes from its registers to the LDS slot, the registers take the load
  // of the tile two ahead (past the last group: the empty range), and the MFMAs read their
  // fragments from the slot, so two tiles are in flight while one is multiplied (one during
  // the group's epilogue).
  __device__ __forceinline__ void run(int gw, int nw, uint4 (&XA)[KS], uint4 (&XB)[KS]) {
    const int iters = gw < NG ? (NG - gw + nw - 1) / nw : 0;
    if constexpr (!DUAL) {
      for (int i = 0; i < iters; ++i) {
        const int g = gw + i * nw;
        const int gn = i + 1 < iters ? g + nw : NG;
        stage_tile(XA);
        tile_load(g, 1, XA);
        __builtin_amdgcn_sched_barrier(0);
        const float gu = draw(g);   // (after the load is out: Philox overlaps it)
        mma<0>();
        store_z<0>(g);
        stage_tile(XA);
        tile_load(g, 2, XA);
        __builtin_amdgcn_sched_barrier(0);
        mma<1>();
        store_z<1>(g);
        stage_tile(XA);
        tile_load(g, 3, XA);
        __builtin_amdgcn_sched_barrier(0);
        mma<2>();
        store_z<2>(g);
        stage_tile(XA);
        tile_load(gn, 0, XA);
        __builtin_amdgcn_sched_barrier(0);
        mma<3>();
        store_z<3>(g);
        group_end(g, gu);
      }
      return;
    }
    for (int i = 0; i < iters; ++i) {
      const int g = gw + i * nw;
      const int gn = i + 1 < iters ? g + nw : NG;
      stage_tile(XA);
      tile_load(g, 2, XA);
      __builtin_amdgcn_sched_barrier(0);
      const float gu = draw(g);   // (after the load is out: Philox overlaps it)
      mma<0>();
      store_z<0>(g);
      stage_tile(XB);
      tile_load(g, 3, XB);
      __builtin_amdgcn_sched_barrier(0);
      mma<1>();
      store_z<1>(g);
      stage_tile(XA);
      tile_load(gn, 0, XA);
      __builtin_amdgcn_sched_barrier(0);
      mma<2>();
      store_z<2>(g);
      stage_tile(XB);
      mma<3>();
      store_z<3>(g);
      group_end(g, gu);
      tile_load(gn, 1, XB);   // after the epilogue, whose registers it would otherwise hold
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // merge the four waves' states per activation row: one Partial per row per workgroup
  __device__ __forceinline__ void write_partials(int wg) {
    __syncthreads();   // the staged activations are no longer read
    Partial* rec = reinterpret_cast<Partial*>(smem);
    const int m = qd * 16 + col;
    if (qd < NCB && m < Mx) {
      Partial p;
      p.m = rm;
      p.s = rsum;
      p.gscore = gbest;
      p.g = gid;
      p.zmax = bz;
      p.zid = bi;
      p.xz = -INFINITY;
      p.pad1 = 0.f;
      rec[w * NC + m] = p;
    }
    __syncthreads();
    int32_t* winner = reinterpret_cast<int32_t*>(reinterpret_cast<char*>(smem) + kTileWaves * NC * 32);
    for (int r = threadIdx.x; r < Mx; r += kTileThreads) {
      Partial p = rec[r];
      int32_t wv = 0;
#pragma unroll
      for (int ww = 1; ww < kTileWaves; ++ww) {
        const Partial q = rec[ww * NC + r];
        if (q.gscore > p.gscore || (q.gscore == p.gscore && q.g < p.g)) wv = ww;   // as partial_merge
        partial_merge(p, q);
      }
      a.partials[static_cast<int64_t>(r) * a.partials_ld + wg] = p;
      if constexpr (SIDE) winner[r] = wv;
    }
    if constexpr (SIDE) {
      if (a.gz != nullptr) {
        // each row's best group of the workgroup: the winning wave's copy goes to the side buffer
        __syncthreads();
        for (int i = threadIdx.x; i < Mx * (kGroup / 4); i += kTileThreads) {
          const int m = i / (kGroup / 4), q = i % (kGroup / 4);
          reinterpret_cast<float4*>(a.gz + (static_cast<int64_t>(m) * a.gz_ld + wg) * kGroup)[q] = side_copy(winner[m], m)[q];
        }
      }
    }
  }
};

template <int NCB, int KS, bool ZOUT, int EPI>
__global__ __launch_bounds__(kTileThreads, 1) void k_head_tile(TileArgs a) {
  extern __shared__ uint4 smem[];
  TilePass<NCB, KS, ZOUT, EPI> p(a, smem);
  const int gw = static_cast<int>(blockIdx.x) * kTileWaves + p.w;
  const int nw = static_cast<int>(gridDim.x) * kTileWaves;
  uint4 XA[KS], XB[KS];
  {
    uint4 xv[TilePass<NCB, KS, ZOUT, EPI>::XPER];
    p.stage_issue(xv);
    p.tile_load(gw < p.NG ? gw : p.NG, 0, XA);
    if constexpr (TilePass<NCB, KS, ZOUT, EPI>::DUAL) p.tile_load(gw < p.NG ? gw : p.NG, 1, XB);
    __builtin_amdgcn_sched_barrier(0);
    p.hist_clear();   // (made visible by the staging barrier)
    p.stage_finish(xv);
    __syncthreads();   // the weight slots reuse the staged activations' space
  }
  p.run(gw, nw, XA, XB);
  if constexpr (TilePass<NCB, KS, ZOUT, EPI>::STATS || TilePass<NCB, KS, ZOUT, EPI>::AMAX)
    p.write_partials(static_cast<int>(blockIdx.x));
  p.hist_flush();
}

// ----------------------------------------------------------------------------------------
// Finalize of one row from its producers' Partials: lse, greedy token, or the two-level draw
// recomputing the winning group's logits.
// NT threads of the workgroup take part; zs holds 64 floats, rec NT/64 Partials.
// ----------------------------------------------------------------------------------------
// The Partials of the NT threads merged by the workgroup, the result in every thread.  Each wave
// reduces the fields separately: the largest m by a max butterfly, each lane's s rescaled to it
// once and summed by an add butterfly, the group score and the argmax by compare butterflies (no
// exponential inside a butterfly); the waves' records then merge through LDS.
template <int NT>
__device__ __forceinline__ Partial block_partial_merge(const Partial& a, Partial* rec) {
  const int l = lane_id(), w = wave_id();
  constexpr int nwaves = NT / kWave;
  float mw = a.m;
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) mw = fmaxf(mw, xor_lane(mw, s));
  float sw = a.m == -INFINITY ? 0.f : a.s * __expf(a.m - mw);
  float gs = a.gscore, zm = a.zmax;
  int32_t gi = a.g, zi = a.zid;
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) {
    sw += xor_lane(sw, s);
    argmax_merge(gs, gi, xor_lane(gs, s), xor_lane(gi, s));
    argmax_merge(zm, zi, xor_lane(zm, s), xor_lane(zi, s));
  }
  if (l == 0) {
    Partial p = partial_empty();
    p.m = mw;
    p.s = sw;
    p.gscore = gs;
    p.g = gi;
    p.zmax = zm;
    p.zid = zi;
    rec[w] = p;
  }
  __syncthreads();
  Partial r = rec[0];
#pragma unroll
  for (int i = 1; i < nwaves; ++i) partial_merge(r, rec[i]);
  return r;
}

// Sums over the wave of 16 values per lane, transposed: four exchanges that each halve the
// values a lane holds, then two full ones, leave lane L with the total of value (L >> 2) mod 16
// (17 exchanges instead of 16 x 6).
__device__ __forceinline__ float wave_sum16(const float (&v)[16]) {
  const int l = lane_id();
  float a[8], b[4], c[2];
  const bool h5 = (l & 32) != 0, h4 = (l & 16) != 0, h3 = (l & 8) != 0, h2 = (l & 4) != 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) a[i] = (h5 ? v[i + 8] : v[i]) + xor_lane(h5 ? v[i] : v[i + 8], 32);
#pragma unroll
  for (int i = 0; i < 4; ++i) b[i] = (h4 ? a[i + 4] : a[i]) + xor_lane(h4 ? a[i] : a[i + 4], 16);
#pragma unroll
  for (int i = 0; i < 2; ++i) c[i] = (h3 ? b[i + 2] : b[i]) + xor_lane(h3 ? b[i] : b[i + 2], 8);
  float d = (h2 ? c[1] : c[0]) + xor_lane(h2 ? c[0] : c[1], 4);
  d += xor_lane(d, 2);
  d += xor_lane(d, 1);
  return d;
}

template <bool BF16, int NT>
__device__ __forceinline__ void finalize_row(const FinalizeArgs& f, int m, float* zs, Partial* rec) {
  const int l = lane_id(), w = wave_id();
  constexpr int nthreads = NT, nwaves = NT / kWave;
  Partial acc = partial_empty();
  const Partial* pp = f.partials + static_cast<int64_t>(m) * f.partials_ld;
  for (int p = threadIdx.x; p < f.P; p += nthreads) partial_merge(acc, pp[p]);
  acc = block_partial_merge<NT>(acc, rec);
  const float lse = acc.m + logf(acc.s);

  int32_t tok;
  float ytok;
  if (f.mode == 0) {
    tok = acc.zid;
    ytok = acc.zmax * f.invT;
  } else if (f.gz != nullptr) {
    // the K-chunked pass kept each workgroup's best group: read the winning group's logits
    // from its owner, workgroup p of the P producers owning groups [p NG / P, (p + 1) NG / P)
    if (w != 0) return;   // the element draw is one wave's work (no barrier follows)
    const int64_t NG = (f.V + kGroup - 1) / kGroup;
    const int64_t g = acc.g == 0x7fffffff ? 0 : acc.g;
    // owner of group g: a consecutive range per workgroup (K-chunked pass), or the wave stride
    // of the tile pass (group g on wave g mod 4P, workgroup (g mod 4P) / 4)
    const int64_t p = f.gz_map == 0 ? ((g + 1) * f.P + NG - 1) / NG - 1 : (g % (int64_t{kTileWaves} * f.P)) / kTileWaves;
    const int64_t gbase = g * kGroup;
    const float z = f.gz[(static_cast<int64_t>(m) * f.gz_ld + p) * kGroup + l];
    const float gel = gumbel(philox_uniform(f.seed, f.offset, kDraftElem, static_cast<uint64_t>(m),
                                            static_cast<uint64_t>(gbase + l)));
    const bool valid = gbase + l < f.V;
    const float y = z * f.invT;
    float e = valid ? y + gel : -INFINITY;
    int32_t ei = valid ? l : 0x7fffffff;
    wave_argmax(e, ei);
    const int el = ei == 0x7fffffff ? 0 : ei;
    tok = static_cast<int32_t>(gbase + el);
    ytok = __shfl(y, el);
  } else {
    // recompute the 64 logits of the winning group, 64 / nwaves rows per wave, loads together
    const int rpw = kGroup / nwaves;
    const int C = static_cast<int>(f.K * (BF16 ? 2 : 4) / 16);   // chunks of each row's used prefix
    const int CPL = (C + kWave - 1) / kWave;
    const uint32_t rowbytes = static_cast<uint32_t>((f.ld > 0 ? f.ld : f.K) * (BF16 ? 2 : 4));   // row stride
    const int64_t gbase = static_cast<int64_t>(acc.g == 0x7fffffff ? 0 : acc.g) * kGroup;
    const int64_t r0 = gbase + w * rpw;
    const int nrows = f.V - r0 >= rpw ? rpw : (f.V - r0 > 0 ? static_cast<int>(f.V - r0) : 0);
    const rsrc_t wrs = make_rsrc(static_cast<const char*>(f.W) + static_cast<size_t>(nrows > 0 ? r0 : 0) * rowbytes,
                                 static_cast<uint32_t>(nrows) * rowbytes);
    const rsrc_t xrs = make_rsrc(static_cast<const char*>(f.x) + static_cast<size_t>(m) * rowbytes,
                                 static_cast<uint32_t>(C) * 16);
    // wave 0: the element Gumbel of row gbase + l, computed while the first loads are in flight
    float gel = 0.f;
    bool gel_done = w != 0;
    // RB rows and QB chunks per lane of each row per batch: RB * QB + QB loads issued together
    constexpr int RB = kGroup / (NT / kWave) < 16 ? kGroup / (NT / kWave) : 16;
    constexpr int QB = 16 / RB > 1 ? 16 / RB : 1;
    for (int j0 = 0; j0 < rpw; j0 += RB) {
      float z[RB];
#pragma unroll
      for (int j = 0; j < RB; ++j) z[j] = 0.f;
      for (int q0 = 0; q0 < CPL; q0 += QB) {
        uint4 xv[QB], wv[QB][RB];
#pragma unroll
        for (int qq = 0; qq < QB; ++qq) {
          const int c = (q0 + qq) * kWave + l;
          const bool cok = q0 + qq < CPL && c < C;
          xv[qq] = buffer_load16(xrs, cok ? static_cast<uint32_t>(c) * 16 : kOutOfRange);
#pragma unroll
          for (int j = 0; j < RB; ++j)
            wv[qq][j] = buffer_load16(wrs, cok ? static_cast<uint32_t>(j0 + j) * rowbytes + static_cast<uint32_t>(c) * 16
                                               : kOutOfRange);
        }
        if (!gel_done) {
          gel = gumbel(philox_uniform(f.seed, f.offset, kDraftElem, static_cast<uint64_t>(m),
                                      static_cast<uint64_t>(gbase + l)));
          gel_done = true;
        }
#pragma unroll
        for (int qq = 0; qq < QB; ++qq)
#pragma unroll
          for (int j = 0; j < RB; ++j) z[j] = chunk_dot<BF16>(wv[qq][j], xv[qq], z[j]);
      }
      if constexpr (RB == 16) {
        const float s = wave_sum16(z);
        if ((l & 3) == 0) zs[w * rpw + j0 + (l >> 2)] = s;
      } else {
#pragma unroll
        for (int j = 0; j < RB; ++j) {
          const float s = wave_sum(z[j]);
          if (l == 0) zs[w * rpw + j0 + j] = s;
        }
      }
    }
    __syncthreads();
    if (w != 0) return;   // the element draw is one wave's work
    if (!gel_done)
      gel = gumbel(philox_uniform(f.seed, f.offset, kDraftElem, static_cast<uint64_t>(m), static_cast<uint64_t>(gbase + l)));
    const int64_t row = gbase + l;
    const bool valid = row < f.V;
    const float y = zs[l] * f.invT;
    float e = valid ? y + gel : -INFINITY;
    int32_t ei = valid ? l : 0x7fffffff;
    wave_argmax(e, ei);
    const int el = ei == 0x7fffffff ? 0 : ei;
    tok = static_cast<int32_t>(gbase + el);
    ytok = __shfl(y, el);
  }
  if (threadIdx.x == 0) {
    // a trimmed head reports the vocabulary id of the chosen kept row
    f.token[m] = (f.id_map != nullptr && tok >= 0 && tok < f.V) ? f.id_map[tok] : tok;
    if (f.lse) f.lse[m] = lse;
    if (f.logprob) f.logprob[m] = ytok - lse;
  }
}

constexpr int kHfThreads = 256;

template <bool BF16>
__global__ __launch_bounds__(kHfThreads) void k_head_fin(FinalizeArgs f) {
  __shared__ Partial rec[kHfThreads / kWave];
  __shared__ float zs[kGroup];
  finalize_row<BF16, kHfThreads>(f, static_cast<int>(blockIdx.x), zs, rec);
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
  const int rec = kTileWaves * ncb * 16 * static_cast<int>(sizeof(Partial));
  const int slots = kTileWaves * 16 * (ks * 4 + 1) * 16;
  const int m = stage > rec ? stage : rec;
  return m > slots ? m : slots;
}

template <int NCB, int KS, bool ZOUT, int EPI>
hipError_t run_tile(const TileArgs& a, int grid, hipStream_t st) {
  constexpr int lds = TilePass<NCB, KS, ZOUT, EPI>::kLds;
  hipError_t e = allow_lds_tile(k_head_tile<NCB, KS, ZOUT, EPI>, lds);
  if (e != hipSuccess) return e;
  // the launch stamps the trace events itself: their interval is the kernel's execution
  TraceScope ts("head_tile", st, true);
  hipExtLaunchKernelGGL((k_head_tile<NCB, KS, ZOUT, EPI>), dim3(static_cast<unsigned>(grid)), dim3(kTileThreads), lds,
                        st, ts.start(), ts.stop(), 0, a);
  return hipGetLastError();
}

template <int NCB, int KS>
hipError_t run_tile_mode(const TileArgs& a, int grid, hipStream_t st) {
  const int epi = (a.want_stats ? kEpiStats : 0) | (a.want_argmax ? kEpiArgmax : 0);
  if (a.hist != nullptr) {   // raw scores with their histogram (the SpecVocab scorer)
    if constexpr (NCB == 1) {
      if (a.zout != nullptr && epi == 0 && a.M <= kTileHistRows) return run_tile<1, KS, true, kEpiHist>(a, grid, st);
    }
    return hipErrorInvalidValue;
  }
  if (a.zout != nullptr) {
    switch (epi) {
      case 0: return run_tile<NCB, KS, true, 0>(a, grid, st);
      case kEpiStats: return run_tile<NCB, KS, true, kEpiStats>(a, grid, st);
      case kEpiArgmax: return run_tile<NCB, KS, true, kEpiArgmax>(a, grid, st);
      default: return run_tile<NCB, KS, true, kEpiStats | kEpiArgmax>(a, grid, st);
    }
  }
  if (a.gz != nullptr) {   // sampling with the side copy of each row's best group
    if constexpr (NCB <= kTileSideMaxNcb) {
      if (a.sample != 0 && epi == kEpiStats) return run_tile<NCB, KS, false, kEpiStats | kEpiSide>(a, grid, st);
    }
    return hipErrorInvalidValue;
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

bool head_tile_supported(int64_t M, int64_t K, int64_t V, bool bf16, int64_t ld) {
  if (ld <= 0) ld = K;
  if (!bf16 || M < 1 || M > kTileMaxRows || K < 1 || K * 2 > 1024 || ld < K || ld % 8 != 0) return false;
  if (K % 32 != 0 || tile_ks(K) * 32 != K) return false;   // rows of exactly KS 32-wide k-steps
  if (V < 1 || V * ld * 2 > int64_t{0xFFFFFFF0}) return false;   // 32-bit buffer ranges
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
  int64_t grid = (NG + kTileWaves - 1) / kTileWaves;
  if (grid > di.cus) grid = di.cus;
  if (grid > kTileMaxGrid) grid = kTileMaxGrid;
  return static_cast<int>(grid < 1 ? 1 : grid);
}

hipError_t launch_head_tile(const TileArgs& a, int grid, hipStream_t st) {
  if (!head_tile_supported(a.M, a.K, a.V, true, a.ld)) return hipErrorInvalidValue;
  if (a.gz != nullptr && (a.M > kTileSideMaxRows || a.gz_ld < grid || grid > kTileMaxGrid || a.zout != nullptr))
    return hipErrorInvalidValue;
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
