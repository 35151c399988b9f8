// Drafter LM-head kernels for gfx950.
//
//   k_rowdot        h_r = round(W_down h): the SlimSpec d -> r map (SlimSpec write-up,
//                   section 三) and the SpecVocab d -> d' map (SpecVocab write-up, 2.2.1);
//                   fp32 on VALU, bf16 on MFMA (k_rowdot_tile in one pass for up to 64 rows,
//                   k_rowdot_mfma + k_rowdot_reduce split over K beyond that).
//   k_stream_valu   skinny head product (M <= 8 rows): coalesced 16-byte weight streaming,
//                   one 64-row vocabulary group per wave at a time.
//   k_stream_mfma16 the same contract once the rows make the product dense (M > 8):
//                   v_mfma_f32_16x16x32_bf16, weights HBM -> VGPR, activations in LDS
//                   (staged whole, or in K chunks for large d).
//   k_stream_mfma   32x32x16 variant, faster for 17..64 rows with small d.
//   k_head_finalize per row: argmax from the per-workgroup partials (greedy), or the row
//                   lse and the two-level draw from the per-group log-sum-exps (sampling).
//
// The streaming kernels fold each 64-row group into one log-sum-exp per row, L_g, written
// to the workspace; everything that needs random numbers (the group scores L_g + Gumbel(u_g)
// and the element draw inside the winning group) runs once per row in the finalize kernel.
//
// Loads use buffer descriptors whose byte range makes out-of-range lanes read zero, so no
// load sits behind a branch; the streaming loops keep one batch of loads in flight while
// the previous batch is consumed (ping-pong buffers, no register copies between them).
#include <mutex>

#include "device_common.h"
#include "launch.h"
#include "trace.h"

namespace sh {


// Copy `items` 16-byte words fetch(i) -> lds[i] with BATCH loads in flight per thread.
// fetch(-1) must return a harmless (zero) value.
template <int BATCH, typename F>
__device__ __forceinline__ void stage16(uint4* lds, int items, F fetch) {
  for (int base = threadIdx.x; base < items; base += blockDim.x * BATCH) {
    uint4 v[BATCH];
#pragma unroll
    for (int b = 0; b < BATCH; ++b) {
      const int i = base + b * static_cast<int>(blockDim.x);
      v[b] = fetch(i < items ? i : -1);
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
constexpr int64_t kRowdotVecMaxM = 2;   // bf16 input rows that take the VALU kernel (measured: faster at 1-2, slower at 6)

template <bool BF16>
__global__ __launch_bounds__(256) void k_rowdot(const void* __restrict__ Wd,
                                                const void* __restrict__ x, int R, int C, int M,
                                                void* __restrict__ out, uint32_t* __restrict__ zero,
                                                int64_t zero_words) {
  extern __shared__ uint4 xs[];  // [kRowdotM][C]
  if (zero != nullptr) {
    // side job: clear a scratch block a later kernel of the same call accumulates into
    const int64_t nwg = static_cast<int64_t>(gridDim.x) * gridDim.y;
    const int64_t per = (zero_words + nwg - 1) / nwg;
    const int64_t z0 = (static_cast<int64_t>(blockIdx.y) * gridDim.x + blockIdx.x) * per;
    const int64_t z1 = z0 + per < zero_words ? z0 + per : zero_words;
    for (int64_t i = z0 + threadIdx.x; i < z1; i += blockDim.x) zero[i] = 0u;
  }
  const int m0 = blockIdx.y * kRowdotM;
  const int l = lane_id(), w = wave_id();
  const int j0 = blockIdx.x * kRowdotRows + w * 2;
  const int CPL = (C + kWave - 1) / kWave;
  const uint32_t rowbytes = static_cast<uint32_t>(C) * 16;
  // the two weight rows of this wave (zero past R), issued before the staging below
  const int wrows = j0 + 2 <= R ? 2 : (j0 < R ? 1 : 0);
  const rsrc_t wrs = make_rsrc(static_cast<const char*>(Wd) + static_cast<size_t>(j0 < R ? j0 : 0) * rowbytes,
                               static_cast<uint32_t>(wrows) * rowbytes);
  uint4 wr0[kRowdotMaxCPL], wr1[kRowdotMaxCPL];
#pragma unroll
  for (int q = 0; q < kRowdotMaxCPL; ++q) {
    const int c = q * kWave + l;
    const bool ok = q < CPL && c < C;
    wr0[q] = buffer_load16(wrs, ok ? static_cast<uint32_t>(c) * 16 : kOutOfRange);
    wr1[q] = buffer_load16(wrs, ok ? rowbytes + static_cast<uint32_t>(c) * 16 : kOutOfRange);
  }
  const int mrows = M - m0 < kRowdotM ? M - m0 : kRowdotM;
  const rsrc_t xrs = make_rsrc(static_cast<const char*>(x) + static_cast<size_t>(m0) * rowbytes,
                               static_cast<uint32_t>(mrows) * rowbytes);
  stage16<8>(xs, kRowdotM * C, [&](int i) {
    return buffer_load16(xrs, i >= 0 ? static_cast<uint32_t>(i) * 16 : kOutOfRange);
  });
  __syncthreads();
  for (int mm = 0; mm < mrows; ++mm) {
    const int m = m0 + mm;
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
// k_rowdot_few: bf16 with XM (1 or 2) input rows.  One weight row per wave, four per
// workgroup, so R / 4 workgroups share the read; the input rows are loaded straight into
// registers (no LDS staging), every load of a lane issued before the first dot.
// ----------------------------------------------------------------------------------------
template <int XM, int CPL>
__global__ __launch_bounds__(256) void k_rowdot_few(const void* __restrict__ Wd, const void* __restrict__ x, int R,
                                                   int C, uint16_t* __restrict__ out, uint32_t* __restrict__ zero,
                                                   int64_t zero_words) {
  if (zero != nullptr) {
    // side job: clear a scratch block a later kernel of the same call accumulates into
    const int64_t nwg = gridDim.x;
    const int64_t per = (zero_words + nwg - 1) / nwg;
    const int64_t z0 = static_cast<int64_t>(blockIdx.x) * per;
    const int64_t z1 = z0 + per < zero_words ? z0 + per : zero_words;
    for (int64_t i = z0 + threadIdx.x; i < z1; i += blockDim.x) zero[i] = 0u;
  }
  const int l = lane_id(), w = wave_id();
  const int j = blockIdx.x * 4 + w;
  const uint32_t rowbytes = static_cast<uint32_t>(C) * 16;
  const rsrc_t wrs = make_rsrc(static_cast<const char*>(Wd) + static_cast<size_t>(j < R ? j : 0) * rowbytes,
                               j < R ? rowbytes : 0u);
  const rsrc_t xrs = make_rsrc(x, static_cast<uint32_t>(XM) * rowbytes);
  uint4 wv[CPL], xv[XM][CPL];
#pragma unroll
  for (int q = 0; q < CPL; ++q) {
    const int c = q * kWave + l;
    const uint32_t off = c < C ? static_cast<uint32_t>(c) * 16 : kOutOfRange;
    wv[q] = buffer_load16(wrs, off);
#pragma unroll
    for (int mm = 0; mm < XM; ++mm) xv[mm][q] = buffer_load16(xrs, c < C ? mm * rowbytes + off : kOutOfRange);
  }
#pragma unroll
  for (int mm = 0; mm < XM; ++mm) {
    float a = 0.f;
#pragma unroll
    for (int q = 0; q < CPL; ++q) a = chunk_dot_bf16(wv[q], xv[mm][q], a);
    a = wave_sum(a);
    if (l == 0 && j < R) out[static_cast<size_t>(mm) * R + j] = f32_to_bf16_rne(a);
  }
}

template <int XM>
hipError_t run_rowdot_few(const void* Wd, const void* x, int64_t R, int C, uint16_t* out, uint32_t* zero,
                          int64_t zero_words, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>((R + 3) / 4));
  const int cpl = (C + kWave - 1) / kWave;
#define SH_FEW(N)                                                                                                \
  hipLaunchKernelGGL((k_rowdot_few<XM, N>), grid, dim3(256), 0, st, Wd, x, static_cast<int>(R), C, out, zero, \
                     zero_words)
  if (cpl <= 2) SH_FEW(2);
  else if (cpl <= 4) SH_FEW(4);
  else if (cpl <= 8) SH_FEW(8);
  else SH_FEW(16);
#undef SH_FEW
  return hipGetLastError();
}

// ----------------------------------------------------------------------------------------
// bf16 down-projection on MFMA, split over K:
//   k_rowdot_mfma    grid (ceil(R/32), ksplit, row chunks): workgroup = 4 waves; each wave
//                    multiplies a 32-row tile of Wd by up to 32*NCB input rows over
//                    kRdKSW k-steps of 16 (v_mfma_f32_32x32x16_bf16, fragments straight from
//                    global memory), the 4 waves' tiles are summed in LDS in a fixed order and
//                    written as one fp32 partial [ksplit][M][R].
//   k_rowdot_reduce  sums the ksplit partials of every output in a fixed order and rounds
//                    once to bf16; also clears a scratch block for a later kernel.
// ----------------------------------------------------------------------------------------
constexpr int kRdKSW = 8;                     // k-steps per wave
constexpr int kRdKWG = 4 * kRdKSW;            // k-steps per workgroup

int rowdot_ksplit(int64_t K) { return static_cast<int>(((K + 15) / 16 + kRdKWG - 1) / kRdKWG); }

template <int NCB>
__global__ __launch_bounds__(256) void k_rowdot_mfma(const void* __restrict__ Wd, const void* __restrict__ x,
                                                     int R, int K, int M, float* __restrict__ part) {
  extern __shared__ float red[];   // [4 waves][NCB][16][64]
  const int l = lane_id(), w = wave_id();
  const int n = l & 31, hf = l >> 5;
  const int j0 = blockIdx.x * 32;
  const int m0 = blockIdx.z * 32 * NCB;
  const int ksp = blockIdx.y;
  const uint32_t rowbytes = static_cast<uint32_t>(K) * 2;
  const int jrows = R - j0 < 32 ? R - j0 : 32;
  const int mrows = M - m0 < 32 * NCB ? M - m0 : 32 * NCB;
  const rsrc_t wrs = make_rsrc(static_cast<const char*>(Wd) + static_cast<size_t>(j0) * rowbytes,
                               static_cast<uint32_t>(jrows) * rowbytes);
  const rsrc_t xrs = make_rsrc(static_cast<const char*>(x) + static_cast<size_t>(m0) * rowbytes,
                               static_cast<uint32_t>(mrows) * rowbytes);
  const int ks0 = (ksp * 4 + w) * kRdKSW;
  uint4 A[kRdKSW], B[kRdKSW][NCB];
#pragma unroll
  for (int t = 0; t < kRdKSW; ++t) {
    const int k = (ks0 + t) * 16 + hf * 8;
    const bool kok = k < K;
    A[t] = buffer_load16(wrs, kok ? static_cast<uint32_t>(n) * rowbytes + static_cast<uint32_t>(k) * 2 : kOutOfRange);
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
      B[t][cb] = buffer_load16(xrs, kok ? static_cast<uint32_t>(cb * 32 + n) * rowbytes + static_cast<uint32_t>(k) * 2
                                        : kOutOfRange);
  }
  f32x16_t acc[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[cb][v] = 0.f;
#pragma unroll
  for (int t = 0; t < kRdKSW; ++t)
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
      acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, A[t]),
                                                        __builtin_bit_cast(bf16x8_t, B[t][cb]), acc[cb], 0, 0, 0);
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
    for (int v = 0; v < 16; ++v) red[((w * NCB + cb) * 16 + v) * kWave + l] = acc[cb][v];
  __syncthreads();
  // thread -> (cb, v, lane): sum the 4 waves in order
  for (int e = threadIdx.x; e < NCB * 16 * kWave; e += blockDim.x) {
    const int ll = e & (kWave - 1);
    const int v = (e / kWave) & 15;
    const int cb = e / (16 * kWave);
    float sum = red[e];
#pragma unroll
    for (int ww = 1; ww < 4; ++ww) sum += red[ww * NCB * 16 * kWave + e];
    const int j = j0 + 8 * (v >> 2) + 4 * (ll >> 5) + (v & 3);
    const int m = m0 + cb * 32 + (ll & 31);
    if (j < R && m < M) part[(static_cast<int64_t>(ksp) * M + m) * R + j] = sum;
  }
}

__global__ __launch_bounds__(256) void k_rowdot_reduce(const float* __restrict__ part, int ksplit, int64_t MR,
                                                       uint16_t* __restrict__ out, uint32_t* __restrict__ zero,
                                                       int64_t zero_words) {
  const int64_t o = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (o < MR) {
    float sum = part[o];
    for (int i = 1; i < ksplit; ++i) sum += part[i * MR + o];
    out[o] = f32_to_bf16_rne(sum);
  }
  if (zero != nullptr) {
    const int64_t nwg = gridDim.x;
    const int64_t per = (zero_words + nwg - 1) / nwg;
    const int64_t z0 = static_cast<int64_t>(blockIdx.x) * per;
    const int64_t z1 = z0 + per < zero_words ? z0 + per : zero_words;
    for (int64_t i = z0 + threadIdx.x; i < z1; i += blockDim.x) zero[i] = 0u;
  }
}

// ----------------------------------------------------------------------------------------
// bf16 down-projection for at most kRdTileMaxM input rows, in one kernel:
//   k_rowdot_tile    one workgroup per JR x MR output tile (JR rows of Wd by MR input rows,
//                    8 or 16 of Wd by 8, 16 or 32 of x, chosen per shape so the pass fills the
//                    CUs with the least per-workgroup reading), ceil(R/JR) * ceil(M/MR) of
//                    them: a workgroup of 8 waves owns its tile over the whole of K (a tile
//                    narrower than the 16 x 16 MFMA leaves the rest of the product unused; 32
//                    input rows are two MFMA column blocks sharing each Wd fragment).  Workgroups are
//                    dealt to the 8 XCDs round-robin by index, so the tiles are numbered
//                    Wd-tile-major and each XCD takes one contiguous run of that order: it
//                    reads its eighth of Wd and all input rows once (dealt in row-major
//                    order, every XCD read all of Wd and all input rows whenever the tile
//                    columns were not a multiple of 8).  K is
//                    walked in chunks of 512 elements; every chunk of both matrices is read
//                    with whole 1 KB row segments per wave instruction (full cache lines),
//                    all chunks of a batch of 4 issued up front, and passed through a
//                    double-buffered, XOR-swizzled LDS tile from which the 8 waves read
//                    their v_mfma_f32_16x16x32_bf16 fragments (two 32-wide k-steps each per
//                    chunk).  The waves' accumulators are summed in LDS in a fixed order and
//                    rounded once to bf16.  No split over workgroups, so no second pass and
//                    no scratch; also clears a scratch block for a later kernel.
// ----------------------------------------------------------------------------------------
constexpr int kRdtWaves = 8;
constexpr int kRdtThreads = kRdtWaves * kWave;
constexpr int kRdtChunk = 512;                      // elements of K per chunk
constexpr int kRdtCpr = kRdtChunk * 2 / 16;         // 16-byte pieces per row per chunk (64)
// chunks whose loads are in flight together (measured: 4 against 8, Llama 48 rows 9.4 -> 9.1 us,
// GPT-OSS 12.2 -> 11.8; 2 slower at the Llama shape)
constexpr int kRdtBatch = 4;
constexpr int64_t kRdTileMaxM = 256;
static_assert(kRdTileMaxM >= kRowdotRanksMaxM, "one rank per row of a one-pass launch");
static_assert(kRdtCpr / 4 == 2 * kRdtWaves, "two k-steps per wave per chunk");

typedef float rd_f32x4_t __attribute__((ext_vector_type(4)));

// per-row output counts (position-adaptive rank: row m keeps its first r[m] outputs)
struct RowRanks {
  int32_t r[kRdTileMaxM];
};

template <int JR, int MR>
__global__ __launch_bounds__(kRdtThreads) void k_rowdot_tile(const void* __restrict__ Wd,
                                                             const void* __restrict__ x, int R, int K, int M,
                                                             uint16_t* __restrict__ out,
                                                             uint32_t* __restrict__ zero, int64_t zero_words,
                                                             RowRanks rk) {
  static_assert((JR == 8 || JR == 16) && (MR == 8 || MR == 16 || MR == 32), "tile rows");
  constexpr int PER = (JR + MR) / 8;   // 16-byte pieces per thread per chunk
  constexpr int MB = MR > 16 ? 2 : 1;  // 16-column MFMA blocks of the input rows
  // [buffer][tile row][piece slot], slot = piece ^ (row & 7): rows 0..15 hold Wd, rows 16 + 16 b
  // .. hold block b of x; rows past JR (Wd) or MR (x) are never written: they only feed outputs
  // that are not stored
  __shared__ uint4 tile[2][16 + 16 * MB][kRdtCpr];
  __shared__ float red[kRdtWaves][MB][4][kWave];
  const int nwg = static_cast<int>(gridDim.x);
  if (zero != nullptr) {
    const int64_t per = (zero_words + nwg - 1) / nwg;
    const int64_t z0 = static_cast<int64_t>(blockIdx.x) * per;
    const int64_t z1 = z0 + per < zero_words ? z0 + per : zero_words;
    for (int64_t i = z0 + threadIdx.x; i < z1; i += blockDim.x) zero[i] = 0u;
  }
  const int l = lane_id(), w = wave_id();
  const int tid = static_cast<int>(threadIdx.x);
  // workgroup b runs on XCD b mod 8 as its (b / 8)-th: XCD x owns tiles [start(x), start(x + 1))
  // of the Wd-tile-major order, the first nwg mod 8 XCDs one tile more than the others
  int ot;   // this workgroup's output tile
  {
    const int xcd = static_cast<int>(blockIdx.x) % kXcds, local = static_cast<int>(blockIdx.x) / kXcds;
    const int base = nwg / kXcds, extra = nwg % kXcds;
    ot = (xcd < extra ? xcd * (base + 1) : extra * (base + 1) + (xcd - extra) * base) + local;
  }
  const int mt = (M + MR - 1) / MR;
  const int j0 = (ot / mt) * JR, m0 = (ot % mt) * MR;
  const uint32_t rowbytes = static_cast<uint32_t>(K) * 2;
  const int jrows = R - j0 < JR ? R - j0 : JR;
  const int mrows = M - m0 < MR ? M - m0 : MR;
  const rsrc_t rs[2] = {make_rsrc(static_cast<const char*>(Wd) + static_cast<size_t>(j0) * rowbytes,
                                  static_cast<uint32_t>(jrows) * rowbytes),
                        make_rsrc(static_cast<const char*>(x) + static_cast<size_t>(m0) * rowbytes,
                                  static_cast<uint32_t>(mrows) * rowbytes)};
  const int nc = (K + kRdtChunk - 1) / kRdtChunk;
  // piece i of this thread in a chunk: the chunk's rows are the JR rows of Wd then the MR rows of
  // x, 64 pieces (1 KB) each; piece i * 512 + tid is row 8 i + tid / 64 (one row per wave)
  static_assert(kRdtThreads == 8 * kRdtCpr, "piece layout");
  auto piece = [&](int i, int& mat, int& row, int& pc) {
    const int gr = 8 * i + tid / kRdtCpr;
    mat = gr < JR ? 0 : 1;
    row = gr < JR ? gr : gr - JR;
    pc = tid % kRdtCpr;
  };
  auto slot_row = [&](int mat, int row) { return mat == 0 ? row : 16 + row; };
  auto issue = [&](int c, uint4 (&v)[PER]) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      int mat, row, pc;
      piece(i, mat, row, pc);
      const int k = c * kRdtChunk + pc * 8;
      v[i] = buffer_load16(rs[mat], (c < nc && k < K) ? static_cast<uint32_t>(row) * rowbytes + static_cast<uint32_t>(k) * 2
                                                      : kOutOfRange);
    }
  };
  rd_f32x4_t acc[MB];
#pragma unroll
  for (int b = 0; b < MB; ++b) acc[b] = rd_f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int row = l & 15, q = l >> 4;
  for (int cb = 0; cb < nc; cb += kRdtBatch) {
    uint4 v[kRdtBatch][PER];
#pragma unroll
    for (int c = 0; c < kRdtBatch; ++c) issue(cb + c, v[c]);
#pragma unroll
    for (int c = 0; c < kRdtBatch; ++c) {
      if (cb + c < nc) {   // uniform over the workgroup
        const int buf = c & 1;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
          int mat, rr, pc;
          piece(i, mat, rr, pc);
          tile[buf][slot_row(mat, rr)][pc ^ (rr & 7)] = v[c][i];
        }
        __syncthreads();
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int pc = (2 * w + t) * 4 + q;   // k-step 2w + t of the chunk, lane quarter q
          const uint4 a = tile[buf][row][pc ^ (row & 7)];
#pragma unroll
          for (int b = 0; b < MB; ++b) {
            const uint4 bx = tile[buf][16 + 16 * b + row][pc ^ (row & 7)];
            acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                             __builtin_bit_cast(bf16x8_t, bx), acc[b], 0, 0, 0);
          }
        }
      }
    }
  }
  // lane l holds rows j0 + 4 (l / 16) + v of column m0 + 16 b + l % 16 (block b)
#pragma unroll
  for (int b = 0; b < MB; ++b)
#pragma unroll
    for (int v = 0; v < 4; ++v) red[w][b][v][l] = acc[b][v];
  __syncthreads();
  if (threadIdx.x < MB * 4 * kWave) {
    const int b = threadIdx.x / (4 * kWave), v = (threadIdx.x / kWave) % 4, ll = threadIdx.x % kWave;
    float sum = red[0][b][v][ll];
#pragma unroll
    for (int ww = 1; ww < kRdtWaves; ++ww) sum += red[ww][b][v][ll];
    const int jj = 4 * (ll >> 4) + v, mm = 16 * b + (ll & 15);
    const int j = j0 + jj, m = m0 + mm;
    if (jj < JR && mm < MR && j < R && m < M)
      out[static_cast<int64_t>(m) * R + j] = j < rk.r[m] ? f32_to_bf16_rne(sum) : uint16_t{0};
  }
}

// ----------------------------------------------------------------------------------------
// Workgroup-level combine of per-wave argmax states into one Partial per row.
// ----------------------------------------------------------------------------------------
__device__ __forceinline__ void wg_argmax_store(Partial* rec, float z, int32_t id, bool holds,
                                                int m_of_lane, int M, Partial* partials, int64_t ld) {
  const int w = wave_id(), nw = blockDim.x / kWave;
  if (holds) {
    Partial p = partial_empty();
    p.zmax = z;
    p.zid = id;
    rec[w * M + m_of_lane] = p;
  }
  __syncthreads();
  for (int m = threadIdx.x; m < M; m += blockDim.x) {
    Partial p = rec[m];
    for (int i = 1; i < nw; ++i) argmax_merge(p.zmax, p.zid, rec[i * M + m].zmax, rec[i * M + m].zid);
    partials[static_cast<int64_t>(m) * ld + blockIdx.x] = p;
  }
}

// Halving step of the transposed reduction: lanes with bit s clear end with lo + lo[l ^ s],
// lanes with bit s set with hi + hi[l ^ s].  One permlane swap plus one add for s = 32, 16.
template <int S>
__device__ __forceinline__ float pair_fold(float lo, float hi) {
  if constexpr (S == 32) {
    const u32x2_t r = __builtin_amdgcn_permlane32_swap(__float_as_uint(lo), __float_as_uint(hi), false, false);
    return __uint_as_float(r.x) + __uint_as_float(r.y);
  } else if constexpr (S == 16) {
    const u32x2_t r = __builtin_amdgcn_permlane16_swap(__float_as_uint(lo), __float_as_uint(hi), false, false);
    return __uint_as_float(r.x) + __uint_as_float(r.y);
  } else {
    const float a = lo + xor_lane(lo, S);
    const float b = hi + xor_lane(hi, S);
    return (lane_id() & S) ? b : a;
  }
}

__device__ __forceinline__ float pair_fold_rt(float lo, float hi, int s) {
  switch (s) {
    case 32: return pair_fold<32>(lo, hi);
    case 16: return pair_fold<16>(lo, hi);
    case 8: return pair_fold<8>(lo, hi);
    case 4: return pair_fold<4>(lo, hi);
    case 2: return pair_fold<2>(lo, hi);
    default: return pair_fold<1>(lo, hi);
  }
}

// ----------------------------------------------------------------------------------------
// k_stream_valu: M <= MB <= 8 rows.
//   A row of the weight matrix is C = K*esize/16 chunks of 16 bytes.  LPR lanes share a row
//   (LPR = 64 when C >= 64, else the next power of two >= C), so one load instruction reads
//   RPI = 64/LPR rows.  A row-block is 8 load-instructions deep; its per-lane partial sums
//   acc[8][MB] are reduced with a halving (transposed) butterfly so that afterwards each lane
//   holds one finished row: the row-slot given by its top 3 lane bits inside the segment.
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
  const uint32_t rowbytes = static_cast<uint32_t>(C) * 16;
  {
    const rsrc_t xrs = make_rsrc(a.x, static_cast<uint32_t>(a.M) * rowbytes);
    stage16<4>(xs, MB * C, [&](int i) {
      return buffer_load16(xrs, i >= 0 ? static_cast<uint32_t>(i) * 16 : kOutOfRange);
    });
  }
  __syncthreads();

  const int l = lane_id(), w = wave_id();
  const int lr = l % LPR;
  const int ri = l / LPR;
  const int jslot = lr / DUP;
  const bool leader = (lr % DUP) == 0;
  const int V32 = static_cast<int>(a.V);
  const int NG = (V32 + kGroup - 1) / kGroup;
  const int nwt = static_cast<int>(gridDim.x) * (blockDim.x / kWave);
  const char* Wb = static_cast<const char*>(a.W);
  const float c2 = a.invT * kLog2e;   // exp(y - ym) = exp2((z - zm) * c2)

  uint4 xr[MB];
#pragma unroll
  for (int m = 0; m < MB; ++m) xr[m] = (ONE && lr < C) ? xs[m * C + lr] : zero16();

  float run_z = -INFINITY;     // lane m: running argmax of row m
  int32_t run_i = 0x7fffffff;
  float vals[NRB][MB];         // the lane's finished z of each row-block of the group
  float gz[MB];
  int32_t gi[MB];

  // reduce acc over the row's lanes, then record the finished row
  auto finish_rb = [&](float (&acc)[RB][MB], int g, auto rbc) {
    constexpr int rb = decltype(rbc)::value;
#pragma unroll
    for (int step = 0; step < 3; ++step) {
      const int half = RB >> (step + 1);
      const int s = LPR >> (step + 1);
#pragma unroll
      for (int i = 0; i < half; ++i)
#pragma unroll
        for (int m = 0; m < MB; ++m) acc[i][m] = pair_fold_rt(acc[i][m], acc[i + half][m], s);
    }
#pragma unroll
    for (int s = LPR >> 4; s >= 1; s >>= 1)
#pragma unroll
      for (int m = 0; m < MB; ++m) acc[0][m] += xor_lane(acc[0][m], s);
    const int row = g * kGroup + rb * ROWS_RB + jslot * RPI + ri;
    const bool valid = row < V32;
    if (a.zout != nullptr && leader && valid) {
#pragma unroll
      for (int m = 0; m < MB; ++m)
        if (m < a.M) a.zout[static_cast<int64_t>(m) * a.zout_ld + row] = acc[0][m];
    }
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      const float z = valid ? acc[0][m] : -INFINITY;
      vals[rb][m] = z;
      if (z > gz[m]) {   // rows of a lane increase with rb: strict > keeps the lowest on ties
        gz[m] = z;
        gi[m] = row;
      }
    }
  };

  auto group_end = [&](int g) {
    if (a.lg != nullptr) {
#pragma unroll
      for (int m = 0; m < MB; ++m) {
        float mx = vals[0][m];
#pragma unroll
        for (int rb = 1; rb < NRB; ++rb) mx = fmaxf(mx, vals[rb][m]);
#pragma unroll
        for (int s = DUP; s < kWave; s <<= 1) mx = fmaxf(mx, xor_lane(mx, s));
        float sm = 0.f;
        if (mx != -INFINITY) {
#pragma unroll
          for (int rb = 0; rb < NRB; ++rb) sm += fast_exp2((vals[rb][m] - mx) * c2);
        }
#pragma unroll
        for (int s = DUP; s < kWave; s <<= 1) sm += xor_lane(sm, s);
        if (l == m && m < a.M) a.lg[static_cast<int64_t>(m) * a.lg_ld + g] = mx * a.invT + log2f(sm) * kLn2;
      }
    }
    if (a.want_argmax) {
#pragma unroll
      for (int m = 0; m < MB; ++m) {
#pragma unroll
        for (int s = DUP; s < kWave; s <<= 1) {
          const float z2 = xor_lane(gz[m], s);
          const int32_t i2 = xor_lane(gi[m], s);
          argmax_merge(gz[m], gi[m], z2, i2);
        }
        if (l == m) argmax_merge(run_z, run_i, gz[m], gi[m]);
      }
    }
  };

  auto group_reset = [&]() {
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      gz[m] = -INFINITY;
      gi[m] = 0x7fffffff;
    }
  };

  // descriptor over one group's rows: rows past V read as zero
  auto group_rsrc = [&](int g) {
    const int g0 = g * kGroup;
    const int rows = V32 - g0 < kGroup ? V32 - g0 : kGroup;
    return make_rsrc(Wb + static_cast<size_t>(g0) * rowbytes, static_cast<uint32_t>(rows) * rowbytes);
  };

  const int gw = static_cast<int>(blockIdx.x) * (blockDim.x / kWave) + w;
  if constexpr (ONE) {
    auto load_rb = [&](int g, int rb, uint4 (&wv)[RB]) {
      const rsrc_t rs = group_rsrc(g);
#pragma unroll
      for (int j = 0; j < RB; ++j) {
        const int rin = rb * ROWS_RB + j * RPI + ri;
        wv[j] = buffer_load16(rs, lr < C ? static_cast<uint32_t>(rin) * rowbytes + static_cast<uint32_t>(lr) * 16 : kOutOfRange);
      }
    };
    // Row-blocks are unrolled so that every index is static.  Each step prefetches the next
    // row-block into the other buffer before consuming its own; the prefetch is
    // unconditional (after the wave's last block it re-reads the current, cache-resident
    // block) so the wait before the consumption leaves exactly those loads in flight.
    uint4 bufA[RB], bufB[RB];
    auto consume = [&](uint4 (&use)[RB], int g, int rb_for_row, auto rbc) {
      constexpr int rb = decltype(rbc)::value;
      (void)rb_for_row;
      float acc[RB][MB];
#pragma unroll
      for (int j = 0; j < RB; ++j)
#pragma unroll
        for (int m = 0; m < MB; ++m) acc[j][m] = chunk_dot<BF16>(use[j], xr[m], 0.f);
      finish_rb(acc, g, rbc);
    };
    int g = gw;
    if (g < NG) load_rb(g, 0, bufA);
    while (g < NG) {
      group_reset();
      const int gnext = g + nwt;
      static_for<0, NRB>([&](auto rbc) {
        constexpr int rb = decltype(rbc)::value;
        // one descriptor per prefetch, built from the already-selected group
        const bool more = gnext < NG;
        const int pg = rb + 1 < NRB ? g : (more ? gnext : g);
        const int prb = rb + 1 < NRB ? rb + 1 : (more ? 0 : rb);
        if constexpr (rb % 2 == 0) {
          load_rb(pg, prb, bufB);
          consume(bufA, g, rb, rbc);
        } else {
          load_rb(pg, prb, bufA);
          consume(bufB, g, rb, rbc);
        }
      });
      group_end(g);
      if constexpr (NRB % 2 == 1) {
        // the next group's first block landed in bufB
#pragma unroll
        for (int j = 0; j < RB; ++j) bufA[j] = bufB[j];
      }
      g = gnext;
    }
  } else {
    for (int g = gw; g < NG; g += nwt) {
      group_reset();
      const rsrc_t rs = group_rsrc(g);
      static_for<0, NRB>([&](auto rbc) {
        constexpr int rb = decltype(rbc)::value;
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
            wv[j] = buffer_load16(rs, cok ? static_cast<uint32_t>(rin) * rowbytes + static_cast<uint32_t>(c) * 16 : kOutOfRange);
          }
          uint4 xq[MB];
#pragma unroll
          for (int m = 0; m < MB; ++m) xq[m] = cok ? xs[m * C + c] : zero16();
#pragma unroll
          for (int j = 0; j < RB; ++j)
#pragma unroll
            for (int m = 0; m < MB; ++m) acc[j][m] = chunk_dot<BF16>(wv[j], xq[m], acc[j][m]);
        }
        finish_rb(acc, g, rbc);
      });
      group_end(g);
    }
  }
  if (!a.want_argmax) return;
  __syncthreads();
  wg_argmax_store(reinterpret_cast<Partial*>(xs), run_z, run_i, l < a.M, l, a.M, a.partials, a.partials_ld);
}

// ----------------------------------------------------------------------------------------
// k_stream_mfma16: bf16, M <= 16*NCB rows.  Built on v_mfma_f32_16x16x32_bf16: per 32-wide
// k-step a wave multiplies the four 16-row weight tiles of its 64-row vocabulary group (A,
// straight from HBM: one 16-byte load per lane per tile covers 16 rows x 64 contiguous
// bytes) by NCB 16-row activation tiles (B, pre-swizzled in LDS as [k-step][tile][lane], one
// conflict-free 16-byte read per lane).  Output tile layout: lane l holds column l % 16
// (an activation row m) for the 4 weight rows 4*(l/16) + v of each tile.
//   CHUNKED = false: all K fits in LDS; fragments are staged once, waves walk their groups
//                    independently with the weight loads one batch ahead across groups.
//   CHUNKED = true:  K is staged in chunks of kch k-steps; the workgroup restages per chunk
//                    (uniform trip counts, every wave takes part in every barrier).
// The epilogue folds each group into the row's group log-sum-exp L_g and argmax, as in the
// VALU kernel.
// ----------------------------------------------------------------------------------------
typedef float f32x4_t __attribute__((ext_vector_type(4)));

template <int NCB, bool CHUNKED>
__global__ __launch_bounds__(256, NCB <= 3 ? 3 : 1) void k_stream_mfma16(StreamArgs a, int kch) {
  // k-steps per load batch: 8 loads per lane in flight, 4 when the accumulators are large
  constexpr int kM16KB = NCB <= 8 ? 2 : 1;
  extern __shared__ uint4 bs[];   // [kch][NCB][64] fragments; Partial records at the end
  const int l = lane_id(), w = wave_id();
  const int NW = blockDim.x / kWave;
  const int col = l & 15, qd = l >> 4;
  const int K = static_cast<int>(a.K);
  const int KS = (K + 31) / 32;
  const uint32_t rowbytes = static_cast<uint32_t>(K) * 2;
  const int V32 = static_cast<int>(a.V);
  const int NG = (V32 + kGroup - 1) / kGroup;
  const int nwt = static_cast<int>(gridDim.x) * NW;
  const char* Wb = static_cast<const char*>(a.W);
  const int Mx = a.M;
  const float c2 = a.invT * kLog2e;
  const rsrc_t xrs = make_rsrc(a.x, static_cast<uint32_t>(Mx) * rowbytes);

  float run_z[NCB];
  int32_t run_i[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    run_z[cb] = -INFINITY;
    run_i[cb] = 0x7fffffff;
  }
  f32x4_t acc[4][NCB];

  auto group_rsrc = [&](int g) {
    const int g0 = g * kGroup;
    const int rows = V32 - g0 < kGroup ? V32 - g0 : kGroup;
    return make_rsrc(Wb + static_cast<size_t>(g0) * rowbytes, static_cast<uint32_t>(rows) * rowbytes);
  };
  auto load_batch = [&](const rsrc_t& rs, int ks0, uint4 (&X)[kM16KB][4]) {
#pragma unroll
    for (int j = 0; j < kM16KB; ++j) {
      const int k = (ks0 + j) * 32 + qd * 8;
#pragma unroll
      for (int t = 0; t < 4; ++t)
        X[j][t] = buffer_load16(rs, k < K ? static_cast<uint32_t>(t * 16 + col) * rowbytes + static_cast<uint32_t>(k) * 2
                                          : kOutOfRange);
    }
  };
  // B fragments of k-steps [ks0, ks0 + nks): item (kk, cb, lane) -> bs[(kk * NCB + cb) * 64 + lane]
  auto stage = [&](int ks0, int nks) {
    stage16<8>(bs, nks * NCB * kWave, [&](int it) {
      if (it < 0) return buffer_load16(xrs, kOutOfRange);
      const int kk = it / (NCB * kWave);
      const int cb = (it / kWave) % NCB;
      const int ll = it & (kWave - 1);
      const int m = cb * 16 + (ll & 15);
      const int k = (ks0 + kk) * 32 + (ll >> 4) * 8;
      return buffer_load16(xrs, (m < Mx && k < K) ? static_cast<uint32_t>(m) * rowbytes + static_cast<uint32_t>(k) * 2
                                                  : kOutOfRange);
    });
  };
  auto zero_acc = [&]() {
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) acc[t][cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  };
  // k-steps [ks0, ks0 + kM16KB) of a batch; kk0 = index of ks0 inside the staged chunk
  auto mma_batch = [&](const uint4 (&X)[kM16KB][4], int ks0, int kk0, int ks_end) {
#pragma unroll
    for (int j = 0; j < kM16KB; ++j) {
      if (ks0 + j < ks_end) {
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
          const bf16x8_t bf = __builtin_bit_cast(bf16x8_t, bs[((kk0 + j) * NCB + cb) * kWave + l]);
#pragma unroll
          for (int t = 0; t < 4; ++t)
            acc[t][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, X[j][t]), bf,
                                                                 acc[t][cb], 0, 0, 0);
        }
      }
    }
  };
  auto epilogue = [&](int g) {
    const int gbase = g * kGroup;
    const bool full = gbase + kGroup <= V32;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      const int m = cb * 16 + col;
      float vals[16];
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int v = 0; v < 4; ++v) vals[t * 4 + v] = acc[t][cb][v];
      if (!full) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (gbase + (i >> 2) * 16 + qd * 4 + (i & 3) >= V32) vals[i] = -INFINITY;
      }
      if (a.zout != nullptr && m < Mx) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int row = gbase + (i >> 2) * 16 + qd * 4 + (i & 3);
          if (row < V32) a.zout[static_cast<int64_t>(m) * a.zout_ld + row] = vals[i];
        }
      }
      float zm = vals[0];
#pragma unroll
      for (int i = 1; i < 16; ++i) zm = fmaxf(zm, vals[i]);
      float ss = 0.f;
      if (a.lg != nullptr && zm != -INFINITY) {
        const float off = zm * c2;
#pragma unroll
        for (int i = 0; i < 16; ++i) ss += fast_exp2(fmaf(vals[i], c2, -off));
      }
      int32_t zi = 0x7fffffff;
      if (a.want_argmax) {
        int bi = 15;
#pragma unroll
        for (int i = 15; i >= 0; --i)   // the lane's rows rise with i: keep the lowest
          if (vals[i] == zm) bi = i;
        zi = zm == -INFINITY ? 0x7fffffff : gbase + (bi >> 2) * 16 + qd * 4 + (bi & 3);
      }
      // the four lanes col, col + 16, col + 32, col + 48 hold the group's 64 rows of column m
#pragma unroll
      for (int o = 16; o <= 32; o <<= 1) {
        const float zm2 = xor_lane(zm, o), ss2 = xor_lane(ss, o);
        const float mx = fmaxf(zm, zm2);
        if (a.lg != nullptr)
          ss = mx == -INFINITY ? 0.f : ss * fast_exp2((zm - mx) * c2) + ss2 * fast_exp2((zm2 - mx) * c2);
        if (a.want_argmax) {
          const int32_t zi2 = xor_lane(zi, o);
          argmax_merge(zm, zi, zm2, zi2);
        }
        zm = mx;
      }
      if (m < Mx) {
        if (a.lg != nullptr && qd == 0) a.lg[static_cast<int64_t>(m) * a.lg_ld + g] = zm * a.invT + log2f(ss) * kLn2;
        if (a.want_argmax) argmax_merge(run_z[cb], run_i[cb], zm, zi);
      }
    }
  };

  const int gw = static_cast<int>(blockIdx.x) * NW + w;
  if constexpr (!CHUNKED) {
    const int nb = (KS + kM16KB - 1) / kM16KB;
    uint4 XA[kM16KB][4], XB[kM16KB][4];
    int g = gw, b = 0;
    rsrc_t rs = group_rsrc(g < NG ? g : 0);
    if (g < NG) load_batch(rs, 0, XA);
    stage(0, KS);
    __syncthreads();
    // one step consumes batch b of group g from U while batch b+1 (or the next group's
    // first) lands in F; past the wave's last group the current batch is re-read
    auto step = [&](uint4 (&U)[kM16KB][4], uint4 (&F)[kM16KB][4]) -> bool {
      int g2 = g, b2 = b + 1;
      if (b2 == nb) {
        b2 = 0;
        g2 = g + nwt;
      }
      const rsrc_t rs2 = g2 < NG ? group_rsrc(g2) : rs;
      load_batch(rs2, g2 < NG ? b2 * kM16KB : b * kM16KB, F);
      if (b == 0) zero_acc();
      mma_batch(U, b * kM16KB, b * kM16KB, KS);
      if (b == nb - 1) epilogue(g);
      g = g2;
      b = b2;
      rs = rs2;
      return g < NG;
    };
    if (g < NG) {
      for (;;) {
        if (!step(XA, XB)) break;
        if (!step(XB, XA)) break;
      }
    }
  } else {
    const int iters = (NG + nwt - 1) / nwt;
    for (int it = 0; it < iters; ++it) {
      const int g = gw + it * nwt;
      const bool valid = g < NG;
      const rsrc_t rs = group_rsrc(valid ? g : 0);
      zero_acc();
      for (int c0 = 0; c0 < KS; c0 += kch) {
        const int nks = KS - c0 < kch ? KS - c0 : kch;
        uint4 XA[kM16KB][4], XB[kM16KB][4];
        if (valid) load_batch(rs, c0, XA);
        __syncthreads();   // the previous chunk's fragments are no longer read
        stage(c0, nks);
        __syncthreads();
        if (valid) {
          for (int kk = 0; kk < nks; kk += 2 * kM16KB) {
            load_batch(rs, c0 + kk + kM16KB, XB);
            mma_batch(XA, c0 + kk, kk, c0 + nks);
            load_batch(rs, c0 + kk + 2 * kM16KB, XA);
            mma_batch(XB, c0 + kk + kM16KB, kk + kM16KB, c0 + nks);
          }
        }
      }
      if (valid) epilogue(g);
    }
  }
  if (!a.want_argmax) return;
  __syncthreads();
  Partial* rec = reinterpret_cast<Partial*>(bs);
  if (qd == 0) {
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      const int m = cb * 16 + col;
      if (m < Mx) {
        Partial p = partial_empty();
        p.zmax = run_z[cb];
        p.zid = run_i[cb];
        rec[w * Mx + m] = p;
      }
    }
  }
  __syncthreads();
  for (int m = threadIdx.x; m < Mx; m += blockDim.x) {
    Partial p = rec[m];
    for (int i = 1; i < NW; ++i) argmax_merge(p.zmax, p.zid, rec[i * Mx + m].zmax, rec[i * Mx + m].zid);
    a.partials[static_cast<int64_t>(m) * a.partials_ld + blockIdx.x] = p;
  }
}

// ----------------------------------------------------------------------------------------
// k_stream_mfma: the same contract on v_mfma_f32_32x32x16_bf16 for 17..64 rows (NCB column
// blocks of 32) whose fragments fit in LDS.  Each load reads 32 rows x 32 bytes; the eight
// k-steps of a batch complete every 128-byte line they touch.  The group's two 32-row tiles
// are computed one after the other, with the weight loads one batch ahead across tile and
// group boundaries.
// ----------------------------------------------------------------------------------------
template <int NCB, bool BG>
__global__ __launch_bounds__(256) void k_stream_mfma(StreamArgs a) {
  constexpr int KB = BG ? (NCB >= 5 ? 2 : 4) : 8;
  extern __shared__ uint4 bs[];
  const int l = lane_id(), w = wave_id();
  const int NW = blockDim.x / kWave;
  const int n = l & 31, hf = l >> 5;
  const int K = static_cast<int>(a.K);
  const int KS = (K + 15) / 16;
  const int nb = (KS + KB - 1) / KB;
  const uint32_t rowbytes = static_cast<uint32_t>(K) * 2;
  const int V32 = static_cast<int>(a.V);
  const int NG = (V32 + kGroup - 1) / kGroup;
  const int nwt = static_cast<int>(gridDim.x) * NW;
  const char* Wb = static_cast<const char*>(a.W);
  const int Mx = a.M;
  const float c2 = a.invT * kLog2e;
  const rsrc_t xrs = make_rsrc(a.x, static_cast<uint32_t>(Mx) * rowbytes);

  float run_z[NCB];
  int32_t run_i[NCB];
  float hm[NCB], hs[NCB], hz[NCB];
  int32_t hi[NCB];
  f32x16_t acc[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    run_z[cb] = -INFINITY;
    run_i[cb] = 0x7fffffff;
  }

  auto load_batch = [&](int g, int t, int b, uint4 (&X)[KB], uint4 (&Y)[KB][NCB]) {
    const int g0 = g * kGroup;
    const int rows = V32 - g0 < kGroup ? V32 - g0 : kGroup;
    const rsrc_t rs = make_rsrc(Wb + static_cast<size_t>(g0) * rowbytes, static_cast<uint32_t>(rows) * rowbytes);
    const uint32_t rbase = static_cast<uint32_t>(t * 32 + n) * rowbytes;
#pragma unroll
    for (int j = 0; j < KB; ++j) {
      const int ks = b * KB + j;
      const int k = ks * 16 + hf * 8;
      const bool kok = ks < KS && k < K;
      X[j] = buffer_load16(rs, kok ? rbase + static_cast<uint32_t>(k) * 2 : kOutOfRange);
      if constexpr (BG) {
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
          const int m = cb * 32 + n;
          Y[j][cb] = buffer_load16(xrs, (kok && m < Mx) ? static_cast<uint32_t>(m) * rowbytes + static_cast<uint32_t>(k) * 2
                                                        : kOutOfRange);
        }
      }
    }
  };

  auto epilogue_tile = [&](int g, int t) {
    const int tbase = g * kGroup + t * 32;
    const bool full = tbase + 32 <= V32;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      const int m = cb * 32 + n;
      if (!full) {
#pragma unroll
        for (int v = 0; v < 16; ++v)
          if (tbase + 8 * (v >> 2) + 4 * hf + (v & 3) >= V32) acc[cb][v] = -INFINITY;
      }
      if (a.zout != nullptr && m < a.M) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int row = tbase + 8 * (v >> 2) + 4 * hf + (v & 3);
          if (row < V32) a.zout[static_cast<int64_t>(m) * a.zout_ld + row] = acc[cb][v];
        }
      }
      float zm = acc[cb][0];
#pragma unroll
      for (int v = 1; v < 16; ++v) zm = fmaxf(zm, acc[cb][v]);
      int32_t zi = 0x7fffffff;
      if (a.want_argmax) {
        int bv = 0;
#pragma unroll
        for (int v = 15; v >= 0; --v)
          if (acc[cb][v] == zm) bv = v;
        zi = zm == -INFINITY ? 0x7fffffff : tbase + 8 * (bv >> 2) + 4 * hf + (bv & 3);
      }
      float ss = 0.f;
      if (a.lg != nullptr && zm != -INFINITY) {
        const float off = zm * c2;
#pragma unroll
        for (int v = 0; v < 16; ++v) ss += fast_exp2(fmaf(acc[cb][v], c2, -off));
      }
      const float zm2 = xor_lane(zm, 32), ss2 = xor_lane(ss, 32);
      const int32_t zi2 = xor_lane(zi, 32);
      const float gmx = fmaxf(zm, zm2);
      float gsm = 0.f;
      if (gmx != -INFINITY) gsm = ss * fast_exp2((zm - gmx) * c2) + ss2 * fast_exp2((zm2 - gmx) * c2);
      argmax_merge(zm, zi, zm2, zi2);
      if (t == 0) {
        hm[cb] = gmx;
        hs[cb] = gsm;
        hz[cb] = zm;
        hi[cb] = zi;
        continue;
      }
      const float tm = fmaxf(gmx, hm[cb]);
      float ts = 0.f;
      if (tm != -INFINITY) ts = gsm * fast_exp2((gmx - tm) * c2) + hs[cb] * fast_exp2((hm[cb] - tm) * c2);
      argmax_merge(zm, zi, hz[cb], hi[cb]);
      if (m < a.M) {
        if (a.lg != nullptr && hf == 0) a.lg[static_cast<int64_t>(m) * a.lg_ld + g] = tm * a.invT + log2f(ts) * kLn2;
        if (a.want_argmax) argmax_merge(run_z[cb], run_i[cb], zm, zi);
      }
    }
  };

  int g = static_cast<int>(blockIdx.x) * NW + w;
  int t = 0, b = 0;
  uint4 XA[KB], XB[KB];
  uint4 YA[KB][NCB], YB[KB][NCB];
  if (g < NG) load_batch(g, 0, 0, XA, YA);

  if constexpr (!BG) {
    // fragments of all nb * KB k-steps (zero past K) so every MFMA of a batch is unconditional
    stage16<8>(bs, nb * KB * NCB * kWave, [&](int it) {
      if (it < 0) return buffer_load16(xrs, kOutOfRange);
      const int ks = it / (NCB * kWave);
      const int cb = (it / kWave) % NCB;
      const int ll = it & (kWave - 1);
      const int m = cb * 32 + (ll & 31);
      const int k = ks * 16 + (ll >> 5) * 8;
      return buffer_load16(xrs, (m < Mx && k < K) ? static_cast<uint32_t>(m) * rowbytes + static_cast<uint32_t>(k) * 2
                                                  : kOutOfRange);
    });
    __syncthreads();
  }

  auto step = [&](uint4 (&UX)[KB], uint4 (&UY)[KB][NCB], uint4 (&FX)[KB], uint4 (&FY)[KB][NCB]) -> bool {
    int g2 = g, t2 = t, b2 = b + 1;
    if (b2 == nb) {
      b2 = 0;
      t2 = t + 1;
      if (t2 == 2) {
        t2 = 0;
        g2 = g + nwt;
      }
    }
    // one straight-line load sequence: past the wave's last group the current batch is
    // re-read (cache-resident), so the wait before each MFMA below leaves exactly the
    // prefetched batch in flight
    const bool more = g2 < NG;
    load_batch(more ? g2 : g, more ? t2 : t, more ? b2 : b, FX, FY);
    if (b == 0) {
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[cb][v] = 0.f;
    }
#pragma unroll
    for (int j = 0; j < KB; ++j) {
      const int ks = b * KB + j;   // k-steps past K hold zero fragments on both sides
      const bf16x8_t af = __builtin_bit_cast(bf16x8_t, UX[j]);
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        const uint4 bv = BG ? UY[j][cb] : bs[(ks * NCB + cb) * kWave + l];
        acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, __builtin_bit_cast(bf16x8_t, bv), acc[cb], 0, 0, 0);
      }
    }
    if (b == nb - 1) epilogue_tile(g, t);
    g = g2;
    t = t2;
    b = b2;
    return g < NG;
  };
  if (g < NG) {
    for (;;) {
      if (!step(XA, YA, XB, YB)) break;
      if (!step(XB, YB, XA, YA)) break;
    }
  }
  if (!a.want_argmax) return;
  __syncthreads();
  Partial* rec = reinterpret_cast<Partial*>(bs);
  if (hf == 0) {
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      const int m = cb * 32 + n;
      if (m < a.M) {
        Partial p = partial_empty();
        p.zmax = run_z[cb];
        p.zid = run_i[cb];
        rec[w * a.M + m] = p;
      }
    }
  }
  __syncthreads();
  for (int m = threadIdx.x; m < a.M; m += blockDim.x) {
    Partial p = rec[m];
    for (int i = 1; i < NW; ++i) argmax_merge(p.zmax, p.zid, rec[i * a.M + m].zmax, rec[i * a.M + m].zid);
    a.partials[static_cast<int64_t>(m) * a.partials_ld + blockIdx.x] = p;
  }
}

// ----------------------------------------------------------------------------------------
// k_head_finalize: one workgroup (16 waves) per row.
//   greedy:  token = argmax over the producers' partials; lse (if wanted) over the L_g.
//   sample:  lse over the L_g; group g* = argmax_g L_g + Gumbel(u_g) with one Philox block
//            per four groups; then the 64 logits of g* are recomputed and the element draw
//            argmax_i y_i + Gumbel(u_i) picks the token.
// ----------------------------------------------------------------------------------------
constexpr int kFinThreads = 1024;
constexpr int kFinWaves = kFinThreads / kWave;
constexpr int kFinPerThread = (kMaxPartials + kFinThreads - 1) / kFinThreads;
constexpr int kFinRowsPerWave = kGroup / kFinWaves;   // 4

// (m, s) log-sum-exp pairs and (value, index) argmax pairs of the kFinWaves waves, written to
// LDS by lane 0 of each wave, merged by every wave at once: lane i takes pair i, a butterfly
// over kFinWaves lanes, and lane 0's result (the same in every wave) is returned.
__device__ __forceinline__ void fin_merge_waves(const float* rm, const float* rs, const float* rb,
                                                const int32_t* ri, float& m, float& s, float& b,
                                                int32_t& bi) {
  const int l = lane_id();
  m = -INFINITY;
  s = 0.f;
  b = -INFINITY;
  bi = 0x7fffffff;
  if (l < kFinWaves) {
    m = rm[l];
    s = rs[l];
    b = rb[l];
    bi = ri[l];
  }
#pragma unroll
  for (int o = 1; o < kFinWaves; o <<= 1) {
    const float m2 = xor_lane(m, o), s2 = xor_lane(s, o), b2 = xor_lane(b, o);
    const int32_t i2 = xor_lane(bi, o);
    lse_merge(m, s, m2, s2);
    argmax_merge(b, bi, b2, i2);
  }
  m = __shfl(m, 0);
  s = __shfl(s, 0);
  b = __shfl(b, 0);
  bi = __shfl(bi, 0);
}

template <bool BF16>
__global__ __launch_bounds__(kFinThreads) void k_head_finalize(FinalizeArgs f) {
  __shared__ float redm[kFinWaves], reds[kFinWaves], redb[kFinWaves];
  __shared__ int32_t redi[kFinWaves];
  __shared__ float zs[kGroup];
  const int m = blockIdx.x;
  const int l = lane_id(), w = wave_id();
  const int NG = static_cast<int>((f.V + kGroup - 1) / kGroup);
  const bool want_lse = f.lse != nullptr || f.logprob != nullptr || f.mode == 1;
  const float* lgr = f.lg + static_cast<int64_t>(m) * f.lg_ld;

  // (greedy) this thread's argmax partials, loaded before anything else
  float bv = -INFINITY;
  int32_t bi = 0x7fffffff;
  if (f.mode == 0) {
    const Partial* pp = f.partials + static_cast<int64_t>(m) * f.partials_ld;
#pragma unroll
    for (int i = 0; i < kFinPerThread; ++i) {
      const int idx = threadIdx.x + i * kFinThreads;
      if (idx < f.P) {
        const float2 zz = *reinterpret_cast<const float2*>(&pp[idx].zmax);
        argmax_merge(bv, bi, zz.x, __float_as_int(zz.y));
      }
    }
  }
  // ---- row lse and (sampling) the group scores, four groups per thread per pass
  float lmx = -INFINITY, lsm = 0.f;
  if (want_lse) {
    for (int q = threadIdx.x; q * 4 < NG; q += kFinThreads) {
      const float4 L4 = reinterpret_cast<const float4*>(lgr)[q];   // rows padded to 4 groups
      const float L[4] = {L4.x, q * 4 + 1 < NG ? L4.y : -INFINITY, q * 4 + 2 < NG ? L4.z : -INFINITY,
                          q * 4 + 3 < NG ? L4.w : -INFINITY};
      const float qm = fmaxf(fmaxf(L[0], L[1]), fmaxf(L[2], L[3]));
      float qs = 0.f;
      if (qm != -INFINITY) {
#pragma unroll
        for (int j = 0; j < 4; ++j) qs += __expf(L[j] - qm);
      }
      lse_merge(lmx, lsm, qm, qs);
      if (f.mode == 1) {
        uint64_t words[4];
        philox_block(f.seed, f.offset, kDraftGroup, static_cast<uint64_t>(m), static_cast<uint64_t>(q) * 4, words);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (L[j] != -INFINITY) argmax_merge(bv, bi, L[j] + gumbel(word_to_uniform(words[j])), q * 4 + j);
      }
    }
  }
  // one butterfly per wave, one LDS exchange, one parallel merge of the waves
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) {
    const float m2 = xor_lane(lmx, s), s2 = xor_lane(lsm, s);
    lse_merge(lmx, lsm, m2, s2);
    const float b2 = xor_lane(bv, s);
    const int32_t i2 = xor_lane(bi, s);
    argmax_merge(bv, bi, b2, i2);
  }
  if (l == 0) {
    redm[w] = lmx;
    reds[w] = lsm;
    redb[w] = bv;
    redi[w] = bi;
  }
  __syncthreads();
  fin_merge_waves(redm, reds, redb, redi, lmx, lsm, bv, bi);
  const float lse = lmx + logf(lsm);

  int32_t tok;
  float ytok;
  if (f.mode == 0) {
    tok = bi;
    ytok = bv * f.invT;
  } else {
    const int32_t bg = bi;
    // recompute the 64 logits of the winning group (4 rows per wave, loads issued together)
    const int C = static_cast<int>(f.K * (BF16 ? 2 : 4) / 16);
    const int CPL = (C + kWave - 1) / kWave;
    const uint32_t rowbytes = static_cast<uint32_t>(C) * 16;
    const int64_t gbase = static_cast<int64_t>(bg == 0x7fffffff ? 0 : bg) * kGroup;
    const int64_t r0 = gbase + w * kFinRowsPerWave;
    const int nrows = f.V - r0 >= kFinRowsPerWave ? kFinRowsPerWave : (f.V - r0 > 0 ? static_cast<int>(f.V - r0) : 0);
    const rsrc_t wrs = make_rsrc(static_cast<const char*>(f.W) + static_cast<size_t>(nrows > 0 ? r0 : 0) * rowbytes,
                                 static_cast<uint32_t>(nrows) * rowbytes);
    const rsrc_t xrs = make_rsrc(static_cast<const char*>(f.x) + static_cast<size_t>(m) * rowbytes, rowbytes);
    float z[kFinRowsPerWave];
#pragma unroll
    for (int j = 0; j < kFinRowsPerWave; ++j) z[j] = 0.f;
    for (int q0 = 0; q0 < CPL; q0 += 4) {
      uint4 xv[4], wv[4][kFinRowsPerWave];
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const int c = (q0 + qq) * kWave + l;
        const bool cok = q0 + qq < CPL && c < C;
        xv[qq] = buffer_load16(xrs, cok ? static_cast<uint32_t>(c) * 16 : kOutOfRange);
#pragma unroll
        for (int j = 0; j < kFinRowsPerWave; ++j)
          wv[qq][j] = buffer_load16(wrs, cok ? static_cast<uint32_t>(j) * rowbytes + static_cast<uint32_t>(c) * 16 : kOutOfRange);
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
    // a trimmed head reports the vocabulary id of the chosen kept row
    f.token[m] = (f.id_map != nullptr && tok >= 0 && tok < f.V) ? f.id_map[tok] : tok;
    if (f.lse) f.lse[m] = lse;
    if (f.logprob) f.logprob[m] = ytok - lse;
  }
}

// ----------------------------------------------------------------------------------------
// host launchers
// ----------------------------------------------------------------------------------------
hipError_t device_info(DeviceInfo* out) {
  // per-device attributes, filled once; the mutex makes concurrent first calls from several
  // host threads safe (later calls read the filled entry under the same lock)
  static std::mutex mu;
  static DeviceInfo cache[64];
  static bool have[64] = {false};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const bool cached = dev >= 0 && dev < 64;
  if (cached) {
    std::lock_guard<std::mutex> g(mu);
    if (have[dev]) {
      *out = cache[dev];
      return hipSuccess;
    }
  }
  DeviceInfo di;
  e = hipDeviceGetAttribute(&di.cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  int lds = 0;
  e = hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
  if (e != hipSuccess) return e;
  di.max_lds = lds;
  if (cached) {
    std::lock_guard<std::mutex> g(mu);
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

template <int NCB>
static hipError_t run_rowdot_mfma(const void* Wd, const void* x, int R, int K, int M, float* part, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>((R + 31) / 32), static_cast<unsigned>(rowdot_ksplit(K)),
                  static_cast<unsigned>((M + 32 * NCB - 1) / (32 * NCB)));
  const int lds = 4 * NCB * 16 * kWave * 4;
  hipError_t e = allow_lds(k_rowdot_mfma<NCB>, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_rowdot_mfma<NCB>, grid, dim3(256), lds, st, Wd, x, R, K, M, part);
  return hipGetLastError();
}

// Tile shape of the one-pass down-projection: JR rows of Wd by MR input rows per workgroup.
// Smaller tiles cut what each workgroup reads (the pass is bound by per-CU ingest and latency,
// not by its MFMAs) at the price of more workgroups and re-reads that the L2 serves.
template <int JR, int MR>
hipError_t run_rowdot_tile_shape(const void* Wd, const void* x, int64_t R, int64_t K, int64_t M, uint16_t* out,
                                 uint32_t* zero, int64_t zero_words, const RowRanks& rk, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(((R + JR - 1) / JR) * ((M + MR - 1) / MR)));
  TraceScope ts("rowdot_tile", st);
  hipLaunchKernelGGL((k_rowdot_tile<JR, MR>), grid, dim3(kRdtThreads), 0, st, Wd, x, static_cast<int>(R),
                     static_cast<int>(K), static_cast<int>(M), out, zero, zero_words, rk);
  return hipGetLastError();
}

// The shape with the most workgroups that still fit one per CU (fewer bytes per workgroup on
// ties); when every shape has more, the one with the fewest.  Measured (event-timed pass):
// 48 x 512 rows 10.7 -> 9.5 us with 16 x 8 tiles, 6 x 512 9.9 -> 8.1 and 16 x 256 11.7 -> 8.8
// with 8 x 8; at 192 x 360 the 16 x 32 tiles (138 workgroups) take 12.1 us where the 276
// 16 x 16 tiles, some CUs running two in turn, took 13.6 (and 8 x 8 tiles 15.9).
hipError_t run_rowdot_tile(const void* Wd, const void* x, int64_t R, int64_t K, int64_t M, uint16_t* out,
                           uint32_t* zero, int64_t zero_words, const RowRanks& rk, hipStream_t st) {
  DeviceInfo di;
  if (device_info(&di) != hipSuccess) di.cus = 256;
  static constexpr int kShapes[5][2] = {{8, 8}, {16, 8}, {8, 16}, {16, 16}, {16, 32}};
  int best = -1;
  int64_t best_n = 0;
  for (int i = 0; i < 5; ++i) {
    const int64_t n = ((R + kShapes[i][0] - 1) / kShapes[i][0]) * ((M + kShapes[i][1] - 1) / kShapes[i][1]);
    const bool fits = n <= di.cus;
    const bool better = best < 0 || (fits && (best_n > di.cus || n > best_n)) || (!fits && best_n > di.cus && n < best_n);
    if (better) {
      best = i;
      best_n = n;
    }
  }
  switch (best) {
    case 0: return run_rowdot_tile_shape<8, 8>(Wd, x, R, K, M, out, zero, zero_words, rk, st);
    case 1: return run_rowdot_tile_shape<16, 8>(Wd, x, R, K, M, out, zero, zero_words, rk, st);
    case 2: return run_rowdot_tile_shape<8, 16>(Wd, x, R, K, M, out, zero, zero_words, rk, st);
    case 3: return run_rowdot_tile_shape<16, 16>(Wd, x, R, K, M, out, zero, zero_words, rk, st);
    default: return run_rowdot_tile_shape<16, 32>(Wd, x, R, K, M, out, zero, zero_words, rk, st);
  }
}

size_t rowdot_scratch_bytes(int64_t M, int64_t R, int64_t K) {
  return static_cast<size_t>(rowdot_ksplit(K)) * static_cast<size_t>(M * R) * 4;
}

hipError_t launch_rowdot(const void* Wd, const void* x, int64_t R, int64_t K, int64_t M, bool bf16,
                         void* out, float* scratch, hipStream_t st, uint32_t* zero, int64_t zero_words) {
  if (bf16 && M <= kRowdotVecMaxM && K * 2 <= kRowdotMaxCPL * kWave * 16) {
    // one or two input rows: one weight row per wave on the VALU, four per workgroup (R / 4
    // workgroups instead of R / 16 MFMA tiles that each pull 16 rows), inputs in registers
    const int C = static_cast<int>(K * 2 / 16);
    TraceScope ts("rowdot", st);
    return M == 1 ? run_rowdot_few<1>(Wd, x, R, C, static_cast<uint16_t*>(out), zero, zero_words, st)
                  : run_rowdot_few<2>(Wd, x, R, C, static_cast<uint16_t*>(out), zero, zero_words, st);
  }
  if (bf16 && M <= kRdTileMaxM) {
    RowRanks rk;
    for (int m = 0; m < kRdTileMaxM; ++m) rk.r[m] = static_cast<int32_t>(R);
    return run_rowdot_tile(Wd, x, R, K, M, static_cast<uint16_t*>(out), zero, zero_words, rk, st);
  }
  if (bf16) {
    const int ncb = static_cast<int>((M + 31) / 32) < 6 ? static_cast<int>((M + 31) / 32) : 6;
    hipError_t e;
    {
      TraceScope ts("rowdot", st);
      switch (ncb) {
        case 1: e = run_rowdot_mfma<1>(Wd, x, static_cast<int>(R), static_cast<int>(K), static_cast<int>(M), scratch, st); break;
        case 2: e = run_rowdot_mfma<2>(Wd, x, static_cast<int>(R), static_cast<int>(K), static_cast<int>(M), scratch, st); break;
        case 3: e = run_rowdot_mfma<3>(Wd, x, static_cast<int>(R), static_cast<int>(K), static_cast<int>(M), scratch, st); break;
        case 4: e = run_rowdot_mfma<4>(Wd, x, static_cast<int>(R), static_cast<int>(K), static_cast<int>(M), scratch, st); break;
        case 5: e = run_rowdot_mfma<5>(Wd, x, static_cast<int>(R), static_cast<int>(K), static_cast<int>(M), scratch, st); break;
        default: e = run_rowdot_mfma<6>(Wd, x, static_cast<int>(R), static_cast<int>(K), static_cast<int>(M), scratch, st); break;
      }
    }
    if (e != hipSuccess) return e;
    const int64_t MR = M * R;
    int64_t blocks = (MR + 255) / 256;
    if (blocks < 1) blocks = 1;
    TraceScope ts("rowdot_reduce", st);
    hipLaunchKernelGGL(k_rowdot_reduce, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st, scratch,
                       rowdot_ksplit(K), MR, static_cast<uint16_t*>(out), zero, zero_words);
    return hipGetLastError();
  }
  const int C = static_cast<int>(K * 4 / 16);
  const dim3 grid(static_cast<unsigned>((R + kRowdotRows - 1) / kRowdotRows),
                  static_cast<unsigned>((M + kRowdotM - 1) / kRowdotM));
  const int lds = kRowdotM * C * 16;
  TraceScope ts("rowdot", st);
  hipError_t e = allow_lds(k_rowdot<false>, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_rowdot<false>, grid, dim3(256), lds, st, Wd, x, static_cast<int>(R), C,
                     static_cast<int>(M), out, zero, zero_words);
  return hipGetLastError();
}

hipError_t launch_rowdot_ranked(const void* Wd, const void* x, int64_t R, int64_t K, int64_t M,
                                const int32_t* ranks, void* out, hipStream_t st) {
  if (M < 1 || M > kRdTileMaxM) return hipErrorInvalidValue;
  RowRanks rk;
  for (int m = 0; m < kRdTileMaxM; ++m) rk.r[m] = m < M ? ranks[m] : 0;
  return run_rowdot_tile(Wd, x, R, K, M, static_cast<uint16_t*>(out), nullptr, int64_t{0}, rk, st);
}

template <bool BF16, int MB, int LPR, bool ONE>
static hipError_t run_valu(const StreamArgs& a, int grid, int nw, int lds, hipStream_t st) {
  const int rec = nw * MB * static_cast<int>(sizeof(Partial));
  const int bytes = lds > rec ? lds : rec;
  hipError_t e = allow_lds(k_stream_valu<BF16, MB, LPR, ONE>, bytes);
  if (e != hipSuccess) return e;
  TraceScope ts("stream_valu", st);
  hipLaunchKernelGGL((k_stream_valu<BF16, MB, LPR, ONE>), dim3(grid), dim3(nw * kWave), bytes, st, a);
  return hipGetLastError();
}

template <bool BF16, int MB>
static hipError_t dispatch_lpr(const StreamArgs& a, int lpr, bool one, int grid, int nw, int lds, hipStream_t st) {
  switch (lpr) {
    case 8: return run_valu<BF16, MB, 8, true>(a, grid, nw, lds, st);
    case 16: return run_valu<BF16, MB, 16, true>(a, grid, nw, lds, st);
    case 32: return run_valu<BF16, MB, 32, true>(a, grid, nw, lds, st);
    default:
      return one ? run_valu<BF16, MB, 64, true>(a, grid, nw, lds, st)
                 : run_valu<BF16, MB, 64, false>(a, grid, nw, lds, st);
  }
}

template <bool BF16>
static hipError_t dispatch_mb(const StreamArgs& a, int lpr, bool one, int grid, int nw, int lds, hipStream_t st) {
  if (a.M <= 1) return dispatch_lpr<BF16, 1>(a, lpr, one, grid, nw, lds, st);
  if (a.M <= 2) return dispatch_lpr<BF16, 2>(a, lpr, one, grid, nw, lds, st);
  if (a.M <= 4) return dispatch_lpr<BF16, 4>(a, lpr, one, grid, nw, lds, st);
  if (a.M <= 6) return dispatch_lpr<BF16, 6>(a, lpr, one, grid, nw, lds, st);
  return dispatch_lpr<BF16, 8>(a, lpr, one, grid, nw, lds, st);
}

template <int NCB>
static hipError_t run_mfma(const StreamArgs& a, int grid, hipStream_t st) {
  const int nw = 4;
  const int rec = nw * a.M * static_cast<int>(sizeof(Partial));
  const int KS = static_cast<int>((a.K + 15) / 16);
  constexpr int KB = 8;   // k-steps per load batch of k_stream_mfma<NCB, false>
  const int frag = (KS + KB - 1) / KB * KB * NCB * 1024;
  const int bytes = frag > rec ? frag : rec;
  TraceScope ts("stream_mfma", st);
  hipError_t e = allow_lds(k_stream_mfma<NCB, false>, bytes);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_stream_mfma<NCB, false>), dim3(grid), dim3(nw * kWave), bytes, st, a);
  return hipGetLastError();
}

// Fragments of the whole K are staged once when they take at most kM16Resident bytes (two
// workgroups per CU); larger K is staged in chunks of at most kM16Chunk bytes.
constexpr int kM16Resident = 80 * 1024;
constexpr int kM16Chunk = 64 * 1024;

template <int NCB>
static hipError_t run_mfma16(const StreamArgs& a, int grid, int nw, hipStream_t st) {
  const int KS = static_cast<int>((a.K + 31) / 32);
  const int rec = nw * a.M * static_cast<int>(sizeof(Partial));
  const int per_ks = NCB * kWave * 16;
  const bool chunked = KS * per_ks > kM16Resident;
  int kch = chunked ? kM16Chunk / per_ks : KS;
  if (kch < 1) kch = 1;
  const int frag = kch * per_ks;
  const int bytes = frag > rec ? frag : rec;
  TraceScope ts("stream_mfma", st);
  hipError_t e;
  if (chunked) {
    e = allow_lds(k_stream_mfma16<NCB, true>, bytes);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((k_stream_mfma16<NCB, true>), dim3(grid), dim3(nw * kWave), bytes, st, a, kch);
  } else {
    e = allow_lds(k_stream_mfma16<NCB, false>, bytes);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((k_stream_mfma16<NCB, false>), dim3(grid), dim3(nw * kWave), bytes, st, a, kch);
  }
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
  // few groups (a trimmed vocabulary): fewer waves per workgroup in the VALU and 16x16x32
  // kernels, so the workgroups still cover every CU
  int nw16 = 4;
  if (NG < 4 * static_cast<int64_t>(di.cus)) nw16 = NG < 2 * static_cast<int64_t>(di.cus) ? 1 : 2;
  const int64_t grid16 = (NG + nw16 - 1) / nw16 < kMaxPartials ? (NG + nw16 - 1) / nw16 : kMaxPartials;
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
    *producers = static_cast<int>(grid16);   // the same few-groups rule as below
    return a.bf16 ? dispatch_mb<true>(a, lpr, one, static_cast<int>(grid16), nw16, lds, st)
                  : dispatch_mb<false>(a, lpr, one, static_cast<int>(grid16), nw16, lds, st);
  }
  // Measured on MI355X: for 17..64 rows whose 32x32 fragments fit in LDS the 32x32x16 kernel
  // (32 rows x 32 bytes per load, four loads completing each 128-byte line in one batch) is
  // the faster one; otherwise the 16x16x32 kernel.
  const int KS16 = static_cast<int>((a.K + 15) / 16);
  if (a.M > 16 && a.M <= 64 && static_cast<int64_t>((KS16 + 7) / 8 * 8) * ((a.M + 31) / 32) * 1024 <= di.max_lds)
    return a.M <= 32 ? run_mfma<1>(a, static_cast<int>(grid), st) : run_mfma<2>(a, static_cast<int>(grid), st);
  const int ncb = (a.M + 15) / 16;
  *producers = static_cast<int>(grid16);
  const int g16 = static_cast<int>(grid16);
  switch (ncb) {
    case 1: return run_mfma16<1>(a, g16, nw16, st);
    case 2: return run_mfma16<2>(a, g16, nw16, st);
    case 3: return run_mfma16<3>(a, g16, nw16, st);
    case 4: return run_mfma16<4>(a, g16, nw16, st);
    case 5: return run_mfma16<5>(a, g16, nw16, st);
    case 6: return run_mfma16<6>(a, g16, nw16, st);
    case 7: return run_mfma16<7>(a, g16, nw16, st);
    case 8: return run_mfma16<8>(a, g16, nw16, st);
    case 9: return run_mfma16<9>(a, g16, nw16, st);
    case 10: return run_mfma16<10>(a, g16, nw16, st);
    case 11: return run_mfma16<11>(a, g16, nw16, st);
    case 12: return run_mfma16<12>(a, g16, nw16, st);
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
