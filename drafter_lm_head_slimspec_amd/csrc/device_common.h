// Device-side helpers shared by the head, top-k and verification kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace sh {

// f(std::integral_constant<int, I>{}) for I = B .. E-1, fully unrolled
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

constexpr int kWave = 64;
constexpr int kXcds = 8;   // accelerator complex dies: workgroup b of a launch runs on die b mod 8
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// 2^x by the hardware instruction alone (no scaling for denormal results): used for sums of
// exponentials of non-positive arguments, where a result below 2^-126 is negligible.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
constexpr int kGroup = 64;           // sampling group: 64 consecutive candidates
constexpr int kMaxPartials = 2048;   // upper bound on producer workgroups per row

// ---------------------------------------------------------------------------------------
// Per-row partial result of a streaming pass over part of the vocabulary.
//   (m, s):      online log-sum-exp of y = z / T over the rows seen: lse = m + log s
//   (gscore, g): best group score L_g + Gumbel(u_g) and its group id (sampling)
//   (zmax, zid): largest raw logit and its id, lowest id on ties (greedy)
//   xz:          verification rows: the raw logit at the row's draft token when the token
//                lies in this part of the vocabulary, else -inf
// ---------------------------------------------------------------------------------------
struct alignas(16) Partial {
  float m, s, gscore;
  int32_t g;
  float zmax;
  int32_t zid;
  float xz, pad1;
};

__device__ __forceinline__ Partial partial_empty() {
  Partial p;
  p.m = -INFINITY;
  p.s = 0.f;
  p.gscore = -INFINITY;
  p.g = 0x7fffffff;
  p.zmax = -INFINITY;
  p.zid = 0x7fffffff;
  p.xz = -INFINITY;
  p.pad1 = 0.f;
  return p;
}

__device__ __forceinline__ void lse_merge(float& m, float& s, float m2, float s2) {
  // branch-free: both exponentials are NaN only when both maxima are -inf, and then the
  // select discards them
  const float mn = fmaxf(m, m2);
  const float a = __expf(m - mn), b = __expf(m2 - mn);
  s = mn == -INFINITY ? 0.f : s * a + s2 * b;
  m = mn;
}

// larger value wins, lower index on ties
__device__ __forceinline__ void argmax_merge(float& v, int32_t& i, float v2, int32_t i2) {
  if (v2 > v || (v2 == v && i2 < i)) {
    v = v2;
    i = i2;
  }
}

__device__ __forceinline__ void partial_merge(Partial& a, const Partial& b) {
  lse_merge(a.m, a.s, b.m, b.s);
  argmax_merge(a.gscore, a.g, b.gscore, b.g);
  argmax_merge(a.zmax, a.zid, b.zmax, b.zid);
}

// ---------------------------------------------------------------------------------------
// bf16
// ---------------------------------------------------------------------------------------
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t v) {
  return __uint_as_float(static_cast<uint32_t>(v) << 16);
}

// a.lo*b.lo + a.hi*b.hi + acc (bf16 pairs, float accumulate)
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), acc, false);
}

// 16-byte chunk dot products: 8 bf16 or 4 f32 elements
__device__ __forceinline__ float chunk_dot_bf16(const uint4& w, const uint4& x, float acc) {
  acc = dot2_bf16(w.x, x.x, acc);
  acc = dot2_bf16(w.y, x.y, acc);
  acc = dot2_bf16(w.z, x.z, acc);
  acc = dot2_bf16(w.w, x.w, acc);
  return acc;
}
__device__ __forceinline__ float chunk_dot_f32(const uint4& w, const uint4& x, float acc) {
  acc = fmaf(__uint_as_float(w.x), __uint_as_float(x.x), acc);
  acc = fmaf(__uint_as_float(w.y), __uint_as_float(x.y), acc);
  acc = fmaf(__uint_as_float(w.z), __uint_as_float(x.z), acc);
  acc = fmaf(__uint_as_float(w.w), __uint_as_float(x.w), acc);
  return acc;
}
template <bool BF16>
__device__ __forceinline__ float chunk_dot(const uint4& w, const uint4& x, float acc) {
  if constexpr (BF16)
    return chunk_dot_bf16(w, x, acc);
  else
    return chunk_dot_f32(w, x, acc);
}

// float -> bf16 bits, round to nearest even (finite inputs; NaN stays NaN)
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return static_cast<uint16_t>((u >> 16) | 0x40u);
  const uint32_t r = u + 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(r >> 16);
}

// ---------------------------------------------------------------------------------------
// Philox4x64-10 (Salmon, Moraes, Dror, Shaw, SC'11): key (seed, 0),
// counter (index / 4, row, purpose, offset); the draw is word index % 4 mapped to
// ((w >> 41) + 0.5) * 2^-23, exact in float32 and strictly inside (0, 1).
// ---------------------------------------------------------------------------------------
enum Purpose : uint32_t {
  kDraftGroup = 0,
  kDraftElem = 1,
  kAccept = 2,
  kResidGroup = 3,
  kResidElem = 4,
  kBonusGroup = 5,
  kBonusElem = 6
};

__device__ __forceinline__ uint64_t philox_word(uint64_t seed, uint64_t offset, uint32_t purpose,
                                                uint64_t row, uint64_t index) {
  const uint64_t kM0 = 0xD2E7470EE14C6C93ull, kM1 = 0xCA5A826395121157ull;
  const uint64_t kW0 = 0x9E3779B97F4A7C15ull, kW1 = 0xBB67AE8584CAA73Bull;
  uint64_t c0 = index >> 2, c1 = row, c2 = purpose, c3 = offset;
  uint64_t k0 = seed, k1 = 0;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += kW0;
      k1 += kW1;
    }
    const uint64_t hi0 = __umul64hi(kM0, c0), lo0 = kM0 * c0;
    const uint64_t hi1 = __umul64hi(kM1, c2), lo1 = kM1 * c2;
    const uint64_t n0 = hi1 ^ c1 ^ k0;
    const uint64_t n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
  }
  const uint32_t sel = static_cast<uint32_t>(index & 3);
  return sel == 0 ? c0 : sel == 1 ? c1 : sel == 2 ? c2 : c3;
}

// all four words of the block holding `index4` (a multiple of 4)
__device__ __forceinline__ void philox_block(uint64_t seed, uint64_t offset, uint32_t purpose, uint64_t row,
                                             uint64_t index4, uint64_t (&out)[4]) {
  const uint64_t kM0 = 0xD2E7470EE14C6C93ull, kM1 = 0xCA5A826395121157ull;
  const uint64_t kW0 = 0x9E3779B97F4A7C15ull, kW1 = 0xBB67AE8584CAA73Bull;
  uint64_t c0 = index4 >> 2, c1 = row, c2 = purpose, c3 = offset;
  uint64_t k0 = seed, k1 = 0;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += kW0;
      k1 += kW1;
    }
    const uint64_t hi0 = __umul64hi(kM0, c0), lo0 = kM0 * c0;
    const uint64_t hi1 = __umul64hi(kM1, c2), lo1 = kM1 * c2;
    const uint64_t n0 = hi1 ^ c1 ^ k0;
    const uint64_t n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
  }
  out[0] = c0;
  out[1] = c1;
  out[2] = c2;
  out[3] = c3;
}
__device__ __forceinline__ float word_to_uniform(uint64_t w) {
  return (static_cast<float>(static_cast<uint32_t>(w >> 41)) + 0.5f) * 0x1p-23f;
}

__device__ __forceinline__ float philox_uniform(uint64_t seed, uint64_t offset, uint32_t purpose,
                                                uint64_t row, uint64_t index) {
  const uint64_t w = philox_word(seed, offset, purpose, row, index);
  return (static_cast<float>(static_cast<uint32_t>(w >> 41)) + 0.5f) * 0x1p-23f;
}

// standard Gumbel variate from a uniform in (0,1)
__device__ __forceinline__ float gumbel(float u) { return -logf(-logf(u)); }

// ---------------------------------------------------------------------------------------
// wave helpers
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ int lane_id() { return static_cast<int>(threadIdx.x) & (kWave - 1); }
// uniform across the wave; read from one lane so the compiler keeps what derives from it
// (group indices, descriptors, loop bounds) in scalar registers
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
}

// Value of lane (l ^ S) without going through LDS: DPP quad permutes for S = 1, 2, DPP row
// shifts for S = 4, 8, and the gfx950 v_permlane16_swap / v_permlane32_swap for S = 16, 32.
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
template <int S>
__device__ __forceinline__ uint32_t xor_lane_u32(uint32_t v) {
  if constexpr (S == 1) {
    return __builtin_amdgcn_update_dpp(0u, v, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
  } else if constexpr (S == 2) {
    return __builtin_amdgcn_update_dpp(0u, v, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
  } else if constexpr (S == 4 || S == 8) {
    const uint32_t up = __builtin_amdgcn_update_dpp(0u, v, 0x100 + S, 0xF, 0xF, false);  // row_shl
    const uint32_t dn = __builtin_amdgcn_update_dpp(0u, v, 0x110 + S, 0xF, 0xF, false);  // row_shr
    return (lane_id() & S) ? dn : up;
  } else if constexpr (S == 16) {
    const u32x2_t r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return ((lane_id() >> 4) & 1) ? r.x : r.y;
  } else {
    static_assert(S == 32, "xor distance must be a power of two below 64");
    const u32x2_t r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return (lane_id() >> 5) ? r.x : r.y;
  }
}
// runtime distance (folds to one case once loops over s are unrolled)
__device__ __forceinline__ uint32_t xor_lane_u32(uint32_t v, int s) {
  switch (s) {
    case 1: return xor_lane_u32<1>(v);
    case 2: return xor_lane_u32<2>(v);
    case 4: return xor_lane_u32<4>(v);
    case 8: return xor_lane_u32<8>(v);
    case 16: return xor_lane_u32<16>(v);
    default: return xor_lane_u32<32>(v);
  }
}
__device__ __forceinline__ float xor_lane(float v, int s) {
  return __uint_as_float(xor_lane_u32(__float_as_uint(v), s));
}
__device__ __forceinline__ int32_t xor_lane(int32_t v, int s) {
  return static_cast<int32_t>(xor_lane_u32(static_cast<uint32_t>(v), s));
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) v += xor_lane(v, s);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) v = fmaxf(v, xor_lane(v, s));
  return v;
}
// wave-wide argmax, lowest index on ties; every lane gets the result
__device__ __forceinline__ void wave_argmax(float& v, int32_t& i) {
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) {
    const float v2 = xor_lane(v, s);
    const int32_t i2 = xor_lane(i, s);
    argmax_merge(v, i, v2, i2);
  }
}
// merge of Partials across the wave (xor tree); every lane gets the result
__device__ __forceinline__ void wave_partial_merge(Partial& p) {
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
}

// order-preserving map float -> uint32 (larger float -> larger key); -0 is treated as +0
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u << 1) == 0u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
constexpr int kTkBins = 4096;   // top-k histogram: bins of the top 12 key bits
constexpr int kTkShift = 20;    // key >> 20 = top 12 bits

// Buffer loads: a resource descriptor (base, byte range) lets the hardware return zero for
// offsets outside the range, so ragged tails need no branch around the load.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kOutOfRange = 0x80000000u;   // above any range used here
// base and bytes must be the same in every active lane of the wave (all descriptors here are
// per wave, per workgroup or per call).  They are moved to scalar registers explicitly so the
// compiler never wraps a load in a loop over distinct descriptors.
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a >> 32));
  const uint64_t ua = (static_cast<uint64_t>(hi) << 32) | lo;
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(ua), static_cast<short>(0),
                                           static_cast<int>(__builtin_amdgcn_readfirstlane(bytes)),
                                           0x00020000);
}
__device__ __forceinline__ uint4 buffer_load16(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ uint32_t buffer_load4(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}

// Branch-free 16-byte load: reads the clamped (always valid) address and returns zero when
// `ok` is false, so that loads stay unconditional and their waits can be counted exactly.
__device__ __forceinline__ uint4 load16_or_zero(const char* base_valid, const char* p, bool ok) {
  const uint4 v = *reinterpret_cast<const uint4*>(ok ? p : base_valid);
  return ok ? v : make_uint4(0u, 0u, 0u, 0u);
}

// ---------------------------------------------------------------------------------------
// Last-arriver hand-off between the workgroups of one kernel.  Each workgroup writes what
// the last one needs with device-coherent stores (sc1: written through the issuing XCD's L2),
// waits until they are complete, then adds one to a counter with a device-scope atomic; the
// workgroup whose addition completes the count reads everything back with device-coherent
// loads (sc1) and finishes the job.  Nobody waits for anybody, so no spin and no grid-wide
// barrier; the XCD caches never need a whole-cache write-back.  The counter must be zero when
// the kernel starts (an earlier kernel of the call clears it); the last arriver puts it back.
// ---------------------------------------------------------------------------------------
constexpr int kCoherent = 16;   // buffer-instruction cache policy: sc1 (device scope)
__device__ __forceinline__ void coherent_store(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void coherent_store(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void coherent_store(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t coherent_load(const uint32_t* p) {
  return __hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// true in every thread of the workgroup that arrives last of n; *flag is a shared word
__device__ __forceinline__ bool arrive_last(uint32_t* counter, uint32_t n, uint32_t* flag) {
  __builtin_amdgcn_s_waitcnt(0);   // this thread's coherent stores have completed
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t old = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint32_t last = old == n - 1u ? 1u : 0u;
    if (last) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *flag = last;
  }
  __syncthreads();
  return *flag != 0u;
}

__device__ __forceinline__ uint4 load16(const void* p) {
  return *reinterpret_cast<const uint4*>(p);
}
__device__ __forceinline__ uint4 zero16() { return make_uint4(0u, 0u, 0u, 0u); }

}  // namespace sh
