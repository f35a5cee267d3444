// Device helpers shared by the FlashHead kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fh_internal.h"
#include "fh_trace.h"

namespace fh {

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// number formats
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Dot product of one 16-byte chunk with the matching h values.
template <typename T> struct Chunk;
template <> struct Chunk<float> {
  static constexpr int kElems = 4;
  __device__ __forceinline__ static void unpack(const uint4& w, float* out) {
    out[0] = __uint_as_float(w.x); out[1] = __uint_as_float(w.y);
    out[2] = __uint_as_float(w.z); out[3] = __uint_as_float(w.w);
  }
  __device__ __forceinline__ static float dot(const uint4& w, const float* h, float acc) {
    acc = fmaf(__uint_as_float(w.x), h[0], acc);
    acc = fmaf(__uint_as_float(w.y), h[1], acc);
    acc = fmaf(__uint_as_float(w.z), h[2], acc);
    acc = fmaf(__uint_as_float(w.w), h[3], acc);
    return acc;
  }
};
struct bf16_t {};  // storage tag: 16-bit brain float
// h is kept as its raw bf16 pairs (one 32-bit word per pair, bit-cast to
// float storage); each word of a row chunk meets the matching word of h in
// one two-way dot-product instruction: both bf16 x bf16 products are exact
// in fp32 and are added to the fp32 accumulator by the instruction.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float dot2_bf16(uint32_t w, float h, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w),
                                         __builtin_bit_cast(bf16x2_t, h), acc, false);
}
template <> struct Chunk<bf16_t> {
  static constexpr int kElems = 4;
  __device__ __forceinline__ static void unpack(const uint4& w, float* out) {
    out[0] = __uint_as_float(w.x); out[1] = __uint_as_float(w.y);
    out[2] = __uint_as_float(w.z); out[3] = __uint_as_float(w.w);
  }
  __device__ __forceinline__ static float dot(const uint4& w, const float* h, float acc) {
    acc = dot2_bf16(w.x, h[0], acc);
    acc = dot2_bf16(w.y, h[1], acc);
    acc = dot2_bf16(w.z, h[2], acc);
    acc = dot2_bf16(w.w, h[3], acc);
    return acc;
  }
};

// INT4 codes: eight signed 4-bit values per 32-bit word, low nibble first.
__device__ __forceinline__ float int4_at(uint32_t w, int i) {
  return (float)(((int32_t)(w << (28 - 4 * i))) >> 28);
}
// sum_i code_i * h[i] over one word (products of small integers and bf16
// values are exact in fp32)
__device__ __forceinline__ float int4_dot_word(uint32_t w, const float* h) {
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) s = fmaf(int4_at(w, i), h[i], s);
  return s;
}
// one lane's 32 codes of a group against the matching 32 h values
__device__ __forceinline__ float int4_dot_chunk(const uint4& w, const float* h) {
  float part = int4_dot_word(w.x, h);
  part += int4_dot_word(w.y, h + 8);
  part += int4_dot_word(w.z, h + 16);
  part += int4_dot_word(w.w, h + 24);
  return part;
}

// ---------------------------------------------------------------------------
// order-preserving keys.  Larger float -> larger uint32; -0 and +0 collapse.
// The 64-bit decode key puts the ordered value above (0xFFFFFFFF - id), so an
// unsigned max picks the largest value and, among equal values, the lowest
// id.  Zero is below every key of a finite value (the "empty" state).
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t ordered_u32(float f) {
  uint32_t u = __float_as_uint(f == 0.0f ? 0.0f : f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ uint64_t decode_key(float f, uint32_t id) {
  return ((uint64_t)ordered_u32(f) << 32) | (uint64_t)(0xFFFFFFFFu - id);
}
__device__ __forceinline__ uint32_t key_id(uint64_t k) {
  return 0xFFFFFFFFu - (uint32_t)(k & 0xFFFFFFFFull);
}

// ---------------------------------------------------------------------------
// Philox4x32-10 (Salmon et al., SC'11) and the Gumbel transform.
// key = (lo32(seed), hi32(seed)); counter = (idx >> 2, stream, 0, 0);
// the draw for idx is output word idx & 3.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint4 philox4x32_10(uint4 x, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) { k0 += 0x9E3779B9u; k1 += 0xBB67AE85u; }
    const uint32_t lo0 = 0xD2511F53u * x.x, hi0 = __umulhi(0xD2511F53u, x.x);
    const uint32_t lo1 = 0xCD9E8D57u * x.z, hi1 = __umulhi(0xCD9E8D57u, x.z);
    x = make_uint4(hi1 ^ x.y ^ k0, lo1, hi0 ^ x.w ^ k1, lo0);
  }
  return x;
}
__device__ __forceinline__ uint32_t philox_word(uint64_t seed, uint32_t stream, uint32_t idx) {
  const uint4 o = philox4x32_10(make_uint4(idx >> 2, stream, 0u, 0u), (uint32_t)seed,
                                (uint32_t)(seed >> 32));
  const uint32_t w = idx & 3u;
  return w == 0 ? o.x : (w == 1 ? o.y : (w == 2 ? o.z : o.w));
}
// u = (2*(x >> 9) + 1) * 2^-24 lies in (0,1) and is exact in fp32.
__device__ __forceinline__ float gumbel_of_word(uint32_t x) {
  const float u = (float)(2u * (x >> 9) + 1u) * 5.9604644775390625e-08f;
  return -logf(-logf(u));
}
__device__ __forceinline__ float gumbel(uint64_t seed, uint32_t stream, uint32_t idx) {
  return gumbel_of_word(philox_word(seed, stream, idx));
}
// the noise of ids 4 m .. 4 m + 3 from one Philox block (the same values as
// gumbel() for each id)
__device__ __forceinline__ float4 gumbel4(uint64_t seed, uint32_t stream, uint32_t m) {
  const uint4 o = philox4x32_10(make_uint4(m, stream, 0u, 0u), (uint32_t)seed,
                                (uint32_t)(seed >> 32));
  return make_float4(gumbel_of_word(o.x), gumbel_of_word(o.y), gumbel_of_word(o.z),
                     gumbel_of_word(o.w));
}
constexpr uint32_t kStreamCluster = 0;
constexpr uint32_t kStreamToken = 1;

// ---------------------------------------------------------------------------
// wave reductions.  The sums, maxima and log-sum-exp merges run on DPP
// (row_shr 1, 2, 4, 8 inside each 16-lane row, then row_bcast 15 and 31
// across rows), which moves data between lanes inside the vector ALU; the
// result is lane 63's, read into a scalar register, so every lane gets it.
// A butterfly of cross-lane shuffles would take six dependent trips through
// the LDS crossbar instead.  Every lane of the wave must be active; the
// order of the operations is fixed, so the results are reproducible.
// ---------------------------------------------------------------------------
template <typename T, typename Op>
__device__ __forceinline__ T wave_reduce_dpp(T x, T identity, Op op) {
  static_assert(sizeof(T) == 4, "32-bit lanes");
  const int id = __builtin_bit_cast(int, identity);
  T v = x;
#define FH_DPP_STEP(ctrl, rmask)                                                           \
  v = op(v, __builtin_bit_cast(                                                            \
                T, __builtin_amdgcn_update_dpp(id, __builtin_bit_cast(int, v), ctrl, rmask, \
                                               0xf, false)));
  FH_DPP_STEP(0x111, 0xf)  // row_shr:1
  FH_DPP_STEP(0x112, 0xf)  // row_shr:2
  FH_DPP_STEP(0x114, 0xf)  // row_shr:4
  FH_DPP_STEP(0x118, 0xf)  // row_shr:8: lane 15 of each row holds the row's result
  FH_DPP_STEP(0x142, 0xa)  // row_bcast:15 into rows 1 and 3
  FH_DPP_STEP(0x143, 0xc)  // row_bcast:31 into rows 2 and 3: lane 63 holds all
#undef FH_DPP_STEP
  return __builtin_bit_cast(T, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

__device__ __forceinline__ float wave_sum(float x) {
  return wave_reduce_dpp(x, 0.0f, [](float a, float b) { return a + b; });
}
__device__ __forceinline__ float wave_max(float x) {
  return wave_reduce_dpp(x, -INFINITY, [](float a, float b) { return fmaxf(a, b); });
}
__device__ __forceinline__ float wave_min(float x) {
  return wave_reduce_dpp(x, INFINITY, [](float a, float b) { return fminf(a, b); });
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
  return wave_reduce_dpp(x, 0u, [](uint32_t a, uint32_t b) { return a > b ? a : b; });
}
// the largest 64-bit value: the largest high word, then the largest low word
// among the lanes that hold it
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t x) {
  const uint32_t hi = (uint32_t)(x >> 32), lo = (uint32_t)x;
  const uint32_t mh = wave_max_u32(hi);
  const uint32_t ml = wave_max_u32(hi == mh ? lo : 0u);
  return ((uint64_t)mh << 32) | ml;
}
// inclusive prefix sum across the wave (lane order)
__device__ __forceinline__ int wave_incl_scan(int x, int lane) {
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int y = __shfl_up(x, o, kWave);
    if (lane >= o) x += y;
  }
  return x;
}

// ---------------------------------------------------------------------------
// DPP (data-parallel primitives) versions: row_shr steps within 16-lane rows,
// then row_bcast:15 / row_bcast:31 across rows.  No LDS traffic.
// ---------------------------------------------------------------------------
// inclusive prefix sum across the wave (lane order)
__device__ __forceinline__ int wave_incl_scan_dpp(int x) {
  int v = x;
  v += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, x, 0x113, 0xf, 0xf, true);  // row_shr:3
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xe, false);  // row_shr:4, lanes 4..15
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xc, false);  // row_shr:8, lanes 8..15
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15 -> rows 1, 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31 -> rows 2, 3
  return v;
}
// Online log-sum-exp state (max m, scaled sum s = sum exp(x - m)).
struct Lse {
  float m, s;
};
__device__ __forceinline__ Lse lse_empty() { return Lse{-INFINITY, 0.0f}; }
__device__ __forceinline__ Lse lse_add(Lse a, float x) {
  if (x > a.m) { a.s = a.s * __expf(a.m - x) + 1.0f; a.m = x; }
  else a.s += __expf(x - a.m);
  return a;
}
__device__ __forceinline__ Lse lse_merge(Lse a, Lse b) {
  if (b.m == -INFINITY) return a;
  if (a.m == -INFINITY) return b;
  if (a.m >= b.m) return Lse{a.m, a.s + b.s * __expf(b.m - a.m)};
  return Lse{b.m, b.s + a.s * __expf(a.m - b.m)};
}
// (the pairs move by DPP as in wave_reduce_dpp; a disabled source lane
// brings the empty state)
__device__ __forceinline__ Lse wave_lse(Lse a) {
  const int ninf = __float_as_int(-INFINITY);
#define FH_DPP_LSE(ctrl, rmask)                                                               \
  {                                                                                           \
    const Lse b{__int_as_float(__builtin_amdgcn_update_dpp(ninf, __float_as_int(a.m), ctrl, \
                                                           rmask, 0xf, false)),            \
                __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(a.s), ctrl,    \
                                                           rmask, 0xf, false))};           \
    a = lse_merge(a, b);                                                                      \
  }
  FH_DPP_LSE(0x111, 0xf)
  FH_DPP_LSE(0x112, 0xf)
  FH_DPP_LSE(0x114, 0xf)
  FH_DPP_LSE(0x118, 0xf)
  FH_DPP_LSE(0x142, 0xa)
  FH_DPP_LSE(0x143, 0xc)
#undef FH_DPP_LSE
  return Lse{__int_as_float(__builtin_amdgcn_readlane(__float_as_int(a.m), 63)),
             __int_as_float(__builtin_amdgcn_readlane(__float_as_int(a.s), 63))};
}

// ---------------------------------------------------------------------------
// Completion of the other workgroups of a grid without same-address
// serialisation.  A workgroup that has made its results visible device-wide
// (device-scope stores, then s_waitcnt) adds 1 to one of kArriveCounters
// counters, each in its own 128-byte line; one designated workgroup polls
// all of them with a single wave until the expected number of arrivals is
// counted, then clears them for the next launch.  Same-address device
// atomics serialise at the memory side (tens of ns each), so spreading the
// arrivals keeps the wait close to one memory round trip.
// ---------------------------------------------------------------------------
constexpr int kArriveSpinLimit = 1 << 22;  // polls before giving up (seconds)

__device__ __forceinline__ void arrive(uint32_t* ctr, int w) {
  __hip_atomic_fetch_add(ctr + (w % kArriveCounters) * kArriveStride, 1u, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t x) {
  return wave_reduce_dpp(x, 0u, [](uint32_t a, uint32_t b) { return a + b; });
}

// Called by all 64 lanes of one wave.  Returns false if the spin limit was
// reached before `expected` arrivals (the caller reports an error).
__device__ __forceinline__ bool wait_arrivals(uint32_t* ctr, uint32_t expected, int lane) {
  uint32_t* mine = ctr + (lane % kArriveCounters) * kArriveStride;
  bool ok = expected == 0;
  for (int it = 0; !ok && it < kArriveSpinLimit; ++it) {
    const uint32_t v =
        lane < kArriveCounters
            ? __hip_atomic_load(mine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
            : 0u;
    const uint32_t tot = wave_sum_u32(v);
    if (tot >= expected) {
      ok = tot == expected;
      break;
    }
    __builtin_amdgcn_s_sleep(2);
  }
  if (lane < kArriveCounters)
    __hip_atomic_store(mine, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return ok;
}

}  // namespace fh
