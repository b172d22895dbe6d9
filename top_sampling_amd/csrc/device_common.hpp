// Device helpers shared by the gfx950 kernels: order-preserving float keys,
// Philox4x32-10, Gumbel noise and deterministic wave/block reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ts {

constexpr int kWave = 64;  // CDNA wavefront width

// ------------------------------------------------------------ float order keys
// Monotone map fp32 -> uint32: a < b (as reals, -0 == +0) iff key(a) < key(b).
// Negative floats have all bits flipped, non-negative ones get the sign bit
// set.  -0 is folded onto +0 first so equal values share one key.  NaNs are
// screened out by the callers before keys are compared.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t b = __float_as_uint(f);
  b = (b == 0x80000000u) ? 0u : b;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ float key_to_float(uint32_t k) {
  uint32_t b = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __uint_as_float(b);
}

// ------------------------------------------------------------- Philox4x32-10
// Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3"
// (SC'11): a 10-round counter-based generator.  Each round takes the 32x32->64
// products of counter words 0 and 2 with two odd multipliers; the new counter
// is (hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0).  The key advances by two Weyl
// increments before every round after the first.
struct U32x4 {
  uint32_t v[4];
};

__device__ __forceinline__ U32x4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2,
                                               uint32_t c3, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r > 0) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint64_t p0 = static_cast<uint64_t>(0xD2511F53u) * c0;
    const uint64_t p1 = static_cast<uint64_t>(0xCD9E8D57u) * c2;
    const uint32_t n0 = static_cast<uint32_t>(p1 >> 32) ^ c1 ^ k0;
    const uint32_t n2 = static_cast<uint32_t>(p0 >> 32) ^ c3 ^ k1;
    c1 = static_cast<uint32_t>(p1);
    c3 = static_cast<uint32_t>(p0);
    c0 = n0;
    c2 = n2;
  }
  U32x4 out;
  out.v[0] = c0;
  out.v[1] = c1;
  out.v[2] = c2;
  out.v[3] = c3;
  return out;
}

// The four words for tokens 4q .. 4q+3 of global row `row`: one Philox call
// with counter (q, row lo, row hi, 0) and key (seed lo, seed hi).
__device__ __forceinline__ U32x4 token_words(uint64_t seed, uint64_t row, uint32_t q) {
  return philox4x32_10(q, static_cast<uint32_t>(row), static_cast<uint32_t>(row >> 32), 0u,
                       static_cast<uint32_t>(seed), static_cast<uint32_t>(seed >> 32));
}

// Word q (0..3, known only at run time) of a Philox block, by selects: an
// indexed read of the four-word array would go through per-lane scratch
// memory, a store and a load in every call.
__device__ __forceinline__ uint32_t word_at(const U32x4& w, int q) {
  const uint32_t lo = (q & 1) ? w.v[1] : w.v[0];
  const uint32_t hi = (q & 1) ? w.v[3] : w.v[2];
  return (q & 2) ? hi : lo;
}

// Standard Gumbel noise from one 32-bit word: u = ((x >> 9) + 1/2) * 2^-23 is
// exact in fp32 and lies in [2^-24, 1 - 2^-24]; g = -ln(-ln u).  Both
// logarithms use the hardware base-2 logarithm (v_log_f32) scaled by ln 2:
// u and -ln u are normal numbers here, and the result's error (a few ulp of
// -ln u, i.e. ~1e-7 relative, so ~1e-6 absolute on g) is far below the
// 1e-4 key gap at which two Gumbel keys count as tied.
constexpr float kLn2 = 0.693147180559945309f;
constexpr float kLog2e = 1.442695040888963407f;

__device__ __forceinline__ float gumbel_from_word(uint32_t x) {
  const float u = (static_cast<float>(x >> 9) + 0.5f) * 1.1920928955078125e-7f;
  const float a = __builtin_amdgcn_logf(u) * -kLn2;  // -ln u > 0
  return __builtin_amdgcn_logf(a) * -kLn2;
}

// A value every lane of the wave holds, moved to a scalar register.
__device__ __forceinline__ float uniform_f32(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, x)));
}

// exp(x) for x <= 0 through the hardware base-2 exponential (v_exp_f32).
__device__ __forceinline__ float fast_exp(float x) {
  return __builtin_amdgcn_exp2f(x * kLog2e);
}

// ------------------------------------------------------------ streaming loads
// Non-temporal loads for data each kernel reads once: the lines are not kept
// in the caches, so a stream does not evict (and write back) other data.  On
// MI355X this doubles the read rate of a one-pass scan.
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float4 load_stream4(const float* p) {
  const f32x4_t t = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p));
  return make_float4(t[0], t[1], t[2], t[3]);
}

__device__ __forceinline__ float load_stream(const float* p) {
  return __builtin_nontemporal_load(p);
}

__device__ __forceinline__ void store_stream4(float* p, const float4& v) {
  const f32x4_t t = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(t, reinterpret_cast<f32x4_t*>(p));
}

// ------------------------------------------------------------ reductions
// Ordering of (key, id) candidates: larger key first, lower id on ties.
__device__ __forceinline__ bool better(float ka, int ia, float kb, int ib) {
  return ka > kb || (ka == kb && ia < ib);
}

__device__ __forceinline__ bool better_u(uint32_t ka, int ia, uint32_t kb, int ib) {
  return ka > kb || (ka == kb && ia < ib);
}

// A DPP move of a 4- or 8-byte value (as one or two 32-bit moves); lanes
// with no source, or outside the row mask, get zero.
template <int CTRL, int ROW_MASK, typename T>
__device__ __forceinline__ T dpp_or_zero(T src) {
  if constexpr (sizeof(T) == 4) {
    return __builtin_bit_cast(
        T, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, src), CTRL, ROW_MASK, 0xF, false));
  } else {
    static_assert(sizeof(T) == 8, "4- or 8-byte values");
    const unsigned long long u = __builtin_bit_cast(unsigned long long, src);
    const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(
        0, static_cast<int>(static_cast<uint32_t>(u)), CTRL, ROW_MASK, 0xF, false));
    const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(
        0, static_cast<int>(static_cast<uint32_t>(u >> 32)), CTRL, ROW_MASK, 0xF, false));
    return __builtin_bit_cast(T, (static_cast<unsigned long long>(hi) << 32) | lo);
  }
}

// Lane 63's value of a 4- or 8-byte value, in scalar registers.
template <typename T>
__device__ __forceinline__ T read_lane63(T v) {
  if constexpr (sizeof(T) == 4) {
    return __builtin_bit_cast(T, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
  } else {
    const unsigned long long u = __builtin_bit_cast(unsigned long long, v);
    const uint32_t lo = __builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(u)), 63);
    const uint32_t hi = __builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(u >> 32)), 63);
    return __builtin_bit_cast(T, (static_cast<unsigned long long>(hi) << 32) | lo);
  }
}

// Sum over the wave, returned to every lane (uniform), by DPP: a butterfly
// within each 16-lane row (quad permutations, then row rotations by 4 and
// 8), then row 1 adds row 0 and row 3 row 2 (broadcast of lane 15), and
// row 3 adds rows 0 + 1 (broadcast of lane 31); lane 63 holds the total.
// Every lane must be active.
template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
  v += dpp_or_zero<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
  v += dpp_or_zero<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
  v += dpp_or_zero<0x124, 0xF>(v);  // row_ror:4
  v += dpp_or_zero<0x128, 0xF>(v);  // row_ror:8
  v += dpp_or_zero<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  v += dpp_or_zero<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
  return read_lane63(v);
}

// One DPP move of a float (ctrl and row_mask are compile-time constants);
// lanes of rows outside row_mask keep `old`.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_f32(float old, float src) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(src),
                                                    CTRL, ROW_MASK, 0xF, false));
}

// Maximum over the wave, returned uniform (in a scalar register), by DPP:
// a butterfly within each 16-lane row, then the rows folded with row
// broadcasts into the last row, read from lane 63.  Every lane must be active.
__device__ __forceinline__ float wave_max_uniform(float v) {
  v = fmaxf(v, dpp_f32<0xB1, 0xF>(v, v));   // quad_perm [1,0,3,2]
  v = fmaxf(v, dpp_f32<0x4E, 0xF>(v, v));   // quad_perm [2,3,0,1]
  v = fmaxf(v, dpp_f32<0x124, 0xF>(v, v));  // row_ror:4
  v = fmaxf(v, dpp_f32<0x128, 0xF>(v, v));  // row_ror:8
  v = fmaxf(v, dpp_f32<0x142, 0xA>(v, v));  // row_bcast:15 into rows 1 and 3
  v = fmaxf(v, dpp_f32<0x143, 0xC>(v, v));  // row_bcast:31 into rows 2 and 3
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// Maximum over the wave (the DPP form above), returned to every lane.
__device__ __forceinline__ float wave_max(float v) { return wave_max_uniform(v); }

// One DPP move of a 64-bit value, as two 32-bit moves (same control).
template <int CTRL, int ROW_MASK, bool BOUND_ZERO>
__device__ __forceinline__ unsigned long long dpp_u64(unsigned long long old,
                                                      unsigned long long src) {
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(
      static_cast<int>(old), static_cast<int>(src), CTRL, ROW_MASK, 0xF, BOUND_ZERO));
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(
      static_cast<int>(old >> 32), static_cast<int>(src >> 32), CTRL, ROW_MASK, 0xF, BOUND_ZERO));
  return (static_cast<unsigned long long>(hi) << 32) | lo;
}

// Maximum of a 64-bit value over the wave, uniform, by DPP (as
// wave_max_uniform).  Every lane must be active.
__device__ __forceinline__ unsigned long long wave_max_u64_uniform(unsigned long long v) {
  unsigned long long t;
  t = dpp_u64<0xB1, 0xF, false>(v, v);   v = t > v ? t : v;  // quad_perm [1,0,3,2]
  t = dpp_u64<0x4E, 0xF, false>(v, v);   v = t > v ? t : v;  // quad_perm [2,3,0,1]
  t = dpp_u64<0x124, 0xF, false>(v, v);  v = t > v ? t : v;  // row_ror:4
  t = dpp_u64<0x128, 0xF, false>(v, v);  v = t > v ? t : v;  // row_ror:8
  t = dpp_u64<0x142, 0xA, false>(v, v);  v = t > v ? t : v;  // row_bcast:15 into rows 1, 3
  t = dpp_u64<0x143, 0xC, false>(v, v);  v = t > v ? t : v;  // row_bcast:31 into rows 2, 3
  const uint32_t lo = __builtin_amdgcn_readlane(static_cast<int>(v), 63);
  const uint32_t hi = __builtin_amdgcn_readlane(static_cast<int>(v >> 32), 63);
  return (static_cast<unsigned long long>(hi) << 32) | lo;
}

// Sum of a 64-bit value over the wave, uniform: the moves of
// wave_max_u64_uniform, with lanes outside a move's row mask adding zero
// (a sum, unlike a maximum, must not take a lane's own value twice).
// Every lane must be active.
__device__ __forceinline__ unsigned long long wave_sum_u64_uniform(unsigned long long v) {
  v += dpp_u64<0xB1, 0xF, false>(0ull, v);   // quad_perm [1,0,3,2]
  v += dpp_u64<0x4E, 0xF, false>(0ull, v);   // quad_perm [2,3,0,1]
  v += dpp_u64<0x124, 0xF, false>(0ull, v);  // row_ror:4
  v += dpp_u64<0x128, 0xF, false>(0ull, v);  // row_ror:8: every lane holds its row's sum
  v += dpp_u64<0x142, 0xA, false>(0ull, v);  // row_bcast:15: rows 1, 3 add rows 0, 2
  v += dpp_u64<0x143, 0xC, false>(0ull, v);  // row_bcast:31: rows 2, 3 add rows 0 + 1
  const uint32_t lo = __builtin_amdgcn_readlane(static_cast<int>(v), 63);
  const uint32_t hi = __builtin_amdgcn_readlane(static_cast<int>(v >> 32), 63);
  return (static_cast<unsigned long long>(hi) << 32) | lo;
}

__device__ __forceinline__ void wave_best(float& k, int& i) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) {
    const float k2 = __shfl_xor(k, o, kWave);
    const int i2 = __shfl_xor(i, o, kWave);
    if (better(k2, i2, k, i)) {
      k = k2;
      i = i2;
    }
  }
}

__device__ __forceinline__ void wave_best_u(uint32_t& k, int& i) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) {
    const uint32_t k2 = __shfl_xor(k, o, kWave);
    const int i2 = __shfl_xor(i, o, kWave);
    if (better_u(k2, i2, k, i)) {
      k = k2;
      i = i2;
    }
  }
}

// Inclusive prefix sum within a wave (lane order), by DPP: shifts right by
// 1, 2, 4 and 8 lanes within each 16-lane row (a lane shifted in from
// outside the row adds zero) give every row its own prefix sums; then row
// 1 adds row 0's total and row 3 row 2's (row broadcast of lane 15), and
// rows 2 and 3 add the first two rows' total (row broadcast of lane 31).
// Six DPP steps instead of six cross-lane shuffles through the LDS
// crossbar.  Every lane must be active.
template <typename T>
__device__ __forceinline__ T wave_inclusive_scan(T v) {
  v += dpp_or_zero<0x111, 0xF>(v);  // row_shr:1
  v += dpp_or_zero<0x112, 0xF>(v);  // row_shr:2
  v += dpp_or_zero<0x114, 0xF>(v);  // row_shr:4
  v += dpp_or_zero<0x118, 0xF>(v);  // row_shr:8
  v += dpp_or_zero<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  v += dpp_or_zero<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
  return v;
}

// Block-wide helpers for a block of NT threads.  `scratch` must hold NT/64
// entries of the value type; every thread of the block must call them.
template <int NT, typename T>
__device__ __forceinline__ T block_sum(T v, T* scratch) {
  constexpr int NW = NT / kWave;
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  v = wave_sum(v);
  __syncthreads();
  if (lane == 0) scratch[w] = v;
  __syncthreads();
  T t = 0;
#pragma unroll
  for (int j = 0; j < NW; ++j) t += scratch[j];  // same order in every thread
  return t;
}

template <int NT>
__device__ __forceinline__ float block_max(float v, float* scratch) {
  constexpr int NW = NT / kWave;
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  v = wave_max(v);
  __syncthreads();
  if (lane == 0) scratch[w] = v;
  __syncthreads();
  float t = scratch[0];
#pragma unroll
  for (int j = 1; j < NW; ++j) t = fmaxf(t, scratch[j]);
  return t;
}

template <int NT>
__device__ __forceinline__ void block_best(float& k, int& i, float* sk, int* si) {
  constexpr int NW = NT / kWave;
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  wave_best(k, i);
  __syncthreads();
  if (lane == 0) {
    sk[w] = k;
    si[w] = i;
  }
  __syncthreads();
  k = sk[0];
  i = si[0];
#pragma unroll
  for (int j = 1; j < NW; ++j)
    if (better(sk[j], si[j], k, i)) {
      k = sk[j];
      i = si[j];
    }
}

template <int NT>
__device__ __forceinline__ void block_best_u(uint32_t& k, int& i, uint32_t* sk, int* si) {
  constexpr int NW = NT / kWave;
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  wave_best_u(k, i);
  __syncthreads();
  if (lane == 0) {
    sk[w] = k;
    si[w] = i;
  }
  __syncthreads();
  k = sk[0];
  i = si[0];
#pragma unroll
  for (int j = 1; j < NW; ++j)
    if (better_u(sk[j], si[j], k, i)) {
      k = sk[j];
      i = si[j];
    }
}

// Bitonic sort of one value per lane across the wave, largest at lane 0
// (compare-exchange through lane shuffles; no LDS, no barrier).
__device__ __forceinline__ float wave_sort_desc(float x) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int k = 2; k <= kWave; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      const float y = __shfl_xor(x, j, kWave);
      const bool desc = (lane & k) == 0;
      const bool lower = (lane & j) == 0;
      x = (desc == lower) ? fmaxf(x, y) : fminf(x, y);
    }
  }
  return x;
}

// Same over four values per lane (256 per wave, element index lane * 4 + i);
// afterwards v[i] of lane l holds rank 4 * l + i.
__device__ __forceinline__ void wave_sort4_desc(float (&v)[4]) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int k = 2; k <= 4 * kWave; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      if (j >= 4) {
        const int lj = j >> 2;
        const bool lower = (lane & lj) == 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int idx = lane * 4 + i;
          const bool desc = (idx & k) == 0;
          const float y = __shfl_xor(v[i], lj, kWave);
          v[i] = (desc == lower) ? fmaxf(v[i], y) : fminf(v[i], y);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (i & j) continue;
          const int idx = lane * 4 + i;
          const bool desc = (idx & k) == 0;
          const float a = v[i], b = v[i + j];
          v[i] = desc ? fmaxf(a, b) : fminf(a, b);
          v[i + j] = desc ? fminf(a, b) : fmaxf(a, b);
        }
      }
    }
  }
}

// Exclusive prefix sum over the block in thread order; returns the block total
// through `total`.
template <int NT, typename T>
__device__ __forceinline__ T block_exclusive_scan(T v, T* scratch, T& total) {
  constexpr int NW = NT / kWave;
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  const T inc = wave_inclusive_scan(v);
  __syncthreads();
  if (lane == kWave - 1) scratch[w] = inc;
  __syncthreads();
  T before = 0, all = 0;
#pragma unroll
  for (int j = 0; j < NW; ++j) {
    before += (j < w) ? scratch[j] : T(0);
    all += scratch[j];
  }
  total = all;
  return before + inc - v;
}

}  // namespace ts
