// Measurement aid for the roofline figures: the shader clock and the bf16
// MFMA rate the part sustains under a dense matrix-core load.  Not a step of
// the sampling path.
//
// Each wave runs `iters` rounds of four independent v_mfma_f32_32x32x16_bf16
// accumulations (enough independent work to keep the matrix pipe issuing back
// to back), eight waves per workgroup (two per SIMD).  Lane 0 of wave 0 reads
// the shader-clock counter (s_memtime) and the constant 100 MHz real-time
// counter (s_memrealtime) before the first round and after the last.  The
// operands are either a few small values (little bit switching) or random
// bit patterns per lane: on this part the matrix cores' sustained rate
// depends on the data, and random operands (like real weights and
// activations) draw more power.
#include "ts_internal.hpp"

namespace ts {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kProbeThreads = 512;

typedef short s16x8 __attribute__((ext_vector_type(8)));

__global__ __launch_bounds__(kProbeThreads) void mfma_clock_kernel(uint64_t* __restrict__ ticks,
                                                                   int64_t iters, int random) {
  const int tid = threadIdx.x;
  bf16x8 a, b;
  if (random) {
    // xorshift32 per lane; exponent bit 14 cleared so no value is Inf or NaN
    uint32_t h = (blockIdx.x * static_cast<uint32_t>(kProbeThreads) + tid) * 2654435761u + 12345u;
    s16x8 ra, rb;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      h ^= h << 13; h ^= h >> 17; h ^= h << 5;
      ra[i] = static_cast<short>(h & 0xbfffu);
      h ^= h << 13; h ^= h >> 17; h ^= h << 5;
      rb[i] = static_cast<short>(h & 0xbfffu);
    }
    a = __builtin_bit_cast(bf16x8, ra);
    b = __builtin_bit_cast(bf16x8, rb);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a[i] = static_cast<__bf16>(0.001f * static_cast<float>((tid + i) & 7));
      b[i] = static_cast<__bf16>(0.002f * static_cast<float>((tid * 3 + i) & 7));
    }
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  __syncthreads();
  const uint64_t m0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  for (int64_t it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, b, c3, 0, 0, 0);
  }
  const uint64_t m1 = __builtin_amdgcn_s_memtime();
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  if (tid == 0) {
    uint64_t* t = ticks + 4 * static_cast<int64_t>(blockIdx.x);
    t[0] = m0;
    t[1] = m1;
    t[2] = r0;
    // The accumulations stay live: a sum no real input can reach marks the
    // record instead of being dropped.
    t[3] = s == -1.0f ? 0ull : r1;
  }
}

}  // namespace

hipError_t launch_mfma_clock_probe(uint64_t* ticks, int workgroups, int64_t iters, int random,
                                   hipStream_t stream) {
  hipLaunchKernelGGL(mfma_clock_kernel, dim3(static_cast<unsigned>(workgroups)),
                     dim3(kProbeThreads), 0, stream, ticks, iters, random);
  return hipGetLastError();
}

}  // namespace ts
