// Check aid: the sampler's fp32 Gumbel-max keys and noise words for listed
// tokens, from the very device functions the sampler decides with
// (token_words, gumbel_from_word, gumbel_key).  Not a step of the path.
#include "sampler_common.hpp"

namespace ts {
namespace {

__global__ __launch_bounds__(256) void gumbel_keys_kernel(
    const float* __restrict__ logits, const float* __restrict__ row_max,
    const float* __restrict__ temperature, const uint64_t* __restrict__ seeds,
    const int64_t* __restrict__ rows, const int32_t* __restrict__ ids, int n,
    float* __restrict__ keys, uint32_t* __restrict__ words) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const int id = ids[i];
  const uint64_t seed = seeds[i], row = static_cast<uint64_t>(rows[i]);
  if (words) {
    const U32x4 w = token_words(seed, row, static_cast<uint32_t>(id) >> 2);
    words[i] = word_at(w, id & 3);
  }
  if (keys) keys[i] = gumbel_key(logits[i], row_max[i], 1.0f / temperature[i], seed, row, id);
}

}  // namespace

hipError_t launch_gumbel_keys(const float* logits, const float* row_max, const float* temperature,
                              const uint64_t* seeds, const int64_t* rows, const int32_t* ids,
                              int n, float* keys, uint32_t* words, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const unsigned grid = static_cast<unsigned>((n + 255) / 256);
  hipLaunchKernelGGL(gumbel_keys_kernel, dim3(grid), dim3(256), 0, stream, logits, row_max,
                     temperature, seeds, rows, ids, n, keys, words);
  return hipGetLastError();
}

}  // namespace ts
