// Receive side of the batch-sharded exchange: stitch the vocabulary slices a
// rank receives into full-vocabulary rows for its slice of requests (page
// "Qwen4Exp batch-sharded sampling: inside vLLM PR #61018", section "What
// batch-sharded sampling is, in one paragraph": ranks swap vocabulary slices
// with an all-to-all).
//
// HBM-bound copy: every byte is read once and written once.  One workgroup
// copies one kAssembleChunk-float column chunk of one slice for a stride of
// rows; 16-byte loads and stores when every slice allows them.
#include "device_common.hpp"
#include "ts_internal.hpp"

namespace ts {
namespace {

constexpr int kAsmThreads = 256;
constexpr int kAsmChunk = static_cast<int>(kAssembleChunk);
static_assert(kAsmChunk % (4 * kAsmThreads) == 0, "whole float4s per thread");

__global__ __launch_bounds__(kAsmThreads) void assemble_kernel(AssembleSlices s, int64_t rows,
                                                               float* __restrict__ out,
                                                               int64_t ld_out) {
  // Read the slice table in place (kernarg segment) rather than copying it.
  const AssembleSlices* sp = &s;
  const int64_t cx = blockIdx.x;
  int sl = 0;
  while (sl + 1 < sp->n && cx >= sp->chunk_start[sl + 1]) ++sl;
  const int64_t c0 = (cx - sp->chunk_start[sl]) * kAsmChunk;
  const int64_t cols = sp->cols[sl];
  const int64_t n = (cols - c0 < kAsmChunk) ? (cols - c0) : kAsmChunk;
  const float* base = sp->ptr[sl];
  const int64_t ld = sp->ld[sl];
  const int64_t off = sp->col_off[sl];
  for (int64_t r = blockIdx.y; r < rows; r += gridDim.y) {
    const float* src = base + r * ld + c0;
    float* dst = out + r * ld_out + off + c0;
    if (sp->vec4) {
      const float4* s4 = reinterpret_cast<const float4*>(src);
      float4* d4 = reinterpret_cast<float4*>(dst);
      const int n4 = static_cast<int>(n >> 2);
      float4 v[kAsmChunk / 4 / kAsmThreads];
#pragma unroll
      for (int j = 0; j < kAsmChunk / 4 / kAsmThreads; ++j) {
        const int i = threadIdx.x + j * kAsmThreads;
        v[j] = load_stream4(reinterpret_cast<const float*>(s4 + (i < n4 ? i : 0)));
      }
#pragma unroll
      for (int j = 0; j < kAsmChunk / 4 / kAsmThreads; ++j) {
        const int i = threadIdx.x + j * kAsmThreads;
        if (i < n4) store_stream4(reinterpret_cast<float*>(d4 + i), v[j]);
      }
    } else {
      for (int i = threadIdx.x; i < n; i += kAsmThreads) dst[i] = src[i];
    }
  }
}

}  // namespace

hipError_t launch_assemble(const AssembleSlices& s, int64_t rows, float* out, int64_t ld_out,
                           hipStream_t stream) {
  const int64_t chunks = s.chunk_start[s.n];
  if (rows == 0 || chunks == 0) return hipSuccess;
  const unsigned gy = static_cast<unsigned>(rows < 65535 ? rows : 65535);
  hipLaunchKernelGGL(assemble_kernel, dim3(static_cast<unsigned>(chunks), gy), dim3(kAsmThreads),
                     0, stream, s, rows, out, ld_out);
  return hipGetLastError();
}

}  // namespace ts
