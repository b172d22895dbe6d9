// Host-side interfaces between the C ABI layer (api.hip) and the kernel files.
// Every launcher assumes its arguments were validated by the ABI layer and
// returns the hipError_t of its launches.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/top_sampling.h"
#include "../../include/top_sampling_measure.h"

namespace ts {

// ---------------------------------------------------------------- projection
hipError_t launch_lmhead_gemm(const uint16_t* hidden, int64_t ld_hidden, const uint16_t* lm_head,
                              int64_t ld_lm_head, float* logits, int64_t ld_logits, int rows,
                              int vocab, int hidden_dim, hipStream_t stream);

// FP8 (OCP E4M3) projection with per-row fp32 scales, and the per-row
// quantization of bf16 hidden states into that form.
hipError_t launch_quantize_rows_e4m3(const uint16_t* in, int64_t ld_in, int rows, int cols,
                                     uint8_t* out, int64_t ld_out, float* scales,
                                     hipStream_t stream);
hipError_t launch_lmhead_e4m3(const uint8_t* hidden, const float* hidden_scales, int64_t ld_hidden,
                              const uint8_t* lm_head, const float* lm_head_scales,
                              int64_t ld_lm_head, float* logits, int64_t ld_logits, int rows,
                              int vocab, int hidden_dim, hipStream_t stream);

// ------------------------------------------------------------------- sampler
// The sampler's logits: n column slices side by side, slice s holding global
// columns [off[s], off[s + 1]) of every row at ptr[s] + row * ld[s].  A single
// buffer is the one-slice case.
struct LogitsView {
  const float* ptr[TS_MAX_SLICES];
  int64_t ld[TS_MAX_SLICES];
  int64_t off[TS_MAX_SLICES + 1];
  int n;
};

struct SamplerArgs {
  LogitsView lv;
  int rows;
  int vocab;
  const ts_row_params* params;
  int64_t row_offset;
  int max_logprobs;
  int32_t* token_ids;
  float* token_logprobs;  // may be null
  int32_t* topn_ids;      // may be null iff max_logprobs == 0
  float* topn_logprobs;
  int32_t* row_status;    // may be null
  int flags;              // TS_LOGPROBS_PROCESSED
  // Optional stitched copy of the logits, out[r * asm_ld + global column],
  // written by the chunk pass as it reads them (null: none).  Only set when
  // sampler_takes_chunk_pass() holds for the call.
  float* asm_out;
  int64_t asm_ld;
};

size_t sampler_workspace_size(int64_t rows, const int64_t* slice_cols, int n_slices,
                              int max_logprobs);
hipError_t launch_sampler(const SamplerArgs& a, void* workspace, size_t workspace_bytes,
                          hipStream_t stream);
// Whether launch_sampler runs the chunk pass (which reads every logit once)
// for these shapes; otherwise every row takes the exact per-row kernel.
bool sampler_takes_chunk_pass(int64_t rows, const int64_t* slice_cols, int n_slices);

// ------------------------------------------------------------------ assembly
struct AssembleSlices {
  const float* ptr[TS_MAX_SLICES];
  int64_t cols[TS_MAX_SLICES];
  int64_t ld[TS_MAX_SLICES];
  int64_t col_off[TS_MAX_SLICES];
  int64_t chunk_start[TS_MAX_SLICES + 1];  // prefix of per-slice column chunks
  int n;
  int vec4;  // every pointer, leading dimension and offset allows float4 copies
};

// Floats of one slice row that one assembly workgroup copies (one float4 per
// thread: many small workgroups keep more copies in flight than fewer large
// ones; 1,024 measured 9% faster than 4,096 on the 640 x 4 x 37,984 exchange).
constexpr int64_t kAssembleChunk = 1024;

hipError_t launch_assemble(const AssembleSlices& s, int64_t rows, float* out, int64_t ld_out,
                           hipStream_t stream);

// ------------------------------------------------------------- measurement
hipError_t launch_mfma_clock_probe(uint64_t* ticks, int workgroups, int64_t iters, int random,
                                   hipStream_t stream);
hipError_t launch_gumbel_keys(const float* logits, const float* row_max, const float* temperature,
                              const uint64_t* seeds, const int64_t* rows, const int32_t* ids,
                              int n, float* keys, uint32_t* words, hipStream_t stream);

}  // namespace ts
