// C ABI of the batch-sharded sampling path (declared in include/top_sampling.h).
//
// Every entry point validates its arguments on the host before touching the
// HIP runtime: invalid configurations are rejected up front with a status
// code and a per-thread message, and nothing is enqueued.  Valid calls only
// enqueue kernels on the caller's stream (no allocation, no synchronisation).
#include <stdarg.h>
#include <stdio.h>

#include "ts_internal.hpp"

namespace {

thread_local char g_last_error[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return code;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return TS_OK;
  return fail(TS_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

constexpr int64_t kMaxDim = 0x7fffffff;

}  // namespace

namespace ts {
// A failure recorded for ts_last_error by other source files of the library.
int fail_message(int code, const char* msg) { return fail(code, "%s", msg); }
}  // namespace ts

extern "C" {

const char* ts_status_string(int status) {
  switch (status) {
    case TS_OK: return "TS_OK";
    case TS_EINVAL: return "TS_EINVAL";
    case TS_EUNSUPPORTED: return "TS_EUNSUPPORTED";
    case TS_EWORKSPACE: return "TS_EWORKSPACE";
    case TS_EHIP: return "TS_EHIP";
    default: return "TS_UNKNOWN";
  }
}

const char* ts_last_error(void) { return g_last_error; }

int ts_mfma_clock_probe(uint64_t* ticks, int32_t workgroups, int64_t iters, int32_t operands,
                        void* stream) {
  if (!ticks) return fail(TS_EINVAL, "NULL ticks");
  if (!aligned(ticks, 8)) return fail(TS_EINVAL, "ticks must be 8-byte aligned");
  if (workgroups < 1 || workgroups > 65536)
    return fail(TS_EINVAL, "workgroups=%d outside 1..65536", workgroups);
  if (iters < 1 || iters > (int64_t{1} << 24))
    return fail(TS_EINVAL, "iters=%lld outside 1..2^24", static_cast<long long>(iters));
  if (operands != TS_PROBE_SMALL_OPERANDS && operands != TS_PROBE_RANDOM_OPERANDS)
    return fail(TS_EINVAL, "operands=%d is neither TS_PROBE_SMALL_OPERANDS nor "
                "TS_PROBE_RANDOM_OPERANDS", operands);
  return hip_status(ts::launch_mfma_clock_probe(ticks, workgroups, iters,
                                                operands == TS_PROBE_RANDOM_OPERANDS ? 1 : 0,
                                                static_cast<hipStream_t>(stream)),
                    "ts_mfma_clock_probe");
}

int ts_gumbel_keys(const float* logits, const float* row_max, const float* temperature,
                   const uint64_t* seeds, const int64_t* rows, const int32_t* ids, int64_t n,
                   float* keys, uint32_t* words, void* stream) {
  if (n < 0) return fail(TS_EINVAL, "n < 0");
  if (n > kMaxDim) return fail(TS_EINVAL, "n above 2^31-1");
  if (n == 0) return TS_OK;
  if (!logits || !row_max || !temperature || !seeds || !rows || !ids)
    return fail(TS_EINVAL, "NULL input");
  if (!aligned(logits, 4) || !aligned(row_max, 4) || !aligned(temperature, 4) ||
      !aligned(seeds, 8) || !aligned(rows, 8) || !aligned(ids, 4) || !aligned(keys, 4) ||
      !aligned(words, 4))
    return fail(TS_EINVAL, "misaligned pointer");
  return hip_status(ts::launch_gumbel_keys(logits, row_max, temperature, seeds, rows, ids,
                                           static_cast<int>(n), keys, words,
                                           static_cast<hipStream_t>(stream)),
                    "ts_gumbel_keys launch");
}

int lmhead_logits_local(const void* hidden, int64_t rows, int64_t hidden_dim, int64_t ld_hidden,
                        const void* lm_head, int64_t vocab_local, int64_t ld_lm_head,
                        float* logits, int64_t ld_logits, void* stream) {
  if (rows < 0 || vocab_local < 0 || hidden_dim < 0)
    return fail(TS_EINVAL, "negative size (rows=%lld vocab_local=%lld hidden_dim=%lld)",
                (long long)rows, (long long)vocab_local, (long long)hidden_dim);
  if (rows > kMaxDim || vocab_local > kMaxDim || hidden_dim > kMaxDim)
    return fail(TS_EUNSUPPORTED, "size above 2^31-1");
  if (rows == 0 || vocab_local == 0) return TS_OK;
  if (hidden_dim == 0) return fail(TS_EINVAL, "hidden_dim == 0 with a non-empty output");
  if (!hidden || !lm_head || !logits) return fail(TS_EINVAL, "NULL pointer");
  if (ld_hidden < hidden_dim || ld_lm_head < hidden_dim || ld_logits < vocab_local)
    return fail(TS_EINVAL, "leading dimension below the row width (ld_hidden=%lld ld_lm_head=%lld "
                "ld_logits=%lld)", (long long)ld_hidden, (long long)ld_lm_head,
                (long long)ld_logits);
  if (hidden_dim % 8 || ld_hidden % 8 || ld_lm_head % 8)
    return fail(TS_EUNSUPPORTED, "hidden_dim, ld_hidden and ld_lm_head must be multiples of 8");
  if (!aligned(hidden, 16) || !aligned(lm_head, 16) || !aligned(logits, 4))
    return fail(TS_EUNSUPPORTED, "hidden/lm_head must be 16-byte aligned, logits 4-byte aligned");
  const hipError_t e = ts::launch_lmhead_gemm(
      static_cast<const uint16_t*>(hidden), ld_hidden, static_cast<const uint16_t*>(lm_head),
      ld_lm_head, logits, ld_logits, static_cast<int>(rows), static_cast<int>(vocab_local),
      static_cast<int>(hidden_dim), static_cast<hipStream_t>(stream));
  return hip_status(e, "lmhead_logits_local launch");
}

int quantize_rows_e4m3(const void* in, int64_t rows, int64_t cols, int64_t ld_in, void* out,
                       int64_t ld_out, float* scales, void* stream) {
  if (rows < 0 || cols < 0)
    return fail(TS_EINVAL, "negative size (rows=%lld cols=%lld)", (long long)rows,
                (long long)cols);
  if (rows > kMaxDim || cols > kMaxDim) return fail(TS_EUNSUPPORTED, "size above 2^31-1");
  if (rows == 0) return TS_OK;
  if (!in || !out || !scales) return fail(TS_EINVAL, "NULL pointer");
  if (ld_in < cols || ld_out < cols)
    return fail(TS_EINVAL, "leading dimension below the row width (ld_in=%lld ld_out=%lld)",
                (long long)ld_in, (long long)ld_out);
  if (!aligned(in, 2) || !aligned(scales, 4))
    return fail(TS_EUNSUPPORTED, "input must be 2-byte aligned, scales 4-byte aligned");
  const hipError_t e = ts::launch_quantize_rows_e4m3(
      static_cast<const uint16_t*>(in), ld_in, static_cast<int>(rows), static_cast<int>(cols),
      static_cast<uint8_t*>(out), ld_out, scales, static_cast<hipStream_t>(stream));
  return hip_status(e, "quantize_rows_e4m3 launch");
}

int lmhead_logits_local_e4m3(const void* hidden, const float* hidden_scales, int64_t rows,
                             int64_t hidden_dim, int64_t ld_hidden, const void* lm_head,
                             const float* lm_head_scales, int64_t vocab_local, int64_t ld_lm_head,
                             float* logits, int64_t ld_logits, void* stream) {
  if (rows < 0 || vocab_local < 0 || hidden_dim < 0)
    return fail(TS_EINVAL, "negative size (rows=%lld vocab_local=%lld hidden_dim=%lld)",
                (long long)rows, (long long)vocab_local, (long long)hidden_dim);
  if (rows > kMaxDim || vocab_local > kMaxDim || hidden_dim > kMaxDim)
    return fail(TS_EUNSUPPORTED, "size above 2^31-1");
  if (rows == 0 || vocab_local == 0) return TS_OK;
  if (hidden_dim == 0) return fail(TS_EINVAL, "hidden_dim == 0 with a non-empty output");
  if (!hidden || !lm_head || !logits || !hidden_scales || !lm_head_scales)
    return fail(TS_EINVAL, "NULL pointer");
  if (ld_hidden < hidden_dim || ld_lm_head < hidden_dim || ld_logits < vocab_local)
    return fail(TS_EINVAL, "leading dimension below the row width (ld_hidden=%lld ld_lm_head=%lld "
                "ld_logits=%lld)", (long long)ld_hidden, (long long)ld_lm_head,
                (long long)ld_logits);
  if (hidden_dim % 128 || ld_hidden % 16 || ld_lm_head % 16)
    return fail(TS_EUNSUPPORTED,
                "hidden_dim must be a multiple of 128, ld_hidden and ld_lm_head of 16");
  if (!aligned(hidden, 16) || !aligned(lm_head, 16) || !aligned(logits, 4) ||
      !aligned(hidden_scales, 4) || !aligned(lm_head_scales, 4))
    return fail(TS_EUNSUPPORTED,
                "codes must be 16-byte aligned, logits and scales 4-byte aligned");
  const hipError_t e = ts::launch_lmhead_e4m3(
      static_cast<const uint8_t*>(hidden), hidden_scales, ld_hidden,
      static_cast<const uint8_t*>(lm_head), lm_head_scales, ld_lm_head, logits, ld_logits,
      static_cast<int>(rows), static_cast<int>(vocab_local), static_cast<int>(hidden_dim),
      static_cast<hipStream_t>(stream));
  return hip_status(e, "lmhead_logits_local_e4m3 launch");
}

size_t sampler_workspace_bytes(int64_t rows, int64_t vocab, int32_t max_logprobs) {
  if (rows < 0 || vocab < 0 || max_logprobs < 0) return 0;
  return ts::sampler_workspace_size(rows, &vocab, 1, max_logprobs);
}

size_t sampler_workspace_bytes_slices(int64_t rows, const int64_t* slice_cols, int32_t n_slices,
                                      int32_t max_logprobs) {
  if (rows < 0 || max_logprobs < 0 || n_slices < 1 || n_slices > TS_MAX_SLICES || !slice_cols)
    return 0;
  for (int i = 0; i < n_slices; ++i)
    if (slice_cols[i] < 0) return 0;
  return ts::sampler_workspace_size(rows, slice_cols, n_slices, max_logprobs);
}

namespace {

// Validates everything but the logits, fills `a` and launches.
// With `stitch` (an assembly the caller validated), the call also writes the
// stitched batch buffer: inside the sampler's chunk pass when the call takes
// it, else by the assembly kernel ahead of the sampler.  Either way nothing
// is enqueued unless every argument is valid.
static int sample_common(ts::SamplerArgs& a, const int64_t* cols, int64_t rows, int64_t vocab,
                         const ts_row_params* params, int64_t row_offset, int32_t max_logprobs,
                         int32_t* token_ids, float* token_logprobs, int32_t* topn_ids,
                         float* topn_logprobs, int32_t* row_status, void* workspace,
                         size_t workspace_bytes, void* stream,
                         const ts::AssembleSlices* stitch = nullptr, float* stitch_out = nullptr,
                         int64_t stitch_ld = 0) {
  if (max_logprobs < 0) return fail(TS_EINVAL, "max_logprobs < 0");
  if (max_logprobs > TS_MAX_LOGPROBS)
    return fail(TS_EUNSUPPORTED, "max_logprobs %d above %d", max_logprobs, TS_MAX_LOGPROBS);
  if (row_offset < 0) return fail(TS_EINVAL, "row_offset < 0");
  if (rows > kMaxDim || vocab > kMaxDim) return fail(TS_EUNSUPPORTED, "size above 2^31-1");
  if (rows == 0) return TS_OK;
  if (vocab == 0) return fail(TS_EINVAL, "vocab == 0 with rows > 0");
  if (!params || !token_ids) return fail(TS_EINVAL, "NULL params/token_ids");
  if (max_logprobs > 0 && (!topn_ids || !topn_logprobs))
    return fail(TS_EINVAL, "NULL top-N outputs with max_logprobs > 0");
  if (!aligned(params, 8) || !aligned(token_ids, 4)) return fail(TS_EUNSUPPORTED, "misaligned pointer");
  const size_t need = ts::sampler_workspace_size(rows, cols, a.lv.n, max_logprobs);
  if (!workspace || workspace_bytes < need)
    return fail(TS_EWORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                workspace ? workspace_bytes : (size_t)0);
  if (!aligned(workspace, 256)) return fail(TS_EUNSUPPORTED, "workspace not 256-byte aligned");
  a.rows = static_cast<int>(rows);
  a.vocab = static_cast<int>(vocab);
  a.params = params;
  a.row_offset = row_offset;
  a.max_logprobs = max_logprobs;
  a.token_ids = token_ids;
  a.token_logprobs = token_logprobs;
  a.topn_ids = topn_ids;
  a.topn_logprobs = topn_logprobs;
  a.row_status = row_status;
  if (stitch != nullptr) {
    if (ts::sampler_takes_chunk_pass(rows, cols, a.lv.n)) {
      a.asm_out = stitch_out;
      a.asm_ld = stitch_ld;
    } else {
      const hipError_t ea = ts::launch_assemble(*stitch, rows, stitch_out, stitch_ld,
                                                static_cast<hipStream_t>(stream));
      if (ea != hipSuccess) return hip_status(ea, "assembly launch");
    }
  }
  const hipError_t e =
      ts::launch_sampler(a, workspace, workspace_bytes, static_cast<hipStream_t>(stream));
  return hip_status(e, "sampler launch");
}

// The slice arrays of a sampler call into a.lv (and a.flags); *total gets the
// summed width.
static int sampler_view(ts::SamplerArgs& a, const float* const* slices,
                        const int64_t* slice_cols, const int64_t* slice_ld, int32_t n_slices,
                        int64_t rows, int32_t flags, int64_t* total_out) {
  if (flags & ~TS_LOGPROBS_PROCESSED) return fail(TS_EINVAL, "unknown flag bits 0x%x", flags);
  if (n_slices < 1 || n_slices > TS_MAX_SLICES)
    return fail(n_slices < 1 ? TS_EINVAL : TS_EUNSUPPORTED, "n_slices %d not in [1, %d]",
                n_slices, TS_MAX_SLICES);
  if (rows < 0) return fail(TS_EINVAL, "rows < 0");
  if (!slices || !slice_cols || !slice_ld) return fail(TS_EINVAL, "NULL slice arrays");
  a.lv.n = n_slices;
  a.flags = flags;
  int64_t total = 0;
  for (int i = 0; i < n_slices; ++i) {
    const int64_t c = slice_cols[i];
    if (c < 0) return fail(TS_EINVAL, "slice %d has negative width", i);
    if (slice_ld[i] < c) return fail(TS_EINVAL, "slice %d leading dimension below its width", i);
    if (rows > 0 && c > 0 && !slices[i]) return fail(TS_EINVAL, "slice %d is NULL", i);
    if (slices[i] && !aligned(slices[i], 4)) return fail(TS_EUNSUPPORTED, "slice %d misaligned", i);
    a.lv.ptr[i] = slices[i];
    a.lv.ld[i] = slice_ld[i];
    a.lv.off[i] = total;
    total += c;
    if (total > kMaxDim) return fail(TS_EUNSUPPORTED, "size above 2^31-1");
  }
  a.lv.off[n_slices] = total;
  *total_out = total;
  return TS_OK;
}

// The arguments of an assembly into s; *work is false when there is nothing
// to copy.
static int assembly_view(ts::AssembleSlices& s, const float* const* slices,
                         const int64_t* slice_cols, const int64_t* slice_ld, int32_t n_slices,
                         int64_t rows, float* out, int64_t ld_out, bool* work) {
  *work = false;
  if (n_slices < 1 || n_slices > TS_MAX_SLICES)
    return fail(n_slices < 1 ? TS_EINVAL : TS_EUNSUPPORTED, "n_slices %d not in [1, %d]",
                n_slices, TS_MAX_SLICES);
  if (rows < 0) return fail(TS_EINVAL, "rows < 0");
  if (!slices || !slice_cols || !slice_ld) return fail(TS_EINVAL, "NULL slice arrays");
  s.n = n_slices;
  int64_t total = 0;
  bool vec4 = aligned(out, 16) && (ld_out % 4 == 0);
  s.chunk_start[0] = 0;
  for (int i = 0; i < n_slices; ++i) {
    const int64_t c = slice_cols[i];
    if (c < 0) return fail(TS_EINVAL, "slice %d has negative width", i);
    if (slice_ld[i] < c) return fail(TS_EINVAL, "slice %d leading dimension below its width", i);
    if (rows > 0 && c > 0 && !slices[i]) return fail(TS_EINVAL, "slice %d is NULL", i);
    if (slices[i] && !aligned(slices[i], 4)) return fail(TS_EUNSUPPORTED, "slice %d misaligned", i);
    s.ptr[i] = slices[i];
    s.cols[i] = c;
    s.ld[i] = slice_ld[i];
    s.col_off[i] = total;
    vec4 = vec4 && aligned(slices[i], 16) && (slice_ld[i] % 4 == 0) && (c % 4 == 0) &&
           (total % 4 == 0);
    s.chunk_start[i + 1] = s.chunk_start[i] + (c + ts::kAssembleChunk - 1) / ts::kAssembleChunk;
    total += c;
  }
  if (ld_out < total) return fail(TS_EINVAL, "ld_out %lld below total width %lld",
                                  (long long)ld_out, (long long)total);
  if (rows == 0 || total == 0) return TS_OK;
  if (!out) return fail(TS_EINVAL, "NULL out");
  if (!aligned(out, 4)) return fail(TS_EUNSUPPORTED, "out misaligned");
  if (s.chunk_start[n_slices] > kMaxDim) return fail(TS_EUNSUPPORTED, "too many column chunks");
  // Slices must not overlap the output rows they are copied into.
  const char* ob = reinterpret_cast<const char*>(out);
  const char* oe = reinterpret_cast<const char*>(out + (rows - 1) * ld_out + total);
  for (int i = 0; i < n_slices; ++i) {
    if (s.cols[i] == 0) continue;
    const char* sb = reinterpret_cast<const char*>(slices[i]);
    const char* se =
        reinterpret_cast<const char*>(slices[i] + (rows - 1) * slice_ld[i] + s.cols[i]);
    if (sb < oe && ob < se) return fail(TS_EINVAL, "slice %d overlaps out", i);
  }
  s.vec4 = vec4 ? 1 : 0;
  *work = true;
  return TS_OK;
}

}  // namespace

int sampler_sample(const float* logits, int64_t rows, int64_t vocab, int64_t ld_logits,
                   const ts_row_params* params, int64_t row_offset, int32_t max_logprobs,
                   int32_t* token_ids, float* token_logprobs, int32_t* topn_ids,
                   float* topn_logprobs, int32_t* row_status, void* workspace,
                   size_t workspace_bytes, void* stream) {
  if (rows < 0 || vocab < 0)
    return fail(TS_EINVAL, "negative size (rows=%lld vocab=%lld)", (long long)rows,
                (long long)vocab);
  if (rows > 0 && vocab > 0) {
    if (ld_logits < vocab)
      return fail(TS_EINVAL, "ld_logits %lld < vocab %lld", (long long)ld_logits,
                  (long long)vocab);
    if (!logits) return fail(TS_EINVAL, "NULL logits");
    if (!aligned(logits, 4)) return fail(TS_EUNSUPPORTED, "misaligned pointer");
  }
  ts::SamplerArgs a{};
  a.lv.n = 1;
  a.lv.ptr[0] = logits;
  a.lv.ld[0] = ld_logits;
  a.lv.off[0] = 0;
  a.lv.off[1] = vocab;
  return sample_common(a, &vocab, rows, vocab, params, row_offset, max_logprobs, token_ids,
                       token_logprobs, topn_ids, topn_logprobs, row_status, workspace,
                       workspace_bytes, stream);
}

int sampler_sample_ex(const float* const* slices, const int64_t* slice_cols,
                      const int64_t* slice_ld, int32_t n_slices, int64_t rows,
                      const ts_row_params* params, int64_t row_offset, int32_t max_logprobs,
                      int32_t flags, int32_t* token_ids, float* token_logprobs, int32_t* topn_ids,
                      float* topn_logprobs, int32_t* row_status, void* workspace,
                      size_t workspace_bytes, void* stream) {
  ts::SamplerArgs a{};
  int64_t total = 0;
  const int st = sampler_view(a, slices, slice_cols, slice_ld, n_slices, rows, flags, &total);
  if (st != TS_OK) return st;
  return sample_common(a, slice_cols, rows, total, params, row_offset, max_logprobs, token_ids,
                       token_logprobs, topn_ids, topn_logprobs, row_status, workspace,
                       workspace_bytes, stream);
}

int sampler_assemble_and_sample(const float* const* slices, const int64_t* slice_cols,
                                const int64_t* slice_ld, int32_t n_slices, int64_t rows,
                                float* out, int64_t ld_out, const ts_row_params* params,
                                int64_t row_offset, int32_t max_logprobs, int32_t flags,
                                int32_t* token_ids, float* token_logprobs, int32_t* topn_ids,
                                float* topn_logprobs, int32_t* row_status, void* workspace,
                                size_t workspace_bytes, void* stream) {
  ts::AssembleSlices s;
  bool work = false;
  int st = assembly_view(s, slices, slice_cols, slice_ld, n_slices, rows, out, ld_out, &work);
  if (st != TS_OK) return st;
  ts::SamplerArgs a{};
  int64_t total = 0;
  st = sampler_view(a, slices, slice_cols, slice_ld, n_slices, rows, flags, &total);
  if (st != TS_OK) return st;
  return sample_common(a, slice_cols, rows, total, params, row_offset, max_logprobs, token_ids,
                       token_logprobs, topn_ids, topn_logprobs, row_status, workspace,
                       workspace_bytes, stream, work ? &s : nullptr, out, ld_out);
}

int sampler_sample_slices(const float* const* slices, const int64_t* slice_cols,
                          const int64_t* slice_ld, int32_t n_slices, int64_t rows,
                          const ts_row_params* params, int64_t row_offset, int32_t max_logprobs,
                          int32_t* token_ids, float* token_logprobs, int32_t* topn_ids,
                          float* topn_logprobs, int32_t* row_status, void* workspace,
                          size_t workspace_bytes, void* stream) {
  return sampler_sample_ex(slices, slice_cols, slice_ld, n_slices, rows, params, row_offset,
                           max_logprobs, 0, token_ids, token_logprobs, topn_ids, topn_logprobs,
                           row_status, workspace, workspace_bytes, stream);
}

int sampler_assemble_vocab_slices(const float* const* slices, const int64_t* slice_cols,
                                  const int64_t* slice_ld, int32_t n_slices, int64_t rows,
                                  float* out, int64_t ld_out, void* stream) {
  ts::AssembleSlices s;
  bool work = false;
  const int st = assembly_view(s, slices, slice_cols, slice_ld, n_slices, rows, out, ld_out, &work);
  if (st != TS_OK || !work) return st;
  const hipError_t e = ts::launch_assemble(s, rows, out, ld_out, static_cast<hipStream_t>(stream));
  return hip_status(e, "sampler_assemble_vocab_slices launch");
}

}  // extern "C"
