// Host-side driver of the C ABI's argument validation, built with
// AddressSanitizer on the host code (device code is not built: every call
// below is rejected, or is a no-op, before any HIP call).  It walks every
// entry point's checks, including the host arrays of the slice calls at their
// largest accepted length, and the workspace-size arithmetic over a range of
// shapes.  Exit status 0 means every return code was the expected one and
// the sanitizer found nothing.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "../../include/top_sampling.h"
#include "../../include/top_sampling_measure.h"

static int failures = 0;

static void expect(int got, int want, const char* what) {
  if (got != want) {
    fprintf(stderr, "FAIL %s: got %d want %d (%s)\n", what, got, want, ts_last_error());
    ++failures;
  }
  if (got != TS_OK && strlen(ts_last_error()) == 0) {
    fprintf(stderr, "FAIL %s: empty ts_last_error\n", what);
    ++failures;
  }
}

int main() {
  void* F = reinterpret_cast<void*>(0x10000);  // aligned, never dereferenced
  float* Ff = static_cast<float*>(F);
  int32_t* Fi = static_cast<int32_t*>(F);
  const ts_row_params* Fp = static_cast<const ts_row_params*>(F);

  // projection
  expect(lmhead_logits_local(F, -1, 256, 256, F, 64, 256, Ff, 64, nullptr), TS_EINVAL, "gemm rows<0");
  expect(lmhead_logits_local(nullptr, 4, 256, 256, F, 64, 256, Ff, 64, nullptr), TS_EINVAL, "gemm null");
  expect(lmhead_logits_local(F, 4, 256, 128, F, 64, 256, Ff, 64, nullptr), TS_EINVAL, "gemm ld");
  expect(lmhead_logits_local(F, 4, 250, 256, F, 64, 256, Ff, 64, nullptr), TS_EUNSUPPORTED, "gemm h%8");
  expect(lmhead_logits_local(static_cast<char*>(F) + 8, 4, 256, 256, F, 64, 256, Ff, 64, nullptr),
         TS_EUNSUPPORTED, "gemm align");
  expect(lmhead_logits_local(nullptr, 0, 256, 256, nullptr, 64, 256, nullptr, 64, nullptr), TS_OK,
         "gemm empty");
  expect(lmhead_logits_local_e4m3(F, Ff, 4, 192, 256, F, Ff, 64, 256, Ff, 64, nullptr),
         TS_EUNSUPPORTED, "fp8 h%128");
  expect(lmhead_logits_local_e4m3(F, nullptr, 4, 256, 256, F, Ff, 64, 256, Ff, 64, nullptr),
         TS_EINVAL, "fp8 null scales");
  expect(quantize_rows_e4m3(F, 4, 8, 7, F, 8, Ff, nullptr), TS_EINVAL, "quant ld");
  expect(quantize_rows_e4m3(static_cast<char*>(F) + 1, 4, 8, 8, F, 8, Ff, nullptr), TS_EUNSUPPORTED,
         "quant align");

  // sampler on one buffer
  expect(sampler_sample(Ff, 8, 100, 100, Fp, 0, -1, Fi, Ff, Fi, Ff, Fi, nullptr, 0, nullptr),
         TS_EINVAL, "sample max_logprobs<0");
  expect(sampler_sample(Ff, 8, 100, 100, Fp, 0, TS_MAX_LOGPROBS + 1, Fi, Ff, Fi, Ff, Fi, nullptr,
                        0, nullptr), TS_EUNSUPPORTED, "sample max_logprobs big");
  expect(sampler_sample(Ff, 8, 100, 99, Fp, 0, 5, Fi, Ff, Fi, Ff, Fi, nullptr, 0, nullptr),
         TS_EINVAL, "sample ld");
  expect(sampler_sample(Ff, 8, 100, 100, Fp, 0, 5, Fi, Ff, nullptr, Ff, Fi, nullptr, 0, nullptr),
         TS_EINVAL, "sample null topn");
  expect(sampler_sample(Ff, 8, 100, 100, Fp, 0, 5, Fi, Ff, Fi, Ff, Fi, nullptr, 0, nullptr),
         TS_EWORKSPACE, "sample no workspace");
  expect(sampler_sample(Ff, 8, 100, 100, Fp, 0, 5, Fi, Ff, Fi, Ff, Fi, F, 1, nullptr),
         TS_EWORKSPACE, "sample small workspace");
  expect(sampler_sample(nullptr, 0, 100, 100, nullptr, 0, 5, nullptr, nullptr, nullptr, nullptr,
                        nullptr, nullptr, 0, nullptr), TS_OK, "sample empty");

  expect(sampler_sample_noalloc(Ff, -1, 100, 100, Fp, 0, 5, Fi, Ff, Fi, Ff, Fi, nullptr), TS_EINVAL,
         "noalloc rows<0");
  expect(sampler_sample_noalloc(Ff, 4096, 262144, 262144, Fp, 0, 20, Fi, Ff, Fi, Ff, Fi, nullptr),
         TS_EUNSUPPORTED, "noalloc too large");
  expect(sampler_sample_noalloc(nullptr, 0, 100, 100, nullptr, 0, 5, nullptr, nullptr, nullptr,
                                nullptr, nullptr, nullptr), TS_OK, "noalloc empty");

  // slice calls with the largest accepted table, and one entry past it
  static const float* ptrs[TS_MAX_SLICES + 1];
  static int64_t cols[TS_MAX_SLICES + 1], lds[TS_MAX_SLICES + 1];
  for (int i = 0; i <= TS_MAX_SLICES; ++i) {
    ptrs[i] = Ff + 1024 * 1024 * (i + 1);
    cols[i] = 2374;
    lds[i] = 2376;
  }
  expect(sampler_sample_slices(ptrs, cols, lds, TS_MAX_SLICES, 8, Fp, 0, 5, Fi, Ff, Fi, Ff, Fi,
                               nullptr, 0, nullptr), TS_EWORKSPACE, "slices 64");
  expect(sampler_sample_slices(ptrs, cols, lds, TS_MAX_SLICES + 1, 8, Fp, 0, 5, Fi, Ff, Fi, Ff,
                               Fi, nullptr, 0, nullptr), TS_EUNSUPPORTED, "slices 65");
  expect(sampler_sample_ex(ptrs, cols, lds, 4, 8, Fp, 0, 5, 2, Fi, Ff, Fi, Ff, Fi, nullptr, 0,
                           nullptr), TS_EINVAL, "ex flags");
  expect(sampler_assemble_vocab_slices(ptrs, cols, lds, TS_MAX_SLICES, 8, nullptr,
                                       TS_MAX_SLICES * 2374, nullptr), TS_EINVAL, "assemble null out");
  expect(sampler_assemble_vocab_slices(ptrs, cols, lds, TS_MAX_SLICES, 8, Ff, 100, nullptr),
         TS_EINVAL, "assemble ld_out");
  expect(sampler_assemble_vocab_slices(ptrs, cols, lds, 0, 8, Ff, 100, nullptr), TS_EINVAL,
         "assemble 0 slices");
  // the one-call assembly + sampler: both tables walked, nothing enqueued
  float* wide = Ff + 1024 * 1024 * (TS_MAX_SLICES + 2);
  expect(sampler_assemble_and_sample(ptrs, cols, lds, TS_MAX_SLICES, 8, wide,
                                     TS_MAX_SLICES * 2374, Fp, 0, 5, 0, Fi, Ff, Fi, Ff, Fi,
                                     nullptr, 0, nullptr), TS_EWORKSPACE, "one call 64");
  expect(sampler_assemble_and_sample(ptrs, cols, lds, TS_MAX_SLICES + 1, 8, wide,
                                     (TS_MAX_SLICES + 1) * 2374, Fp, 0, 5, 0, Fi, Ff, Fi, Ff, Fi,
                                     nullptr, 0, nullptr), TS_EUNSUPPORTED, "one call 65");
  expect(sampler_assemble_and_sample(ptrs, cols, lds, 4, 8, nullptr, 4 * 2374, Fp, 0, 5, 0, Fi,
                                     Ff, Fi, Ff, Fi, nullptr, 0, nullptr), TS_EINVAL,
         "one call null out");
  expect(sampler_assemble_and_sample(ptrs, cols, lds, 4, 8, wide, 100, Fp, 0, 5, 0, Fi, Ff, Fi,
                                     Ff, Fi, nullptr, 0, nullptr), TS_EINVAL, "one call ld_out");
  expect(sampler_assemble_and_sample(ptrs, cols, lds, 4, 8, const_cast<float*>(ptrs[1]),
                                     4 * 2374, Fp, 0, 5, 0, Fi, Ff, Fi, Ff, Fi, nullptr, 0,
                                     nullptr), TS_EINVAL, "one call overlap");
  expect(sampler_assemble_and_sample(ptrs, cols, lds, 4, 8, wide, 4 * 2374, Fp, 0, 5, 4, Fi, Ff,
                                     Fi, Ff, Fi, nullptr, 0, nullptr), TS_EINVAL, "one call flags");
  expect(sampler_assemble_and_sample(ptrs, cols, lds, 4, 0, nullptr, 4 * 2374, nullptr, 0, 5, 0,
                                     nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0,
                                     nullptr), TS_OK, "one call empty");

  // workspace arithmetic over many shapes (host only)
  const int64_t rows_list[] = {0, 1, 3, 64, 640, 1024, 4096, 65536};
  const int64_t vocab_list[] = {1, 3, 4, 1000, 4097, 151936, 262144, 1 << 20};
  for (int64_t r : rows_list)
    for (int64_t v : vocab_list)
      for (int32_t lp : {0, 5, 20, 1024}) {
        const size_t a = sampler_workspace_bytes(r, v, lp);
        int64_t one[1] = {v};
        const size_t b = sampler_workspace_bytes_slices(r, one, 1, lp);
        if (a != b) {
          fprintf(stderr, "FAIL workspace %lld %lld %d: %zu vs %zu\n", (long long)r,
                  (long long)v, lp, a, b);
          ++failures;
        }
        int64_t many[TS_MAX_SLICES];
        for (int i = 0; i < TS_MAX_SLICES; ++i) many[i] = v / TS_MAX_SLICES + (i < v % 64);
        (void)sampler_workspace_bytes_slices(r, many, TS_MAX_SLICES, lp);
      }
  if (sampler_workspace_bytes(-1, 10, 0) != 0 || sampler_workspace_bytes(4, 10, -1) != 0) {
    fprintf(stderr, "FAIL workspace of invalid sizes\n");
    ++failures;
  }

  // measurement aids
  expect(ts_mfma_clock_probe(nullptr, 4, 16, TS_PROBE_RANDOM_OPERANDS, nullptr), TS_EINVAL, "probe");
  expect(ts_gumbel_keys(Ff, Ff, Ff, static_cast<const uint64_t*>(F), static_cast<const int64_t*>(F),
                        Fi, -1, Ff, nullptr, nullptr), TS_EINVAL, "gumbel n<0");
  expect(ts_gumbel_keys(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0, nullptr, nullptr,
                        nullptr), TS_OK, "gumbel empty");

  for (int s : {0, -1, -2, -3, -4, 7})
    if (!ts_status_string(s) || !ts_status_string(s)[0]) ++failures;
  printf("abi_driver: %d failures\n", failures);
  return failures == 0 ? 0 : 1;
}
