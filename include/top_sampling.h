/*
 * top_sampling.h -- C ABI of the MI355X (gfx950) batch-sharded sampling path.
 *
 * One tensor-parallel rank's share of batch-sharded sampling, as described on
 * the page "Qwen4Exp batch-sharded sampling: inside vLLM PR #61018"
 * (orcarouter.ai blog, ja/nl/fr editions):
 *
 *   1. lmhead_logits_local       -- the rank's own vocabulary slice of the
 *      projection, with no gather (sections "What batch-sharded sampling is,
 *      in one paragraph" and "Why three lines were the whole job": the
 *      model's local-logits hook hands back only the rank's vocabulary shard);
 *   2. sampler_assemble_vocab_slices -- the receive side of the all-to-all:
 *      vocabulary slices from every rank stitched into full-vocabulary rows
 *      for the rank's slice of requests (section "What batch-sharded sampling
 *      is, in one paragraph");
 *   3. sampler_sample            -- the per-row sampler over
 *      batch x (speculative tokens + 1) rows: temperature, top-k, top-p,
 *      log-probabilities and seeded sampling (same section; the page names
 *      top-k, top-p and a non-negative max_logprobs, not their arithmetic);
 *   2+3. sampler_assemble_and_sample -- both in one call that reads the
 *      received logits once.
 *
 * Conventions shared by every call
 *   - All pointers to bulk data are DEVICE pointers unless stated otherwise.
 *     The caller owns every buffer; the library never allocates device
 *     memory, never synchronises the host and never prints.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Work is enqueued asynchronously on it.
 *   - A nonzero return value means argument validation failed and NOTHING was
 *     enqueued: invalid configurations are rejected up front rather than
 *     degraded silently.  This follows the fail-fast convention of the
 *     sequence-parallel patch described on the page "Qwen 4 leak: SGLang
 *     shards the Qwen4Exp prefill" (orcarouter.ai blog, ja edition), section
 *     "The cost to you: constraints": unsupported configurations fail during
 *     argument validation.  ts_last_error() then describes the failure for
 *     the calling thread.  TS_EHIP reports a failed kernel launch.
 *   - The preconditions batch-sharded sampling states (page "Qwen4Exp
 *     batch-sharded sampling: inside vLLM PR #61018", section "What
 *     batch-sharded sampling is, in one paragraph") include a non-negative
 *     max_logprobs: max_logprobs < 0 is TS_EINVAL in every sampler call.
 *   - Measurement and check aids that are not steps of the path (clock
 *     probe, noise readout) are declared in top_sampling_measure.h.
 *   - Sizes of zero are valid no-ops.
 *   - Matrices are row-major with an explicit leading dimension (elements).
 */
#ifndef TOP_SAMPLING_H_
#define TOP_SAMPLING_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
enum {
  TS_OK = 0,
  TS_EINVAL = -1,        /* bad sizes, leading dimensions or NULL pointers     */
  TS_EUNSUPPORTED = -2,  /* valid but outside what the kernels take (alignment,
                            limits such as TS_MAX_LOGPROBS)                    */
  TS_EWORKSPACE = -3,    /* workspace NULL or smaller than required            */
  TS_EHIP = -4           /* the HIP runtime rejected a launch                  */
};

/* Per-row status written by sampler_sample. */
enum {
  TS_ROW_OK = 0,
  TS_ROW_BAD_PARAMS = 1,  /* temperature < 0 or not finite; top_k < 0;
                             top_p not in (0, 1]; n_logprobs not in
                             [0, max_logprobs]                               */
  TS_ROW_BAD_LOGITS = 2   /* a NaN or +inf logit, or no finite logit          */
};

#define TS_MAX_LOGPROBS 1024   /* largest accepted max_logprobs              */
#define TS_MAX_SLICES 64       /* largest accepted n_slices                  */
#define TS_GREEDY_EPS 1e-6f    /* temperatures below this sample greedily    */
/* sampler_sample_ex flags */
#define TS_LOGPROBS_PROCESSED 1 /* log-probabilities of the sampled distribution */

/*
 * Sampling parameters of one row (24 bytes, 8-byte aligned; an array of
 * `rows` of them lives in device memory).
 *   temperature  0 (or < TS_GREEDY_EPS): greedy argmax of the raw logits.
 *   top_k        0 or >= vocab: no top-k filter; 1: greedy.  Every token
 *                tied with the k-th largest logit is kept.
 *   top_p        1: no top-p filter.  Otherwise the smallest set of most
 *                likely tokens (of the temperature-scaled distribution
 *                renormalised over the top-k set) whose mass reaches top_p;
 *                the crossing token and its ties are kept.
 *   n_logprobs   how many of the row's largest logits to report (<= the
 *                call's max_logprobs).
 *   seed         RNG key of the row.  Sampling is Gumbel-max:
 *                token = argmax over kept v of (l_v - max l) / T + g_v,
 *                g_v = -ln(-ln u_v), u_v = ((x >> 9) + 1/2) * 2^-23 where x
 *                is word (v & 3) of Philox4x32-10 with key (seed lo32,
 *                seed hi32) and counter (v >> 2, row lo32, row hi32, 0),
 *                row = row_offset + local row (Salmon et al., "Parallel
 *                Random Numbers: As Easy as 1, 2, 3", SC'11).  Lowest id
 *                wins exact ties.
 */
typedef struct ts_row_params {
  float temperature;
  int32_t top_k;
  float top_p;
  int32_t n_logprobs;
  uint64_t seed;
} ts_row_params;

/*
 * lmhead_logits_local: logits[r, v] = sum_h hidden[r, h] * lm_head[v, h].
 *
 * The rank's local vocabulary projection: only the slice of the vocabulary
 * this rank holds (vocab_local rows of lm_head), never gathered.
 *   hidden     bf16 [rows, hidden_dim], leading dimension ld_hidden
 *   lm_head    bf16 [vocab_local, hidden_dim], leading dimension ld_lm_head
 *              (both K-contiguous)
 *   logits     fp32 [rows, vocab_local] written with leading dimension
 *              ld_logits >= vocab_local, so a slice can be written straight
 *              into a wider buffer.
 * Products of bf16 are exact in fp32; accumulation is fp32 (MFMA).
 * Requirements (else TS_EUNSUPPORTED): hidden_dim % 8 == 0, ld_hidden and
 * ld_lm_head multiples of 8, hidden and lm_head 16-byte aligned, logits
 * 4-byte aligned.  rows, vocab_local < 2^31.
 */
int lmhead_logits_local(const void* hidden, int64_t rows, int64_t hidden_dim,
                        int64_t ld_hidden, const void* lm_head, int64_t vocab_local,
                        int64_t ld_lm_head, float* logits, int64_t ld_logits,
                        void* stream);

/*
 * FP8 projection.  The pages' measured deployment is an FP8 checkpoint and
 * their patch cluster unpacks e4m3 bytes (sections "The 1.5% estimate, and
 * the measurement next to it" and "The patch cluster"); they state no
 * scaling scheme.  Reading: W8A8 with one fp32 scale per row on both
 * operands.  A row x is held as OCP E4M3 codes q (one byte each; no
 * infinities, largest magnitude 448, 0x7F/0xFF NaN) with x ~ s * dec(q),
 * s = max|x| / 448.
 *
 * quantize_rows_e4m3: per-row dynamic quantization of bf16 data:
 *   scales[r] = max_c |in[r, c]| / 448 in fp32 (NaN ignored; 1 for a row
 *   of zeros); out[r, c] = the E4M3 code nearest in[r, c] / scales[r]
 *   (quotient in fp32), ties to the even code, saturating at +-448, NaN ->
 *   0x7F.
 *   in      bf16 [rows, cols], leading dimension ld_in (elements)
 *   out     codes [rows, cols], leading dimension ld_out (bytes)
 *   scales  fp32 [rows]
 * Caller-owned device buffers; in 2-byte and scales 4-byte aligned.
 *
 * lmhead_logits_local_e4m3: logits[r, v] = hidden_scales[r] *
 *   lm_head_scales[v] * sum_h dec(hidden[r, h]) * dec(lm_head[v, h]),
 *   fp32 accumulation (every product of two E4M3 values is exact in fp32),
 *   over the rank's own vocabulary slice, never gathered.
 *   hidden          codes [rows, hidden_dim], leading dimension ld_hidden
 *   hidden_scales   fp32 [rows]
 *   lm_head         codes [vocab_local, hidden_dim], leading dimension ld_lm_head
 *   lm_head_scales  fp32 [vocab_local]
 *   logits          fp32 [rows, vocab_local], leading dimension ld_logits
 * Requirements (else TS_EUNSUPPORTED): hidden_dim a multiple of 128,
 * ld_hidden and ld_lm_head multiples of 16, codes 16-byte aligned, logits
 * and scales 4-byte aligned.  Other errors and the empty cases as for
 * lmhead_logits_local.
 */
int quantize_rows_e4m3(const void* in, int64_t rows, int64_t cols, int64_t ld_in, void* out,
                       int64_t ld_out, float* scales, void* stream);
int lmhead_logits_local_e4m3(const void* hidden, const float* hidden_scales, int64_t rows,
                             int64_t hidden_dim, int64_t ld_hidden, const void* lm_head,
                             const float* lm_head_scales, int64_t vocab_local, int64_t ld_lm_head,
                             float* logits, int64_t ld_logits, void* stream);

/*
 * sampler_workspace_bytes: device workspace sampler_sample needs for these
 * sizes (host-only computation; callable without a GPU).  The caller owns
 * the workspace, as every other buffer: serving replays fixed graph buckets
 * (page "Qwen 4 leak: SGLang shards the Qwen4Exp prefill", section "The
 * layout bug they had to fix first": fixed physical CUDA-graph buckets), so
 * the library allocates nothing per call and the caller sizes each bucket's
 * workspace once from this query.  Returns 0 for negative sizes or
 * max_logprobs < 0 (the non-negative max_logprobs precondition of page
 * "Qwen4Exp batch-sharded sampling: inside vLLM PR #61018", section "What
 * batch-sharded sampling is, in one paragraph").
 */
size_t sampler_workspace_bytes(int64_t rows, int64_t vocab, int32_t max_logprobs);

/*
 * sampler_sample: sample one token per row and report log-probabilities.
 *   logits          fp32 [rows, vocab], leading dimension ld_logits; read only.
 *   params          device array of `rows` ts_row_params.
 *   row_offset      global index of local row 0 (keys the RNG, so a rank's
 *                   share of rows draws exactly what the unsharded call would).
 *   max_logprobs    0..TS_MAX_LOGPROBS: width of the top-N outputs.
 *   token_ids       int32 [rows]: sampled token, -1 for a row whose status != 0.
 *   token_logprobs  fp32 [rows] or NULL: raw log_softmax of the sampled token
 *                   (NaN for a bad row).
 *   topn_ids        int32 [rows, max_logprobs] (may be NULL iff max_logprobs
 *                   == 0): the row's n_logprobs largest logits, largest first,
 *                   lower id first on ties; unused slots -1.
 *   topn_logprobs   fp32 [rows, max_logprobs]: their raw log-probabilities;
 *                   unused slots -inf; NaN for a bad row.
 *   row_status      int32 [rows] or NULL: TS_ROW_* per row.
 *   workspace       device scratch of at least sampler_workspace_bytes(...)
 *                   bytes, 256-byte aligned; contents need no initialisation
 *                   and are clobbered.
 * Log-probabilities describe the raw distribution log_softmax(logits)
 * (unscaled, unfiltered).  Calls that share a workspace must be ordered on
 * one stream.  vocab < 2^31.
 */
int sampler_sample(const float* logits, int64_t rows, int64_t vocab, int64_t ld_logits,
                   const ts_row_params* params, int64_t row_offset, int32_t max_logprobs,
                   int32_t* token_ids, float* token_logprobs, int32_t* topn_ids,
                   float* topn_logprobs, int32_t* row_status, void* workspace,
                   size_t workspace_bytes, void* stream);

/*
 * sampler_sample_noalloc: sampler_sample for callers that cannot allocate --
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, outputs and results as sampler_sample, without
 * the workspace: the library keeps a file-scope device array of
 * TS_NOALLOC_SCRATCH_BYTES per GPU (placed when the runtime loads the
 * library on that GPU, held until the process ends) and uses it as the
 * workspace.  The call allocates and frees nothing.
 *   - TS_EUNSUPPORTED if sampler_workspace_bytes(rows, vocab, max_logprobs)
 *     exceeds TS_NOALLOC_SCRATCH_BYTES (e.g. 640 x 151,936 x 20 needs about
 *     43 MB and fits; use sampler_sample with a caller workspace beyond it).
 *   - Every call on a GPU shares that GPU's array: calls that overlap on one
 *     GPU (different streams, or different host threads) race and must be
 *     serialised by the caller.  The array needs no clearing between calls.
 *   - TS_EHIP if no HIP device is current or the array's device address
 *     cannot be obtained.
 */
#define TS_NOALLOC_SCRATCH_BYTES (96ull << 20)
int sampler_sample_noalloc(const float* logits, int64_t rows, int64_t vocab, int64_t ld_logits,
                           const ts_row_params* params, int64_t row_offset, int32_t max_logprobs,
                           int32_t* token_ids, float* token_logprobs, int32_t* topn_ids,
                           float* topn_logprobs, int32_t* row_status, void* stream);

/*
 * sampler_workspace_bytes_slices: device workspace sampler_sample_slices
 * needs (host-only computation).  slice_cols is a HOST array of n_slices
 * entries.
 */
size_t sampler_workspace_bytes_slices(int64_t rows, const int64_t* slice_cols, int32_t n_slices,
                                      int32_t max_logprobs);

/*
 * sampler_sample_slices: sampler_sample over a rank's batch slice that is
 * still held as the vocabulary slices the exchange delivered, without
 * stitching them into one buffer first (the step after the all-to-all on
 * the page "Qwen4Exp batch-sharded sampling: inside vLLM PR #61018", section
 * "What batch-sharded sampling is, in one paragraph": each rank receives the
 * vocabulary slices of its requests).  Global column off_s + c of row r is
 * slices[s][r * slice_ld[s] + c], off_s = slice_cols[0] + ... +
 * slice_cols[s-1]; vocab = the sum of slice_cols.
 *   slices      HOST array of n_slices DEVICE pointers (fp32, read only)
 *   slice_cols, slice_ld   HOST arrays of n_slices entries
 * Every other argument, output and the results are those of sampler_sample
 * on the stitched [rows, vocab] buffer; the workspace is sized by
 * sampler_workspace_bytes_slices.  1 <= n_slices <= TS_MAX_SLICES.  Slices
 * that start at a column not a multiple of 4 take the exact per-row kernel
 * (same results, slower).
 */
int sampler_sample_slices(const float* const* slices, const int64_t* slice_cols,
                          const int64_t* slice_ld, int32_t n_slices, int64_t rows,
                          const ts_row_params* params, int64_t row_offset, int32_t max_logprobs,
                          int32_t* token_ids, float* token_logprobs, int32_t* topn_ids,
                          float* topn_logprobs, int32_t* row_status, void* workspace,
                          size_t workspace_bytes, void* stream);

/*
 * sampler_sample_ex: sampler_sample_slices with a flags word (0 gives
 * sampler_sample_slices exactly; sampler_sample is the one-slice case).
 *   TS_LOGPROBS_PROCESSED  token_logprobs and topn_logprobs describe the
 *       distribution the token is drawn from instead of the raw
 *       log_softmax(logits): (l - m)/T - ln(sum over the kept set of
 *       exp((l - m)/T)) for tokens the filters keep, -inf for the others; a
 *       greedy row is a point mass (0 for the chosen token, -inf for the
 *       rest).  top-N lists the same ids as the raw mode (the N largest
 *       logits).  The pages ask only for a non-negative max_logprobs
 *       (section "What batch-sharded sampling is, in one paragraph"); this
 *       is the processed variant of the same output.  Top-p-only rows whose
 *       nucleus reaches below the listed candidates take the exact per-row
 *       kernel in this mode.
 * Other flag bits: TS_EINVAL.  Workspace: sampler_workspace_bytes_slices.
 */
int sampler_sample_ex(const float* const* slices, const int64_t* slice_cols,
                      const int64_t* slice_ld, int32_t n_slices, int64_t rows,
                      const ts_row_params* params, int64_t row_offset, int32_t max_logprobs,
                      int32_t flags, int32_t* token_ids, float* token_logprobs, int32_t* topn_ids,
                      float* topn_logprobs, int32_t* row_status, void* workspace,
                      size_t workspace_bytes, void* stream);

/*
 * sampler_assemble_vocab_slices: out[r, off_s + c] = slice_s[r, c] with
 * off_s = slice_cols[0] + ... + slice_cols[s-1].
 *   slices      HOST array of n_slices DEVICE pointers, slice s fp32
 *               [rows, slice_cols[s]] with leading dimension slice_ld[s]
 *   slice_cols, slice_ld   HOST arrays of n_slices entries
 *   out         fp32 [rows, sum slice_cols], leading dimension ld_out
 * A bit-exact copy.  1 <= n_slices <= TS_MAX_SLICES.  Slices must not
 * overlap `out`.
 */
int sampler_assemble_vocab_slices(const float* const* slices, const int64_t* slice_cols,
                                  const int64_t* slice_ld, int32_t n_slices, int64_t rows,
                                  float* out, int64_t ld_out, void* stream);

/*
 * sampler_assemble_and_sample: sampler_assemble_vocab_slices followed by
 * sampler_sample_ex on the same received slices, with one read of the
 * logits instead of two.  The rank's step after the exchange on the page
 * "Qwen4Exp batch-sharded sampling: inside vLLM PR #61018", section "What
 * batch-sharded sampling is, in one paragraph", stitches the received
 * vocabulary slices into its batch rows and samples them.  Here the
 * sampler's first pass reads every logit of every row from the slices once,
 * for its row statistics and candidates, and in the same pass writes it to
 * `out`.
 *   out, ld_out   as in sampler_assemble_vocab_slices: fp32
 *                 [rows, sum slice_cols], written in full and bit-exact;
 *                 the slices must not overlap it.
 *   Every other argument and output, and the workspace
 *   (sampler_workspace_bytes_slices), are as in sampler_sample_ex.
 * `out` is exactly what sampler_assemble_vocab_slices writes.  The sampling
 * outputs follow the same definitions as sampler_sample_ex; the call may cut
 * the rows into narrower chunks (8 instead of 16 float4 per thread when
 * that keeps at most 24 chunks per row, which overlaps the extra copy
 * traffic better), so fp32 sums and the log-probabilities may differ from
 * sampler_sample_ex's in the last bits.
 * Shapes whose rows all take the exact per-row kernel (slices that start at
 * a column not a multiple of 4) run the assembly kernel first instead.
 * Arguments of both calls are validated before anything is enqueued.
 */
int sampler_assemble_and_sample(const float* const* slices, const int64_t* slice_cols,
                                const int64_t* slice_ld, int32_t n_slices, int64_t rows,
                                float* out, int64_t ld_out, const ts_row_params* params,
                                int64_t row_offset, int32_t max_logprobs, int32_t flags,
                                int32_t* token_ids, float* token_logprobs, int32_t* topn_ids,
                                float* topn_logprobs, int32_t* row_status, void* workspace,
                                size_t workspace_bytes, void* stream);

/*
 * ts_status_string: name of a TS_* return code (a static string; unknown
 * codes give "TS_UNKNOWN").  ts_last_error: a description of the calling
 * thread's last nonzero return (a per-thread static buffer, overwritten by
 * that thread's next failure).  Both serve the fail-fast convention above:
 * a rejected configuration says why it was rejected (page "Qwen 4 leak:
 * SGLang shards the Qwen4Exp prefill", section "The cost to you:
 * constraints").  Host-only; callable without a GPU.
 */
const char* ts_status_string(int status);
const char* ts_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* TOP_SAMPLING_H_ */
