/*
 * top_sampling_measure.h -- measurement and check aids exported by the same
 * library as top_sampling.h.  None of them is a step of the sampling path;
 * the bench and the tests use them to put the path's figures and arithmetic
 * in context.  Conventions (device pointers, caller-owned buffers, nonzero
 * return = nothing enqueued, ts_last_error) are those of top_sampling.h.
 */
#ifndef TOP_SAMPLING_MEASURE_H_
#define TOP_SAMPLING_MEASURE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * ts_mfma_clock_probe: every workgroup (eight waves, two per SIMD) runs
 * `iters` rounds of four independent bf16 32x32x16 matrix-core accumulations
 * per wave and records the shader-clock counter and the constant 100 MHz
 * real-time counter before the first round and after the last:
 *   ticks       DEVICE uint64 [workgroups, 4]: clock start, clock end,
 *               real-time start, real-time end (caller-owned)
 *   workgroups  1 .. 65536 (one or more per compute unit loads every unit)
 *   iters       1 .. 2^24
 *   operands    TS_PROBE_SMALL_OPERANDS (a few small values: little bit
 *               switching) or TS_PROBE_RANDOM_OPERANDS (random bit patterns
 *               per lane, finite): the sustained rate depends on the data
 * The shader clock under this load is (clock end - clock start) /
 * (real-time end - real-time start) x 100 MHz; the matrix-core rate is
 * workgroups x 8 x iters x 4 x 32768 flop over the launch's duration.  It
 * sets the projection's bf16 roofline figure beside the clock it ran at.
 * TS_EINVAL for a NULL ticks, a misaligned ticks, a size out of range or an
 * unknown operands value.
 */
#define TS_PROBE_SMALL_OPERANDS 0
#define TS_PROBE_RANDOM_OPERANDS 1
int ts_mfma_clock_probe(uint64_t* ticks, int32_t workgroups, int64_t iters, int32_t operands,
                        void* stream);

/*
 * ts_gumbel_keys: the sampler's own fp32 Gumbel-max keys and noise words for
 * listed tokens, computed by the same device functions the sampler decides
 * with, so tests can measure how far the GPU's keys lie from float64 ones
 * (two keys closer than that error cannot be ordered reliably).  For each
 * i < n (all DEVICE arrays of n entries, caller-owned):
 *   words[i] = word (ids[i] & 3) of Philox4x32-10 with key (seeds[i] lo32,
 *              seeds[i] hi32) and counter (ids[i] >> 2, rows[i] lo32,
 *              rows[i] hi32, 0)  -- the noise layout of ts_row_params.seed;
 *   keys[i]  = (logits[i] - row_max[i]) * (1 / temperature[i]) + g,
 *              g = -ln(-ln u), u = ((words[i] >> 9) + 1/2) * 2^-23.
 * logits, row_max, temperature, keys: fp32, 4-byte aligned; seeds (uint64),
 * rows (int64): 8-byte aligned; ids (int32, >= 0), words (uint32): 4-byte
 * aligned.  keys or words may be NULL (not written).  n == 0 is a no-op;
 * n < 0, n >= 2^31 or a NULL input is TS_EINVAL.
 */
int ts_gumbel_keys(const float* logits, const float* row_max, const float* temperature,
                   const uint64_t* seeds, const int64_t* rows, const int32_t* ids, int64_t n,
                   float* keys, uint32_t* words, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TOP_SAMPLING_MEASURE_H_ */
