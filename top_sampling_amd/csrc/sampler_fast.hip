// Single-read sampler for batch-sharded sampling on gfx950.
//
// The sampler runs on the rank's slice of requests: batch x (speculative
// tokens + 1) rows of full-vocabulary fp32 logits (page "Qwen4Exp
// batch-sharded sampling: inside vLLM PR #61018", section "What
// batch-sharded sampling is, in one paragraph").  The logits are read where
// they lie: one buffer, or the vocabulary slices the exchange delivered
// (LogitsView; chunks never straddle two slices).  Every logit is read from
// HBM once by the chunk pass; the probe pass re-reads only the rows that need
// it.
//
// A  chunk pass   one 256-thread workgroup per (row, chunk of <= 16384
//                 logits), the chunk held in registers (16 float4 per
//                 thread).  Per chunk, in one pass over the loaded values:
//                   - max, sum exp(l - max) and, for top-p-only rows, sum
//                     exp((l - max) / T), rescaled as the maximum grows; a
//                     NaN or +inf shows up as a NaN sum;
//                   - a logit candidate list holding at least the chunk's
//                     share of the row's M largest, M = max(n_logprobs,
//                     top_k) (64 for top-p-only rows): the threshold is
//                     bounded by the q-th largest per-thread maximum (or
//                     top-4 value) of each wave, found with one ballot per
//                     key bit, or an LDS radix selection for large M;
//                   - for full-vocabulary and top-p-only rows, Philox4x32-10
//                     Gumbel keys, skipped for tokens whose uniform cannot
//                     lift them over the running bar; every key above the
//                     chunk's floor goes to a short key list.
// B  merge        one 256-thread workgroup per row: log-sum-exp; the union of
//                 logit candidates above the highest chunk threshold is
//                 exactly the row's logits above it.  Short prefixes (top N,
//                 top-k up to 192, the head of a top-p row) are trimmed and
//                 sorted in LDS; longer top-k sets are settled by count- and
//                 mass-weighted radix selection without sorting.  Top-N,
//                 greedy, top-k, top-p and Gumbel-max are exact on the list.
//                 A top-p-only row whose boundary lies below the list takes
//                 its best Gumbel keys as probes.
// P  probe        chunk-parallel re-read of probe rows only: the mass of the
//                 logits strictly above each probe's logit.  Token v is kept
//                 by top-p iff that mass is below p times the total, so the
//                 first probe (by key) that is kept is the Gumbel-max winner.
// X  finish       (sampler_exact.hip) settles probe rows; rows that no fast
//                 route settles (candidate or key overflow, top_k > 1024, no
//                 kept probe) run the exact per-row kernel.
#include <stdlib.h>

#include "sampler_common.hpp"

namespace ts {
namespace {

constexpr int AT = kChunkThreads;
constexpr int AW = AT / kWave;
constexpr int AV = kChunkVec;
constexpr int RB = 2048;
constexpr int BT = 256;
constexpr int BW = BT / kWave;
constexpr int PT = 256;
constexpr int PW = PT / kWave;

__device__ __forceinline__ float lane(const float4& f, int q) {
  return q == 0 ? f.x : (q == 1 ? f.y : (q == 2 ? f.z : f.w));
}

// Threshold below which every logit qualifies: keys at or below the key of
// -inf map to -inf (all lower keys are NaN patterns).
__device__ __forceinline__ float key_floor_value(uint32_t kt) {
  return kt <= 0x007fffffu ? -INFINITY : key_to_float(kt);
}

template <int NT>
__device__ void write_bad(const SamplerArgs& a, int r, int status) {
  const float qnan = __builtin_nanf("");
  for (int j = threadIdx.x; j < a.max_logprobs; j += NT) {
    a.topn_ids[static_cast<int64_t>(r) * a.max_logprobs + j] = -1;
    a.topn_logprobs[static_cast<int64_t>(r) * a.max_logprobs + j] = qnan;
  }
  if (threadIdx.x == 0) {
    a.token_ids[r] = -1;
    if (a.token_logprobs) a.token_logprobs[r] = qnan;
    if (a.row_status) a.row_status[r] = status;
  }
}

// The M-th largest of nk keys in LDS (1 <= M <= nk), by radix selection
// (11/11/10-bit digits).
template <int NT>
__device__ __forceinline__ uint32_t lds_kth_largest(const uint32_t* keys, int nk, uint32_t M, uint32_t* hist,
                                    uint32_t* scratch, uint32_t* sel_d, uint32_t* sel_above) {
  uint32_t prefix = 0u, pmask = 0u, rem = M;
  for (int rd = 0; rd < 3; ++rd) {
    const int shift = rd == 0 ? 21 : (rd == 1 ? 10 : 0);
    const int width = rd == 2 ? 10 : 11;
    const uint32_t dmask = (1u << width) - 1u;
    for (int b = threadIdx.x; b < RB; b += NT) hist[b] = 0u;
    __syncthreads();
    for (int i = threadIdx.x; i < nk; i += NT) {
      const uint32_t k = keys[i];
      if ((k & pmask) == prefix) atomicAdd(&hist[(k >> shift) & dmask], 1u);
    }
    __syncthreads();
    select_digit_top<NT, RB / NT>(hist, 1 << width, rem, scratch, sel_d, sel_above);
    const uint32_t d = *sel_d, ab = *sel_above;
    __syncthreads();
    rem -= ab;
    prefix |= d << shift;
    pmask |= dmask << shift;
  }
  return prefix;
}

// ------------------------------------------------------------------ A: chunks
struct ChunkSmem {
  uint32_t hist[RB];
  uint32_t keys4[4 * AT];  // per-thread top-4 keys (block-level selection)
  int klist[kKeyCap];
  float wthr[AW];
  float wbar[AW];
  float wsec[AW];  // posted second-largest group maxima (top-p key bars)
  float rm[AW], rs[AW], rt[AW];
  int rb[AW];
  float rf[AW];
  int ri[AW];
  uint32_t ru[AW];
  uint32_t sel_d, sel_above;
  int wcnt[AW];
  int ncand, nkey;
};

__device__ __forceinline__ void set_lane(float4& f, int q, float x) {
  if (q == 0) f.x = x;
  else if (q == 1) f.y = x;
  else if (q == 2) f.z = x;
  else f.w = x;
}

// The chunk into registers: logit e = 4 * (j * AT + tid) + q of the chunk in
// lane q of v[j]; slots past the chunk end hold -inf.  Every load is issued
// unconditionally (out-of-range slots re-read the chunk's last element), so
// all sixteen are in flight together, as non-temporal (streaming) loads.
// VEC: 16-byte aligned rows and n % 4 == 0.
template <bool VEC>
__device__ __forceinline__ void load_chunk(float4 (&v)[AV], const float* __restrict__ src, int n,
                                           int tid) {
  if (VEC) {
    const int n4 = n >> 2;
#pragma unroll
    for (int j = 0; j < AV; ++j) {
      const int i4 = j * AT + tid;
      const bool ok = i4 < n4;
      const float4 f = load_stream4(src + 4 * (ok ? i4 : n4 - 1));
      v[j].x = ok ? f.x : -INFINITY;
      v[j].y = ok ? f.y : -INFINITY;
      v[j].z = ok ? f.z : -INFINITY;
      v[j].w = ok ? f.w : -INFINITY;
    }
  } else {
#pragma unroll
    for (int j = 0; j < AV; ++j) {
      const int e = 4 * (j * AT + tid);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const bool ok = e + q < n;
        const float x = load_stream(src + (ok ? e + q : n - 1));
        set_lane(v[j], q, ok ? x : -INFINITY);
      }
    }
  }
}

// (m, s, t): a maximum with sum exp(l - m) and sum exp((l - m) / T); merging
// two rescales both sums to the larger maximum.
__device__ __forceinline__ void merge_stats(float& m, float& s, float& t, float m2, float s2,
                                            float t2, float inv_t) {
  const float mm = fmaxf(m, m2);
  if (mm == -INFINITY) return;  // both empty
  s = s * fast_exp(m - mm) + s2 * fast_exp(m2 - mm);
  t = t * fast_exp((m - mm) * inv_t) + t2 * fast_exp((m2 - mm) * inv_t);
  m = mm;
}

// The q-th largest (1 <= q <= 64) per-thread value of this wave: the largest
// order key K with at least q lanes at or above it, built bit by bit from
// the top with one ballot per bit (no data moves between lanes).
__device__ __forceinline__ float wave_qth(float x, int q) {
  const uint32_t k = order_key(x);
  uint32_t K = 0u;
#pragma unroll
  for (int b = 31; b >= 0; --b) {
    const uint32_t cand = K | (1u << b);
    if (__popcll(__ballot(k >= cand)) >= q) K = cand;
  }
  return key_to_float(K);
}

// Chunk-pass thresholds, built on the top 16 key bits only (sign, exponent
// and 7 mantissa bits): the largest K with zero low 16 bits and at least q
// lanes (or, for the top-4 form, q of the wave's per-thread top-4 values) at
// or above it.  K is at most the exact q-th largest key, so every logit the
// exact threshold admits is admitted too; the extra ones lie within 2^-7
// relative of it.  Half the ballots of the exact search.
__device__ __forceinline__ float wave_qth_hi16(float x, int q) {
  const uint32_t k = order_key(x);
  uint32_t K = 0u;
#pragma unroll
  for (int b = 31; b >= 16; --b) {
    const uint32_t cand = K | (1u << b);
    if (__popcll(__ballot(k >= cand)) >= q) K = cand;
  }
  return key_floor_value(K);
}

__device__ __forceinline__ float wave_qth4_hi16(const float (&t)[4], int q) {
  const uint32_t k0 = order_key(t[0]), k1 = order_key(t[1]), k2 = order_key(t[2]),
                 k3 = order_key(t[3]);
  uint32_t K = 0u;
#pragma unroll
  for (int b = 31; b >= 16; --b) {
    const uint32_t cand = K | (1u << b);
    const int cnt = __popcll(__ballot(k0 >= cand)) + __popcll(__ballot(k1 >= cand)) +
                    __popcll(__ballot(k2 >= cand)) + __popcll(__ballot(k3 >= cand));
    if (cnt >= q) K = cand;
  }
  return key_floor_value(K);
}

// (m & a) | (~m & b) in one v_bfi_b32.  Written as an opaque instruction so
// that a tree of them over a register array is not turned back into an
// indexed access (which would move the array to scratch memory).
__device__ __forceinline__ float bit_blend(uint32_t m, float a, float b) {
  float r;
  asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(r) : "v"(m), "v"(a), "v"(b));
  return r;
}

__device__ __forceinline__ float4 blend4(uint32_t m, const float4& a, const float4& b) {
  return make_float4(bit_blend(m, a.x, b.x), bit_blend(m, a.y, b.y), bit_blend(m, a.z, b.z),
                     bit_blend(m, a.w, b.w));
}

// Element b (= 4 j + q) of the thread's chunk registers, for a per-lane b: a
// blend tree over j, then over q.
__device__ __forceinline__ float pick_logit(const float4 (&v)[AV], int b) {
  static_assert(AV == 16, "the blend tree is written for 16 float4 per thread");
  const uint32_t m0 = 0u - ((b >> 2) & 1u), m1 = 0u - ((b >> 3) & 1u),
                 m2 = 0u - ((b >> 4) & 1u), m3 = 0u - ((b >> 5) & 1u);
  float4 l1[8], l2[4], l3[2];
#pragma unroll
  for (int i = 0; i < 8; ++i) l1[i] = blend4(m0, v[2 * i + 1], v[2 * i]);
#pragma unroll
  for (int i = 0; i < 4; ++i) l2[i] = blend4(m1, l1[2 * i + 1], l1[2 * i]);
#pragma unroll
  for (int i = 0; i < 2; ++i) l3[i] = blend4(m2, l2[2 * i + 1], l2[2 * i]);
  const float4 f = blend4(m3, l3[1], l3[0]);
  const uint32_t q0 = 0u - (b & 1u), q1 = 0u - ((b >> 1) & 1u);
  return bit_blend(q1, bit_blend(q0, f.w, f.z), bit_blend(q0, f.y, f.x));
}

// Smallest 23-bit uniform index m = x >> 9 a token needs so that its key
// x_tok + g(u) can exceed `bar`, given x_tok <= xm: g(u) > bar - x_tok needs
// u > exp(-exp(xm - bar)).  The bound is lowered by a relative 2^-10 and one
// unit, far beyond the error of the hardware exponentials, so no token that
// could exceed the bar is skipped.
__device__ __forceinline__ uint32_t u_floor_bits(float xm, float bar) {
  const float e1 = __builtin_amdgcn_exp2f((xm - bar) * kLog2e);
  const float u0 = __builtin_amdgcn_exp2f(-e1 * kLog2e) * (1.0f - 0.0009765625f);
  const float th = u0 * 8388608.0f - 1.0f;
  return th > 0.0f ? static_cast<uint32_t>(th) : 0u;
}

__device__ __forceinline__ void insert3(float key, int id, float (&k)[3], int (&i)[3]) {
  if (!better(key, id, k[2], i[2])) return;
  if (better(key, id, k[1], i[1])) {
    k[2] = k[1];
    i[2] = i[1];
    if (better(key, id, k[0], i[0])) {
      k[1] = k[0];
      i[1] = i[0];
      k[0] = key;
      i[0] = id;
    } else {
      k[1] = key;
      i[1] = id;
    }
  } else {
    k[2] = key;
    i[2] = id;
  }
}

// ------------------------------------------------------------- Gumbel keys
// Gumbel keys of one chunk of a full-vocabulary or top-p-only row, drawn by
// the chunk pass from the logits in its registers, relative to the chunk
// maximum: x = (l - cmax) / T, key = x + g.  Full rows list the chunk's best
// key (floor: that key); top-p-only rows list every key at or above the
// floor.  Every thread of the workgroup calls it, with sh.nkey zero and
// sh.wsec all -inf.  Returns the number of keys (above kKeyCap: overflow, the
// list is not written).
__device__ __forceinline__ int chunk_keys(const float4 (&v)[AV], float cmax, float inv_t, bool topp,
                                          uint64_t seed, uint64_t grow, int c0,
                                          int* __restrict__ klist_out, ChunkSmem& sh,
                                          float& kfloor) {
  const int tid = threadIdx.x, lane_id = tid & (kWave - 1), wave = tid / kWave;
  kfloor = INFINITY;
  {
    // Full rows keep each thread's best key; the chunk maximum's key is at
    // least the smallest Gumbel value, so no token below that bar needs its
    // noise.  Top-p-only rows keep each thread's best three.  The bar a token
    // must clear is the larger of the thread's own (its best, or its third
    // best) and the wave's, refreshed after five of the sixteen float4s: for
    // full rows the wave's largest best key (a token under it cannot be the
    // chunk's best); for top-p rows a value eight keys of the chunk reach,
    // the larger of two: the smallest of the wave's eight 8-lane group
    // maxima of the best keys, and the smallest of the second-largest group
    // maxima the four waves have posted in LDS (two keys per wave; a stale
    // or missing post is lower, so it still holds).  The top-p key floor
    // below is raised to every wave's bar, so a token skipped under a bar is
    // under the floor and the key list above the floor stays complete; whole
    // waves skip the Gumbel draw once a few good keys are known.
    float kb[3] = {-INFINITY, -INFINITY, -INFINITY};
    int ib[3] = {0x7fffffff, 0x7fffffff, 0x7fffffff};
    float wbar = topp ? -INFINITY : kMinGumbel;
    volatile float* posted = sh.wsec;
#pragma unroll
    for (int j = 0; j < AV; ++j) {
      const int e = 4 * (j * AT + tid);
      float x[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) x[q] = (lane(v[j], q) - cmax) * inv_t;
      const float xm = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
      const float bar = fmaxf(wbar, topp ? kb[2] : kb[0]);
      if (xm + kGumbelMax >= bar) {  // else no key here can clear the bar (or all padding)
        const uint32_t th = u_floor_bits(xm, bar);
        const U32x4 w = token_words(seed, grow, static_cast<uint32_t>(c0 + e) >> 2);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if ((w.v[q] >> 9) < th || x[q] == -INFINITY) continue;
          const float key = x[q] + gumbel_from_word(w.v[q]);
          const int id = c0 + e + q;
          if (topp) {
            insert3(key, id, kb, ib);
          } else if (better(key, id, kb[0], ib[0])) {
            kb[0] = key;
            ib[0] = id;
          }
        }
      }
      // Refreshed early and then less often: the bar rises fastest at first.
      if (j == 0 || j == 1 || j == 3 || j == 7 || j == 11) {
        if (topp) {
          float second;
          const float own = wave_group_floors(kb[0], second);
          if (lane_id == 0) posted[wave] = second;
          float b = posted[0];
#pragma unroll
          for (int w = 1; w < AW; ++w) b = fminf(b, posted[w]);
          wbar = fmaxf(wbar, fmaxf(own, uniform_f32(b)));
        } else {
          wbar = fmaxf(wbar, wave_max_uniform(kb[0]));
        }
      }
    }
    if (!topp) {
      float k1 = kb[0];
      int i1 = ib[0];
      block_best<AT>(k1, i1, sh.rf, sh.ri);
      if (tid == 0 && i1 != 0x7fffffff) {
        klist_out[0] = i1;
        sh.nkey = 1;
      }
      kfloor = k1;
    } else {
      // Floor F >= every thread's third-best key, so the tokens with key >=
      // F all sit in the threads' top-three lists, and F >= every wave's
      // final bar, so no skipped token lies at or above it.  F is also raised
      // to the smallest of the four waves' third-largest best keys to keep
      // the list short (at least twelve entries when that raises it, eight
      // when a wave's bar does).
      const float f0 = block_max<AT>(kb[2], sh.rf);
      const float tw = wave_qth(kb[0], 3);
      if (lane_id == 0) {
        sh.wthr[wave] = tw;
        sh.wbar[wave] = wbar;
      }
      __syncthreads();
      float g = sh.wthr[0], wb = sh.wbar[0];
#pragma unroll
      for (int w = 1; w < AW; ++w) {
        g = fminf(g, sh.wthr[w]);
        wb = fmaxf(wb, sh.wbar[w]);
      }
      kfloor = fmaxf(fmaxf(f0, g), wb);
#pragma unroll
      for (int i = 0; i < 3; ++i) {
        if (ib[i] != 0x7fffffff && kb[i] >= kfloor) {
          const int slot = atomicAdd(&sh.nkey, 1);
          if (slot < kKeyCap) sh.klist[slot] = ib[i];
        }
      }
      __syncthreads();
      if (sh.nkey <= kKeyCap && tid < sh.nkey) klist_out[tid] = sh.klist[tid];
    }
  }
  __syncthreads();
  return sh.nkey;
}

template <bool VEC>
__global__ __launch_bounds__(AT, 4) void chunk_pass_kernel(SamplerArgs a, FastLayout lay,
                                                        uint8_t* __restrict__ ws) {
  __shared__ ChunkSmem sh;
  const int S = lay.S;
  const int bid = blockIdx.x;
  const int r = bid / S, c = bid - r * S;
  const int tid = threadIdx.x, lane_id = tid & (kWave - 1), wave = tid / kWave;
  if (bid == 0 && tid < 2) reinterpret_cast<int*>(ws + lay.off_ctr)[tid] = 0;
  // The chunk's loads go out first, so the parameter read and the row-kind
  // decision overlap them (rows the chunk pass skips waste one chunk read).
  const ChunkGeo geo = chunk_geo(a.lv, lay, r, c);
  const int c0 = geo.gofs;  // global column of the chunk's first logit
  const int n = geo.n;
  float4 v[AV];
  load_chunk<VEC>(v, geo.src, n, tid);
  const ts_row_params p = a.params[r];
  const int V = a.vocab;
  // Row-uniform values in scalar registers, so the per-kind paths below are
  // real branches rather than flattened selects.
  const int kind = __builtin_amdgcn_readfirstlane(row_kind(p, V, a.max_logprobs));
  if (kind == KIND_BAD || kind == KIND_EXACT) return;
  ChunkRec* rec = reinterpret_cast<ChunkRec*>(ws + lay.off_chunk) + bid;
  // The temperature-scaled mass: top-p-only rows, and unfiltered rows when
  // the log-probabilities describe the sampled distribution.
  const bool topp = kind == KIND_TOPP ||
                    ((a.flags & TS_LOGPROBS_PROCESSED) && kind == KIND_FULL);
  const float inv_t = uniform_f32(kind == KIND_GREEDY ? 0.0f : 1.0f / p.temperature);

  // The thread maximum, each float4 taken as soon as it lands (with the
  // thread's four largest values when M > 64); then sum exp(l - max) and, for
  // top-p-only rows, sum exp((l - max) / T) relative to that maximum.  A NaN
  // logit makes the sum NaN; +inf makes it NaN too (inf - inf); a thread
  // holding only -inf and NaN scans for NaN afterwards.
  const int M = __builtin_amdgcn_readfirstlane(chunk_target(cand_target(kind, p, V), S));
  const bool four = M > 64 && M < n;
  float t[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
  float lm = -INFINITY, ls = 0.0f, lt = 0.0f;
  const float sc = inv_t * kLog2e;
  if (four) {
#pragma unroll
    for (int j = 0; j < AV; ++j) {
      const float4 f = v[j];
      lm = fmaxf(lm, fmaxf(fmaxf(f.x, f.y), fmaxf(f.z, f.w)));
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float x = lane(f, q);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float hi = fmaxf(t[i], x);
          x = fminf(t[i], x);
          t[i] = hi;
        }
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < AV; ++j) {
      const float4 f = v[j];
      lm = fmaxf(lm, fmaxf(fmaxf(f.x, f.y), fmaxf(f.z, f.w)));
    }
  }
  if (lm > -INFINITY) {
    // Differences from the maximum first, then the scale: the exponent's
    // rounding error stays proportional to l - m, small where the terms are
    // large (a fused l * c - m * c would round m * c, an error that grows with
    // |m| / T).  The scaled sum forms its difference as (m - l) * -c, the same
    // value but not the same instruction, so the compiler does not keep the
    // first loop's 64 differences alive for the second.
#pragma unroll
    for (int j = 0; j < AV; ++j) {
      const float4 f = v[j];
      ls += fast_exp(f.x - lm) + fast_exp(f.y - lm) + fast_exp(f.z - lm) + fast_exp(f.w - lm);
    }
    if (topp) {
      const float nsc = -sc;
#pragma unroll
      for (int j = 0; j < AV; ++j) {
        const float4 f = v[j];
        lt += __builtin_amdgcn_exp2f((lm - f.x) * nsc) + __builtin_amdgcn_exp2f((lm - f.y) * nsc) +
              __builtin_amdgcn_exp2f((lm - f.z) * nsc) + __builtin_amdgcn_exp2f((lm - f.w) * nsc);
      }
    }
  }
  if (!four) t[0] = lm;
  int flag = lm == INFINITY ? 1 : 0;
  if (lm == -INFINITY) {
#pragma unroll
    for (int j = 0; j < AV; ++j)
      flag |= (isnan(v[j].x) || isnan(v[j].y) || isnan(v[j].z) || isnan(v[j].w)) ? 1 : 0;
  }
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) {
    const float m2 = __shfl_xor(lm, o, kWave), s2 = __shfl_xor(ls, o, kWave),
                t2 = __shfl_xor(lt, o, kWave);
    merge_stats(lm, ls, lt, m2, s2, t2, inv_t);
  }
  flag = __any(flag) ? 1 : 0;
  if (lane_id == 0) {
    sh.rm[wave] = lm;
    sh.rs[wave] = ls;
    sh.rt[wave] = lt;
    sh.rb[wave] = flag;
  }
  if (tid == 0) {
    sh.ncand = 0;
    sh.nkey = 0;
  }
  if (tid < AW) sh.wsec[tid] = -INFINITY;
  // Logit candidate threshold tf: at least M logits of the chunk are >= tf.
  // M <= 64: every wave holds ceil(M/4) per-thread maxima >= its own q-th
  // largest, so the smallest of the four wave values works.  64 < M <= 256:
  // the same over per-thread top-4 values.  M > 256: the M-th largest of the
  // block's 4 * 256 top-4 values, by radix selection in LDS.
  if (M < n && M <= 256) {
    const int q = (M + AW - 1) / AW;
    const float tw = four ? wave_qth4_hi16(t, q) : wave_qth_hi16(t[0], q);
    if (lane_id == 0) sh.wthr[wave] = tw;
  } else if (M < n) {
#pragma unroll
    for (int i = 0; i < 4; ++i) sh.keys4[4 * tid + i] = order_key(t[i]);
  }
  __syncthreads();
  float cmax = sh.rm[0], s = sh.rs[0], tmass = sh.rt[0];
  int bad = sh.rb[0];
#pragma unroll
  for (int w = 1; w < AW; ++w) {
    merge_stats(cmax, s, tmass, sh.rm[w], sh.rs[w], sh.rt[w], inv_t);
    bad |= sh.rb[w];
  }
  if (bad || isnan(s) || cmax == INFINITY) {
    if (tid == 0) rec->status = 1;
    return;
  }
  if (!topp) tmass = 0.0f;
  float tf = -INFINITY;
  if (M < n && M <= 256) {
    tf = sh.wthr[0];
#pragma unroll
    for (int w = 1; w < AW; ++w) tf = fminf(tf, sh.wthr[w]);
  } else if (M < n) {
    const uint32_t kk = lds_kth_largest<AT>(sh.keys4, 4 * AT, static_cast<uint32_t>(M), sh.hist,
                                            sh.ru, &sh.sel_d, &sh.sel_above);
    tf = key_floor_value(kk);
  }

  // Every valid logit >= tf goes to the chunk's candidate list.  Slots come
  // from a block-wide exclusive scan of the per-thread counts, so writing a
  // candidate costs no LDS round trip.
  unsigned long long cm = 0ull;  // bit 4j + q: lane q of v[j] is a candidate
#pragma unroll
  for (int j = 0; j < AV; ++j) {
    const int e = 4 * (j * AT + tid);
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (lane(v[j], q) >= tf && e + q < n) cm |= 1ull << (4 * j + q);
  }
  const int cnt = __popcll(cm);
  int incl = cnt;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int t = __shfl_up(incl, d, kWave);
    if (lane_id >= d) incl += t;
  }
  if (lane_id == kWave - 1) sh.wcnt[wave] = incl;
  __syncthreads();
  int slot = incl - cnt, total = 0;
#pragma unroll
  for (int w = 0; w < AW; ++w) {
    const int c = sh.wcnt[w];
    slot += w < wave ? c : 0;
    total += c;
  }
  unsigned long long* cand = reinterpret_cast<unsigned long long*>(ws + lay.off_cand) +
                             static_cast<size_t>(bid) * lay.cc;
  // One pass per set bit of the thread's mask: the wave loops only as often
  // as its busiest lane has candidates (candidates are sparse).
  while (cm != 0ull) {
    const int b = __builtin_ctzll(cm);
    cm &= cm - 1ull;
    const int e = 4 * ((b >> 2) * AT + tid) + (b & 3);
    if (slot < lay.cc) cand[slot] = pack_cand(order_key(pick_logit(v, b)), c0 + e);
    ++slot;
  }

  // Gumbel keys for the rows that draw them over the whole vocabulary
  // (full-vocabulary rows) or over an unknown nucleus (top-p-only rows).
  const bool ovf = total > lay.cc;
  int nkey = 0;
  float kfloor = INFINITY;
  if ((kind == KIND_FULL || kind == KIND_TOPP) && !ovf) {
    int* klist_out = reinterpret_cast<int*>(ws + lay.off_key) + static_cast<size_t>(bid) * kKeyCap;
    nkey = chunk_keys(v, cmax, inv_t, kind == KIND_TOPP, p.seed,
                      static_cast<uint64_t>(a.row_offset + r), c0, klist_out, sh, kfloor);
  }
  if (tid == 0) {
    const bool key_ovf = nkey > kKeyCap;
    ChunkRec o;
    o.cmax = cmax;
    o.sumexp = s;
    o.tmass = tmass;
    o.kt = order_key(tf);
    o.ncand = ovf ? 0 : total;
    o.status = (ovf || key_ovf) ? 2 : 0;
    o.nkey = key_ovf ? 0 : nkey;
    o.kfloor = kfloor;
#pragma unroll
    for (int i = 0; i < 8; ++i) o.pad[i] = 0;
    *rec = o;
  }
}

// ------------------------------------------------------------------- B: merge
constexpr int kUnionMax = 1 << 20;  // candidates a merge workgroup walks

struct MergeSmem {
  unsigned long long list[kListMax];
  union {
    ChunkRec recs[kMaxChunks];     // read once at the start of the merge
    uint32_t hist[RB];             // radix bins (counts), used afterwards
    unsigned long long mhist[RB];  // radix bins (fixed-point mass)
  };
  int nkey[kMaxChunks];         // the chunks' Gumbel-key list lengths
  int pos[kMaxChunks + 1];
  unsigned long long uscan[BW];
  double dscan[BW];
  unsigned long long sel_above64;
  int sel_found;
  float rf[BW];
  int ri[BW];
  uint32_t ru[BW];
  uint32_t sel_d, sel_above, rmax, sel_cnt;
  int nlist, status, total, nsmall;
  uint32_t skey[BT];             // one radix bin's entries, ranked directly
  unsigned long long smass[BT];
  float m, lse, kmin;
  uint32_t floor_key;
  double z;
};

__device__ __forceinline__ void push_row(int* ctr, int* list, int r) { list[atomicAdd(ctr, 1)] = r; }

// Bitonic sort of n (a power of two, <= kListMax) packed candidates in LDS,
// largest first.  Each thread takes up to kListMax / (2 BT) compare-exchange
// pairs per stage, loads all of them before comparing, so a stage costs one
// LDS round trip and one barrier.
__device__ void lds_bitonic_desc(unsigned long long* s, int n) {
  constexpr int PAIRS = kListMax / (2 * BT);
  const int tid = threadIdx.x, half = n >> 1;
  for (int k = 2; k <= n; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      int lo[PAIRS];
      unsigned long long a[PAIRS], b[PAIRS];
#pragma unroll
      for (int t = 0; t < PAIRS; ++t) {
        const int q = tid + t * BT;
        lo[t] = ((q & ~(j - 1)) << 1) | (q & (j - 1));  // j is a power of two
        if (q < half) {
          a[t] = s[lo[t]];
          b[t] = s[lo[t] + j];
        }
      }
#pragma unroll
      for (int t = 0; t < PAIRS; ++t) {
        const int q = tid + t * BT;
        if (q < half) {
          const bool desc = (lo[t] & k) == 0;
          if (desc ? (a[t] < b[t]) : (a[t] > b[t])) {
            s[lo[t]] = b[t];
            s[lo[t] + j] = a[t];
          }
        }
      }
      __syncthreads();
    }
  }
}


// Largest key offset (key - base) over the entries of sh.list[0, U) with
// key >= base, as a bit count: offsets fit in span_bits bits.
__device__ int list_span_bits(MergeSmem& sh, int U, uint32_t base) {
  const int tid = threadIdx.x;
  uint32_t mx = 0u;
  for (int i = tid; i < U; i += BT) {
    const uint32_t key = cand_key(sh.list[i]);
    if (key >= base) mx = max(mx, key - base);
  }
  if (tid == 0) sh.rmax = 0u;
  __syncthreads();
  atomicMax(&sh.rmax, mx);
  __syncthreads();
  const uint32_t r = sh.rmax;
  __syncthreads();
  return r == 0u ? 0 : 32 - __builtin_clz(r);
}

// High bits (offset >> lowbit) of a key offset; no bits are left above bit 31.
__device__ __forceinline__ uint32_t high_bits(uint32_t off, int lowbit) {
  return lowbit >= 32 ? 0u : (off >> lowbit);
}

// Order key of the k-th largest entry of sh.list[0, U) (1 <= k <= U), every
// key >= base.  Radix selection over the offset key - base with 11-bit digits
// from its top bit down; as soon as the selected bin holds at most BT
// entries, they are gathered and the k-th is found by ranking them directly
// (ties: the key x with #{> x} < k' <= #{>= x} within the bin).
__device__ uint32_t list_kth_key(MergeSmem& sh, int U, int k, uint32_t base) {
  const int tid = threadIdx.x;
  uint32_t prefix = 0u, rem = static_cast<uint32_t>(k), hd = static_cast<uint32_t>(U);
  int lowbit = list_span_bits(sh, U, base);
  while (lowbit > 0 && hd > static_cast<uint32_t>(BT)) {
    const int width = lowbit < 11 ? lowbit : 11;
    const int shift = lowbit - width;
    const uint32_t dmask = (1u << width) - 1u;
    const uint32_t hi = high_bits(prefix, lowbit);
    for (int b = tid; b < RB; b += BT) sh.hist[b] = 0u;
    __syncthreads();
    for (int i = tid; i < U; i += BT) {
      const uint32_t off = cand_key(sh.list[i]) - base;
      if (high_bits(off, lowbit) == hi) atomicAdd(&sh.hist[(off >> shift) & dmask], 1u);
    }
    __syncthreads();
    select_digit_top<BT, RB / BT>(sh.hist, 1 << width, rem, sh.ru, &sh.sel_d, &sh.sel_above);
    const uint32_t d = sh.sel_d;
    rem -= sh.sel_above;
    hd = sh.hist[d];
    __syncthreads();
    prefix |= d << shift;
    lowbit = shift;
  }
  if (lowbit == 0) return base + prefix;
  const uint32_t hi = high_bits(prefix, lowbit);
  if (tid == 0) sh.nsmall = 0;
  __syncthreads();
  for (int i = tid; i < U; i += BT) {
    const uint32_t key = cand_key(sh.list[i]);
    if (high_bits(key - base, lowbit) == hi) sh.skey[atomicAdd(&sh.nsmall, 1)] = key;
  }
  __syncthreads();
  const int ns = sh.nsmall;
  if (tid < ns) {
    const uint32_t x = sh.skey[tid];
    uint32_t gt = 0u, ge = 0u;
    for (int j = 0; j < ns; ++j) {
      const uint32_t y = sh.skey[j];
      gt += y > x ? 1u : 0u;
      ge += y >= x ? 1u : 0u;
    }
    if (gt < rem && rem <= ge) sh.sel_d = x;  // equal keys write the same value
  }
  __syncthreads();
  const uint32_t res = sh.sel_d;
  __syncthreads();
  return res;
}

// Fixed-point (2^-40) temperature-scaled weight exp((l - m) / T) of a listed
// logit, l <= m.
__device__ __forceinline__ unsigned long long list_mass(uint32_t key, float m, float inv_t) {
  return fixed_mass(fast_exp((key_to_float(key) - m) * inv_t));
}

// Top-p boundary among the entries of sh.list[0, U) with key >= kmin: the
// largest key t whose entries at or above it carry mass >= target (fixed
// point), i.e. the key of the first sorted position where the cumulative
// mass reaches the target.  Radix selection with mass-weighted bins over the
// offset key - kmin, from its top bit down (each bin also counts its
// entries, packed above the mass: a bin's mass stays below 2^52); once the
// selected bin holds at most BT entries they are gathered and the boundary
// is found among them directly.  Fixed-point sums are exact, so the result
// does not depend on the order of the additions.  *found = 0 if the
// eligible entries' whole mass stays below the target.
__device__ uint32_t list_mass_key(MergeSmem& sh, int U, uint32_t kmin, float m, float inv_t,
                                  double target, int* found) {
  constexpr int BPT = RB / BT;
  constexpr unsigned long long kCountOne = 1ull << 52;
  constexpr unsigned long long kMassBits = kCountOne - 1ull;
  const int tid = threadIdx.x;
  uint32_t prefix = 0u, hd = static_cast<uint32_t>(U);
  double rem = target;
  int lowbit = list_span_bits(sh, U, kmin);
  bool rounds = false;
  while (lowbit > 0 && hd > static_cast<uint32_t>(BT)) {
    const int width = lowbit < 11 ? lowbit : 11;
    const int shift = lowbit - width;
    const uint32_t dmask = (1u << width) - 1u;
    const int nb = 1 << width;
    const uint32_t hi = high_bits(prefix, lowbit);
    for (int b = tid; b < RB; b += BT) sh.mhist[b] = 0ull;
    if (tid == 0) sh.sel_found = 0;
    __syncthreads();
    for (int i = tid; i < U; i += BT) {
      const uint32_t key = cand_key(sh.list[i]);
      if (key >= kmin && high_bits(key - kmin, lowbit) == hi)
        atomicAdd(&sh.mhist[((key - kmin) >> shift) & dmask],
                  kCountOne + list_mass(key, m, inv_t));
    }
    __syncthreads();
    // Bins from the top digit down, BPT per thread: find d with
    // above(d) < rem <= above(d) + mass(d).
    unsigned long long h[BPT];
    unsigned long long mine = 0ull;
#pragma unroll
    for (int j = 0; j < BPT; ++j) {
      const int b = nb - 1 - (tid * BPT + j);
      h[j] = b >= 0 ? sh.mhist[b] : 0ull;
      mine += h[j] & kMassBits;
    }
    unsigned long long tot;
    unsigned long long ex = block_exclusive_scan<BT, unsigned long long>(mine, sh.uscan, tot);
#pragma unroll
    for (int j = 0; j < BPT; ++j) {
      const int b = nb - 1 - (tid * BPT + j);
      const unsigned long long hm = h[j] & kMassBits;
      if (b >= 0 && static_cast<double>(ex) < rem && rem <= static_cast<double>(ex + hm)) {
        sh.sel_d = static_cast<uint32_t>(b);
        sh.sel_above64 = ex;
        sh.sel_cnt = static_cast<uint32_t>(h[j] >> 52);
        sh.sel_found = 1;
      }
      ex += hm;
    }
    __syncthreads();
    if (!sh.sel_found) {
      *found = 0;
      return 0u;
    }
    const uint32_t d = sh.sel_d;
    rem -= static_cast<double>(sh.sel_above64);
    hd = sh.sel_cnt;
    __syncthreads();
    prefix |= d << shift;
    lowbit = shift;
    rounds = true;
  }
  if (lowbit == 0 && rounds) {
    *found = 1;
    return kmin + prefix;
  }
  if (lowbit == 0) {
    // Every eligible entry has the key kmin (possibly more than BT of them):
    // the boundary is kmin if their whole mass reaches the target.
    unsigned long long mine = 0ull;
    for (int i = tid; i < U; i += BT) {
      const uint32_t key = cand_key(sh.list[i]);
      if (key == kmin) mine += list_mass(key, m, inv_t);
    }
    const unsigned long long tot = block_sum<BT, unsigned long long>(mine, sh.uscan);
    *found = (tot > 0ull && rem <= static_cast<double>(tot)) ? 1 : 0;
    return kmin;
  }
  // Direct search among the (at most BT) eligible entries sharing the
  // selected high bits.
  const uint32_t hi = high_bits(prefix, lowbit);
  if (tid == 0) {
    sh.nsmall = 0;
    sh.sel_found = 0;
  }
  __syncthreads();
  for (int i = tid; i < U; i += BT) {
    const uint32_t key = cand_key(sh.list[i]);
    if (key >= kmin && high_bits(key - kmin, lowbit) == hi) {
      const int slot = atomicAdd(&sh.nsmall, 1);
      sh.skey[slot] = key;
      sh.smass[slot] = list_mass(key, m, inv_t);
    }
  }
  __syncthreads();
  const int ns = sh.nsmall;
  if (tid < ns) {
    const uint32_t x = sh.skey[tid];
    unsigned long long above = 0ull, eq = 0ull;
    for (int j = 0; j < ns; ++j) {
      const uint32_t y = sh.skey[j];
      const unsigned long long w = sh.smass[j];
      above += y > x ? w : 0ull;
      eq += y == x ? w : 0ull;
    }
    if (static_cast<double>(above) < rem && rem <= static_cast<double>(above + eq)) {
      sh.sel_d = x;  // equal keys write the same value
      sh.sel_found = 1;
    }
  }
  __syncthreads();
  const uint32_t res = sh.sel_d;
  *found = sh.sel_found;
  __syncthreads();
  return res;
}


// Keeps the entries of sh.list[0, U) (all with key >= floor_key) that are at
// least the need-th largest, plus whatever shares its radix bin when the list
// is long (at most need + 64 entries, or the power of two the sort pads to,
// unless ties force more), and leaves them
// in sh.list sorted largest first; returns their count.  Radix selection on
// the key offset above the floor, digits from its highest set bit; sorting by
// rank (entries are unique: the low word holds the inverted token id).
__device__ int trim_and_sort(MergeSmem& sh, int U, int need, uint32_t floor_key) {
  const int tid = threadIdx.x;
  int cap = need + 64;
  if (cap > 256) cap = cap <= 1024 ? 1024 : kListMax;  // what the sort pads to anyway
  int C = U;
  if (U > cap) {
    uint32_t rmax = 0u;
    for (int i = tid; i < U; i += BT) rmax = max(rmax, cand_key(sh.list[i]) - floor_key);
    if (tid == 0) sh.rmax = 0u;
    __syncthreads();
    atomicMax(&sh.rmax, rmax);
    __syncthreads();
    rmax = sh.rmax;
    const int hb = rmax == 0u ? -1 : 31 - __builtin_clz(rmax);
    uint32_t prefix = 0u, rem = static_cast<uint32_t>(need), above = 0u;
    int lowbit = hb + 1;
    while (lowbit > 0) {
      const int width = lowbit < 11 ? lowbit : 11;
      const int shift = lowbit - width;
      const uint32_t dmask = (1u << width) - 1u;
      const uint32_t hi_pref = lowbit >= 32 ? 0u : (prefix >> lowbit);
      for (int b = tid; b < RB; b += BT) sh.hist[b] = 0u;
      __syncthreads();
      for (int i = tid; i < U; i += BT) {
        const uint32_t off = cand_key(sh.list[i]) - floor_key;
        if ((lowbit >= 32 ? 0u : (off >> lowbit)) == hi_pref)
          atomicAdd(&sh.hist[(off >> shift) & dmask], 1u);
      }
      __syncthreads();
      select_digit_top<BT, RB / BT>(sh.hist, 1 << width, rem, sh.ru, &sh.sel_d, &sh.sel_above);
      const uint32_t d = sh.sel_d, ab = sh.sel_above, hd = sh.hist[d];
      __syncthreads();
      above += ab;
      rem -= ab;
      prefix |= d << shift;
      lowbit = shift;
      if (above + hd <= static_cast<uint32_t>(cap)) break;
    }
    // Compact the entries >= floor + prefix to the front, in place: every
    // thread reads its entries before any is rewritten.
    const uint32_t fl2 = floor_key + prefix;
    unsigned long long keep[kListMax / BT];
#pragma unroll
    for (int t = 0; t < kListMax / BT; ++t) {
      const int i = tid + t * BT;
      keep[t] = i < U ? sh.list[i] : 0ull;
    }
    if (tid == 0) sh.nlist = 0;
    __syncthreads();
#pragma unroll
    for (int t = 0; t < kListMax / BT; ++t)
      if (keep[t] != 0ull && cand_key(keep[t]) >= fl2) sh.list[atomicAdd(&sh.nlist, 1)] = keep[t];
    __syncthreads();
    C = sh.nlist;
  }
  if (C <= BT) {
    // Rank sort: entry x goes to position #{y > x} (read all, then write).
    const unsigned long long x = tid < C ? sh.list[tid] : 0ull;
    int rank = 0;
    if (tid < C) {
      int j = 0;
      for (; j + 4 <= C; j += 4) {
        rank += (sh.list[j] > x) + (sh.list[j + 1] > x) + (sh.list[j + 2] > x) +
                (sh.list[j + 3] > x);
      }
      for (; j < C; ++j) rank += sh.list[j] > x;
    }
    __syncthreads();
    if (tid < C) sh.list[rank] = x;
    __syncthreads();
    return C;
  }
  int n2 = 1;
  while (n2 < C) n2 <<= 1;
  for (int i = C + tid; i < n2; i += BT) sh.list[i] = 0ull;
  __syncthreads();
  lds_bitonic_desc(sh.list, n2);
  return C;
}

// force: bit 0 sends every top-p-only row through the probe pass (a
// diagnostic route; the result is the same).
__global__ __launch_bounds__(BT) void merge_kernel(SamplerArgs a, FastLayout lay,
                                                   uint8_t* __restrict__ ws, int force) {
  __shared__ MergeSmem sh;
  const int r = blockIdx.x, tid = threadIdx.x, S = lay.S, V = a.vocab;
  const ts_row_params p = a.params[r];
  const int kind = row_kind(p, V, a.max_logprobs);
  const bool proc = (a.flags & TS_LOGPROBS_PROCESSED) != 0;
  int* ctr = reinterpret_cast<int*>(ws + lay.off_ctr);
  int* exact_list = reinterpret_cast<int*>(ws + lay.off_exact);
  int* probe_list = reinterpret_cast<int*>(ws + lay.off_probe);
  if (kind == KIND_BAD) {
    write_bad<BT>(a, r, TS_ROW_BAD_PARAMS);
    return;
  }
  if (kind == KIND_EXACT) {
    if (tid == 0) push_row(&ctr[0], exact_list, r);
    return;
  }
  const ChunkRec* recs = reinterpret_cast<const ChunkRec*>(ws + lay.off_chunk) +
                         static_cast<size_t>(r) * S;
  for (int c = tid; c < S; c += BT) {
    sh.recs[c] = recs[c];
    sh.nkey[c] = recs[c].nkey;
  }
  __syncthreads();
  const float inv_t = kind == KIND_GREEDY ? 0.0f : 1.0f / p.temperature;
  if (tid == 0) {
    int st = 0;
    for (int c = 0; c < S; ++c)
      if (sh.recs[c].status == 1) st = 1;
    if (st == 0)
      for (int c = 0; c < S; ++c)
        if (sh.recs[c].status == 2) st = 2;
    float m = -INFINITY;
    uint32_t fl = 0u;
    int tot = 0;
    if (st != 1) {
      for (int c = 0; c < S; ++c) {
        m = fmaxf(m, sh.recs[c].cmax);
        if (sh.recs[c].kt > fl) fl = sh.recs[c].kt;
        sh.pos[c] = tot;
        tot += sh.recs[c].ncand;
      }
    }
    sh.pos[S] = tot;
    float se = 0.0f;
    double z = 0.0;
    float kmin = -INFINITY;
    if (m > -INFINITY) {
      for (int c = 0; c < S; ++c) {
        if (!(sh.recs[c].cmax > -INFINITY)) continue;
        se += sh.recs[c].sumexp * fast_exp(sh.recs[c].cmax - m);
        if (kind == KIND_TOPP || (proc && kind == KIND_FULL)) {
          const float shift = (sh.recs[c].cmax - m) * inv_t;
          z += static_cast<double>(sh.recs[c].tmass) *
               static_cast<double>(__builtin_amdgcn_exp2f(shift * kLog2e));
          if (kind == KIND_TOPP) kmin = fmaxf(kmin, sh.recs[c].kfloor + shift);
        }
      }
    }
    sh.status = st;
    sh.m = m;
    sh.floor_key = fl;
    sh.total = tot;
    sh.lse = m + logf(se);
    sh.z = z;
    sh.kmin = kmin + kKeyMargin;
    sh.nlist = 0;
    sh.rmax = 0u;
  }
  __syncthreads();
  if (sh.status == 1 || !(sh.m > -INFINITY)) {
    write_bad<BT>(a, r, TS_ROW_BAD_LOGITS);
    return;
  }
  if (sh.status == 2 || sh.total > kUnionMax) {
    if (tid == 0) push_row(&ctr[0], exact_list, r);
    return;
  }
  const float m = sh.m, lse = sh.lse;
  uint32_t floor_key = sh.floor_key;
  const int total = sh.total;

  // The union of the chunks' candidates above the floor holds the row's M
  // largest logits (each chunk listed at least its own M largest).  Passes
  // over it read global memory (L2-resident), four entries in flight per
  // thread.
  const unsigned long long* cand = reinterpret_cast<const unsigned long long*>(ws + lay.off_cand) +
                                   static_cast<size_t>(r) * S * lay.cc;
  auto cand_at = [&](int g) -> unsigned long long {
    int lo = 0, hi = S - 1;  // chunk c with pos[c] <= g < pos[c + 1]
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (sh.pos[mid] <= g) lo = mid; else hi = mid - 1;
    }
    return cand[static_cast<size_t>(lo) * lay.cc + (g - sh.pos[lo])];
  };
  if (total > kListMax) {
    // Raise the floor to the row's M-th largest candidate: radix selection
    // on the key offset above the floor, digits from its highest set bit.
    uint32_t rmax = 0u;
    int mine = 0;
#pragma unroll 4
    for (int g = tid; g < total; g += BT) {
      const uint32_t key = cand_key(cand_at(g));
      if (key >= floor_key) {
        rmax = max(rmax, key - floor_key);
        ++mine;
      }
    }
    atomicMax(&sh.rmax, rmax);
    const int U0 = block_sum<BT, int>(mine, sh.ri);
    rmax = sh.rmax;
    if (U0 > kListMax) {
      const int M = cand_target(kind, p, V);
      const int hb = rmax == 0u ? -1 : 31 - __builtin_clz(rmax);
      uint32_t prefix = 0u, rem = static_cast<uint32_t>(M), above = 0u;
      int lowbit = hb + 1;  // offset bits >= lowbit are resolved
      while (lowbit > 0) {
        const int width = lowbit < 11 ? lowbit : 11;
        const int shift = lowbit - width;
        const uint32_t dmask = (1u << width) - 1u;
        const uint32_t hi_pref = lowbit >= 32 ? 0u : (prefix >> lowbit);
        for (int b = tid; b < RB; b += BT) sh.hist[b] = 0u;
        __syncthreads();
#pragma unroll 4
        for (int g = tid; g < total; g += BT) {
          const uint32_t key = cand_key(cand_at(g));
          if (key < floor_key) continue;
          const uint32_t off = key - floor_key;
          if ((lowbit >= 32 ? 0u : (off >> lowbit)) == hi_pref)
            atomicAdd(&sh.hist[(off >> shift) & dmask], 1u);
        }
        __syncthreads();
        select_digit_top<BT, RB / BT>(sh.hist, 1 << width, rem, sh.ru, &sh.sel_d,
                                      &sh.sel_above);
        const uint32_t d = sh.sel_d, ab = sh.sel_above, hd = sh.hist[d];
        __syncthreads();
        above += ab;
        rem -= ab;
        prefix |= d << shift;
        lowbit = shift;
        if (above + hd <= static_cast<uint32_t>(kListMax)) break;
      }
      floor_key += prefix;
    }
  }
  {
    // Thread t takes g = t, t + BT, ... four at a time (four loads in
    // flight); its chunk index only moves forward, so it walks the chunk
    // offsets instead of searching them.  Slots come one atomic per wave:
    // the wave's count from a ballot, each lane's offset from mbcnt.  The
    // list's order is immaterial (every later step sorts, selects or takes a
    // maximum with id tie-breaks).
    const int lane_id = tid & (kWave - 1);
    int c = 0;
    for (int g0 = tid; g0 < total; g0 += 4 * BT) {
      unsigned long long x[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int g = g0 + u * BT;
        x[u] = 0ull;
        if (g < total) {
          while (sh.pos[c + 1] <= g) ++c;
          x[u] = cand[static_cast<size_t>(c) * lay.cc + (g - sh.pos[c])];
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const bool keep = g0 + u * BT < total && cand_key(x[u]) >= floor_key;
        const unsigned long long bal = __ballot(keep);
        if (bal == 0ull) continue;
        // lane 0 holds the wave's smallest g, so it is active whenever any lane is
        int base = 0;
        if (lane_id == 0) base = atomicAdd(&sh.nlist, __popcll(bal));
        base = __builtin_amdgcn_readfirstlane(base);
        const int slot = base + static_cast<int>(__builtin_amdgcn_mbcnt_hi(
                                    static_cast<uint32_t>(bal >> 32),
                                    __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(bal), 0u)));
        if (keep && slot < kListMax) sh.list[slot] = x[u];
      }
    }
  }
  __syncthreads();
  int U = sh.nlist;
  if (U > kListMax || U < cand_target(kind, p, V)) {
    if (tid == 0) push_row(&ctr[0], exact_list, r);
    return;
  }
  // Most rows use a short prefix of the list: the top N, a top-k set of at
  // most 192, or the 64-entry head of a top-p-only row (its boundary further
  // down goes to the probe pass).  Those lists are trimmed to the prefix and
  // sorted, and the top-p boundary is a prefix sum over them.  Longer top-k
  // sets stay unsorted: the k-th key and the top-p boundary are found by
  // count- and mass-weighted radix selection.
  const int n_eff = p.n_logprobs < V ? p.n_logprobs : V;
  const uint64_t grow = static_cast<uint64_t>(a.row_offset + r);
  int need = n_eff > 1 ? n_eff : 1;
  if (kind == KIND_TOPK && p.top_k > need) need = p.top_k;
  if (kind == KIND_TOPP && need < 64) need = 64;
  bool sorted = need <= 192;
  if (sorted) {
    U = trim_and_sort(sh, U, need < U ? need : U, floor_key);
    sorted = U <= BT;  // long tie runs keep more: those rows take the selection path
  }
  int token = -1;
  bool probe = false;
  // The kept set's smallest key and its temperature-scaled mass (for the
  // processed log-probabilities).
  uint32_t kept_key = 0u;
  double zk = 0.0;
  if (kind == KIND_FULL) {
    zk = sh.z;
    const int* keys = reinterpret_cast<const int*>(ws + lay.off_key) +
                      static_cast<size_t>(r) * S * kKeyCap;
    float gk = -INFINITY;
    int gi = 0x7fffffff;
    for (int c = tid; c < S; c += BT) {
      if (sh.nkey[c] < 1) continue;
      const int id = keys[static_cast<size_t>(c) * kKeyCap];
      const float key = gumbel_key(logit_at(a.lv, r, id), m, inv_t, p.seed, grow, id);
      if (better(key, id, gk, gi)) {
        gk = key;
        gi = id;
      }
    }
    block_best<BT>(gk, gi, sh.rf, sh.ri);
    token = gi;
  } else if (sorted && (kind == KIND_TOPK || kind == KIND_TOPP)) {
    // U <= 256 sorted entries, entry i with thread i.
    const uint32_t kmin = kind == KIND_TOPK ? cand_key(sh.list[p.top_k - 1]) : 0u;
    uint32_t kept = kmin;
    const unsigned long long mine = tid < U ? sh.list[tid] : 0ull;
    if (p.top_p < 1.0f || proc) {
      const double w = (tid < U && cand_key(mine) >= kmin)
                           ? static_cast<double>(fast_exp((key_to_float(cand_key(mine)) - m) * inv_t))
                           : 0.0;
      double total;
      const double ex = block_exclusive_scan<BT, double>(w, sh.dscan, total);
      const double target = static_cast<double>(p.top_p) * (kind == KIND_TOPK ? total : sh.z);
      if (tid == 0) sh.sel_found = 0;
      __syncthreads();
      if (w > 0.0 && ex < target && target <= ex + w) {
        sh.sel_d = cand_key(mine);  // the boundary's key: first cumulative mass >= target
        sh.sel_found = 1;
      }
      __syncthreads();
      if (p.top_p >= 1.0f) {
        // top-k alone: every listed entry at or above the k-th key is kept
      } else if (!sh.sel_found || (kind == KIND_TOPP && (force & 1))) {
        if (kind == KIND_TOPK && !sh.sel_found) {  // cannot happen: the top-k set is all listed
          if (tid == 0) push_row(&ctr[0], exact_list, r);
          return;
        }
        probe = true;
      } else {
        kept = sh.sel_d > kmin ? sh.sel_d : kmin;
      }
      if (proc && !probe) {
        const double wk = (tid < U && cand_key(mine) >= kept) ? w : 0.0;
        zk = block_sum<BT, double>(wk, sh.dscan);
      }
    }
    kept_key = kept;
    if (!probe) {
      float gk = -INFINITY;
      int gi = 0x7fffffff;
      if (tid < U && cand_key(mine) >= kept) {
        gi = cand_id(mine);
        gk = gumbel_key(key_to_float(cand_key(mine)), m, inv_t, p.seed, grow, gi);
      }
      block_best<BT>(gk, gi, sh.rf, sh.ri);
      token = gi;
    }
  } else if (kind == KIND_TOPK || kind == KIND_TOPP) {
    const uint32_t kmin = kind == KIND_TOPK ? list_kth_key(sh, U, p.top_k, floor_key) : 0u;
    uint32_t kept = kmin;
    if (p.top_p < 1.0f) {
      double target;
      if (kind == KIND_TOPK) {
        unsigned long long mine = 0ull;
        for (int i = tid; i < U; i += BT) {
          const uint32_t key = cand_key(sh.list[i]);
          if (key >= kmin) mine += list_mass(key, m, inv_t);
        }
        target = static_cast<double>(p.top_p) *
                 static_cast<double>(block_sum<BT, unsigned long long>(mine, sh.uscan));
      } else {
        target = static_cast<double>(p.top_p) * sh.z * static_cast<double>(kMassScale);
      }
      if (kind == KIND_TOPP && (force & 1)) {
        probe = true;
      } else {
        int found = 0;
        const uint32_t tp = list_mass_key(sh, U, kmin, m, inv_t, target, &found);
        if (!found) {
          if (kind == KIND_TOPK) {  // cannot happen: the top-k set is all listed
            if (tid == 0) push_row(&ctr[0], exact_list, r);
            return;
          }
          probe = true;
        } else {
          kept = tp > kmin ? tp : kmin;
        }
      }
    }
    kept_key = kept;
    if (proc && !probe) {
      unsigned long long mk = 0ull;
      for (int i = tid; i < U; i += BT) {
        const uint32_t key = cand_key(sh.list[i]);
        if (key >= kept) mk += list_mass(key, m, inv_t);
      }
      zk = static_cast<double>(block_sum<BT, unsigned long long>(mk, sh.uscan)) * kMassUnit;
    }
    if (!probe) {
      float gk = -INFINITY;
      int gi = 0x7fffffff;
      for (int i = tid; i < U; i += BT) {
        const unsigned long long e = sh.list[i];
        if (cand_key(e) < kept) continue;
        const int id = cand_id(e);
        const float key = gumbel_key(key_to_float(cand_key(e)), m, inv_t, p.seed, grow, id);
        if (better(key, id, gk, gi)) {
          gk = key;
          gi = id;
        }
      }
      block_best<BT>(gk, gi, sh.rf, sh.ri);
      token = gi;
    }
  }

  // Top-N log-probabilities (and the greedy token): the n_eff largest, sorted.
  if (!sorted && need > 192) {
    const int nt = n_eff > 1 ? n_eff : 1;
    trim_and_sort(sh, U, nt < U ? nt : U, floor_key);
  }
  if (kind == KIND_GREEDY) token = cand_id(sh.list[0]);  // largest logit, lowest id
  if (proc && probe) {  // the kept mass lies beyond the listed logits
    if (tid == 0) push_row(&ctr[0], exact_list, r);
    return;
  }
  // Processed log-probabilities: (l - m) / T - ln(kept mass) inside the kept
  // set, -inf outside it; a greedy row is a point mass on its token.
  const float lzk = (proc && kind != KIND_GREEDY) ? static_cast<float>(log(zk)) : 0.0f;
  const int64_t obase = static_cast<int64_t>(r) * a.max_logprobs;
  for (int j = tid; j < a.max_logprobs; j += BT) {
    if (j < n_eff) {
      const unsigned long long e = sh.list[j];
      const float l = key_to_float(cand_key(e));
      float lp = l - lse;
      if (proc)
        lp = kind == KIND_GREEDY ? (cand_id(e) == token ? 0.0f : -INFINITY)
             : cand_key(e) >= kept_key ? (l - m) * inv_t - lzk : -INFINITY;
      a.topn_ids[obase + j] = cand_id(e);
      a.topn_logprobs[obase + j] = lp;
    } else {
      a.topn_ids[obase + j] = -1;
      a.topn_logprobs[obase + j] = -INFINITY;
    }
  }

  if (probe) {
    // Top-p-only row whose boundary lies below the listed logits: the
    // chunks' key candidates, complete above the highest chunk floor,
    // sorted by row key; the best few become probes.
    const int* keys = reinterpret_cast<const int*>(ws + lay.off_key) +
                      static_cast<size_t>(r) * S * kKeyCap;
    const float kmin = sh.kmin;
    __syncthreads();
    if (tid == 0) sh.nlist = 0;
    __syncthreads();
    const int kspan = S * kKeyCap;
    for (int g = tid; g < kspan; g += BT) {
      const int c = g / kKeyCap, i = g - c * kKeyCap;
      if (i >= sh.nkey[c]) continue;
      const int id = keys[g];
      const float key = gumbel_key(logit_at(a.lv, r, id), m, inv_t, p.seed, grow, id);
      if (key >= kmin) {
        const int slot = atomicAdd(&sh.nlist, 1);
        if (slot < kListMax) sh.list[slot] = pack_cand(order_key(key), id);
      }
    }
    __syncthreads();
    const int nk = sh.nlist;
    if (nk == 0 || nk > kListMax) {
      if (tid == 0) push_row(&ctr[0], exact_list, r);
      return;
    }
    trim_and_sort(sh, nk, nk, 0u);
    if (tid == 0) {
      ProbeRec pr;
      pr.z = sh.z;
      pr.m = m;
      pr.lse = lse;
      pr.inv_t = inv_t;
      pr.npts = nk < kProbes ? nk : kProbes;
      for (int i = 0; i < kProbes; ++i) {
        const int id = i < pr.npts ? cand_id(sh.list[i]) : 0;
        pr.id[i] = id;
        pr.pt[i] = i < pr.npts ? logit_at(a.lv, r, id) : INFINITY;
      }
      reinterpret_cast<ProbeRec*>(ws + lay.off_prec)[r] = pr;
      push_row(&ctr[1], probe_list, r);
    }
    return;
  }
  if (tid == 0) {
    a.token_ids[r] = token;
    if (a.token_logprobs) {
      const float l = logit_at(a.lv, r, token);
      a.token_logprobs[r] = !proc ? l - lse : kind == KIND_GREEDY ? 0.0f : (l - m) * inv_t - lzk;
    }
    if (a.row_status) a.row_status[r] = TS_ROW_OK;
  }
}

// ------------------------------------------------------------------- P: probe
// Mass strictly above each probe logit, per (probe row, chunk).
__global__ __launch_bounds__(PT) void probe_kernel(SamplerArgs a, FastLayout lay,
                                                   uint8_t* __restrict__ ws, int vec) {
  __shared__ double part[kProbes][PW];
  const int S = lay.S;
  const int count = reinterpret_cast<const int*>(ws + lay.off_ctr)[1];
  const int* probe_list = reinterpret_cast<const int*>(ws + lay.off_probe);
  const int tid = threadIdx.x, lane_id = tid & (kWave - 1), wave = tid / kWave;
  for (int w = blockIdx.x; w < count * S; w += gridDim.x) {
    const int li = w / S, c = w - li * S;
    const int r = probe_list[li];
    const ProbeRec pr = reinterpret_cast<const ProbeRec*>(ws + lay.off_prec)[r];
    const ChunkGeo geo = chunk_geo(a.lv, lay, r, c);
    const float* __restrict__ src = geo.src;
    const int n = geo.n;
    const float sc = pr.inv_t * kLog2e;
    float acc[kProbes];
#pragma unroll
    for (int i = 0; i < kProbes; ++i) acc[i] = 0.0f;
    // Four float4 per thread in flight per step (a fourth of the round trips
    // of one at a time); each thread still takes its elements in the order
    // e = 4 tid + 4 PT j, j = 0, 1, ...
    constexpr int U = 4;
    for (int e0 = 4 * tid; e0 < n; e0 += 4 * PT * U) {
      float4 f[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int e = e0 + 4 * PT * u;
        if (vec && e + 3 < n) {
          f[u] = load_stream4(src + e);
        } else {
          f[u].x = e + 0 < n ? load_stream(src + e + 0) : -INFINITY;
          f[u].y = e + 1 < n ? load_stream(src + e + 1) : -INFINITY;
          f[u].z = e + 2 < n ? load_stream(src + e + 2) : -INFINITY;
          f[u].w = e + 3 < n ? load_stream(src + e + 3) : -INFINITY;
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float l = lane(f[u], q);
          const float wt = __builtin_amdgcn_exp2f((l - pr.m) * sc);
#pragma unroll
          for (int i = 0; i < kProbes; ++i) acc[i] += l > pr.pt[i] ? wt : 0.0f;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < kProbes; ++i) {
      const double s = wave_sum(static_cast<double>(acc[i]));
      if (lane_id == 0) part[i][wave] = s;
    }
    __syncthreads();
    if (tid < kProbes) {
      double t = 0.0;
      for (int k = 0; k < PW; ++k) t += part[tid][k];
      reinterpret_cast<double*>(ws + lay.off_part)[(static_cast<size_t>(li) * S + c) * kProbes + tid] = t;
    }
    __syncthreads();
  }
}

// Diagnostic routes (same results): TS_SAMPLER_EXACT=1 samples every row with
// the exact per-row kernel; TS_SAMPLER_FORCE_PROBE=1 sends every top-p-only
// row through the probe pass.
bool env_flag(const char* name) {
  const char* e = getenv(name);
  return e != nullptr && e[0] == '1';
}

}  // namespace

size_t sampler_workspace_size(int64_t rows, const int64_t* slice_cols, int n_slices,
                              int max_logprobs) {
  (void)max_logprobs;
  if (!fast_path_supported(rows, slice_cols, n_slices)) return 256;
  return make_layout(rows, slice_cols, n_slices).total;
}

hipError_t launch_sampler(const SamplerArgs& a, void* workspace, size_t workspace_bytes,
                          hipStream_t stream) {
  (void)workspace_bytes;
  if (a.rows == 0) return hipSuccess;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  int64_t cols[TS_MAX_SLICES];
  for (int s = 0; s < a.lv.n; ++s) cols[s] = a.lv.off[s + 1] - a.lv.off[s];
  if (env_flag("TS_SAMPLER_EXACT") || !fast_path_supported(a.rows, cols, a.lv.n))
    return launch_sampler_finish(a, nullptr, ws, stream);
  const FastLayout lay = make_layout(a.rows, cols, a.lv.n);
  // float4 loads: every slice 16-byte aligned with rows and widths of whole float4s.
  int vec = 1;
  for (int s = 0; s < a.lv.n; ++s) {
    if (cols[s] == 0) continue;
    vec &= (reinterpret_cast<uintptr_t>(a.lv.ptr[s]) % 16 == 0) && (a.lv.ld[s] % 4 == 0) &&
           (cols[s] % 4 == 0);
  }
  const unsigned chunks = static_cast<unsigned>(a.rows) * static_cast<unsigned>(lay.S);
  if (vec)
    hipLaunchKernelGGL(chunk_pass_kernel<true>, dim3(chunks), dim3(AT), 0, stream, a, lay, ws);
  else
    hipLaunchKernelGGL(chunk_pass_kernel<false>, dim3(chunks), dim3(AT), 0, stream, a, lay, ws);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int force = env_flag("TS_SAMPLER_FORCE_PROBE") ? 1 : 0;
  hipLaunchKernelGGL(merge_kernel, dim3(a.rows), dim3(BT), 0, stream, a, lay, ws, force);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const unsigned pgrid = chunks < 2048u ? chunks : 2048u;
  hipLaunchKernelGGL(probe_kernel, dim3(pgrid), dim3(PT), 0, stream, a, lay, ws, vec);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_sampler_finish(a, &lay, ws, stream);
}

}  // namespace ts
