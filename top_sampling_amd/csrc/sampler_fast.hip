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
// O  row order    one workgroup: the order the chunk pass takes the rows in,
//                 rows that draw Gumbel keys over every token first, then
//                 rows with long top-k lists, then the rest (a slow row near
//                 the end of the grid would leave a tail).  Only wide-chunk
//                 calls whose chunk grid takes more than one round of the
//                 GPU launch it.
// A  chunk pass   one 256-thread workgroup per (row, chunk of <= 16384
//                 logits), the chunk held in registers (16 float4 per
//                 thread; 8 in the narrow chunks the one-call assembly +
//                 sampler takes when they stay few, writing each chunk to
//                 the stitched batch buffer as well).  Per chunk:
//                   - max, then sum exp(l - max) and, for top-p-only rows,
//                     sum exp((l - max) / T); lanes and waves are combined by
//                     rescaling to the larger maximum (DPP reductions); a
//                     NaN or +inf shows up as a NaN sum or a flag;
//                   - a logit candidate list holding at least the chunk's
//                     share of the row's M largest, M = max(n_logprobs,
//                     top_k) (64 for top-p-only rows): the threshold is
//                     bounded by the q-th largest per-thread maximum (or
//                     top-4 value) of each wave, found with one ballot per
//                     key bit, or an LDS radix selection for large M;
//                   - for full-vocabulary rows the chunk's best Philox4x32-10
//                     Gumbel key (tokens whose uniform cannot lift them over
//                     the running bar are skipped); for top-p-only rows every
//                     key above a bar set from the chunk's own mass (about 24
//                     on average), the passing tokens queued per wave and
//                     their keys formed together.  Key lists hold the token,
//                     its logit and its Philox word.
// B  merge        one 256-thread workgroup per row: log-sum-exp; the union of
//                 logit candidates above the highest chunk threshold is
//                 exactly the row's logits above it.  Short prefixes (top N,
//                 top-k up to 192, the head of a top-p row) are trimmed and
//                 sorted in LDS; for longer top-k sets the k-th key comes
//                 from radix selection and top-p from the list's best Gumbel
//                 keys checked in key order against the top-k mass (the
//                 mass-weighted boundary search only when none is kept).
//                 Top-N, greedy, top-k, top-p and Gumbel-max are exact on
//                 the list.  A top-p-only row whose boundary lies below the
//                 list takes its best Gumbel keys as probes.
// P  probe        chunk-parallel re-read of probe rows only: the mass of the
//                 logits strictly above each probe's logit.  Token v is kept
//                 by top-p iff that mass is below p times the total, so the
//                 first probe (by key) that is kept is the Gumbel-max winner;
//                 only probes that raise the logit maximum in key order can
//                 be it, and only those are summed.
// X  finish       (sampler_exact.hip) settles probe rows; rows that no fast
//                 route settles (candidate or key overflow, top_k > 2048, no
//                 kept probe) run the exact per-row kernel.
#include <stdlib.h>

#include "sampler_common.hpp"

namespace ts {
namespace {

constexpr int AT = kChunkThreads;
constexpr int AW = AT / kWave;
constexpr int RB = 2048;
constexpr int BT = 256;
constexpr int BW = BT / kWave;
constexpr int kRegList = 2048;  // merge-list entries the register routines take (8 per thread)
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
// Tokens of a top-p-only row whose uniform may lift them over the key bar,
// queued per wave (at most kQueueCap; drained when a float4 step could fill it).
constexpr int kQueueCap = 320;

struct ChunkSmem {
  uint32_t hist[RB];
  uint32_t keys4[4 * AT];  // per-thread top-4 keys (block-level selection)
  KeyRec klist[kKeyCap];
  float wthr[AW];
  float ql[AW][kQueueCap];     // the token's logit
  uint32_t qw[AW][kQueueCap];  // its Philox word
  uint16_t qe[AW][kQueueCap];  // its index in the chunk
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
// all AVW of them are in flight together, as non-temporal (streaming) loads.
// VEC: 16-byte aligned rows and n % 4 == 0.
template <bool VEC, int AVW>
__device__ __forceinline__ void load_chunk(float4 (&v)[AVW], const float* __restrict__ src, int n,
                                           int tid) {
  if (VEC) {
    const int n4 = n >> 2;
#pragma unroll
    for (int j = 0; j < AVW; ++j) {
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
    for (int j = 0; j < AVW; ++j) {
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

// The chunk as load_chunk left it, written to dst (the stitched batch row at
// the chunk's global column): slots past the chunk end are not written.
// VEC4: dst 16-byte aligned and n % 4 == 0 (the chunk starts at a column that
// is a multiple of 4).  Non-temporal stores: nothing reads them back here.
template <int AVW>
__device__ __forceinline__ void store_chunk(const float4 (&v)[AVW], float* __restrict__ dst, int n,
                                            int tid, bool vec4) {
  if (vec4) {
    const int n4 = n >> 2;
#pragma unroll
    for (int j = 0; j < AVW; ++j) {
      const int i4 = j * AT + tid;
      if (i4 < n4) store_stream4(dst + 4 * i4, v[j]);
    }
  } else {
#pragma unroll
    for (int j = 0; j < AVW; ++j) {
      const int e = 4 * (j * AT + tid);
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (e + q < n) __builtin_nontemporal_store(lane(v[j], q), dst + e + q);
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

__device__ __forceinline__ float wave_qth2_hi16(const float (&t)[4], int q) {
  const uint32_t k0 = order_key(t[0]), k1 = order_key(t[1]);
  uint32_t K = 0u;
#pragma unroll
  for (int b = 31; b >= 16; --b) {
    const uint32_t cand = K | (1u << b);
    const int cnt = __popcll(__ballot(k0 >= cand)) + __popcll(__ballot(k1 >= cand));
    if (cnt >= q) K = cand;
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
template <int AVW>
__device__ __forceinline__ float pick_logit(const float4 (&v)[AVW], int b) {
  static_assert(AVW == 16 || AVW == 8, "the blend tree is written for 8 or 16 float4 per thread");
  const uint32_t m0 = 0u - ((b >> 2) & 1u), m1 = 0u - ((b >> 3) & 1u),
                 m2 = 0u - ((b >> 4) & 1u), m3 = 0u - ((b >> 5) & 1u);
  float4 l1[AVW / 2], l2[AVW / 4], l3[AVW / 8];
#pragma unroll
  for (int i = 0; i < AVW / 2; ++i) l1[i] = blend4(m0, v[2 * i + 1], v[2 * i]);
#pragma unroll
  for (int i = 0; i < AVW / 4; ++i) l2[i] = blend4(m1, l1[2 * i + 1], l1[2 * i]);
#pragma unroll
  for (int i = 0; i < AVW / 8; ++i) l3[i] = blend4(m2, l2[2 * i + 1], l2[2 * i]);
  float4 f;
  if constexpr (AVW == 16)
    f = blend4(m3, l3[1], l3[0]);
  else
    f = l3[0];
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

// ------------------------------------------------------------- Gumbel keys
// Best Gumbel key of one chunk of a full-vocabulary row, drawn by the chunk
// pass from the logits in its registers, relative to the chunk maximum:
// x = (l - cmax) / T, key = x + g.  A token needs its noise only if its
// key can clear the bar: the larger of the thread's best key so far and the
// wave's, refreshed after five of the sixteen float4s (the chunk maximum's
// key is at least the smallest Gumbel value, the bar's start).  Every
// thread of the workgroup calls it, with sh.nkey zero.  Returns the number
// of keys listed (1, or 0 for an all-padding chunk); kfloor is the key.
template <int AVW>
__device__ __forceinline__ int chunk_best_key(const float4 (&v)[AVW], float cmax, float inv_t,
                                              uint64_t seed, uint64_t grow, int c0,
                                              KeyRec* __restrict__ klist_out, ChunkSmem& sh,
                                              float& kfloor) {
  const int tid = threadIdx.x;
  float kb = -INFINITY, kl = 0.0f;
  int ib = 0x7fffffff;
  uint32_t kw = 0u;
  float wbar = kMinGumbel;
#pragma unroll
  for (int j = 0; j < AVW; ++j) {
    const int e = 4 * (j * AT + tid);
    float x[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) x[q] = (lane(v[j], q) - cmax) * inv_t;
    const float xm = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    const float bar = fmaxf(wbar, kb);
    if (xm + kGumbelMax >= bar) {  // else no key here can clear the bar (or all padding)
      const uint32_t th = u_floor_bits(xm, bar);
      const U32x4 w = token_words(seed, grow, static_cast<uint32_t>(c0 + e) >> 2);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if ((w.v[q] >> 9) < th || x[q] == -INFINITY) continue;
        const float key = x[q] + gumbel_from_word(w.v[q]);
        const int id = c0 + e + q;
        if (better(key, id, kb, ib)) {
          kb = key;
          ib = id;
          kl = lane(v[j], q);
          kw = w.v[q];
        }
      }
    }
    // Refreshed early and then less often: the bar rises fastest at first.
    if (j == 0 || j == 1 || j == 3 || j == (AVW == 16 ? 7 : 5) || j == 11)
      wbar = fmaxf(wbar, wave_max_uniform(kb));
  }
  const int mine = ib;
  block_best<AT>(kb, ib, sh.rf, sh.ri);
  if (ib != 0x7fffffff) {
    if (mine == ib) klist_out[0] = KeyRec{ib, kl, kw, 0};  // ids are unique: one writer
    if (tid == 0) sh.nkey = 1;
  }
  kfloor = kb;
  __syncthreads();
  return sh.nkey;
}

// Gumbel keys of one chunk of a top-p-only row, relative to the chunk
// maximum as above.  The chunk lists every key at or above the bar
// B = ln(sum of exp x over the chunk) - ln 24.  A token reaches B with
// probability 1 - exp(-exp(x - B)) <= exp(x - B), so at most 24 keys do on
// average; their count is a sum of independent draws, so more than the
// list's 64 has odds below 1e-10 and none at all e^-24 (the merge's floor
// is the highest chunk bar, so the row's union holds about 24 keys or more).
// A token is tested with a floor on its uniform from the largest x of its
// float4; the few that pass are queued per wave in LDS and their keys
// computed together, so a wave runs the two logarithms once per 64 queued
// tokens rather than whenever one lane's token passes.  Every thread of the
// workgroup calls it, with sh.nkey zero.  Returns the number of keys (above
// kKeyCap: overflow, the list is not written); kfloor = B.
template <int AVW>
__device__ __forceinline__ int chunk_keys_topp(const float4 (&v)[AVW], float cmax, float inv_t,
                                               float tmass, uint64_t seed, uint64_t grow, int c0,
                                               KeyRec* __restrict__ klist_out, ChunkSmem& sh,
                                               float& kfloor) {
  const int tid = threadIdx.x, lane_id = tid & (kWave - 1), wave = tid / kWave;
  const float bar = uniform_f32(__builtin_amdgcn_logf(tmass) * kLn2 - kLnKeysPerChunk);
  kfloor = bar;
  float* ql = sh.ql[wave];
  uint32_t* qw = sh.qw[wave];
  uint16_t* qe = sh.qe[wave];
  int qn = 0;  // the wave's queue length (uniform)
  // Lanes read what other lanes wrote: each drain is fenced at wavefront
  // scope before (the writes are seen) and after (later writes cannot
  // overtake the reads).
  auto drain = [&]() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    for (int i = lane_id; i < qn; i += kWave) {
      const float l = ql[i];
      if ((l - cmax) * inv_t + gumbel_from_word(qw[i]) >= bar) {
        const int slot = atomicAdd(&sh.nkey, 1);
        if (slot < kKeyCap) sh.klist[slot] = KeyRec{c0 + qe[i], l, qw[i], 0};
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    qn = 0;
  };
#pragma unroll
  for (int j = 0; j < AVW; ++j) {
    if (qn > kQueueCap - 4 * kWave) drain();
    const int e = 4 * (j * AT + tid);
    float x[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) x[q] = (lane(v[j], q) - cmax) * inv_t;
    const float xm = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    uint32_t wq[4] = {0u, 0u, 0u, 0u};
    bool pass[4] = {false, false, false, false};
    if (xm + kGumbelMax >= bar) {  // else no key here can reach the bar (or all padding)
      const uint32_t th = u_floor_bits(xm, bar);
      const U32x4 w = token_words(seed, grow, static_cast<uint32_t>(c0 + e) >> 2);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        wq[q] = w.v[q];
        pass[q] = (w.v[q] >> 9) >= th && x[q] != -INFINITY;
      }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const unsigned long long bal = __ballot(pass[q]);
      if (bal == 0ull) continue;
      if (pass[q]) {
        const int slot = qn + static_cast<int>(__builtin_amdgcn_mbcnt_hi(
                                  static_cast<uint32_t>(bal >> 32),
                                  __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(bal), 0u)));
        ql[slot] = lane(v[j], q);
        qw[slot] = wq[q];
        qe[slot] = static_cast<uint16_t>(e + q);
      }
      qn += __popcll(bal);
    }
  }
  drain();
  __syncthreads();
  const int nk = sh.nkey;
  if (nk <= kKeyCap && tid < nk) klist_out[tid] = sh.klist[tid];
  return nk;
}

// ------------------------------------------------------------- row order
// The chunk pass's cost per row differs by a factor of three between row
// kinds: rows that draw Gumbel keys over every token (full-vocabulary and
// top-p-only rows) are the slowest, rows with a long top-k list next.  With
// the rows taken in their own order, such rows near the end of the grid
// leave a slow tail; this single workgroup writes the order the chunk pass
// takes them in instead (those classes first, each class in row order).
// It also clears the exact- and probe-row counters of this call.
constexpr int OT = 256;
constexpr unsigned kOneRoundChunks = 1024;  // wide chunk workgroups resident at once (4 per CU x 256)

// The four filter fields of a row's parameters in one 16-byte read (two
// 8-byte loads: rows are 24 bytes apart), issued before any of them is
// tested, so the checks below cost one memory round trip, not four.
__device__ __forceinline__ ts_row_params load_filter_params(const ts_row_params* row) {
  const uint2* q = reinterpret_cast<const uint2*>(row);
  const uint2 x = q[0], y = q[1];
  ts_row_params p;
  p.temperature = __uint_as_float(x.x);
  p.top_k = static_cast<int>(x.y);
  p.top_p = __uint_as_float(y.x);
  p.n_logprobs = static_cast<int>(y.y);
  p.seed = 0;
  return p;
}

__device__ __forceinline__ int chunk_cost_class(const ts_row_params& p, int V, int max_logprobs) {
  const int kind = row_kind(p, V, max_logprobs);
  if (kind == KIND_BAD || kind == KIND_EXACT) return 3;  // the chunk pass skips them
  if (kind == KIND_TOPP || kind == KIND_FULL) return 0;
  return cand_target(kind, p, V) > 256 ? 1 : 2;
}

__global__ __launch_bounds__(OT) void order_rows_kernel(SamplerArgs a, FastLayout lay,
                                                        uint8_t* __restrict__ ws) {
  __shared__ int wsum[OT / kWave][4];
  const int tid = threadIdx.x, lane_id = tid & (kWave - 1), wave = tid / kWave;
  const int rows = static_cast<int>(a.rows);
  if (tid < 2) reinterpret_cast<int*>(ws + lay.off_ctr)[tid] = 0;
  // Thread t takes rows [t * per, (t + 1) * per): counts per class, then a
  // block-wide exclusive scan gives each class's slots in row order.
  const int per = (rows + OT - 1) / OT;
  const int r0 = tid * per, r1 = min(rows, r0 + per);
  // Up to kKeep rows per thread keep their class in registers (one read of
  // the parameters); beyond that the second loop reads them again.
  constexpr int kKeep = 4;
  int cls[kKeep];
  int cnt[4] = {0, 0, 0, 0};
  ts_row_params pk[kKeep];  // all issued before any is tested (rows >= 1)
#pragma unroll
  for (int i = 0; i < kKeep; ++i) pk[i] = load_filter_params(a.params + min(r0 + i, rows - 1));
#pragma unroll
  for (int i = 0; i < kKeep; ++i)
    cls[i] = r0 + i < r1 ? chunk_cost_class(pk[i], a.vocab, a.max_logprobs) : 3;
#pragma unroll
  for (int i = 0; i < kKeep; ++i) {
    if (r0 + i >= r1) break;
    cnt[0] += cls[i] == 0;
    cnt[1] += cls[i] == 1;
    cnt[2] += cls[i] == 2;
    cnt[3] += cls[i] == 3;
  }
  for (int r = r0 + kKeep; r < r1; ++r) {
    const int k = chunk_cost_class(load_filter_params(a.params + r), a.vocab, a.max_logprobs);
    cnt[0] += k == 0;
    cnt[1] += k == 1;
    cnt[2] += k == 2;
    cnt[3] += k == 3;
  }
  int incl[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    incl[k] = wave_inclusive_scan(cnt[k]);
    if (lane_id == kWave - 1) wsum[wave][k] = incl[k];
  }
  __syncthreads();
  int pos[4], base = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    int before = 0, total = 0;
    for (int w = 0; w < OT / kWave; ++w) {
      const int c = wsum[w][k];
      before += w < wave ? c : 0;
      total += c;
    }
    pos[k] = base + before + incl[k] - cnt[k];
    base += total;
  }
  int* order = reinterpret_cast<int*>(ws + lay.off_order);
  for (int r = r0; r < r1; ++r) {
    int k = 3;
#pragma unroll
    for (int i = 0; i < kKeep; ++i)
      if (r == r0 + i) k = cls[i];
    if (r >= r0 + kKeep) k = chunk_cost_class(load_filter_params(a.params + r), a.vocab, a.max_logprobs);
    const int at = k == 0 ? pos[0]++ : (k == 1 ? pos[1]++ : (k == 2 ? pos[2]++ : pos[3]++));
    order[at] = r;
  }
}

template <bool VEC, int AVW>
__global__ __launch_bounds__(AT, AVW == 16 ? 4 : 6) void chunk_pass_kernel(
    SamplerArgs a, FastLayout lay, uint8_t* __restrict__ ws) {
  __shared__ ChunkSmem sh;
  const int S = lay.S;
  // Workgroup -> (row, chunk) through the row order; a chunk's records
  // and lists sit at its own index bid = r * S + c.
  const int wg = blockIdx.x / S, c = blockIdx.x - wg * S;
  const int r = lay.ordered ? __builtin_amdgcn_readfirstlane(
                                  reinterpret_cast<const int*>(ws + lay.off_order)[wg])
                            : wg;
  // Without the pre-pass the first workgroup clears this call's exact- and
  // probe-row counters (the merge, which fills them, starts after this pass).
  if (!lay.ordered && blockIdx.x == 0 && threadIdx.x < 2)
    reinterpret_cast<int*>(ws + lay.off_ctr)[threadIdx.x] = 0;
  const int bid = r * S + c;
  const int tid = threadIdx.x, lane_id = tid & (kWave - 1), wave = tid / kWave;
  // The chunk's loads go out first, so the parameter read and the row-kind
  // decision overlap them (rows the chunk pass skips waste one chunk read).
  const ChunkGeo geo = chunk_geo(a.lv, lay, r, c);
  const int c0 = geo.gofs;  // global column of the chunk's first logit
  const int n = geo.n;
  float4 v[AVW];
  load_chunk<VEC, AVW>(v, geo.src, n, tid);
  const ts_row_params p = a.params[r];
  const int V = a.vocab;
  // Row-uniform values in scalar registers, so the per-kind paths below are
  // real branches rather than flattened selects.
  const int kind = __builtin_amdgcn_readfirstlane(row_kind(p, V, a.max_logprobs));
  // The stitched copy of the received slices, when the call asks for it:
  // every chunk of every row, whatever route the row takes.
  if (a.asm_out != nullptr) {
    float* dst = a.asm_out + static_cast<int64_t>(r) * a.asm_ld + c0;
    store_chunk(v, dst, n, tid, VEC && lay.asm_vec4);
  }
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
  // Per-thread largest values kept for the candidate threshold: the maximum
  // (M <= 64), the two largest (M <= 256) or the four largest (beyond).
  const int tk = (M <= 64 || M >= n) ? 1 : (M <= 256 ? 2 : 4);
  float t[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
  float lm = -INFINITY, ls = 0.0f, lt = 0.0f;
  const float sc = inv_t * kLog2e;
  if (tk == 4) {
#pragma unroll
    for (int j = 0; j < AVW; ++j) {
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
  } else if (tk == 2) {
#pragma unroll
    for (int j = 0; j < AVW; ++j) {
      const float4 f = v[j];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float x = lane(f, q);
        t[1] = fmaxf(t[1], fminf(t[0], x));
        t[0] = fmaxf(t[0], x);
      }
    }
    lm = t[0];
  } else {
#pragma unroll
    for (int j = 0; j < AVW; ++j) {
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
    for (int j = 0; j < AVW; ++j) {
      const float4 f = v[j];
      ls += fast_exp(f.x - lm) + fast_exp(f.y - lm) + fast_exp(f.z - lm) + fast_exp(f.w - lm);
    }
    if (topp) {
      const float nsc = -sc;
#pragma unroll
      for (int j = 0; j < AVW; ++j) {
        const float4 f = v[j];
        lt += __builtin_amdgcn_exp2f((lm - f.x) * nsc) + __builtin_amdgcn_exp2f((lm - f.y) * nsc) +
              __builtin_amdgcn_exp2f((lm - f.z) * nsc) + __builtin_amdgcn_exp2f((lm - f.w) * nsc);
      }
    }
  }
  if (tk == 1) t[0] = lm;
  int flag = lm == INFINITY ? 1 : 0;
  if (lm == -INFINITY) {
#pragma unroll
    for (int j = 0; j < AVW; ++j)
      flag |= (isnan(v[j].x) || isnan(v[j].y) || isnan(v[j].z) || isnan(v[j].w)) ? 1 : 0;
  }
  // The wave's statistics: its maximum by DPP, each lane's sums rescaled to
  // it (a lane's maximum is never NaN: it starts at -inf and fmaxf skips
  // NaN), then DPP sums -- two exponentials per lane instead of four per
  // step of a shuffle butterfly.
  {
    const float wm = wave_max_uniform(lm);
    if (wm > -INFINITY) {
      const bool live = lm > -INFINITY;
      ls = live ? ls * fast_exp(lm - wm) : 0.0f;
      lt = live ? lt * fast_exp((lm - wm) * inv_t) : 0.0f;
    }
    ls = wave_sum(ls);
    lt = wave_sum(lt);
    lm = wm;
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
  // Logit candidate threshold tf: at least M logits of the chunk are >= tf.
  // M <= 64: every wave holds ceil(M/4) per-thread maxima >= its own q-th
  // largest, so the smallest of the four wave values works.  64 < M <= 256:
  // the same over each thread's two largest values.  M > 256: the M-th
  // largest of the block's 4 * 256 top-4 values, by radix selection in LDS.
  if (M < n && M <= 256) {
    const int q = (M + AW - 1) / AW;
    const float tw = tk == 4   ? wave_qth4_hi16(t, q)
                     : tk == 2 ? wave_qth2_hi16(t, q)
                               : wave_qth_hi16(t[0], q);
    if (lane_id == 0) sh.wthr[wave] = tw;
  } else if (M < n && M <= 4 * AT) {
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
  } else if (M < n && M <= 4 * AT) {
    const uint32_t kk = lds_kth_largest<AT>(sh.keys4, 4 * AT, static_cast<uint32_t>(M), sh.hist,
                                            sh.ru, &sh.sel_d, &sh.sel_above);
    tf = key_floor_value(kk);
  }  // a larger target than the block's 4 * AT top-4 values lists the whole chunk

  // Every valid logit >= tf goes to the chunk's candidate list.  Slots come
  // from a block-wide exclusive scan of the per-thread counts, so writing a
  // candidate costs no LDS round trip.
  unsigned long long cm = 0ull;  // bit 4j + q: lane q of v[j] is a candidate
#pragma unroll
  for (int j = 0; j < AVW; ++j) {
    const int e = 4 * (j * AT + tid);
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (lane(v[j], q) >= tf && e + q < n) cm |= 1ull << (4 * j + q);
  }
  const int cnt = __popcll(cm);
  const int incl = wave_inclusive_scan(cnt);
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
    KeyRec* klist_out = reinterpret_cast<KeyRec*>(ws + lay.off_key) + static_cast<size_t>(bid) * kKeyCap;
    const uint64_t grow = static_cast<uint64_t>(a.row_offset + r);
    nkey = kind == KIND_TOPP
               ? chunk_keys_topp(v, cmax, inv_t, tmass, p.seed, grow, c0, klist_out, sh, kfloor)
               : chunk_best_key(v, cmax, inv_t, p.seed, grow, c0, klist_out, sh, kfloor);
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
    struct {                       // a top-k row's in-list probes (no radix round runs then)
      unsigned long long key[kProbes];         // best Gumbel keys, packed with the ids
      uint32_t logit[kProbes];                 // their logits' order keys
      unsigned long long psum[BW][kProbes + 1];  // per-wave mass sums
    } pr;
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
  // The radix-bin union as 4,096 words (kListMax): scratch for per-entry
  // values when no radix round runs.
  __device__ uint32_t* hist4() { return reinterpret_cast<uint32_t*>(mhist); }
};
static_assert(2 * RB >= kListMax, "the radix-bin union holds a word per list entry");
// Three merge workgroups share a CU at this size; 384 bytes more (53,824)
// left room for only two, measured as 6-8 us more per merge call.
static_assert(sizeof(MergeSmem) <= 53440, "three merge workgroups per CU");


__device__ __forceinline__ void push_row(int* ctr, int* list, int r) { list[atomicAdd(ctr, 1)] = r; }

// One compare-exchange stage between entries J apart within a lane's P
// registers (J a compile-time constant, so the registers are never indexed
// at run time).
template <int P, int J>
__device__ __forceinline__ void sort_lane_stage(unsigned long long (&v)[P], int base, int k) {
#pragma unroll
  for (int i = 0; i < P; ++i) {
    if ((i & J) || i + J >= P) continue;
    const unsigned long long a = v[i], b = v[i + J];
    const unsigned long long hi = a > b ? a : b, lo = a > b ? b : a;
    const bool desc = ((base + i) & k) == 0;
    v[i] = desc ? hi : lo;
    v[i + J] = desc ? lo : hi;
  }
}

// Bitonic sort, largest first, of the 256 * P packed candidates in s (LDS;
// P = 2, 4, 8 or 16).  Wave w holds entries w * 64P .. (w + 1) * 64P - 1, lane l
// of it P consecutive ones in registers, so the compare-exchange stages
// between entries of one lane run in registers, those within a wave by lane
// shuffles, and only the few stages that pair entries of different waves go
// through LDS (the power-of-two strides of an all-LDS network crowd a few
// banks).  Every thread of the workgroup calls it.
template <int P>
__device__ void block_sort_desc(unsigned long long* s) {
  constexpr int N = BT * P;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), w = tid / kWave;
  const int base = w * kWave * P + lane * P;
  unsigned long long v[P];
#pragma unroll
  for (int i = 0; i < P; ++i) v[i] = s[base + i];
  for (int k = 2; k <= N; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      if (j >= kWave * P) {
        __syncthreads();
#pragma unroll
        for (int i = 0; i < P; ++i) s[base + i] = v[i];
        __syncthreads();
#pragma unroll
        for (int i = 0; i < P; ++i) {
          const int x = base + i;
          const unsigned long long y = s[x ^ j];
          const bool keep_max = ((x & k) == 0) == ((x & j) == 0);
          v[i] = keep_max ? (v[i] > y ? v[i] : y) : (v[i] < y ? v[i] : y);
        }
      } else if (j >= P) {
        const int lm = j / P;
#pragma unroll
        for (int i = 0; i < P; ++i) {
          const int x = base + i;
          const unsigned long long y = shfl_xor_u64(v[i], lm);
          const bool keep_max = ((x & k) == 0) == ((x & j) == 0);
          v[i] = keep_max ? (v[i] > y ? v[i] : y) : (v[i] < y ? v[i] : y);
        }
      } else if (j == 8) {
        sort_lane_stage<P, 8>(v, base, k);
      } else if (j == 4) {
        sort_lane_stage<P, 4>(v, base, k);
      } else if (j == 2) {
        sort_lane_stage<P, 2>(v, base, k);
      } else {
        sort_lane_stage<P, 1>(v, base, k);
      }
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < P; ++i) s[base + i] = v[i];
  __syncthreads();
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

// Radix descent over the offsets key - base of the entries of sh.list[0, U)
// (every key >= base), 10-bit digits from the offsets' top bit down: each
// round keeps the digit whose bin holds the rem-th largest of the entries
// that share the digits kept so far.  Three barriers per round: the next
// round's bins are cleared while this round's fill (two buffers), the wave
// totals and the kept digit alternate between two buffers too, and the
// scan runs by DPP.  It stops when the kept bin holds at most `cap` entries
// (with the entries above it when WITH_ABOVE) or no bits are left; on
// return prefix holds the kept digits above bit `lowbit`, rem the rank
// left within the kept bin, above the entries above it and hd its count.
// Uses the radix-bin union; every thread of the block calls it.
template <bool WITH_ABOVE>
__device__ void radix_descend(MergeSmem& sh, int U, uint32_t base, uint32_t cap, int& lowbit,
                              uint32_t& prefix, uint32_t& rem, uint32_t& above, uint32_t& hd) {
  constexpr int NB = 1024;         // bins per round (10-bit digits)
  constexpr int BPT = NB / BT;     // bins per thread
  const int tid = threadIdx.x, lane = tid & (kWave - 1), w = tid / kWave;
  uint32_t* bins = sh.hist4();     // [2][NB] bins, then the posts below
  uint32_t* wpost = bins + 2 * NB;           // [BW] wave maxima
  uint32_t* wtot = wpost + BW;               // [2][BW] wave totals
  uint32_t* sel = wtot + 2 * BW;             // [2][4] digit, count above, count in bin
  static_assert(2 * NB + 3 * BW + 8 <= 2 * RB, "bins and posts fit the radix-bin union");
  // The span of the offsets (a DPP wave maximum, one post per wave), with
  // the first round's bins cleared in the same phase.
  uint32_t mx = 0u;
  for (int i = tid; i < U; i += BT) {
    const uint32_t key = cand_key(sh.list[i]);
    if (key >= base) mx = max(mx, key - base);
  }
  mx = static_cast<uint32_t>(wave_max_u64_uniform(mx));
  for (int b = tid; b < NB; b += BT) bins[b] = 0u;
  if (lane == 0) wpost[w] = mx;
  __syncthreads();
#pragma unroll
  for (int x = 0; x < BW; ++x) mx = max(mx, wpost[x]);
  prefix = 0u;
  above = 0u;
  hd = static_cast<uint32_t>(U);
  lowbit = mx == 0u ? 0 : 32 - __builtin_clz(mx);
  int buf = 0;
  while (lowbit > 0 && (WITH_ABOVE ? above + hd : hd) > cap) {
    const int width = lowbit < 10 ? lowbit : 10;
    const int shift = lowbit - width;
    const uint32_t dmask = (1u << width) - 1u;
    const int nb = 1 << width;
    const uint32_t hi = high_bits(prefix, lowbit);
    uint32_t* h = bins + buf * NB;
    uint32_t* hn = bins + (buf ^ 1) * NB;
    for (int i = tid; i < U; i += BT) {
      const uint32_t key = cand_key(sh.list[i]);
      if (key < base) continue;
      const uint32_t off = key - base;
      if (high_bits(off, lowbit) == hi) atomicAdd(&h[(off >> shift) & dmask], 1u);
    }
    for (int b = tid; b < NB; b += BT) hn[b] = 0u;  // the next round's bins
    __syncthreads();
    // Bins from the top digit down, BPT per thread: the digit d with
    // above(d) < rem <= above(d) + count(d).
    uint32_t hc[BPT], sum = 0u;
#pragma unroll
    for (int j = 0; j < BPT; ++j) {
      const int b = nb - 1 - (tid * BPT + j);
      hc[j] = b >= 0 ? h[b] : 0u;
      sum += hc[j];
    }
    const uint32_t inc = wave_inclusive_scan(sum);
    if (lane == kWave - 1) wtot[buf * BW + w] = inc;
    __syncthreads();
    uint32_t ex = inc - sum;
#pragma unroll
    for (int x = 0; x < BW; ++x) ex += x < w ? wtot[buf * BW + x] : 0u;
#pragma unroll
    for (int j = 0; j < BPT; ++j) {
      const int b = nb - 1 - (tid * BPT + j);
      if (b >= 0 && ex < rem && rem <= ex + hc[j]) {
        sel[buf * 4 + 0] = static_cast<uint32_t>(b);
        sel[buf * 4 + 1] = ex;
        sel[buf * 4 + 2] = hc[j];
      }
      ex += hc[j];
    }
    __syncthreads();
    const uint32_t ab = sel[buf * 4 + 1];
    prefix |= sel[buf * 4 + 0] << shift;
    rem -= ab;
    above += ab;
    hd = sel[buf * 4 + 2];
    lowbit = shift;
    buf ^= 1;
  }
  __syncthreads();  // the posts are reused by the caller
}

// Order key of the k-th largest entry of sh.list[0, U) (1 <= k <= U), every
// key >= base: radix descent until the kept bin holds at most BT entries,
// which are then gathered and ranked directly (ties: the key x with
// #{> x} < k' <= #{>= x} within the bin).
__device__ uint32_t list_kth_key(MergeSmem& sh, int U, int k, uint32_t base) {
  const int tid = threadIdx.x;
  int lowbit;
  uint32_t prefix, rem = static_cast<uint32_t>(k), above, hd;
  radix_descend<false>(sh, U, base, static_cast<uint32_t>(BT), lowbit, prefix, rem, above, hd);
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


// The n (1 <= n <= 64) largest of the nonzero 64-bit values the threads hold
// in registers (P per thread, 0 for none, all distinct), largest first, into
// out[0, ...), with each one's 32-bit payload into out_pay when PAY.  A lower
// bound of the n-th largest comes from the waves: each has ceil(n / 4)
// threads whose largest value reaches its own bound (built on the top 16 bits
// of the high word, one ballot per bit), so at least n values reach the
// smallest of the four bounds.  The values at or above it are gathered and
// ranked directly.  Returns the number written, min(n, #values), or -1 when
// more than BT values reach the bound (nothing written: the caller takes
// another route).  A few thousand cycles where rounds of a block maximum
// cost about 1,600 each.  Scratch: sh.smass, sh.skey, sh.ru, sh.nsmall.
// Every thread of the block calls it; out may be sh.list, since the values
// are in registers by then.
template <int P, bool PAY>
__device__ int top_n_regs(const unsigned long long (&v)[P], const uint32_t (&pay)[P], int n,
                          unsigned long long* out, uint32_t* out_pay, MergeSmem& sh) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), w = tid / kWave;
  unsigned long long mx = 0ull;
#pragma unroll
  for (int q = 0; q < P; ++q) mx = v[q] > mx ? v[q] : mx;
  const int qn = (n + BW - 1) / BW;
  const uint32_t mh = static_cast<uint32_t>(mx >> 32);
  uint32_t K = 0u;
#pragma unroll
  for (int b = 31; b >= 16; --b) {
    const uint32_t cand = K | (1u << b);
    if (__popcll(__ballot(mh >= cand)) >= qn) K = cand;
  }
  if (lane == 0) sh.ru[w] = K;
  if (tid == 0) sh.nsmall = 0;
  __syncthreads();
  uint32_t t = sh.ru[0];
#pragma unroll
  for (int j = 1; j < BW; ++j) t = min(t, sh.ru[j]);
  const unsigned long long tb = static_cast<unsigned long long>(t) << 32;
  // Gathered with one atomic per wave: the wave's count from ballots, each
  // lane's offset from the earlier ballots' counts and mbcnt (every lane is
  // active here).
  unsigned long long bal[P];
  int wn = 0;
#pragma unroll
  for (int q = 0; q < P; ++q) {
    bal[q] = __ballot(v[q] != 0ull && v[q] >= tb);
    wn += __popcll(bal[q]);
  }
  int base = 0;
  if (wn > 0) {
    if (lane == 0) base = atomicAdd(&sh.nsmall, wn);
    base = __builtin_amdgcn_readfirstlane(base);
  }
#pragma unroll
  for (int q = 0; q < P; ++q) {
    if (bal[q] == 0ull) continue;
    const int slot = base + static_cast<int>(__builtin_amdgcn_mbcnt_hi(
                                static_cast<uint32_t>(bal[q] >> 32),
                                __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(bal[q]), 0u)));
    if (((bal[q] >> lane) & 1ull) && slot < BT) {
      sh.smass[slot] = v[q];
      if (PAY) sh.skey[slot] = pay[q];
    }
    base += __popcll(bal[q]);
  }
  __syncthreads();
  const int C = sh.nsmall;
  if (C > BT) {
    __syncthreads();
    return -1;
  }
  const int nn = n < C ? n : C;
  if (tid < C) {
    const unsigned long long x = sh.smass[tid];
    int rank = 0;
    for (int j = 0; j < C; ++j) rank += sh.smass[j] > x ? 1 : 0;
    if (rank < nn) {
      out[rank] = x;
      if (PAY) out_pay[rank] = sh.skey[tid];
    }
  }
  __syncthreads();
  return nn;
}

// Top-p over a long top-k list without locating the boundary.  The list's
// best few Gumbel keys over the entries at or above the k-th key (kmin) are
// taken in key order; token v is kept iff the entries with a larger logit
// carry less than p times the top-k mass, which is exactly the set the
// boundary search keeps (its boundary is the largest key whose entries at
// or above it reach that mass).  The first kept one is therefore the
// Gumbel-max winner over the kept set.  Masses in the same 2^-40 fixed point
// and compared in the same double arithmetic as the boundary search, so the
// decision is the same.  Returns the winner's id, or -1 when none of the
// probes is kept or the list is longer than kRegList (then the caller
// searches the boundary).

__device__ int topk_probe_winner(MergeSmem& sh, int U, uint32_t kmin, float m, float inv_t,
                                 float top_p, uint64_t seed, uint64_t grow) {
  constexpr int P = kRegList / BT;
  if (U > kRegList) return -1;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), w = tid / kWave;
  unsigned long long gk[P], wm[P];
  uint32_t lk[P];
  unsigned long long tot = 0ull;
#pragma unroll
  for (int q = 0; q < P; ++q) {
    gk[q] = 0ull;
    wm[q] = 0ull;
    lk[q] = 0u;
    const int i = tid + q * BT;
    if (q * BT < U && i < U) {
      const unsigned long long e = sh.list[i];
      const uint32_t key = cand_key(e);
      if (key >= kmin) {
        const int id = cand_id(e);
        gk[q] = pack_cand(order_key(gumbel_key(key_to_float(key), m, inv_t, seed, grow, id)), id);
        lk[q] = key;
        wm[q] = list_mass(key, m, inv_t);
        tot += wm[q];
      }
    }
  }
  const int np = top_n_regs<P, true>(gk, lk, kProbes, sh.pr.key, sh.pr.logit, sh);
  if (np <= 0) return -1;
  // Only a probe whose logit exceeds every earlier probe's can be the first
  // kept one (a probe at or below an earlier, unkept one's logit has at
  // least its mass above it): usually two or three of the eight.
  uint32_t pl[kProbes];
  uint32_t rec = 0u, hi = 0u;
#pragma unroll
  for (int j = 0; j < kProbes; ++j) {
    pl[j] = __builtin_amdgcn_readfirstlane(j < np ? sh.pr.logit[j] : 0xffffffffu);
    if (j < np && (j == 0 || pl[j] > hi)) {
      rec |= 1u << j;
      hi = pl[j];
    }
  }
  rec = __builtin_amdgcn_readfirstlane(rec);  // the same in every lane: scalar branches below
  unsigned long long acc[kProbes];
#pragma unroll
  for (int j = 0; j < kProbes; ++j) acc[j] = 0ull;
#pragma unroll
  for (int q = 0; q < P; ++q) {
    if (q * BT >= U) continue;
#pragma unroll
    for (int j = 0; j < kProbes; ++j)
      if ((rec >> j) & 1u) acc[j] += lk[q] > pl[j] ? wm[q] : 0ull;
  }
#pragma unroll
  for (int j = 0; j < kProbes; ++j)
    if ((rec >> j) & 1u) acc[j] = wave_sum_u64_uniform(acc[j]);
  tot = wave_sum_u64_uniform(tot);
  if (lane == 0) {
#pragma unroll
    for (int j = 0; j < kProbes; ++j) sh.pr.psum[w][j] = acc[j];
    sh.pr.psum[w][kProbes] = tot;
  }
  __syncthreads();
  unsigned long long all = 0ull;
#pragma unroll
  for (int x = 0; x < BW; ++x) all += sh.pr.psum[x][kProbes];
  const double target = static_cast<double>(top_p) * static_cast<double>(all);
  int id = -1;
  for (int j = 0; j < np; ++j) {
    if (!((rec >> j) & 1u)) continue;
    unsigned long long a = 0ull;
#pragma unroll
    for (int x = 0; x < BW; ++x) a += sh.pr.psum[x][j];
    if (static_cast<double>(a) < target) {
      id = cand_id(sh.pr.key[j]);
      break;
    }
  }
  __syncthreads();
  return id;
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
  if (cap > 256) cap = cap <= 1024 ? 1024 : 2048;  // what the sort pads to anyway
  int C = U;
  if (U > cap && U > BT) {  // up to one entry per thread is ranked directly instead
    int lowbit;
    uint32_t prefix, rem = static_cast<uint32_t>(need), above, hd;
    radix_descend<true>(sh, U, floor_key, static_cast<uint32_t>(cap), lowbit, prefix, rem, above,
                        hd);
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
    // Rank sort: entry x goes to position #{y > x} (read all, then write);
    // eight entries per step in flight, two per 16-byte read.
    typedef unsigned long long u64x2 __attribute__((ext_vector_type(2)));
    const unsigned long long x = tid < C ? sh.list[tid] : 0ull;
    int rank = 0;
    if (tid < C) {
      const u64x2* l2 = reinterpret_cast<const u64x2*>(sh.list);
      int j = 0;
      for (; j + 8 <= C; j += 8) {
        const u64x2 a = l2[j / 2], b = l2[j / 2 + 1], c = l2[j / 2 + 2], d = l2[j / 2 + 3];
        rank += (a.x > x) + (a.y > x) + (b.x > x) + (b.y > x) + (c.x > x) + (c.y > x) +
                (d.x > x) + (d.y > x);
      }
      for (; j < C; ++j) rank += sh.list[j] > x;
    }
    __syncthreads();
    if (tid < C) sh.list[rank] = x;
    __syncthreads();
    return C;
  }
  int n2 = 2 * BT;
  while (n2 < C) n2 <<= 1;
  for (int i = C + tid; i < n2; i += BT) sh.list[i] = 0ull;
  __syncthreads();
  if (n2 == 2 * BT) block_sort_desc<2>(sh.list);
  else if (n2 == 4 * BT) block_sort_desc<4>(sh.list);
  else if (n2 == 8 * BT) block_sort_desc<8>(sh.list);
  else block_sort_desc<16>(sh.list);  // long tie runs only
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
  if (S <= kWave) {
    // One chunk per lane of the first wave: the row's statistics by wave
    // reductions rather than a walk over the records by one thread.
    if (tid < kWave) {
      const bool has = tid < S;
      const ChunkRec& rc = sh.recs[has ? tid : 0];
      const int status = has ? rc.status : 0;
      const int st = __any(status == 1) ? 1 : (__any(status == 2) ? 2 : 0);
      const float cm = has ? rc.cmax : -INFINITY;
      float m = -INFINITY;
      uint32_t fl = 0u;
      int tot = 0;
      if (st != 1) {
        m = wave_max(cm);
        fl = has ? rc.kt : 0u;
#pragma unroll
        for (int o = kWave / 2; o > 0; o >>= 1) fl = max(fl, static_cast<uint32_t>(__shfl_xor(static_cast<int>(fl), o, kWave)));
        const int nc = has ? rc.ncand : 0;
        const int inc = wave_inclusive_scan(nc);
        if (has) sh.pos[tid] = inc - nc;
        tot = __shfl(inc, kWave - 1, kWave);
      }
      float se = 0.0f, kf = -INFINITY;
      double z = 0.0;
      if (m > -INFINITY && has && cm > -INFINITY) {
        se = rc.sumexp * fast_exp(cm - m);
        if (kind == KIND_TOPP || (proc && kind == KIND_FULL)) {
          const float shift = (cm - m) * inv_t;
          z = static_cast<double>(rc.tmass) * static_cast<double>(__builtin_amdgcn_exp2f(shift * kLog2e));
          if (kind == KIND_TOPP) kf = rc.kfloor + shift;
        }
      }
      se = wave_sum(se);
      z = wave_sum(z);
      kf = wave_max(kf);
      if (tid == 0) {
        sh.status = st;
        sh.m = m;
        sh.floor_key = fl;
        sh.total = tot;
        sh.pos[S] = tot;
        sh.lse = m + logf(se);
        sh.z = z;
        sh.kmin = kf + kKeyMargin;
        sh.nlist = 0;
        sh.rmax = 0u;
      }
    }
    __syncthreads();
  } else {
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
  }
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
    // Thread t takes g = t, t + BT, ... eight at a time (eight loads in
    // flight: a long top-k row's union, one to three thousand entries, in
    // one round trip); its chunk index only moves forward, so it walks the chunk
    // offsets instead of searching them.  Slots come one atomic per wave:
    // the wave's count from a ballot, each lane's offset from mbcnt.  The
    // list's order is immaterial (every later step sorts, selects or takes a
    // maximum with id tie-breaks).
    const int lane_id = tid & (kWave - 1);
    int c = 0;
    constexpr int kGather = 8;
    for (int g0 = tid; g0 < total; g0 += kGather * BT) {
      unsigned long long x[kGather];
#pragma unroll
      for (int u = 0; u < kGather; ++u) {
        const int g = g0 + u * BT;
        x[u] = 0ull;
        if (g < total) {
          while (sh.pos[c + 1] <= g) ++c;
          x[u] = cand[static_cast<size_t>(c) * lay.cc + (g - sh.pos[c])];
        }
      }
      // One atomic per wave per round: the wave's count from the ballots,
      // each lane's offset from the earlier ballots' counts and mbcnt (lane
      // 0 holds the wave's smallest g, so it is active whenever any lane is).
      unsigned long long bal[kGather];
      int wn = 0;
#pragma unroll
      for (int u = 0; u < kGather; ++u) {
        bal[u] = __ballot(g0 + u * BT < total && cand_key(x[u]) >= floor_key);
        wn += __popcll(bal[u]);
      }
      if (wn == 0) continue;
      int base = 0;
      if (lane_id == 0) base = atomicAdd(&sh.nlist, wn);
      base = __builtin_amdgcn_readfirstlane(base);
#pragma unroll
      for (int u = 0; u < kGather; ++u) {
        if (bal[u] == 0ull) continue;
        const int slot = base + static_cast<int>(__builtin_amdgcn_mbcnt_hi(
                                    static_cast<uint32_t>(bal[u] >> 32),
                                    __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(bal[u]), 0u)));
        if (((bal[u] >> lane_id) & 1ull) && slot < kListMax) sh.list[slot] = x[u];
        base += __popcll(bal[u]);
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
  // Most rows use a short prefix of the list: the top N, a top-k set of at
  // most 192, or the 64-entry head of a top-p-only row (its boundary further
  // down goes to the probe pass).  Those lists are trimmed to the prefix and
  // sorted, and the top-p boundary is a prefix sum over them.  Longer top-k
  // sets stay unsorted: the k-th key and the top-p boundary are found by
  // count- and mass-weighted radix selection (sorting a list of a few
  // thousand entries in one workgroup costs several times more).
  // A top-p-only row whose listed logits carry less than p times the row's
  // mass has its boundary below the list: it goes to the probe pass without
  // sorting its head (only its top N are needed here).
  bool early_probe = false;
  if (kind == KIND_TOPP && need <= 192) {
    double wsum = 0.0;
    for (int i = tid; i < U; i += BT)
      wsum += static_cast<double>(fast_exp((key_to_float(cand_key(sh.list[i])) - m) * inv_t));
    const double wlist = block_sum<BT, double>(wsum, sh.dscan);
    early_probe = (force & 1) || wlist < static_cast<double>(p.top_p) * sh.z;
  }
  bool sorted = need <= 192 && !early_probe;
  if (sorted) {
    U = trim_and_sort(sh, U, need < U ? need : U, floor_key);
    sorted = U <= BT;  // long tie runs keep more: those rows take the selection path
  }
  int token = -1;
  bool probe = early_probe;
  // The kept set's smallest key and its temperature-scaled mass (for the
  // processed log-probabilities).
  uint32_t kept_key = 0u;
  double zk = 0.0;
  if (kind == KIND_FULL) {
    zk = sh.z;
    const KeyRec* keys = reinterpret_cast<const KeyRec*>(ws + lay.off_key) +
                         static_cast<size_t>(r) * S * kKeyCap;
    float gk = -INFINITY;
    int gi = 0x7fffffff;
    for (int c = tid; c < S; c += BT) {
      if (sh.nkey[c] < 1) continue;
      const KeyRec k = keys[static_cast<size_t>(c) * kKeyCap];
      const int id = k.id;
      const float key = key_of(k, m, inv_t);
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
  } else if (!early_probe && (kind == KIND_TOPK || kind == KIND_TOPP)) {
    const uint32_t kmin = kind == KIND_TOPK ? list_kth_key(sh, U, p.top_k, floor_key) : 0u;
    uint32_t kept = kmin;
    // Top-k with top-p, plain log-probabilities: the list's best Gumbel keys
    // settle most rows without the boundary search.
    if (kind == KIND_TOPK && p.top_p < 1.0f && !proc)
      token = topk_probe_winner(sh, U, kmin, m, inv_t, p.top_p, p.seed, grow);
    if (token < 0 && p.top_p < 1.0f) {
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
    if (proc && !probe) {  // (no probe winner: proc rows never take that route)
      unsigned long long mk = 0ull;
      for (int i = tid; i < U; i += BT) {
        const uint32_t key = cand_key(sh.list[i]);
        if (key >= kept) mk += list_mass(key, m, inv_t);
      }
      zk = static_cast<double>(block_sum<BT, unsigned long long>(mk, sh.uscan)) * kMassUnit;
    }
    if (!probe && token < 0) {
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
  if (!sorted && (need > 192 || early_probe)) {
    const int nt = n_eff > 1 ? n_eff : 1;
    int got = -1;
    if (nt <= 64 && U <= kRegList) {
      constexpr int kPer = kRegList / BT;
      unsigned long long mine[kPer];
      uint32_t none[kPer];
#pragma unroll
      for (int q = 0; q < kPer; ++q) {
        mine[q] = tid + q * BT < U ? sh.list[tid + q * BT] : 0ull;
        none[q] = 0u;
      }
      got = top_n_regs<kPer, false>(mine, none, nt, sh.list, nullptr, sh);
    }
    if (got < 0) trim_and_sort(sh, U, nt < U ? nt : U, floor_key);
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
    const KeyRec* keys = reinterpret_cast<const KeyRec*>(ws + lay.off_key) +
                         static_cast<size_t>(r) * S * kKeyCap;
    const float kmin = sh.kmin;
    // The listed keys' logits ride along in the radix-bin space (free here).
    uint32_t* klog = sh.hist4();
    __syncthreads();
    if (tid == 0) sh.nlist = 0;
    __syncthreads();
    const int kspan = S * kKeyCap;
    for (int g = tid; g < kspan; g += BT) {
      const int c = g / kKeyCap, i = g - c * kKeyCap;
      if (i >= sh.nkey[c]) continue;
      const KeyRec k = keys[g];
      const float key = key_of(k, m, inv_t);
      if (key >= kmin) {
        const int slot = atomicAdd(&sh.nlist, 1);
        if (slot < kListMax) {
          sh.list[slot] = pack_cand(order_key(key), k.id);
          klog[slot] = __float_as_uint(k.logit);
        }
      }
    }
    __syncthreads();
    const int nk = sh.nlist;
    if (nk == 0 || nk > kListMax) {
      if (tid == 0) push_row(&ctr[0], exact_list, r);
      return;
    }
    int got = -1;
    if (nk <= kRegList) {
      constexpr int kPer = kRegList / BT;
      unsigned long long mine[kPer];
      uint32_t lg[kPer];
#pragma unroll
      for (int q = 0; q < kPer; ++q) {
        const int i = tid + q * BT;
        mine[q] = i < nk ? sh.list[i] : 0ull;
        lg[q] = i < nk ? klog[i] : 0u;
      }
      got = top_n_regs<kPer, true>(mine, lg, kProbes, sh.list, sh.pr.logit, sh);
    }
    if (got < 0) trim_and_sort(sh, nk, nk, 0u);  // (logits read again below)
    const int np = nk < kProbes ? nk : kProbes;
    if (tid == 0) {
      // Written field by field into the record (a local copy indexed by the
      // running count would live in per-lane scratch memory).
      ProbeRec* dst = reinterpret_cast<ProbeRec*>(ws + lay.off_prec) + r;
      dst->z = sh.z;
      dst->m = m;
      dst->lse = lse;
      dst->inv_t = inv_t;
      // Only a probe whose logit exceeds every earlier probe's can be the
      // first kept one: top-p keeps the logits from a boundary up, so a
      // probe at or below an earlier, unkept probe's logit is not kept
      // either (the probe pass's sums keep that order: a sum of more
      // nonnegative terms never rounds below one of fewer).  The kept list
      // is therefore increasing in logit and usually two or three long.
      int pid[kProbes];
      float pl[kProbes];
#pragma unroll
      for (int i = 0; i < kProbes; ++i) {
        pid[i] = i < np ? cand_id(sh.list[i]) : 0;
        pl[i] = i >= np ? -INFINITY
                : got >= 0 ? __uint_as_float(sh.pr.logit[i])
                           : logit_at(a.lv, r, pid[i]);
      }
      int nh = 0;
      float hi = -INFINITY;
#pragma unroll
      for (int i = 0; i < kProbes; ++i) {
        if (i < np && (i == 0 || pl[i] > hi)) {
          dst->id[nh] = pid[i];
          dst->pt[nh] = pl[i];
          hi = pl[i];
          ++nh;
        }
      }
      for (int i = nh; i < kProbes; ++i) {
        dst->id[i] = 0;
        dst->pt[i] = INFINITY;
      }
      dst->npts = nh;
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
// This thread's sums of the weights exp((l - m) / T) of the chunk's logits
// above each of the row's NP probe logits.  Four float4 per thread in flight
// per step (a fourth of the round trips of one at a time); each thread
// still takes its elements in the order e = 4 tid + 4 PT j, j = 0, 1, ...
template <int NP>
__device__ __forceinline__ void probe_sums(const float* __restrict__ src, int n, int vec,
                                           const ProbeRec& pr, float (&acc)[kProbes]) {
  const int tid = threadIdx.x;
  const float sc = pr.inv_t * kLog2e;
  float pt[NP];
#pragma unroll
  for (int i = 0; i < NP; ++i) pt[i] = pr.pt[i];
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
        for (int i = 0; i < NP; ++i) acc[i] += l > pt[i] ? wt : 0.0f;
      }
    }
  }
}

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
    float acc[kProbes];
#pragma unroll
    for (int i = 0; i < kProbes; ++i) acc[i] = 0.0f;
    // The row's probe count (1..kProbes, most often two or three) fixes how
    // many comparisons each logit takes.
    const int np = __builtin_amdgcn_readfirstlane(pr.npts);
    switch (np) {
      case 1: probe_sums<1>(geo.src, geo.n, vec, pr, acc); break;
      case 2: probe_sums<2>(geo.src, geo.n, vec, pr, acc); break;
      case 3: probe_sums<3>(geo.src, geo.n, vec, pr, acc); break;
      case 4: probe_sums<4>(geo.src, geo.n, vec, pr, acc); break;
      case 5: probe_sums<5>(geo.src, geo.n, vec, pr, acc); break;
      case 6: probe_sums<6>(geo.src, geo.n, vec, pr, acc); break;
      case 7: probe_sums<7>(geo.src, geo.n, vec, pr, acc); break;
      default: probe_sums<kProbes>(geo.src, geo.n, vec, pr, acc); break;
    }
#pragma unroll
    for (int i = 0; i < kProbes; ++i) {
      if (i >= np) break;
      const double s = wave_sum(static_cast<double>(acc[i]));
      if (lane_id == 0) part[i][wave] = s;
    }
    __syncthreads();
    if (tid < np) {
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

bool sampler_takes_chunk_pass(int64_t rows, const int64_t* slice_cols, int n_slices) {
  return rows > 0 && !env_flag("TS_SAMPLER_EXACT") &&
         fast_path_supported(rows, slice_cols, n_slices);
}

// The chunk width of a call: narrow chunks (twice the chunk workgroups, six
// per CU instead of four) when the call also writes the stitched copy and
// the narrow layout stays short.  The copy doubles the chunk pass's memory
// traffic, and more resident workgroups overlap it with the arithmetic
// better, but twice the chunks make the merge's union of chunk lists twice as
// long.  Measured on MI355X (assembly + sampler): four 37,984-column slices,
// 20 narrow chunks per row: 0.186 against 0.197 ms at 640 rows, 0.101 against
// 0.108 ms at 256 rows; eight 31,040-column slices, 32 chunks: 0.329 against
// 0.292 ms.
constexpr int kNarrowMaxChunks = 24;

FastLayout call_layout(int64_t rows, const int64_t* cols, int n, int max_logprobs, bool stitch) {
  if (stitch) {
    const FastLayout narrow = make_layout(rows, cols, n, max_logprobs, kChunkVecNarrow);
    if (narrow.S > 0 && narrow.S <= kNarrowMaxChunks) return narrow;
  }
  return make_layout(rows, cols, n, max_logprobs, kChunkVec);
}

size_t sampler_workspace_size(int64_t rows, const int64_t* slice_cols, int n_slices,
                              int max_logprobs) {
  if (!fast_path_supported(rows, slice_cols, n_slices)) return 256;
  // Either layout a call may take fits.
  const size_t wide = call_layout(rows, slice_cols, n_slices, max_logprobs, false).total;
  const size_t any = call_layout(rows, slice_cols, n_slices, max_logprobs, true).total;
  return wide > any ? wide : any;
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
  FastLayout lay = call_layout(a.rows, cols, a.lv.n, a.max_logprobs, a.asm_out != nullptr);
  // float4 loads: every slice 16-byte aligned with rows and widths of whole float4s.
  int vec = 1;
  for (int s = 0; s < a.lv.n; ++s) {
    if (cols[s] == 0) continue;
    vec &= (reinterpret_cast<uintptr_t>(a.lv.ptr[s]) % 16 == 0) && (a.lv.ld[s] % 4 == 0) &&
           (cols[s] % 4 == 0);
  }
  lay.asm_vec4 = a.asm_out != nullptr && reinterpret_cast<uintptr_t>(a.asm_out) % 16 == 0 &&
                 a.asm_ld % 4 == 0;
  const unsigned chunks = static_cast<unsigned>(a.rows) * static_cast<unsigned>(lay.S);
  // The row order only matters when the chunk workgroups take more than one
  // round of the GPU (four per CU on 256 CUs); a smaller grid runs at once
  // and skips the pre-pass launch (about 4 us, a tenth of a 64-row call).
  // The narrow chunk pass of the one-call assembly + sampler, whose stitched
  // copy gives every chunk the same store traffic, was measured faster in
  // the rows' own order at every size (spec_decode 0.183 against 0.188 ms).
  lay.ordered = (lay.vec == kChunkVecNarrow || chunks <= kOneRoundChunks) ? 0 : 1;
  if (lay.ordered) hipLaunchKernelGGL(order_rows_kernel, dim3(1), dim3(OT), 0, stream, a, lay, ws);
  if (lay.vec == kChunkVecNarrow) {
    if (vec)
      hipLaunchKernelGGL((chunk_pass_kernel<true, kChunkVecNarrow>), dim3(chunks), dim3(AT), 0,
                         stream, a, lay, ws);
    else
      hipLaunchKernelGGL((chunk_pass_kernel<false, kChunkVecNarrow>), dim3(chunks), dim3(AT), 0,
                         stream, a, lay, ws);
  } else {
    if (vec)
      hipLaunchKernelGGL((chunk_pass_kernel<true, kChunkVec>), dim3(chunks), dim3(AT), 0, stream,
                         a, lay, ws);
    else
      hipLaunchKernelGGL((chunk_pass_kernel<false, kChunkVec>), dim3(chunks), dim3(AT), 0, stream,
                         a, lay, ws);
  }
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
