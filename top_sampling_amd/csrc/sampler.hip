// Per-row sampler for batch-sharded sampling on gfx950.
//
// The sampler runs on the rank's slice of requests, batch x (speculative
// tokens + 1) rows of full-vocabulary fp32 logits, and does temperature,
// top-k, top-p, log-probabilities and seeded sampling (page "Qwen4Exp
// batch-sharded sampling: inside vLLM PR #61018", orcarouter.ai blog, section
// "What batch-sharded sampling is, in one paragraph"; the page names the
// filters and a non-negative max_logprobs, not their arithmetic).  Semantics
// implemented here:
//   * log-probabilities are the raw log_softmax of the row;
//   * greedy (temperature < TS_GREEDY_EPS or top_k == 1): argmax, lowest id;
//   * otherwise temperature, then top-k (every token tied with the k-th
//     largest logit kept), then top-p on the temperature-scaled distribution
//     renormalised over the top-k set (the token whose cumulative mass first
//     reaches p is kept, with its ties), then Gumbel-max over the kept set
//     with Philox4x32-10 noise keyed on (seed, global row, token id).
//
// Exact kernel: one 1024-thread workgroup per row, radix selection on
// order-preserving 32-bit keys with LDS histograms (11/11/10-bit digits), and
// a top-p threshold search over the same digits with fixed-point (2^-40)
// masses, so every sum is exact integer arithmetic and independent of the
// order of atomics.  The row is re-read per pass from cache.
#include <float.h>
#include <math.h>

#include "device_common.hpp"
#include "ts_internal.hpp"

namespace ts {
namespace {

constexpr int XT = 1024;          // threads per row
constexpr int XW = XT / kWave;    // waves per row
constexpr int RBINS = 2048;       // radix bins (11-bit digit)
constexpr float kMassScale = 1099511627776.0f;  // 2^40: fixed-point unit of a weight

struct ExactSmem {
  uint32_t cnt[RBINS];
  unsigned long long mass[RBINS];
  float rf[XW];
  int ri[XW];
  uint32_t ru[XW];
  unsigned long long rq[XW];
  uint32_t list_key[TS_MAX_LOGPROBS];
  int list_id[TS_MAX_LOGPROBS];
  uint32_t sel_digit;
  uint32_t sel_above;
  unsigned long long sel_above_q;
  int list_n;
};

__device__ __forceinline__ int digit_shift(int rd) { return rd == 0 ? 21 : (rd == 1 ? 10 : 0); }
__device__ __forceinline__ int digit_width(int rd) { return rd == 2 ? 10 : 11; }

__device__ __forceinline__ unsigned long long fixed_mass(float w) {
  return static_cast<unsigned long long>(w * kMassScale);  // w in [0, 1]
}

// Pick the digit whose bin holds the `rem`-th largest element, counting from
// the top bin down; sets sel_digit and sel_above (count strictly above it).
__device__ void select_digit_count(ExactSmem& sh, int nb, uint32_t rem) {
  const int t = threadIdx.x;
  const int b0 = nb - 1 - 2 * t, b1 = nb - 2 - 2 * t;
  const uint32_t h0 = b0 >= 0 ? sh.cnt[b0] : 0u;
  const uint32_t h1 = b1 >= 0 ? sh.cnt[b1] : 0u;
  uint32_t total;
  const uint32_t ex = block_exclusive_scan<XT, uint32_t>(h0 + h1, sh.ru, total);
  if (b0 >= 0 && ex < rem && rem <= ex + h0) {
    sh.sel_digit = static_cast<uint32_t>(b0);
    sh.sel_above = ex;
  } else if (b1 >= 0 && ex + h0 < rem && rem <= ex + h0 + h1) {
    sh.sel_digit = static_cast<uint32_t>(b1);
    sh.sel_above = ex + h0;
  }
  __syncthreads();
}

// Same search over fixed-point masses: the bin where the mass counted from the
// top first reaches `rem`.
__device__ void select_digit_mass(ExactSmem& sh, int nb, unsigned long long rem) {
  const int t = threadIdx.x;
  const int b0 = nb - 1 - 2 * t, b1 = nb - 2 - 2 * t;
  const unsigned long long h0 = b0 >= 0 ? sh.mass[b0] : 0ull;
  const unsigned long long h1 = b1 >= 0 ? sh.mass[b1] : 0ull;
  unsigned long long total;
  const unsigned long long ex = block_exclusive_scan<XT, unsigned long long>(h0 + h1, sh.rq, total);
  if (b0 >= 0 && ex < rem && rem <= ex + h0) {
    sh.sel_digit = static_cast<uint32_t>(b0);
    sh.sel_above_q = ex;
  } else if (b1 >= 0 && ex + h0 < rem && rem <= ex + h0 + h1) {
    sh.sel_digit = static_cast<uint32_t>(b1);
    sh.sel_above_q = ex + h0;
  }
  __syncthreads();
}

// The k-th largest key of the row (1 <= k <= V): K with
// #(key > K) < k <= #(key >= K).  Returns K, gt = #(key > K), eq = #(key == K).
__device__ void radix_kth(const float* __restrict__ row, int V, uint32_t k, ExactSmem& sh,
                          uint32_t& K, uint32_t& gt, uint32_t& eq) {
  uint32_t prefix = 0, pmask = 0, rem = k, above = 0, last = 0;
  for (int rd = 0; rd < 3; ++rd) {
    const int shift = digit_shift(rd), width = digit_width(rd);
    const uint32_t dmask = (1u << width) - 1u;
    for (int b = threadIdx.x; b < RBINS; b += XT) sh.cnt[b] = 0u;
    __syncthreads();
    for (int i = threadIdx.x; i < V; i += XT) {
      const uint32_t key = order_key(row[i]);
      if ((key & pmask) == prefix) atomicAdd(&sh.cnt[(key >> shift) & dmask], 1u);
    }
    __syncthreads();
    select_digit_count(sh, 1 << width, rem);
    const uint32_t d = sh.sel_digit, a = sh.sel_above;
    last = sh.cnt[d];
    __syncthreads();
    rem -= a;
    above += a;
    prefix |= d << shift;
    pmask |= dmask << shift;
  }
  K = prefix;
  gt = above;
  eq = last;
}

// The largest key K such that the fixed-point mass of {key >= max(K, floor)}
// reaches `target` (1 <= target <= mass of {key >= floor}).
__device__ uint32_t radix_mass(const float* __restrict__ row, int V, uint32_t floor_key, float m,
                               float inv_t, unsigned long long target, ExactSmem& sh) {
  uint32_t prefix = 0, pmask = 0;
  unsigned long long rem = target;
  for (int rd = 0; rd < 3; ++rd) {
    const int shift = digit_shift(rd), width = digit_width(rd);
    const uint32_t dmask = (1u << width) - 1u;
    for (int b = threadIdx.x; b < RBINS; b += XT) sh.mass[b] = 0ull;
    __syncthreads();
    for (int i = threadIdx.x; i < V; i += XT) {
      const float l = row[i];
      const uint32_t key = order_key(l);
      if (key >= floor_key && (key & pmask) == prefix)
        atomicAdd(&sh.mass[(key >> shift) & dmask], fixed_mass(expf((l - m) * inv_t)));
    }
    __syncthreads();
    select_digit_mass(sh, 1 << width, rem);
    const uint32_t d = sh.sel_digit;
    const unsigned long long a = sh.sel_above_q;
    __syncthreads();
    rem -= a;
    prefix |= d << shift;
    pmask |= dmask << shift;
  }
  return prefix;
}

__device__ void write_bad_row(const SamplerArgs& a, int r, int status) {
  const float qnan = __builtin_nanf("");
  for (int j = threadIdx.x; j < a.max_logprobs; j += XT) {
    a.topn_ids[static_cast<int64_t>(r) * a.max_logprobs + j] = -1;
    a.topn_logprobs[static_cast<int64_t>(r) * a.max_logprobs + j] = qnan;
  }
  if (threadIdx.x == 0) {
    a.token_ids[r] = -1;
    if (a.token_logprobs) a.token_logprobs[r] = qnan;
    if (a.row_status) a.row_status[r] = status;
  }
}

__device__ bool params_ok(const ts_row_params& p, int max_logprobs) {
  if (!(p.temperature >= 0.0f) || isinf(p.temperature)) return false;
  if (p.top_k < 0) return false;
  if (!(p.top_p > 0.0f && p.top_p <= 1.0f)) return false;
  if (p.n_logprobs < 0 || p.n_logprobs > max_logprobs) return false;
  return true;
}

// One workgroup samples one row.  `row_list` (optional) maps blockIdx.x to a
// local row; `row_count` (optional, device) bounds the list.
__global__ __launch_bounds__(XT) void sampler_exact_kernel(SamplerArgs a, const int* row_list,
                                                           const int* row_count) {
  __shared__ ExactSmem sh;
  int r = blockIdx.x;
  if (row_count != nullptr && r >= *row_count) return;
  if (row_list != nullptr) r = row_list[r];
  const int tid = threadIdx.x;
  const int V = a.vocab;
  const float* __restrict__ row = a.logits + static_cast<int64_t>(r) * a.ld;
  const ts_row_params p = a.params[r];

  if (!params_ok(p, a.max_logprobs)) {
    write_bad_row(a, r, TS_ROW_BAD_PARAMS);
    return;
  }

  // Pass 1: maximum key with its lowest id; screen NaN and +inf.
  uint32_t bk = 0u;
  int bi = 0x7fffffff;
  int bad = 0;
  for (int i = tid; i < V; i += XT) {
    const float l = row[i];
    bad |= (isnan(l) || (isinf(l) && l > 0.0f)) ? 1 : 0;
    const uint32_t key = order_key(l);
    if (better_u(key, i, bk, bi)) {
      bk = key;
      bi = i;
    }
  }
  bad = block_sum<XT, int>(bad, sh.ri);
  block_best_u<XT>(bk, bi, sh.ru, sh.ri);
  const float m = key_to_float(bk);
  if (bad != 0 || isinf(m)) {  // NaN/+inf present, or every logit is -inf
    write_bad_row(a, r, TS_ROW_BAD_LOGITS);
    return;
  }
  const int argmax_id = bi;

  // Pass 2: log-sum-exp of the raw logits (fixed per-thread order, fixed tree).
  float s = 0.0f;
  for (int i = tid; i < V; i += XT) s += expf(row[i] - m);
  s = block_sum<XT, float>(s, sh.rf);
  const float lse = m + logf(s);

  // Top-N log-probabilities.
  const int n = p.n_logprobs < V ? p.n_logprobs : V;
  const int64_t obase = static_cast<int64_t>(r) * a.max_logprobs;
  for (int j = n + tid; j < a.max_logprobs; j += XT) {
    a.topn_ids[obase + j] = -1;
    a.topn_logprobs[obase + j] = -INFINITY;
  }
  if (n > 0) {
    uint32_t kn, gt, eq;
    radix_kth(row, V, static_cast<uint32_t>(n), sh, kn, gt, eq);
    const uint32_t need = static_cast<uint32_t>(n) - gt;  // ties at kn taken by lowest id
    if (tid == 0) sh.list_n = 0;
    __syncthreads();
    for (int i = tid; i < V; i += XT) {
      const uint32_t key = order_key(row[i]);
      if (key > kn || (eq == need && key == kn)) {
        const int slot = atomicAdd(&sh.list_n, 1);
        sh.list_key[slot] = key;
        sh.list_id[slot] = i;
      }
    }
    if (eq != need) {
      uint32_t taken = 0;
      for (int base = 0; base < V && taken < need; base += XT) {
        const int i = base + tid;
        const bool f = i < V && order_key(row[i]) == kn;
        uint32_t tot;
        const uint32_t ex = block_exclusive_scan<XT, uint32_t>(f ? 1u : 0u, sh.ru, tot);
        if (f && taken + ex < need) {
          const int slot = atomicAdd(&sh.list_n, 1);
          sh.list_key[slot] = kn;
          sh.list_id[slot] = i;
        }
        taken += tot;
      }
    }
    __syncthreads();
    for (int t = tid; t < n; t += XT) {
      const uint32_t kt = sh.list_key[t];
      const int it = sh.list_id[t];
      int rank = 0;
      for (int j = 0; j < n; ++j) rank += better_u(sh.list_key[j], sh.list_id[j], kt, it) ? 1 : 0;
      a.topn_ids[obase + rank] = it;
      a.topn_logprobs[obase + rank] = key_to_float(kt) - lse;
    }
  }

  int token;
  if (p.temperature < TS_GREEDY_EPS || p.top_k == 1) {
    token = argmax_id;
  } else {
    const float inv_t = 1.0f / p.temperature;
    // Top-k threshold key (0 keeps every non-NaN key).
    uint32_t kk = 0u;
    if (p.top_k > 0 && p.top_k < V) {
      uint32_t gt, eq;
      radix_kth(row, V, static_cast<uint32_t>(p.top_k), sh, kk, gt, eq);
    }
    // Top-p threshold key on the temperature-scaled top-k distribution.
    uint32_t kp = 0u;
    if (p.top_p < 1.0f) {
      unsigned long long z = 0ull;
      for (int i = tid; i < V; i += XT) {
        const float l = row[i];
        if (order_key(l) >= kk) z += fixed_mass(expf((l - m) * inv_t));
      }
      z = block_sum<XT, unsigned long long>(z, sh.rq);
      double tgt = ceil(static_cast<double>(p.top_p) * static_cast<double>(z));
      unsigned long long target = static_cast<unsigned long long>(tgt);
      if (target < 1ull) target = 1ull;
      if (target > z) target = z;
      kp = radix_mass(row, V, kk, m, inv_t, target, sh);
    }
    const uint32_t thr = kk > kp ? kk : kp;
    // Gumbel-max over the kept set, four consecutive tokens per Philox call.
    const uint64_t grow = static_cast<uint64_t>(a.row_offset + r);
    float gk = -INFINITY;
    int gi = 0x7fffffff;
    const int nq = (V + 3) >> 2;
    for (int q = tid; q < nq; q += XT) {
      float l4[4];
      bool in[4];
      bool any = false;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int v = 4 * q + j;
        l4[j] = v < V ? row[v] : -INFINITY;
        in[j] = v < V && order_key(l4[j]) >= thr;
        any |= in[j];
      }
      if (!any) continue;
      const U32x4 w = token_words(p.seed, grow, static_cast<uint32_t>(q));
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (!in[j]) continue;
        const float key = (l4[j] - m) * inv_t + gumbel_from_word(w.v[j]);
        if (better(key, 4 * q + j, gk, gi)) {
          gk = key;
          gi = 4 * q + j;
        }
      }
    }
    block_best<XT>(gk, gi, sh.rf, sh.ri);
    token = gi;
  }
  if (tid == 0) {
    a.token_ids[r] = token;
    if (a.token_logprobs) a.token_logprobs[r] = row[token] - lse;
    if (a.row_status) a.row_status[r] = TS_ROW_OK;
  }
}

}  // namespace

size_t sampler_workspace_size(int64_t rows, int64_t vocab, int max_logprobs) {
  (void)rows;
  (void)vocab;
  (void)max_logprobs;
  return 256;
}

hipError_t launch_sampler(const SamplerArgs& a, void* workspace, size_t workspace_bytes,
                          hipStream_t stream) {
  (void)workspace;
  (void)workspace_bytes;
  if (a.rows == 0) return hipSuccess;
  hipLaunchKernelGGL(sampler_exact_kernel, dim3(a.rows), dim3(XT), 0, stream, a,
                     static_cast<const int*>(nullptr), static_cast<const int*>(nullptr));
  return hipGetLastError();
}

}  // namespace ts
