// Finishing kernel of the sampler and the exact per-row sampler (gfx950).
//
// One 1024-thread workgroup per row that the single-read fast path leaves
// open:
//   probe rows: top-p-only rows whose boundary lies below the listed logits.
//     The probe pass has summed, per probe token v (the row's best Gumbel
//     keys, best first), the temperature-scaled mass of the logits strictly
//     above l_v.  v is kept by top-p iff that mass is below p times the
//     total, so the first kept probe is the Gumbel-max winner over the kept
//     set.  If no probe is kept, the row is computed exactly.
//   exact rows (candidate overflow, top_k > 1024, heavy ties): the whole row
//     from scratch with radix selection on order-preserving keys (11/11/10-bit
//     digits in LDS) and a top-p threshold search over the same digits with
//     fixed-point (2^-40) masses, so every sum is exact integer arithmetic.
//     With TS_SAMPLER_EXACT=1 every row takes this route.
#include <float.h>

#include "sampler_common.hpp"

namespace ts {
namespace {

constexpr int XT = 1024;        // threads per row
constexpr int XW = XT / kWave;  // waves per row
constexpr int RBINS = 2048;     // radix bins (11-bit digit)

struct ExactSmem {
  uint32_t cnt[RBINS];
  unsigned long long mass[RBINS];
  uint32_t list_key[TS_MAX_LOGPROBS];
  int list_id[TS_MAX_LOGPROBS];
};

struct FallbackSmem {
  ExactSmem ex;
  float rf_[XW];
  int ri[XW];
  uint32_t ru[XW];
  unsigned long long rq[XW];
  uint32_t sel_digit;
  uint32_t sel_above;
  unsigned long long sel_above_q;
  int list_n;
  double pabove[kProbes];  // probe rows: mass above each probe
  double pstage[kMaxChunks * kProbes];  // probe rows: every chunk's partial masses
  LogitsView lv;  // the slice table, read with per-thread indices from here
};

// Copies the slice table out of the kernel arguments with constant indices
// only.  Indexing the by-value argument with a run-time slice number makes the
// compiler copy the whole argument block into per-lane scratch memory.
__device__ __forceinline__ void stage_view(const LogitsView& src, LogitsView& dst) {
  if (threadIdx.x == 0) {
    dst.n = src.n;
    dst.off[0] = src.off[0];
#pragma unroll
    for (int s = 0; s < TS_MAX_SLICES; ++s) {
      if (s < src.n) {
        dst.ptr[s] = src.ptr[s];
        dst.ld[s] = src.ld[s];
        dst.off[s + 1] = src.off[s + 1];
      }
    }
  }
  __syncthreads();
}

__device__ __forceinline__ int digit_shift(int rd) { return rd == 0 ? 21 : (rd == 1 ? 10 : 0); }
__device__ __forceinline__ int digit_width(int rd) { return rd == 2 ? 10 : 11; }

// Same search over fixed-point masses: the bin where the mass counted from the
// top first reaches `rem`.
__device__ __forceinline__ void select_digit_mass(FallbackSmem& sh, int nb, unsigned long long rem) {
  const int t = threadIdx.x;
  const int b0 = nb - 1 - 2 * t, b1 = nb - 2 - 2 * t;
  const unsigned long long h0 = b0 >= 0 ? sh.ex.mass[b0] : 0ull;
  const unsigned long long h1 = b1 >= 0 ? sh.ex.mass[b1] : 0ull;
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

// Calls f(i, l) for the logits of row r, each thread taking every XT-th
// column of each slice, in increasing column order.  The loads run kRowLoads
// columns ahead of the calls (one wave's load covers 64 consecutive columns),
// so a pass over a row is not one memory round trip per column step.
constexpr int kRowLoads = 16;
template <typename F>
__device__ __forceinline__ void for_row(const LogitsView& lv, int r, F&& f) {
  for (int s = 0; s < lv.n; ++s) {
    const float* __restrict__ src = lv.ptr[s] + static_cast<int64_t>(r) * lv.ld[s];
    const int base = static_cast<int>(lv.off[s]);
    const int cols = static_cast<int>(lv.off[s + 1] - lv.off[s]);
    int j = threadIdx.x;
    for (; j + (kRowLoads - 1) * XT < cols; j += kRowLoads * XT) {
      float x[kRowLoads];
#pragma unroll
      for (int u = 0; u < kRowLoads; ++u) x[u] = src[j + u * XT];
#pragma unroll
      for (int u = 0; u < kRowLoads; ++u) f(base + j + u * XT, x[u]);
    }
    for (; j < cols; j += XT) f(base + j, src[j]);
  }
}

// The k-th largest key of the row (1 <= k <= V): K with
// #(key > K) < k <= #(key >= K).  Returns K, gt = #(key > K), eq = #(key == K).
__device__ __forceinline__ void radix_kth(const LogitsView& lv, int r, uint32_t k, FallbackSmem& sh,
                          uint32_t& K, uint32_t& gt, uint32_t& eq) {
  uint32_t prefix = 0, pmask = 0, rem = k, above = 0, last = 0;
  for (int rd = 0; rd < 3; ++rd) {
    const int shift = digit_shift(rd), width = digit_width(rd);
    const uint32_t dmask = (1u << width) - 1u;
    for (int b = threadIdx.x; b < RBINS; b += XT) sh.ex.cnt[b] = 0u;
    __syncthreads();
    for_row(lv, r, [&](int, float l) {
      const uint32_t key = order_key(l);
      if ((key & pmask) == prefix) atomicAdd(&sh.ex.cnt[(key >> shift) & dmask], 1u);
    });
    __syncthreads();
    select_digit_top<XT, 2>(sh.ex.cnt, 1 << width, rem, sh.ru, &sh.sel_digit, &sh.sel_above);
    const uint32_t d = sh.sel_digit, a = sh.sel_above;
    last = sh.ex.cnt[d];
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
__device__ __forceinline__ uint32_t radix_mass(const LogitsView& lv, int r, uint32_t floor_key, float m,
                               float inv_t, unsigned long long target, FallbackSmem& sh) {
  uint32_t prefix = 0, pmask = 0;
  unsigned long long rem = target;
  for (int rd = 0; rd < 3; ++rd) {
    const int shift = digit_shift(rd), width = digit_width(rd);
    const uint32_t dmask = (1u << width) - 1u;
    for (int b = threadIdx.x; b < RBINS; b += XT) sh.ex.mass[b] = 0ull;
    __syncthreads();
    for_row(lv, r, [&](int, float l) {
      const uint32_t key = order_key(l);
      if (key >= floor_key && (key & pmask) == prefix)
        atomicAdd(&sh.ex.mass[(key >> shift) & dmask], fixed_mass(fast_exp((l - m) * inv_t)));
    });
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

__device__ __forceinline__ void write_bad_row(const SamplerArgs& a, int r, int status) {
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

// The whole row from scratch.
__device__ __forceinline__ void exact_row(const SamplerArgs& a, int r, FallbackSmem& sh) {
  const int tid = threadIdx.x;
  const int V = a.vocab;
  const LogitsView& lv = sh.lv;
  const ts_row_params p = a.params[r];

  if (!params_ok(p, a.max_logprobs)) {
    write_bad_row(a, r, TS_ROW_BAD_PARAMS);
    return;
  }

  // Pass 1: maximum key with its lowest id; screen NaN and +inf; and each
  // thread's sum of exp(l - its running maximum), rescaled as that maximum
  // grows (fixed per-thread order, fixed tree), for the log-sum-exp.
  uint32_t bk = 0u;
  int bi = 0x7fffffff;
  int bad = 0;
  float mt = -INFINITY, st = 0.0f;
  for_row(lv, r, [&](int i, float l) {
    bad |= (isnan(l) || (isinf(l) && l > 0.0f)) ? 1 : 0;
    const uint32_t key = order_key(l);
    if (better_u(key, i, bk, bi)) {
      bk = key;
      bi = i;
    }
    if (l > mt) {
      st = st * fast_exp(mt - l) + 1.0f;
      mt = l;
    } else if (l > -INFINITY) {
      st += fast_exp(l - mt);
    }
  });
  bad = block_sum<XT, int>(bad, sh.ri);
  block_best_u<XT>(bk, bi, sh.ru, sh.ri);
  const float m = key_to_float(bk);
  if (bad != 0 || isinf(m)) {  // NaN/+inf present, or every logit is -inf
    write_bad_row(a, r, TS_ROW_BAD_LOGITS);
    return;
  }
  const int argmax_id = bi;
  const float s = block_sum<XT, float>(mt > -INFINITY ? st * fast_exp(mt - m) : 0.0f, sh.rf_);
  const float lse = m + logf(s);

  // The sampled token first: the processed log-probabilities need the kept
  // set it is drawn from.
  int token;
  const bool greedy = p.temperature < TS_GREEDY_EPS || p.top_k == 1;
  float inv_t = 0.0f;
  uint32_t thr = 0u;  // the kept set's smallest key
  if (greedy) {
    token = argmax_id;
  } else {
    inv_t = 1.0f / p.temperature;
    // Top-k threshold key (0 keeps every non-NaN key).
    uint32_t kk = 0u;
    if (p.top_k > 0 && p.top_k < V) {
      uint32_t gt, eq;
      radix_kth(lv, r, static_cast<uint32_t>(p.top_k), sh, kk, gt, eq);
    }
    // Top-p threshold key on the temperature-scaled top-k distribution.
    uint32_t kp = 0u;
    if (p.top_p < 1.0f) {
      unsigned long long z = 0ull;
      for_row(lv, r, [&](int, float l) {
        if (order_key(l) >= kk) z += fixed_mass(fast_exp((l - m) * inv_t));
      });
      z = block_sum<XT, unsigned long long>(z, sh.rq);
      const double tgt = ceil(static_cast<double>(p.top_p) * static_cast<double>(z));
      unsigned long long target = static_cast<unsigned long long>(tgt);
      if (target < 1ull) target = 1ull;
      if (target > z) target = z;
      kp = radix_mass(lv, r, kk, m, inv_t, target, sh);
    }
    thr = kk > kp ? kk : kp;
    // Gumbel-max over the kept set, four consecutive tokens per Philox call.
    const uint64_t grow = static_cast<uint64_t>(a.row_offset + r);
    float gk = -INFINITY;
    int gi = 0x7fffffff;
    // Thread t takes the groups q = t, t + XT, ..., the logits of four
    // groups loaded before any is used.
    const int nq = (V + 3) >> 2;
    constexpr int QG = 4;
    for (int q0 = tid; q0 < nq; q0 += QG * XT) {
      float l4[QG][4];
#pragma unroll
      for (int u = 0; u < QG; ++u) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int v = 4 * (q0 + u * XT) + j;
          l4[u][j] = v < V ? logit_at(lv, r, v) : -INFINITY;
        }
      }
#pragma unroll
      for (int u = 0; u < QG; ++u) {
        const int q = q0 + u * XT;
        bool in[4];
        bool any = false;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          in[j] = 4 * q + j < V && order_key(l4[u][j]) >= thr;
          any |= in[j];
        }
        if (!any) continue;
        const U32x4 w = token_words(p.seed, grow, static_cast<uint32_t>(q));
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (!in[j]) continue;
          const float key = (l4[u][j] - m) * inv_t + gumbel_from_word(w.v[j]);
          if (better(key, 4 * q + j, gk, gi)) {
            gk = key;
            gi = 4 * q + j;
          }
        }
      }
    }
    block_best<XT>(gk, gi, sh.rf_, sh.ri);
    token = gi;
  }
  // Processed log-probabilities: (l - m) / T - ln(kept mass) inside the kept
  // set, -inf outside it; a greedy row is a point mass on its token.
  const bool proc = (a.flags & TS_LOGPROBS_PROCESSED) != 0;
  float lzk = 0.0f;
  if (proc && !greedy) {
    float z = 0.0f;
    for_row(lv, r, [&](int, float l) {
      if (order_key(l) >= thr) z += fast_exp((l - m) * inv_t);
    });
    lzk = logf(block_sum<XT, float>(z, sh.rf_));
  }
  auto out_lp = [&](uint32_t key, int id) -> float {
    const float l = key_to_float(key);
    if (!proc) return l - lse;
    if (greedy) return id == token ? 0.0f : -INFINITY;
    return key >= thr ? (l - m) * inv_t - lzk : -INFINITY;
  };

  // Top-N log-probabilities.
  const int n = p.n_logprobs < V ? p.n_logprobs : V;
  const int64_t obase = static_cast<int64_t>(r) * a.max_logprobs;
  for (int j = n + tid; j < a.max_logprobs; j += XT) {
    a.topn_ids[obase + j] = -1;
    a.topn_logprobs[obase + j] = -INFINITY;
  }
  if (n > 0) {
    uint32_t kn, gt, eq;
    radix_kth(lv, r, static_cast<uint32_t>(n), sh, kn, gt, eq);
    const uint32_t need = static_cast<uint32_t>(n) - gt;  // ties at kn taken by lowest id
    if (tid == 0) sh.list_n = 0;
    __syncthreads();
    for_row(lv, r, [&](int i, float l) {
      const uint32_t key = order_key(l);
      if (key > kn || (eq == need && key == kn)) {
        const int slot = atomicAdd(&sh.list_n, 1);
        sh.ex.list_key[slot] = key;
        sh.ex.list_id[slot] = i;
      }
    });
    if (eq != need) {
      uint32_t taken = 0;
      for (int base = 0; base < V && taken < need; base += XT) {
        const int i = base + tid;
        const bool f = i < V && order_key(logit_at(lv, r, i)) == kn;
        uint32_t tot;
        const uint32_t ex = block_exclusive_scan<XT, uint32_t>(f ? 1u : 0u, sh.ru, tot);
        if (f && taken + ex < need) {
          const int slot = atomicAdd(&sh.list_n, 1);
          sh.ex.list_key[slot] = kn;
          sh.ex.list_id[slot] = i;
        }
        taken += tot;
      }
    }
    __syncthreads();
    for (int t = tid; t < n; t += XT) {
      const uint32_t kt = sh.ex.list_key[t];
      const int it = sh.ex.list_id[t];
      int rank = 0;
      for (int j = 0; j < n; ++j)
        rank += better_u(sh.ex.list_key[j], sh.ex.list_id[j], kt, it) ? 1 : 0;
      a.topn_ids[obase + rank] = it;
      a.topn_logprobs[obase + rank] = out_lp(kt, it);
    }
  }

  if (tid == 0) {
    a.token_ids[r] = token;
    if (a.token_logprobs) a.token_logprobs[r] = out_lp(order_key(logit_at(lv, r, token)), token);
    if (a.row_status) a.row_status[r] = TS_ROW_OK;
  }
}

// Probe row: the first probe (best Gumbel key first) whose mass-above is below
// p times the total is the winner.
__device__ __forceinline__ void finish_probe_row(const SamplerArgs& a, const FastLayout& lay, const uint8_t* ws,
                                 int li, int r, FallbackSmem& sh) {
  const ProbeRec& pr = reinterpret_cast<const ProbeRec*>(ws + lay.off_prec)[r];
  const ts_row_params p = a.params[r];
  const double* part = reinterpret_cast<const double*>(ws + lay.off_part) +
                       static_cast<size_t>(li) * lay.S * kProbes;
  // Every chunk's partials are fetched at once (thread t takes chunk t / np,
  // probe t % np), then thread i sums probe i's over the chunks in chunk
  // order, the additions of a serial walk without its chain of loads.
  const int np = pr.npts;
  const int nstage = lay.S * np;  // at most kMaxChunks * kProbes <= XT
  for (int t = threadIdx.x; t < nstage; t += XT) {
    const int c = t / np;
    sh.pstage[t] = part[static_cast<size_t>(c) * kProbes + (t - c * np)];
  }
  __syncthreads();
  if (static_cast<int>(threadIdx.x) < np) {
    double above = 0.0;
    for (int c = 0; c < lay.S; ++c) above += sh.pstage[c * np + threadIdx.x];
    sh.pabove[threadIdx.x] = above;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    const double target = static_cast<double>(p.top_p) * pr.z;
    int win = -1;
    for (int i = 0; i < np; ++i) {
      if (sh.pabove[i] < target) {
        win = i;
        break;
      }
    }
    sh.list_n = win;
  }
  __syncthreads();
  const int win = sh.list_n;
  __syncthreads();
  if (win < 0) {
    exact_row(a, r, sh);
    return;
  }
  if (threadIdx.x == 0) {
    a.token_ids[r] = pr.id[win];
    if (a.token_logprobs) a.token_logprobs[r] = pr.pt[win] - pr.lse;  // pt: the probe's logit
    if (a.row_status) a.row_status[r] = TS_ROW_OK;
  }
}

// Workgroup b finishes probe row b, then exact row b - (probe rows); with
// all_rows every row is computed exactly.
__global__ __launch_bounds__(XT) void sampler_finish_kernel(SamplerArgs a, FastLayout lay,
                                                            uint8_t* ws, int all_rows) {
  __shared__ FallbackSmem sh;
  const int b = blockIdx.x;
  const int* ctr = reinterpret_cast<const int*>(ws + lay.off_ctr);
  const int n_exact = all_rows ? 0 : ctr[0], n_probe = all_rows ? 0 : ctr[1];
  if (!all_rows && b >= n_probe + n_exact) return;  // nothing left for this workgroup
  stage_view(a.lv, sh.lv);
  if (all_rows) {
    exact_row(a, b, sh);
  } else if (b < n_probe) {
    finish_probe_row(a, lay, ws, b, reinterpret_cast<const int*>(ws + lay.off_probe)[b], sh);
  } else {
    exact_row(a, reinterpret_cast<const int*>(ws + lay.off_exact)[b - n_probe], sh);
  }
}

}  // namespace

hipError_t launch_sampler_finish(const SamplerArgs& a, const FastLayout* lay, uint8_t* ws,
                                 hipStream_t stream) {
  const FastLayout l = lay ? *lay : FastLayout{};
  hipLaunchKernelGGL(sampler_finish_kernel, dim3(a.rows), dim3(XT), 0, stream, a, l, ws,
                     lay ? 0 : 1);
  return hipGetLastError();
}

}  // namespace ts
