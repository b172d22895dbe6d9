// Definitions shared by the sampler kernels (fast path and exact path).
//
// Semantics (the page "Qwen4Exp batch-sharded sampling: inside vLLM PR
// #61018", section "What batch-sharded sampling is, in one paragraph", names
// top-k, top-p and log-probabilities but not their arithmetic; the readings
// below are the ones the C ABI documents):
//   * log-probabilities: raw log_softmax of the row;
//   * greedy (temperature < TS_GREEDY_EPS or top_k == 1): argmax, lowest id;
//   * otherwise temperature, then top-k (ties with the k-th largest kept),
//     then top-p over the temperature-scaled distribution renormalised on the
//     top-k set (the crossing token and its ties kept), then Gumbel-max with
//     key (l - max) / T + g, g from Philox4x32-10 keyed on (seed, global row,
//     token id), lowest id on exact ties.
#pragma once

#include <math.h>

#include "device_common.hpp"
#include "ts_internal.hpp"

namespace ts {

// ------------------------------------------------------------------ row kinds
enum RowKind : int {
  KIND_BAD = 0,     // invalid parameters
  KIND_GREEDY = 1,  // argmax
  KIND_TOPK = 2,    // 0 < top_k < V (top_k <= kFastTopKMax), any top_p
  KIND_FULL = 3,    // no filter: Gumbel-max over every token
  KIND_TOPP = 4,    // top-p only
  KIND_EXACT = 5    // handled by the exact per-row kernel (large top_k)
};

constexpr int kFastTopKMax = 2048;

__device__ __forceinline__ bool params_ok(const ts_row_params& p, int max_logprobs) {
  if (!(p.temperature >= 0.0f) || isinf(p.temperature)) return false;
  if (p.top_k < 0) return false;
  if (!(p.top_p > 0.0f && p.top_p <= 1.0f)) return false;
  if (p.n_logprobs < 0 || p.n_logprobs > max_logprobs) return false;
  return true;
}

// How many of a chunk's largest logits its candidate list must hold.
__device__ __forceinline__ int cand_target(int kind, const ts_row_params& p, int V) {
  const int n_eff = p.n_logprobs < V ? p.n_logprobs : V;
  int M = n_eff > 1 ? n_eff : 1;
  if (kind == 2 && p.top_k > M) M = p.top_k;         // KIND_TOPK
  if (kind == 4 && 64 > M) M = 64;                   // KIND_TOPP
  return M < V ? M : V;
}

// How many of its largest logits one of S chunks lists.  Up to 64 every chunk
// lists the row's whole target M, so the union of the lists holds the row's M
// largest whatever their distribution.  Above 64 a chunk lists 1.5 times its
// share, at least 64: the union then holds the row's M largest unless they
// crowd into a few chunks, which the merge detects (fewer than M entries
// above the highest chunk threshold) and hands to the exact kernel.
__device__ __forceinline__ int chunk_target(int M, int S) {
  if (M <= 64) return M;
  int mc = (3 * M + 2 * S - 1) / (2 * S);
  mc = mc > 64 ? mc : 64;
  return mc < M ? mc : M;
}

__device__ __forceinline__ int row_kind(const ts_row_params& p, int V, int max_logprobs) {
  if (!params_ok(p, max_logprobs)) return KIND_BAD;
  if (p.temperature < TS_GREEDY_EPS || p.top_k == 1) return KIND_GREEDY;
  if (p.top_k > 0 && p.top_k < V) return p.top_k <= kFastTopKMax ? KIND_TOPK : KIND_EXACT;
  return p.top_p < 1.0f ? KIND_TOPP : KIND_FULL;
}

// ------------------------------------------------------------------- numerics
constexpr float kMassScale = 1099511627776.0f;  // 2^40: fixed-point unit of a weight in [0, 1]
constexpr double kMassUnit = 1.0 / 1099511627776.0;
constexpr float kGumbelMax = 16.7f;  // above every Gumbel value a 23-bit uniform can give
constexpr float kMinGumbel = -2.9f;  // below every such Gumbel value (-ln(-ln 2^-24) = -2.81)

__device__ __forceinline__ unsigned long long fixed_mass(float w) {
  return static_cast<unsigned long long>(w * kMassScale);
}

// A candidate packed so that a larger value means "earlier in the order
// (logit descending, token id ascending)": key in the high word, inverted id
// in the low word.  Zero means "no candidate" (every real key is > 0).
__device__ __forceinline__ unsigned long long pack_cand(uint32_t key, int id) {
  return (static_cast<unsigned long long>(key) << 32) | static_cast<uint32_t>(~id);
}
__device__ __forceinline__ uint32_t cand_key(unsigned long long c) {
  return static_cast<uint32_t>(c >> 32);
}
__device__ __forceinline__ int cand_id(unsigned long long c) {
  return static_cast<int>(~static_cast<uint32_t>(c));
}

// Gumbel key of token `id` (logit l) of a row with maximum m.
__device__ __forceinline__ float gumbel_key(float l, float m, float inv_t, uint64_t seed,
                                            uint64_t grow, int id) {
  const U32x4 w = token_words(seed, grow, static_cast<uint32_t>(id) >> 2);
  return (l - m) * inv_t + gumbel_from_word(word_at(w, id & 3));
}

// ------------------------------------------------------------ workspace layout
constexpr int kKeyCap = 64;       // Gumbel-key candidates per chunk (top-p-only rows)
constexpr int kProbes = 8;        // probe points per top-p-only row

constexpr int kMaxChunks = 128;   // chunks per row
constexpr int kChunkThreads = 256;
constexpr int kChunkVec = 16;     // float4 per thread
constexpr int kChunkVecNarrow = 8;  // float4 per thread in a narrow chunk
constexpr int kChunkMax = kChunkThreads * kChunkVec * 4;  // 16384 logits
constexpr int kListMax = 4096;    // merged candidates a row may keep in LDS
constexpr float kKeyMargin = 1e-4f;  // rounding margin between chunk-local and row keys
constexpr float kLnKeysPerChunk = 3.17805383f;  // ln 24: a top-p chunk's expected key count at most 24

struct ChunkRec {  // one per (row, chunk); 64 bytes
  float cmax;      // chunk maximum
  float sumexp;    // sum exp(l - cmax)
  float tmass;     // sum exp((l - cmax) / T)                (top-p-only rows)
  uint32_t kt;     // logit candidate threshold: every logit with key >= kt is listed
  int ncand;       // listed logit candidates
  int status;      // 0 ok, 1 NaN/+inf seen, 2 candidate overflow
  int nkey;        // listed Gumbel-key candidates (full and top-p-only rows)
  float kfloor;    // every token whose key (l - cmax)/T + g >= kfloor is listed
  int pad[8];
};
static_assert(sizeof(ChunkRec) == 64, "64-byte chunk records");

// A Gumbel-key candidate as the chunk pass lists it: the token, its logit and
// its Philox word, so the merge forms the key (l - m) / T + g without reading
// the logit or drawing the word again.
struct KeyRec {
  int id;
  float logit;
  uint32_t word;
  int pad;
};
static_assert(sizeof(KeyRec) == 16, "16-byte key records");

__device__ __forceinline__ float key_of(const KeyRec& k, float m, float inv_t) {
  return (k.logit - m) * inv_t + gumbel_from_word(k.word);
}

struct ProbeRec {  // a top-p-only row whose boundary lies below the listed logits
  double z;        // total temperature-scaled mass, relative to the row maximum
  float m, lse, inv_t;
  int npts;        // probe tokens, best Gumbel key first
  int id[kProbes];
  float pt[kProbes];  // their logits
};

struct FastLayout {
  int S;  // chunks per row
  int L;  // the longest chunk (logits, a multiple of 4)
  int Ls[TS_MAX_SLICES];  // chunk length in slice s (multiple of 4; its last chunk may be shorter)
  int cc;  // candidate slots per chunk (cand_slots)
  int nsl;                      // column slices
  int cbase[TS_MAX_SLICES + 1];  // first chunk of each slice (chunks never straddle slices)
  size_t off_ctr, off_order, off_exact, off_probe, off_chunk, off_cand, off_key, off_prec, off_part,
      total;
  int vec;      // float4 per thread of the chunk pass (kChunkVec or kChunkVecNarrow)
  int ordered;  // the chunk pass takes rows in the row-order pre-pass's order (else row order)
  int asm_vec4;  // the stitched copy takes 16-byte stores (aligned base, ld a multiple of 4)
};

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Chunks per row: at most 4 * vec * kChunkThreads logits each (kChunkMax for
// the wide chunks), at least about one chunk workgroup per compute unit
// (kWantChunks), chunks of at least 1024 logits, at most kMaxChunks; every slice is cut into chunks of its own.  Few rows get no
// more chunks than that: the merge of a row walks every chunk's candidates,
// so for small batches it, not the read, sets the time.  S == 0 marks a shape
// the chunked path does not take.
constexpr int64_t kWantChunks = 256;

// Candidate slots per chunk: a chunk lists every logit at or above a
// threshold that at least its target count reach (chunk_target of the row's
// need, at most max(kFastTopKMax, max_logprobs, 64)); twice the largest
// target plus 64 leaves room for the logits that tie with or lie just above
// the threshold.  A chunk that lists more is an overflow: its row takes the
// exact per-row kernel (same results).
inline int cand_slots(int L, int S, int max_logprobs) {
  int64_t M = kFastTopKMax;
  if (max_logprobs > M) M = max_logprobs;
  int64_t mc = M;
  if (M > 64) {
    mc = (3 * M + 2 * S - 1) / (2 * S);
    if (mc < 64) mc = 64;
    if (mc > M) mc = M;
  }
  int64_t cc = (2 * mc + 64 + 63) / 64 * 64;
  return static_cast<int>(cc < L ? cc : L);
}

inline FastLayout make_layout(int64_t rows, const int64_t* cols, int n, int max_logprobs,
                              int vec = kChunkVec) {
  FastLayout l{};
  l.vec = vec;
  const int64_t chunk_max = static_cast<int64_t>(kChunkThreads) * vec * 4;
  int64_t vocab = 0;
  for (int s = 0; s < n; ++s) vocab += cols[s];
  int64_t S = (vocab + chunk_max - 1) / chunk_max;
  int64_t want = rows > 0 ? (kWantChunks + rows - 1) / rows : 1;
  int64_t most = vocab / 1024 > 0 ? vocab / 1024 : 1;
  if (want > most) want = most;
  if (want > kMaxChunks) want = kMaxChunks;
  if (S < want) S = want;
  if (S < 1) S = 1;
  int64_t L = (vocab + S - 1) / S;
  if (n > 1 && n < kMaxChunks) {
    // Each slice adds at most one partial chunk: keep the total within kMaxChunks.
    const int64_t Lmin = (vocab + (kMaxChunks - n) - 1) / (kMaxChunks - n);
    if (L < Lmin) L = Lmin;
  }
  L = (L + 3) / 4 * 4;
  if (L < 4) L = 4;
  l.nsl = n;
  // A slice takes as many chunks as the target length L needs, of equal
  // length (a slice of 37,984 at L = 15,194: three of 12,664, not two full
  // chunks and one half-empty one).
  int64_t total = 0, longest = 4;
  l.cbase[0] = 0;
  for (int s = 0; s < n; ++s) {
    const int64_t k = cols[s] > 0 ? (cols[s] + L - 1) / L : 0;
    int64_t Ls = k > 0 ? ((cols[s] + k - 1) / k + 3) / 4 * 4 : 4;
    if (Ls > L) Ls = L;
    l.Ls[s] = static_cast<int>(Ls);
    if (Ls > longest) longest = Ls;
    total += (cols[s] + Ls - 1) / Ls;
    l.cbase[s + 1] = static_cast<int>(total < (1 << 30) ? total : (1 << 30));
  }
  l.L = static_cast<int>(longest);
  l.S = (L > chunk_max || total > kMaxChunks || n >= kMaxChunks || total < 1)
            ? 0
            : static_cast<int>(total);
  l.cc = cand_slots(l.L, l.S > 0 ? l.S : 1, max_logprobs);
  const size_t R = static_cast<size_t>(rows);
  const size_t RS = R * static_cast<size_t>(l.S);
  size_t off = 0;
  l.off_ctr = off;  // [0] exact rows, [1] probe rows
  off = align_up(off + 256, 256);
  l.off_order = off;  // the chunk pass's row order (heaviest rows first)
  off = align_up(off + R * sizeof(int), 256);
  l.off_exact = off;
  off = align_up(off + R * sizeof(int), 256);
  l.off_probe = off;
  off = align_up(off + R * sizeof(int), 256);
  l.off_chunk = off;
  off = align_up(off + RS * sizeof(ChunkRec), 256);
  l.off_cand = off;
  off = align_up(off + RS * static_cast<size_t>(l.cc) * sizeof(unsigned long long), 256);
  l.off_key = off;
  off = align_up(off + RS * kKeyCap * sizeof(KeyRec), 256);
  l.off_prec = off;
  off = align_up(off + R * sizeof(ProbeRec), 256);
  l.off_part = off;
  off = align_up(off + RS * kProbes * sizeof(double), 256);
  l.total = off;
  return l;
}

// The chunked path needs every slice to start at a column that is a multiple
// of 4 (a float4 of a chunk then holds one Philox block of four tokens).
inline bool fast_path_supported(int64_t rows, const int64_t* cols, int n) {
  const FastLayout l = make_layout(rows, cols, n, 0);
  if (l.S == 0) return false;
  int64_t off = 0;
  for (int s = 0; s < n; ++s) {
    if (cols[s] > 0 && off % 4 != 0) return false;
    off += cols[s];
  }
  return rows * static_cast<int64_t>(l.S) <= 0x7fffffff;
}

// --------------------------------------------------------- logits access
// Slice holding global column col (empty slices are skipped).
__device__ __forceinline__ int slice_of(const LogitsView& lv, int col) {
  int lo = 0, hi = lv.n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (lv.off[mid] <= col) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

__device__ __forceinline__ float logit_at(const LogitsView& lv, int r, int col) {
  const int s = slice_of(lv, col);
  return lv.ptr[s][static_cast<int64_t>(r) * lv.ld[s] + (col - lv.off[s])];
}

// Chunk c of row r: its first logit, its length and its first global column.
struct ChunkGeo {
  const float* src;
  int n;
  int gofs;
};

__device__ __forceinline__ ChunkGeo chunk_geo(const LogitsView& lv, const FastLayout& lay, int r,
                                              int c) {
  int s = 0;
  while (s + 1 < lay.nsl && c >= lay.cbase[s + 1]) ++s;
  const int c0 = (c - lay.cbase[s]) * lay.Ls[s];
  const int cols = static_cast<int>(lv.off[s + 1] - lv.off[s]);
  ChunkGeo g;
  g.n = min(lay.Ls[s], cols - c0);
  g.gofs = static_cast<int>(lv.off[s]) + c0;
  g.src = lv.ptr[s] + static_cast<int64_t>(r) * lv.ld[s] + c0;
  return g;
}

// ---------------------------------------------------------- block utilities
typedef double double4v __attribute__((ext_vector_type(4)));
typedef double double2v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ unsigned long long shfl_xor_u64(unsigned long long v, int mask) {
  const uint32_t lo = __shfl_xor(static_cast<uint32_t>(v), mask, kWave);
  const uint32_t hi = __shfl_xor(static_cast<uint32_t>(v >> 32), mask, kWave);
  return (static_cast<unsigned long long>(hi) << 32) | lo;
}

__device__ __forceinline__ int next_pow2(int x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}

// Radix digit search from the top bin down over `nb` LDS counts (NT threads,
// nb <= NT * BPT): finds d with above(d) < rem <= above(d) + cnt[d], where
// above(d) counts bins > d.  Writes d and above(d) to *sel_d / *sel_above.
template <int NT, int BPT>
__device__ void select_digit_top(const uint32_t* cnt, int nb, uint32_t rem, uint32_t* scratch,
                                 uint32_t* sel_d, uint32_t* sel_above) {
  uint32_t h[BPT];
  uint32_t s = 0;
#pragma unroll
  for (int j = 0; j < BPT; ++j) {
    const int b = nb - 1 - (static_cast<int>(threadIdx.x) * BPT + j);
    h[j] = b >= 0 ? cnt[b] : 0u;
    s += h[j];
  }
  uint32_t total;
  uint32_t ex = block_exclusive_scan<NT, uint32_t>(s, scratch, total);
#pragma unroll
  for (int j = 0; j < BPT; ++j) {
    const int b = nb - 1 - (static_cast<int>(threadIdx.x) * BPT + j);
    if (b >= 0 && ex < rem && rem <= ex + h[j]) {
      *sel_d = static_cast<uint32_t>(b);
      *sel_above = ex;
    }
    ex += h[j];
  }
  __syncthreads();
}

// ----------------------------------------------------------------- launchers
// Finishes probe rows and computes exact rows (all rows when lay == nullptr).
hipError_t launch_sampler_finish(const SamplerArgs& a, const FastLayout* lay, uint8_t* ws,
                                 hipStream_t stream);

}  // namespace ts
