// Local vocabulary projection for batch-sharded sampling on gfx950:
// logits[r, v] = sum_h hidden[r, h] * lm_head[v, h] over the rank's own
// vocabulary slice, fp32 out, never gathered (page "Qwen4Exp batch-sharded
// sampling: inside vLLM PR #61018", sections "What batch-sharded sampling is,
// in one paragraph" and "Why three lines were the whole job").
//
// A dense bf16 contraction, so it runs on the matrix cores:
// v_mfma_f32_32x32x16_bf16 (gfx950), fp32 accumulation.  Both operands are
// K-contiguous ("NT").  A workgroup owns a BM x BN output tile and walks K in
// steps of 64 through double-buffered LDS, one barrier per step, the next
// step's loads in flight during the current step's MFMAs.  The main kernel
// loads global memory straight into LDS; a register-staged kernel covers
// hidden sizes that are not a multiple of 64.  LDS rows are 128 bytes (64
// bf16) with the 16-byte chunk index XOR-swizzled by the row pair, so the
// fragment reads of 32 consecutive rows spread over all banks.  The fp32
// logits leave through LDS: each wave turns its accumulator blocks into row
// segments and writes them with 16-byte non-temporal stores, a quarter of the
// store instructions of writing them from the MFMA layout (that epilogue cost
// about a fifth of the kernel at 640 x 151,936 x 4,096; outputs whose rows
// cannot take 16-byte stores keep the direct 4-byte path).  Tiles are ordered so that the
// workgroups sharing one lm_head strip run on the same XCD back to back (the
// strip is then read from HBM once and reused from that XCD's L2).
#include <stdlib.h>

#include "ts_internal.hpp"
#include "tile_store.hpp"

namespace ts {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kGemmThreads = 256;
constexpr int kBK = 64;        // K per LDS stage
constexpr int kChunks = kBK / 8;  // 16-byte chunks per LDS row
constexpr int kXcds = 8;

// LDS rows are 128 bytes, so consecutive rows start alternately at bank 0 and
// bank 32; XOR-ing the chunk with (row / 2) % 8 gives the 16 rows one
// ds_read_b128 pass serves 16 distinct (half, chunk) slots: no bank conflicts.
__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ ((row >> 1) & 7); }

template <int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(kGemmThreads, 1) void lmhead_gemm_kernel(
    const uint16_t* __restrict__ X, int64_t ldx, const uint16_t* __restrict__ W, int64_t ldw,
    float* __restrict__ C, int64_t ldc, int M, int N, int K, int tiles_m, int tiles_total,
    int tiles_per_xcd) {
  constexpr int WAVES_N = BN / WN;
  constexpr int TM = WM / 32, TN = WN / 32;
  constexpr int A_LOADS = BM * kChunks / kGemmThreads;
  constexpr int B_LOADS = BN * kChunks / kGemmThreads;
  static_assert((BM / WM) * (BN / WN) == 4, "4 waves per workgroup");
  static_assert(A_LOADS >= 1 && B_LOADS >= 1, "tile too small");

  __shared__ uint4 lds[2][(BM + BN) * kChunks];

  // XCD-aware tile order: dispatch places workgroup i on XCD i % 8; give each
  // XCD a contiguous run of tiles, M fastest, so an lm_head strip's M tiles
  // run together on one XCD.
  const int bid = blockIdx.x;
  const int tile = (bid % kXcds) * tiles_per_xcd + bid / kXcds;
  if (tile >= tiles_total) return;
  const int tm = tile % tiles_m, tn = tile / tiles_m;
  const int m0 = tm * BM, n0 = tn * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm0 = (wave / WAVES_N) * WM, wn0 = (wave % WAVES_N) * WN;

  // Global -> register staging of one K stage.
  uint4 ra[A_LOADS], rb[B_LOADS];
  auto load_stage = [&](int k0) {
#pragma unroll
    for (int j = 0; j < A_LOADS; ++j) {
      const int idx = tid + j * kGemmThreads;
      const int r = idx / kChunks, c = idx % kChunks;
      const int gr = m0 + r, gk = k0 + c * 8;
      ra[j] = (gr < M && gk < K) ? *reinterpret_cast<const uint4*>(X + gr * ldx + gk)
                                 : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < B_LOADS; ++j) {
      const int idx = tid + j * kGemmThreads;
      const int r = idx / kChunks, c = idx % kChunks;
      const int gr = n0 + r, gk = k0 + c * 8;
      rb[j] = (gr < N && gk < K) ? *reinterpret_cast<const uint4*>(W + gr * ldw + gk)
                                 : make_uint4(0, 0, 0, 0);
    }
  };
  auto store_stage = [&](int buf) {
#pragma unroll
    for (int j = 0; j < A_LOADS; ++j) {
      const int idx = tid + j * kGemmThreads;
      const int r = idx / kChunks, c = idx % kChunks;
      lds[buf][r * kChunks + swz(r, c)] = ra[j];
    }
#pragma unroll
    for (int j = 0; j < B_LOADS; ++j) {
      const int idx = tid + j * kGemmThreads;
      const int r = idx / kChunks, c = idx % kChunks;
      lds[buf][(BM + r) * kChunks + swz(r, c)] = rb[j];
    }
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  const int ksteps = (K + kBK - 1) / kBK;
  load_stage(0);
  store_stage(0);
  __syncthreads();

  // Fragment of a 32-row block: lane holds row (lane % 32) and 8 consecutive
  // K values starting at (lane / 32) * 8 within the 16-wide K slice.
  const int frow = lane & 31, fhalf = lane >> 5;
  for (int ks = 0; ks < ksteps; ++ks) {
    const int cur = ks & 1;
    if (ks + 1 < ksteps) load_stage((ks + 1) * kBK);
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      const int chunk = kk * 2 + fhalf;
      bf16x8 af[TM], bfr[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int r = wm0 + i * 32 + frow;
        af[i] = *reinterpret_cast<const bf16x8*>(&lds[cur][r * kChunks + swz(r, chunk)]);
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int r = wn0 + j * 32 + frow;
        bfr[j] = *reinterpret_cast<const bf16x8*>(&lds[cur][(BM + r) * kChunks + swz(r, chunk)]);
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (ks + 1 < ksteps) store_stage(cur ^ 1);
    __syncthreads();
  }

  // Epilogue: accumulator element e of a 32x32 block sits at row
  // 8 * (e / 4) + 4 * (lane / 32) + (e % 4), column lane % 32.
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int col = n0 + wn0 + j * 32 + frow;
      if (col >= N) continue;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = m0 + wm0 + i * 32 + 8 * (e >> 2) + 4 * fhalf + (e & 3);
        if (row < M) __builtin_nontemporal_store(acc[i][j][e], C + static_cast<int64_t>(row) * ldc + col);
      }
    }
  }
}

// One K stage of a wave's direct-to-LDS loads (a plain function: the host
// pass does not emit the kernel stub when the builtin sits in a lambda).
template <int LOADS, int A_LOADS, int NW, int NTLOAD>
__device__ __forceinline__ void issue_stage(const uint16_t* const* src, uint8_t* stage,
                                            int wave, int k0) {
#pragma unroll
  for (int q = 0; q < A_LOADS; ++q)
    __builtin_amdgcn_global_load_lds(src[q] + k0, stage + (wave + NW * q) * 1024, 16, 0, 0);
#pragma unroll
  for (int q = A_LOADS; q < LOADS; ++q)
    __builtin_amdgcn_global_load_lds(src[q] + k0, stage + (wave + NW * q) * 1024, 16, 0,
                                     NTLOAD ? 2 : 0);
}

template <int TM, int TN>
constexpr int kMfmaPerRead = (TM * TN) / (TM + TN) > 0 ? (TM * TN) / (TM + TN) : 1;

// ---------------------------------------------------------------------------
// Main kernel (K a multiple of 64): operands go from global memory straight
// into LDS (global_load_lds_dwordx4, no register staging), double-buffered.
// Each wave load fills one 1 KB block of LDS = 8 rows x 8 chunks, lane i
// writing slot i; the swizzle is applied by choosing which global chunk lane i
// fetches.  Rows past M or N re-read the last valid row (their results are
// never stored).  NTLOAD streams the lm_head rows past the caches (for one
// row tile, where nothing re-reads them).  Per 64-wide K step every wave reads its fragments for the
// next 16-wide slice while the MFMAs of the current slice run.
template <int BM, int BN, int WAVES_M, int WAVES_N, int NTLOAD>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N, 1) void lmhead_gemm_dl_kernel(
    const uint16_t* __restrict__ X, int64_t ldx, const uint16_t* __restrict__ W, int64_t ldw,
    float* __restrict__ C, int64_t ldc, int M, int N, int K, int tiles_m, int tiles_total,
    int tiles_per_xcd, int vec_out) {
  constexpr int NW = WAVES_M * WAVES_N;
  constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  constexpr int TM = WM / 32, TN = WN / 32;
  constexpr int ROWS = BM + BN;
  constexpr int STAGE = ROWS * 128;  // bytes per LDS stage
  constexpr int BLOCKS = ROWS / 8;   // 1 KB blocks per stage
  constexpr int LOADS = BLOCKS / NW; // wave loads per stage
  static_assert(BLOCKS % NW == 0 && (BM / 8) % NW == 0, "blocks must split evenly over the waves");
  constexpr int A_LOADS = BM / 8 / NW;  // the first A_LOADS of a wave's loads are hidden rows
  static_assert(WM % 32 == 0 && WN % 32 == 0, "wave tile of whole 32x32 blocks");

  __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * STAGE];

  const int bid = blockIdx.x;
  const int tile = (bid % kXcds) * tiles_per_xcd + bid / kXcds;
  if (tile >= tiles_total) return;
  const int tm = tile % tiles_m, tn = tile / tiles_m;
  const int m0 = tm * BM, n0 = tn * BN;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm0 = (wave / WAVES_N) * WM, wn0 = (wave % WAVES_N) * WN;

  // Source of this lane's 16 bytes in each of the wave's LOADS blocks.
  const uint16_t* src[LOADS];
#pragma unroll
  for (int q = 0; q < LOADS; ++q) {
    const int row = 8 * (wave + NW * q) + (lane >> 3);
    const int c = (lane & 7) ^ ((row >> 1) & 7);
    if (q < A_LOADS) {
      const int gr = min(m0 + row, M - 1);
      src[q] = X + static_cast<int64_t>(gr) * ldx + c * 8;
    } else {
      const int gr = min(n0 + row - BM, N - 1);
      src[q] = W + static_cast<int64_t>(gr) * ldw + c * 8;
    }
  }

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  const int frow = lane & 31, fhalf = lane >> 5;
  // Byte offsets (within a stage) of this lane's fragment rows, chunk 0.
  int aoff[TM], boff[TN], aswz[TM], bswz[TN];
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int r = wm0 + i * 32 + frow;
    aoff[i] = r * 128;
    aswz[i] = (r >> 1) & 7;
  }
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int r = BM + wn0 + j * 32 + frow;
    boff[j] = r * 128;
    bswz[j] = (r >> 1) & 7;
  }
  auto frags = [&](int buf, int kk, bf16x8 (&af)[TM], bf16x8 (&bfr)[TN]) {
    const int chunk = kk * 2 + fhalf;
    const uint8_t* base = lds + buf * STAGE;
#pragma unroll
    for (int i = 0; i < TM; ++i)
      af[i] = *reinterpret_cast<const bf16x8*>(base + aoff[i] + ((chunk ^ aswz[i]) << 4));
#pragma unroll
    for (int j = 0; j < TN; ++j)
      bfr[j] = *reinterpret_cast<const bf16x8*>(base + boff[j] + ((chunk ^ bswz[j]) << 4));
  };

  const int ksteps = K / kBK;
  issue_stage<LOADS, A_LOADS, NW, NTLOAD>(src, lds, wave, 0);
  for (int ks = 0; ks < ksteps; ++ks) {
    const int cur = ks & 1;
    __builtin_amdgcn_s_waitcnt(0);  // this step's loads have landed in LDS
    __syncthreads();                // ... for every wave; the other buffer is free
    if (ks + 1 < ksteps)
      issue_stage<LOADS, A_LOADS, NW, NTLOAD>(src, lds + (cur ^ 1) * STAGE, wave, (ks + 1) * kBK);
    bf16x8 af[2][TM], bfr[2][TN];
    frags(cur, 0, af[0], bfr[0]);
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      if (kk + 1 < kBK / 16) frags(cur, kk + 1, af[(kk + 1) & 1], bfr[(kk + 1) & 1]);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[kk & 1][i], bfr[kk & 1][j],
                                                               acc[i][j], 0, 0, 0);
    }
    // Schedule: this step's first fragments, then per 16-wide slice its MFMAs
    // with the next slice's fragment reads spread between them.
    __builtin_amdgcn_sched_group_barrier(0x100, TM + TN, 0);
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      if (kk + 1 < kBK / 16) {
#pragma unroll
        for (int t = 0; t < TM + TN; ++t) {
          __builtin_amdgcn_sched_group_barrier(0x008, kMfmaPerRead<TM, TN>, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        if (TM * TN > kMfmaPerRead<TM, TN> * (TM + TN))
          __builtin_amdgcn_sched_group_barrier(0x008, TM * TN - kMfmaPerRead<TM, TN> * (TM + TN), 0);
      } else {
        __builtin_amdgcn_sched_group_barrier(0x008, TM * TN, 0);
      }
    }
  }

  if (vec_out) {
    // Scratch in the stage buffer the last step did not use, when one buffer
    // holds every wave's: every wave was done reading it at that step's
    // barrier and nothing was loaded into it, so each wave starts its
    // epilogue as soon as its own MFMAs are issued.  Otherwise the scratch
    // spans both buffers, after a barrier.
    if constexpr (NW * kTileStoreFloats * 4 <= STAGE) {
      store_tile_rows<false>(acc, reinterpret_cast<float*>(lds + (((ksteps - 1) & 1) ^ 1) * STAGE),
                             wave, lane, C, ldc, m0 + wm0, n0 + wn0, M, N, nullptr, nullptr);
    } else {
      static_assert(NW * kTileStoreFloats * 4 <= 2 * STAGE, "tile-store scratch fits the stages");
      __syncthreads();  // every wave is done reading the stage buffers
      store_tile_rows<false>(acc, reinterpret_cast<float*>(lds), wave, lane, C, ldc, m0 + wm0,
                             n0 + wn0, M, N, nullptr, nullptr);
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int col = n0 + wn0 + j * 32 + frow;
      if (col >= N) continue;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = m0 + wm0 + i * 32 + 8 * (e >> 2) + 4 * fhalf + (e & 3);
        if (row < M)
          __builtin_nontemporal_store(acc[i][j][e], C + static_cast<int64_t>(row) * ldc + col);
      }
    }
  }
}

template <int BM, int BN, int WAVES_M, int WAVES_N, int NTLOAD>
hipError_t launch_dl(const uint16_t* X, int64_t ldx, const uint16_t* W, int64_t ldw, float* C,
                     int64_t ldc, int M, int N, int K, hipStream_t stream) {
  const int tiles_m = (M + BM - 1) / BM;
  const int tiles_n = (N + BN - 1) / BN;
  const int total = tiles_m * tiles_n;
  const int per_xcd = (total + kXcds - 1) / kXcds;
  const int vec_out = rows_take_vector_stores(C, ldc);
  hipLaunchKernelGGL((lmhead_gemm_dl_kernel<BM, BN, WAVES_M, WAVES_N, NTLOAD>),
                     dim3(per_xcd * kXcds), dim3(64 * WAVES_M * WAVES_N), 0, stream, X, ldx, W, ldw,
                     C, ldc, M, N, K, tiles_m, total, per_xcd, vec_out);
  return hipGetLastError();
}

template <int BM, int BN, int WM, int WN>
hipError_t launch_cfg(const uint16_t* X, int64_t ldx, const uint16_t* W, int64_t ldw, float* C,
                      int64_t ldc, int M, int N, int K, hipStream_t stream) {
  const int tiles_m = (M + BM - 1) / BM;
  const int tiles_n = (N + BN - 1) / BN;
  const int total = tiles_m * tiles_n;
  const int per_xcd = (total + kXcds - 1) / kXcds;
  hipLaunchKernelGGL((lmhead_gemm_kernel<BM, BN, WM, WN>), dim3(per_xcd * kXcds),
                     dim3(kGemmThreads), 0, stream, X, ldx, W, ldw, C, ldc, M, N, K, tiles_m,
                     total, per_xcd);
  return hipGetLastError();
}

}  // namespace

// Tile shapes (rows x vocab per workgroup, waves): the default picks the
// shape that pads the row count least; TS_GEMM_TILE=<n> forces shape n (the
// tests run every shape).  1: 64x128/4 waves and 2: 128x128/8 waves stream
// the lm_head past the caches (one row tile reads it once; 128-wide strips
// give twice the workgroups of 256-wide ones, so the last round over the
// CUs is not left a third full at a 151,936-row lm_head); 3: 256x256/8;
// 4: 320x256/8; 5: the register-staged kernel (also used when the hidden size
// is not a multiple of 64).
hipError_t launch_lmhead_gemm(const uint16_t* hidden, int64_t ld_hidden, const uint16_t* lm_head,
                              int64_t ld_lm_head, float* logits, int64_t ld_logits, int rows,
                              int vocab, int hidden_dim, hipStream_t stream) {
  if (rows == 0 || vocab == 0) return hipSuccess;
  const char* env = getenv("TS_GEMM_TILE");
  int sel = env ? atoi(env) : 0;
  if (hidden_dim % kBK != 0) sel = 5;
  if (sel < 1 || sel > 5) {
    const int64_t pad256 = (rows + 255) / 256 * 256, pad320 = (rows + 319) / 320 * 320;
    sel = rows <= 64 ? 1 : (rows <= 128 ? 2 : (pad320 < pad256 ? 4 : 3));
  }
  switch (sel) {
    case 1:
      return launch_dl<64, 128, 1, 4, 1>(hidden, ld_hidden, lm_head, ld_lm_head, logits, ld_logits,
                                         rows, vocab, hidden_dim, stream);
    case 2:
      return launch_dl<128, 128, 2, 4, 1>(hidden, ld_hidden, lm_head, ld_lm_head, logits, ld_logits,
                                          rows, vocab, hidden_dim, stream);
    case 3:
      return launch_dl<256, 256, 2, 4, 0>(hidden, ld_hidden, lm_head, ld_lm_head, logits, ld_logits,
                                          rows, vocab, hidden_dim, stream);
    case 4:
      return launch_dl<320, 256, 2, 4, 0>(hidden, ld_hidden, lm_head, ld_lm_head, logits, ld_logits,
                                          rows, vocab, hidden_dim, stream);
    default:
      break;
  }
  if (rows <= 64)
    return launch_cfg<64, 256, 64, 64>(hidden, ld_hidden, lm_head, ld_lm_head, logits, ld_logits,
                                       rows, vocab, hidden_dim, stream);
  if (rows <= 128)
    return launch_cfg<128, 256, 64, 128>(hidden, ld_hidden, lm_head, ld_lm_head, logits,
                                         ld_logits, rows, vocab, hidden_dim, stream);
  return launch_cfg<256, 256, 128, 128>(hidden, ld_hidden, lm_head, ld_lm_head, logits, ld_logits,
                                        rows, vocab, hidden_dim, stream);
}

}  // namespace ts
