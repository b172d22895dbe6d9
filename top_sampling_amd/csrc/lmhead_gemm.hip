// Local vocabulary projection for batch-sharded sampling on gfx950:
// logits[r, v] = sum_h hidden[r, h] * lm_head[v, h] over the rank's own
// vocabulary slice, fp32 out, never gathered (page "Qwen4Exp batch-sharded
// sampling: inside vLLM PR #61018", sections "What batch-sharded sampling is,
// in one paragraph" and "Why three lines were the whole job").
//
// A dense bf16 contraction, so it runs on the matrix cores:
// v_mfma_f32_32x32x16_bf16 (gfx950), fp32 accumulation.  Both operands are
// K-contiguous ("NT").  A workgroup of 4 waves owns a BM x BN output tile and
// walks K in steps of 64 through double-buffered LDS (one barrier per step,
// the next step's global loads in flight during the current step's MFMAs).
// LDS rows are 128 bytes (64 bf16) with the 16-byte chunk index XOR-swizzled
// by the row, so the fragment reads of 32 consecutive rows spread over banks.
// Tiles are ordered so that the workgroups sharing one lm_head strip run on
// the same XCD back to back (the strip is then read from HBM once and reused
// from that XCD's L2).
#include "ts_internal.hpp"

namespace ts {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kGemmThreads = 256;
constexpr int kBK = 64;        // K per LDS stage
constexpr int kChunks = kBK / 8;  // 16-byte chunks per LDS row
constexpr int kXcds = 8;

__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ (row & 7); }

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
        if (row < M) C[static_cast<int64_t>(row) * ldc + col] = acc[i][j][e];
      }
    }
  }
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

hipError_t launch_lmhead_gemm(const uint16_t* hidden, int64_t ld_hidden, const uint16_t* lm_head,
                              int64_t ld_lm_head, float* logits, int64_t ld_logits, int rows,
                              int vocab, int hidden_dim, hipStream_t stream) {
  if (rows == 0 || vocab == 0) return hipSuccess;
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
