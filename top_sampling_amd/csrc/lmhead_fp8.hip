// FP8 local vocabulary projection for batch-sharded sampling on gfx950.
//
// The pages' measured deployment is an FP8 checkpoint and their patch cluster
// unpacks e4m3 bytes (page "Qwen4Exp batch-sharded sampling: inside vLLM PR
// #61018", sections "The 1.5% estimate, and the measurement next to it" and
// "The patch cluster"); the scaling scheme is not stated.  Reading: W8A8 with
// one fp32 scale per row on both operands.  Every lm_head row and every
// hidden-state row is held as OCP E4M3 codes (no infinities, largest 448)
// times its own scale amax / 448, and
//   logits[r, v] = s_x[r] * s_w[v] * sum_h q_x[r, h] * q_w[v, h],
// over the rank's own vocabulary slice, fp32 out, never gathered.
//
// quantize_rows_e4m3_kernel turns bf16 hidden states into codes and scales
// (one workgroup per row: amax, then every element divided by the scale in
// fp32 and rounded to the nearest code, ties to even, saturating at 448).
//
// lmhead_e4m3_kernel is the contraction on the matrix cores:
// v_mfma_f32_32x32x64_f8f6f4 with both operands e4m3 (gfx950), fp32
// accumulation; products of two e4m3 values are exact in fp32.  The layout
// follows the bf16 kernel: K-contiguous operands go from global memory
// straight into double-buffered LDS (global_load_lds_dwordx4), rows of 128
// bytes (here 128 codes, so a stage covers K = 128), the 16-byte chunk index
// XOR-swizzled by the row pair.  An MFMA takes 64 K per row: a lane and the
// lane 32 above it hold 32 codes each, read as two 16-byte chunks.  The
// lm_head fragments of a 64-wide slice stay in registers while the hidden
// fragments stream one ahead of their MFMAs, which keeps the wave within 256
// registers at a 160 x 64 wave tile.  Both scales are applied when the
// accumulators are stored, which goes through LDS as in the bf16 kernel:
// row segments, 16-byte non-temporal stores.
#include <stdlib.h>

#include "ts_internal.hpp"
#include "tile_store.hpp"

namespace ts {
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kXcds = 8;
constexpr int kFbk = 128;  // codes per LDS row and per K stage
constexpr float kE4m3Max = 448.0f;

// ------------------------------------------------------------ quantization
// fp32 -> OCP E4M3 code: nearest value, ties to the even code, magnitudes of
// 448 and above (infinities included) saturate to 448, NaN gives 0x7F, the
// sign bit is the input's.  Exact: normal values round their 23-bit mantissa
// to 3 bits on the integer bits; subnormal codes count units of 2^-9.
__device__ __forceinline__ uint32_t encode_e4m3(float q) {
  const uint32_t u = __float_as_uint(q);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return 0x7fu;          // NaN
  if (a >= 0x43e00000u) return sign | 0x7eu;  // |q| >= 448
  if (a < 0x3c800000u) {                      // |q| < 2^-6: m * 2^-9, m = 0..8
    const float m = __builtin_rintf(__uint_as_float(a) * 512.0f);
    return sign | static_cast<uint32_t>(m);
  }
  uint32_t e = (a >> 23) - 127u + 7u;  // 1..15
  uint32_t keep = (a >> 20) & 7u;
  const uint32_t rest = a & 0xfffffu;
  if (rest > 0x80000u || (rest == 0x80000u && (keep & 1u))) ++keep;
  if (keep == 8u) {
    keep = 0u;
    ++e;
  }
  return sign | (e << 3) | keep;
}

constexpr int QT = 256;

__global__ __launch_bounds__(QT) void quantize_rows_e4m3_kernel(
    const uint16_t* __restrict__ in, int64_t ld_in, int cols, uint8_t* __restrict__ out,
    int64_t ld_out, float* __restrict__ scales) {
  __shared__ float red[QT / 64];
  const int r = blockIdx.x, tid = threadIdx.x;
  const uint16_t* row = in + static_cast<int64_t>(r) * ld_in;
  uint8_t* orow = out + static_cast<int64_t>(r) * ld_out;
  float amax = 0.0f;  // fmaxf drops NaN
  for (int c = tid; c < cols; c += QT)
    amax = fmaxf(amax, fabsf(__uint_as_float(static_cast<uint32_t>(row[c]) << 16)));
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
  if ((tid & 63) == 0) red[tid >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float scale = amax > 0.0f ? __fdiv_rn(amax, kE4m3Max) : 1.0f;
  if (tid == 0) scales[r] = scale;
  // Four codes per thread and store where the row allows it, one at a time
  // in the tail.
  const int c4 = (cols & ~3);
  for (int c = 4 * tid; c < c4; c += 4 * QT) {
    uint32_t w = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float x = __uint_as_float(static_cast<uint32_t>(row[c + q]) << 16);
      w |= encode_e4m3(__fdiv_rn(x, scale)) << (8 * q);
    }
    if ((reinterpret_cast<uintptr_t>(orow + c) & 3) == 0)
      *reinterpret_cast<uint32_t*>(orow + c) = w;
    else
#pragma unroll
      for (int q = 0; q < 4; ++q) orow[c + q] = static_cast<uint8_t>(w >> (8 * q));
  }
  for (int c = c4 + tid; c < cols; c += QT) {
    const float x = __uint_as_float(static_cast<uint32_t>(row[c]) << 16);
    orow[c] = static_cast<uint8_t>(encode_e4m3(__fdiv_rn(x, scale)));
  }
}

// ------------------------------------------------------------- projection
// One K stage of a wave's direct-to-LDS loads (a plain function: the host pass
// does not emit the kernel stub when the builtin sits in a lambda).
template <int LOADS, int A_LOADS, int NW, int NTLOAD>
__device__ __forceinline__ void issue_stage_e4m3(const uint8_t* const* src, uint8_t* stage,
                                                 int wave, int k0) {
#pragma unroll
  for (int q = 0; q < A_LOADS; ++q)
    __builtin_amdgcn_global_load_lds(src[q] + k0, stage + (wave + NW * q) * 1024, 16, 0, 0);
#pragma unroll
  for (int q = A_LOADS; q < LOADS; ++q)
    __builtin_amdgcn_global_load_lds(src[q] + k0, stage + (wave + NW * q) * 1024, 16, 0,
                                     NTLOAD ? 2 : 0);
}

// 32 codes of one fragment row: logical chunks 4 kk + 2 half and the next
// one, each at its swizzled slot.
__device__ __forceinline__ i32x8 frag_e4m3(const uint8_t* row_base, int swz, int kk, int half) {
  const int c0 = 4 * kk + 2 * half;
  const i32x4 lo = *reinterpret_cast<const i32x4*>(row_base + ((c0 ^ swz) << 4));
  const i32x4 hi = *reinterpret_cast<const i32x4*>(row_base + (((c0 + 1) ^ swz) << 4));
  return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

template <int BM, int BN, int WAVES_M, int WAVES_N, int NTLOAD>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N, 1) void lmhead_e4m3_kernel(
    const uint8_t* __restrict__ X, const float* __restrict__ xs, int64_t ldx,
    const uint8_t* __restrict__ W, const float* __restrict__ wsc, int64_t ldw,
    float* __restrict__ C, int64_t ldc, int M, int N, int K, int tiles_m, int tiles_total,
    int tiles_per_xcd, int vec_out) {
  constexpr int NW = WAVES_M * WAVES_N;
  constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  constexpr int TM = WM / 32, TN = WN / 32;
  constexpr int ROWS = BM + BN;
  constexpr int STAGE = ROWS * 128;  // bytes per LDS stage
  constexpr int BLOCKS = ROWS / 8;   // 1 KB blocks per stage
  constexpr int LOADS = BLOCKS / NW;
  constexpr int A_LOADS = BM / 8 / NW;
  static_assert(BLOCKS % NW == 0 && (BM / 8) % NW == 0, "blocks must split evenly over the waves");
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

  // Source of this lane's 16 bytes in each of the wave's LOADS blocks (8 rows
  // x 8 chunks per block; rows past M or N re-read the last valid row).
  const uint8_t* src[LOADS];
#pragma unroll
  for (int q = 0; q < LOADS; ++q) {
    const int row = 8 * (wave + NW * q) + (lane >> 3);
    const int c = (lane & 7) ^ ((row >> 1) & 7);
    if (q < A_LOADS)
      src[q] = X + static_cast<int64_t>(min(m0 + row, M - 1)) * ldx + c * 16;
    else
      src[q] = W + static_cast<int64_t>(min(n0 + row - BM, N - 1)) * ldw + c * 16;
  }

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  const int frow = lane & 31, fhalf = lane >> 5;
  const int arow0 = wm0 + frow, brow0 = BM + wn0 + frow;
  const int aswz = (arow0 >> 1) & 7, bswz = (brow0 >> 1) & 7;  // rows 32 apart share it

  const int ksteps = K / kFbk;
  issue_stage_e4m3<LOADS, A_LOADS, NW, NTLOAD>(src, lds, wave, 0);
  for (int ks = 0; ks < ksteps; ++ks) {
    const int cur = ks & 1;
    __builtin_amdgcn_s_waitcnt(0);  // this step's loads have landed in LDS
    __syncthreads();                // ... for every wave; the other buffer is free
    if (ks + 1 < ksteps)
      issue_stage_e4m3<LOADS, A_LOADS, NW, NTLOAD>(src, lds + (cur ^ 1) * STAGE, wave,
                                                   (ks + 1) * kFbk);
    const uint8_t* base = lds + cur * STAGE;
#pragma unroll
    for (int kk = 0; kk < kFbk / 64; ++kk) {
      i32x8 bfr[TN];
#pragma unroll
      for (int j = 0; j < TN; ++j) bfr[j] = frag_e4m3(base + (brow0 + 32 * j) * 128, bswz, kk, fhalf);
      i32x8 a_next = frag_e4m3(base + arow0 * 128, aswz, kk, fhalf);
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const i32x8 a = a_next;
        if (i + 1 < TM) a_next = frag_e4m3(base + (arow0 + 32 * (i + 1)) * 128, aswz, kk, fhalf);
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, bfr[j], acc[i][j], 0, 0,
                                                                       0, 0, 0, 0);
      }
    }
    // Schedule per 64-wide slice: the B fragments and the first A fragment
    // (two 16-byte LDS reads each), then for every row block the next A
    // fragment's reads ahead of this block's MFMAs, so each LDS read has a
    // block of MFMAs to hide behind.
#pragma unroll
    for (int kk = 0; kk < kFbk / 64; ++kk) {
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * TN + 2, 0);
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        if (i + 1 < TM) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, TN, 0);
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
      store_tile_rows<true>(acc, reinterpret_cast<float*>(lds + (((ksteps - 1) & 1) ^ 1) * STAGE),
                             wave, lane, C, ldc, m0 + wm0, n0 + wn0, M, N, xs, wsc);
    } else {
      static_assert(NW * kTileStoreFloats * 4 <= 2 * STAGE, "tile-store scratch fits the stages");
      __syncthreads();  // every wave is done reading the stage buffers
      store_tile_rows<true>(acc, reinterpret_cast<float*>(lds), wave, lane, C, ldc, m0 + wm0,
                             n0 + wn0, M, N, xs, wsc);
    }
    return;
  }
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int col = n0 + wn0 + j * 32 + frow;
    if (col >= N) continue;
    const float sw = wsc[col];
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = m0 + wm0 + i * 32 + 8 * (e >> 2) + 4 * fhalf + (e & 3);
        if (row < M)
          __builtin_nontemporal_store(acc[i][j][e] * (xs[row] * sw),
                                      C + static_cast<int64_t>(row) * ldc + col);
      }
    }
  }
}

template <int BM, int BN, int WAVES_M, int WAVES_N, int NTLOAD>
hipError_t launch_e4m3(const uint8_t* X, const float* xs, int64_t ldx, const uint8_t* W,
                       const float* wsc, int64_t ldw, float* C, int64_t ldc, int M, int N, int K,
                       hipStream_t stream) {
  const int tiles_m = (M + BM - 1) / BM;
  const int tiles_n = (N + BN - 1) / BN;
  const int total = tiles_m * tiles_n;
  const int per_xcd = (total + kXcds - 1) / kXcds;
  const int vec_out = rows_take_vector_stores(C, ldc);
  hipLaunchKernelGGL((lmhead_e4m3_kernel<BM, BN, WAVES_M, WAVES_N, NTLOAD>), dim3(per_xcd * kXcds),
                     dim3(64 * WAVES_M * WAVES_N), 0, stream, X, xs, ldx, W, wsc, ldw, C, ldc, M,
                     N, K, tiles_m, total, per_xcd, vec_out);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize_rows_e4m3(const uint16_t* in, int64_t ld_in, int rows, int cols,
                                     uint8_t* out, int64_t ld_out, float* scales,
                                     hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(quantize_rows_e4m3_kernel, dim3(rows), dim3(QT), 0, stream, in, ld_in, cols,
                     out, ld_out, scales);
  return hipGetLastError();
}

// Tile shapes as for the bf16 projection: 64 x 256 (4 waves) up to 64 rows and
// 128 x 256 (8 waves) up to 128 rows, both streaming the lm_head past the
// caches; above that 320 x 256 or 256 x 256 (8 waves), whichever pads the rows
// least.  TS_GEMM_TILE=1..4 forces one (the tests run every shape).
hipError_t launch_lmhead_e4m3(const uint8_t* hidden, const float* hidden_scales, int64_t ld_hidden,
                              const uint8_t* lm_head, const float* lm_head_scales,
                              int64_t ld_lm_head, float* logits, int64_t ld_logits, int rows,
                              int vocab, int hidden_dim, hipStream_t stream) {
  if (rows == 0 || vocab == 0) return hipSuccess;
  const char* env = getenv("TS_GEMM_TILE");
  int sel = env ? atoi(env) : 0;
  if (sel < 1 || sel > 4) {
    const int64_t pad256 = (rows + 255) / 256 * 256, pad320 = (rows + 319) / 320 * 320;
    sel = rows <= 64 ? 1 : (rows <= 128 ? 2 : (pad320 < pad256 ? 4 : 3));
  }
  switch (sel) {
    case 1:
      return launch_e4m3<64, 256, 1, 4, 1>(hidden, hidden_scales, ld_hidden, lm_head,
                                           lm_head_scales, ld_lm_head, logits, ld_logits, rows,
                                           vocab, hidden_dim, stream);
    case 2:
      return launch_e4m3<128, 256, 2, 4, 1>(hidden, hidden_scales, ld_hidden, lm_head,
                                            lm_head_scales, ld_lm_head, logits, ld_logits, rows,
                                            vocab, hidden_dim, stream);
    case 3:
      return launch_e4m3<256, 256, 2, 4, 0>(hidden, hidden_scales, ld_hidden, lm_head,
                                            lm_head_scales, ld_lm_head, logits, ld_logits, rows,
                                            vocab, hidden_dim, stream);
    default:
      return launch_e4m3<320, 256, 2, 4, 0>(hidden, hidden_scales, ld_hidden, lm_head,
                                            lm_head_scales, ld_lm_head, logits, ld_logits, rows,
                                            vocab, hidden_dim, stream);
  }
}

}  // namespace ts
