// Output tiles of the projection kernels, written a logit row at a time.
//
// A 32 x 32 MFMA accumulator block leaves each lane holding one column (lane
// % 32) and sixteen rows of it (8 (e / 4) + 4 (lane / 32) + e % 4 for value
// e), so storing it straight from registers takes one 4-byte store per value
// per lane.  Passing the block through a small LDS scratch turns it into row
// segments: each lane then holds four consecutive columns of one row and
// writes them with a single 16-byte store, a quarter of the store
// instructions for the same bytes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ts {

// Host side: whether rows of C can take 16-byte stores (16-byte aligned base,
// leading dimension a multiple of 4 floats).
inline int rows_take_vector_stores(const float* C, int64_t ldc) {
  return (reinterpret_cast<uintptr_t>(C) % 16 == 0 && ldc % 4 == 0) ? 1 : 0;
}

// Floats of LDS scratch per wave (a 32 x 36 block: 16-byte aligned rows).
constexpr int kTileStoreStride = 36;
constexpr int kTileStoreFloats = 32 * kTileStoreStride;

// One wave writes its TM x TN accumulator blocks, block (i, j) covering rows
// row0 + 32 i .. +31 and columns col0 + 32 j .. +31 of C (row-major, leading
// dimension ldc, rows >= M and columns >= N dropped).  With SCALED, every value
// is multiplied by row_scale[row] * col_scale[col] (that product first); the
// wave reads all the scales it needs up front, in one round trip, rather than
// a few per block (one memory latency per block made the FP8 epilogue a third
// of that kernel).  The wave's scratch is lds + wave * kTileStoreFloats; every
// wave of the workgroup must be past its last read of that LDS before any
// wave calls this.  The 16-byte row stores are ordinary (write-back) stores:
// non-temporal ones were slower for the FP8 kernel and no faster for the bf16
// one.  A ragged column tail falls back to 4-byte stores.
template <bool SCALED, int TM, int TN, typename Acc>
__device__ __forceinline__ void store_tile_rows(const Acc (&acc)[TM][TN], float* lds, int wave,
                                                int lane, float* __restrict__ C, int64_t ldc,
                                                int row0, int col0, int M, int N,
                                                const float* __restrict__ row_scale,
                                                const float* __restrict__ col_scale) {
  typedef float f32x4v __attribute__((ext_vector_type(4)));
  constexpr int SP = kTileStoreStride;
  float* scr = lds + wave * kTileStoreFloats;
  const int frow = lane & 31, fhalf = lane >> 5;
  const int c0 = (lane & 7) * 4;  // this lane's four columns within a block row
  // Scales of this lane's rows (four per row block) and columns (four per
  // column block); a column past N gets 0 (never stored), a row past M 1.
  float rsv[TM][4], csv[TN][4];
  if (SCALED) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int row = row0 + i * 32 + (lane >> 3) + 8 * q;
        rsv[i][q] = row < M ? row_scale[row] : 1.0f;
      }
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int col = col0 + j * 32 + c0 + t;
        csv[j][t] = col < N ? col_scale[col] : 0.0f;
      }
  }
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      // In by columns (the accumulator layout), out by rows.  Lanes read
      // what other lanes wrote, so each exchange is fenced at wavefront
      // scope: after the writes (the reads below see them) and after the
      // reads (the next block's writes cannot overtake them).
#pragma unroll
      for (int e = 0; e < 16; ++e)
        scr[(8 * (e >> 2) + 4 * fhalf + (e & 3)) * SP + frow] = acc[i][j][e];
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      const int col = col0 + j * 32 + c0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int rr = (lane >> 3) + 8 * q;
        const int row = row0 + i * 32 + rr;
        f32x4v v = *reinterpret_cast<const f32x4v*>(scr + rr * SP + c0);
        if (row >= M || col >= N) continue;
        if (SCALED) {
#pragma unroll
          for (int t = 0; t < 4; ++t) v[t] = v[t] * (rsv[i][q] * csv[j][t]);
        }
        float* dst = C + static_cast<int64_t>(row) * ldc + col;
        if (col + 3 < N) {
          *reinterpret_cast<f32x4v*>(dst) = v;
        } else {
#pragma unroll
          for (int t = 0; t < 4; ++t)
            if (col + t < N) dst[t] = v[t];
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
  }
}

}  // namespace ts
