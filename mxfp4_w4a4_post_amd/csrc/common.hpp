// Shared device-side definitions of the MACaQ HIP library (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace macaq {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

// E2M1 element code of the MXFP4 format in the MFMA format selectors.
constexpr int kFmtFp4 = 4;

// Number of XCDs on MI355X: consecutive workgroups are dispatched round-robin
// over them, and each XCD has its own L2.
constexpr int kNumXcd = 8;

// GEMM layout of a packed MXFP4 operand (rows x K elements): rows padded to
// a multiple of 64, K to a multiple of 128, padding all zero.
//   codes: 16 rows x 128 elements per 1024-byte block, blocks ordered
//          (row block, k block); inside a block row r at r * 64, element
//          pair (2j, 2j+1) at byte j (low nibble first).
//   scales: 64 rows x 4 groups per 256-byte block, blocks ordered
//          (64-row block, k block); inside a block row r at r * 4 + g.
constexpr int kTileRows = 16;
constexpr int kTileK = 128;
constexpr int kCodeBlock = kTileRows * kTileK / 2;     // 1024
constexpr int kScaleRows = 64;
constexpr int kScaleBlock = kScaleRows * kTileK / 32;  // 256
constexpr int kRowPad = 64;

__host__ __device__ inline int64_t pad_rows(int64_t r) { return (r + kRowPad - 1) / kRowPad * kRowPad; }
__host__ __device__ inline int64_t pad_k(int64_t k) { return (k + kTileK - 1) / kTileK * kTileK; }
__host__ __device__ inline int64_t tiled_codes_bytes(int64_t rows, int64_t K) { return pad_rows(rows) * pad_k(K) / 2; }
__host__ __device__ inline int64_t tiled_scales_bytes(int64_t rows, int64_t K) { return pad_rows(rows) * pad_k(K) / 32; }

struct QuantArgs {
  const void* x;         // bf16 or fp32 rows [M, ldx]
  int64_t M, K, ldx;
  const float* mult;     // [K] or [E, K] (grouped); nullptr = no multiply
  const int32_t* offsets;  // grouped only: [E+1], rows of expert e
  int E;
  uint8_t* codes;        // [M, K/2] row-major, or the GEMM layout
  uint8_t* scales;       // [M, K/32] row-major, or the GEMM layout
  bool tiled;            // write the GEMM layout (with its zero padding)
  int64_t kpad;          // pad_k(K)
};

hipError_t launch_calibrate(const void* xcal, int64_t R, int64_t K, int64_t ldx, float* s, hipStream_t stream);
hipError_t launch_multipliers(const float* s, int64_t K, float cb, float* a, float* r, hipStream_t stream);
// x_is_f32: input rows are fp32 (weights) instead of bf16.
hipError_t launch_quant_rows(const QuantArgs& q, int b, bool x_is_f32, hipStream_t stream);

struct GemmArgs {
  const uint8_t* a_codes;   // [M, K/2]
  const uint8_t* a_scales;  // [M, K/32]
  const uint8_t* b_codes;   // [N, K/2] (per expert when grouped)
  const uint8_t* b_scales;  // [N, K/32]
  int64_t M, N, K;
  void* y;                  // [M, ldy]
  int64_t ldy;
  bool y_bf16;
  float* partial;           // split-K partial sums [splits, M, N] (workspace)
  int splits;
  // grouped
  const int32_t* offsets;   // [E+1] or nullptr
  int32_t* tile_map;        // workspace: per m-tile (expert, first row)
  int E;
  int64_t max_mtiles;
};

struct GemmPlan {
  int cfg;         // tile configuration index
  int bm, bn;      // tile sizes
  int splits;      // split-K factor
  size_t partial_bytes;
};

GemmPlan plan_gemm(int64_t M, int64_t N, int64_t K);
GemmPlan plan_gemm_grouped(int64_t T, int E, int64_t N, int64_t K);
hipError_t launch_gemm(const GemmArgs& g, const GemmPlan& p, hipStream_t stream);
hipError_t launch_gemm_grouped(const GemmArgs& g, const GemmPlan& p, hipStream_t stream);

}  // namespace macaq
