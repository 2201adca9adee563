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

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// bf16(lo) | bf16(hi) << 16, each rounded to nearest even (NaN stays NaN):
// one packed conversion instruction on gfx950.
__device__ __forceinline__ uint32_t bf16x2_rne(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// E2M1 element code of the MXFP4 format in the MFMA format selectors.
constexpr int kFmtFp4 = 4;

// Number of XCDs on MI355X: consecutive workgroups are dispatched round-robin
// over them, and each XCD has its own L2.
constexpr int kNumXcd = 8;

// GEMM layout of a packed MXFP4 operand (rows x K elements): rows padded to a
// multiple of 32, K to a multiple of 256, padding all zero. The operand is cut
// into blocks of 32 rows x 256 elements, ordered (row group, k block). Inside
// a block the 8 chunks of 32 elements of a row are numbered c = 2h + j
// (h = 0..3, j = 0..1), and
//   codes:  4096 bytes; chunk (r, c) holds 16 bytes at h*1024 + (32j + r)*16
//           (element pair (2i, 2i+1) of the chunk at byte i, low nibble first);
//   scales: 256 bytes; the E8M0 byte of chunk (r, c) at (32j + r)*4 + h.
// So 1 KiB of codes (h fixed) is exactly the operand of one scaled-FP4 MFMA
// 32x32x64 over K elements [64h, 64h + 64) of the block (lane l = 32j + r), and
// one dword per lane holds the lane's scales for the 4 MFMAs of the block.
constexpr int kGroupRows = 32;
constexpr int kBlockK = 256;
constexpr int kCodeBlock = kGroupRows * kBlockK / 2;      // 4096
constexpr int kCodeHalf = kCodeBlock / 4;                 // 1024: one MFMA operand
constexpr int kScaleBlock = kGroupRows * kBlockK / 32;    // 256

__host__ __device__ inline int64_t pad_rows(int64_t r) { return (r + kGroupRows - 1) / kGroupRows * kGroupRows; }
__host__ __device__ inline int64_t pad_k(int64_t k) { return (k + kBlockK - 1) / kBlockK * kBlockK; }
__host__ __device__ inline int64_t tiled_codes_bytes(int64_t rows, int64_t K) { return pad_rows(rows) * pad_k(K) / 2; }
__host__ __device__ inline int64_t tiled_scales_bytes(int64_t rows, int64_t K) { return pad_rows(rows) * pad_k(K) / 32; }

// Byte offsets of element k's code byte and of its group's scale for row r.
__host__ __device__ inline int64_t tiled_code_offset(int64_t r, int64_t k, int64_t kpad) {
  const int64_t c = (k % kBlockK) / 32;
  return ((r / kGroupRows) * (kpad / kBlockK) + k / kBlockK) * kCodeBlock + (c >> 1) * kCodeHalf +
         ((c & 1) * kGroupRows + r % kGroupRows) * 16 + (k % 32) / 2;
}
__host__ __device__ inline int64_t tiled_scale_offset(int64_t r, int64_t k, int64_t kpad) {
  const int64_t c = (k % kBlockK) / 32;
  return ((r / kGroupRows) * (kpad / kBlockK) + k / kBlockK) * kScaleBlock +
         ((c & 1) * kGroupRows + r % kGroupRows) * 4 + (c >> 1);
}

struct QuantArgs {
  const void* x;         // bf16 or fp32 rows [M, ldx]
  int64_t M, K, ldx;
  const float* mult;     // [K] or [E, K] (grouped); nullptr = no multiply
  const int32_t* row_expert;  // grouped only: [M], the expert of each row (its multipliers' row)
  uint8_t* codes;        // [M, K/2] row-major, or the GEMM layout
  uint8_t* scales;       // [M, K/32] row-major, or the GEMM layout
  bool tiled;            // write the GEMM layout (with its zero padding)
  int64_t kpad;          // pad_k(K)
  const int32_t* gather;  // optional: row r reads x row gather[r] (clamped to [0, src_rows))
  int64_t src_rows;
};

// s = (column max of |xcal|)^(quarters / 4), quarters in {0, 1, 2, 4}
hipError_t launch_calibrate(const void* xcal, int64_t R, int64_t K, int64_t ldx, int quarters, float* s,
                            hipStream_t stream);
hipError_t launch_multipliers(const float* s, int64_t K, float cb, float* a, float* r, hipStream_t stream);
// x_is_f32: input rows are fp32 (weights) instead of bf16.
hipError_t launch_quant_rows(const QuantArgs& q, int b, bool x_is_f32, hipStream_t stream);
// out[r] = the expert of row r of an expert-major row set (the largest e < E
// with off[e] <= r), for rows r in [0, rows).
hipError_t launch_row_expert(const int32_t* off, int E, int64_t rows, int32_t* out, hipStream_t stream);

struct GemmArgs {
  const uint8_t* a_codes;   // GEMM layout, M rows (T rows when grouped)
  const uint8_t* a_scales;
  const uint8_t* b_codes;   // GEMM layout, N rows (per expert when grouped)
  const uint8_t* b_scales;
  int64_t M, N, K;
  void* y;                  // [M, ldy]
  int64_t ldy;
  bool y_bf16;
  float* partial;           // split-K partial sums [splits, M, N] (workspace)
  int splits;
  // grouped
  const int32_t* offsets;   // [E+1] or nullptr
  int32_t* tile_map;        // workspace: per m-tile (expert, first row), then the used count
  int E;
  int64_t max_mtiles;
  bool map_ready;           // grouped: tile_map already holds the map of these offsets
  // grouped SwiGLU epilogue (MoE gate/up): instead of Y, write the down
  // projection's MXFP4 input h = SiLU(gate) * up through its multiplier and
  // block-Hadamard; B's rows alternate blocks of 32 gate and 32 up rows
  bool swiglu;
  uint8_t* q_codes;         // GEMM layout [M, q_F]
  uint8_t* q_scales;
  const float* q_mult;      // [E, q_F] or nullptr
  int64_t q_F;              // channels (N = 2 q_F)
  int q_b;                  // Hadamard block of the down input
  // set by the launcher: outputs may be stored as 4-element vectors
  bool vec_y, vec_partial, vec16_y;
};

struct GemmPlan {
  int cfg;         // tile configuration index
  int bm, bn;      // tile sizes
  int splits;      // split-K factor
  size_t partial_bytes;
};

GemmPlan plan_gemm(int64_t M, int64_t N, int64_t K);
// swiglu: the MoE gate/up GEMM with the SwiGLU epilogue (its own tile shape)
GemmPlan plan_gemm_grouped(int64_t T, int E, int64_t N, int64_t K, bool swiglu = false);
hipError_t launch_gemm(const GemmArgs& g, const GemmPlan& p, hipStream_t stream);
// Upper bound on the workgroups of every persistent GEMM launch (0: the
// planned grid); the stress hook of the tests.
void set_workgroup_cap(int32_t n);
hipError_t launch_gemm_grouped(const GemmArgs& g, const GemmPlan& p, hipStream_t stream);

// Exclusive prefix sum of v over a workgroup of NTH threads (Hillis-Steele
// in the LDS array sh[NTH]); *total receives the sum of every thread's v.
// Every thread of the workgroup must call it.
template <int NTH>
__device__ __forceinline__ int block_exclusive_scan(int v, int* sh, int* total) {
  const int tid = threadIdx.x;
  sh[tid] = v;
  __syncthreads();
  for (int d = 1; d < NTH; d <<= 1) {
    const int t = tid >= d ? sh[tid - d] : 0;
    __syncthreads();
    sh[tid] += t;
    __syncthreads();
  }
  const int incl = sh[tid];
  *total = sh[NTH - 1];
  __syncthreads();
  return incl - v;
}

// MoE block: routing (chunks of 1024 entries, at most kMaxExperts experts;
// counts: int32 scratch [moe_route_chunks(T*k), E]) and the weighted combine
// of bf16 expert rows.
constexpr int kMaxExperts = 4096;
int64_t moe_route_chunks(int64_t n);
// Tile maps of grouped GEMMs over the routed rows that the routing can write
// as it goes (map[i] == nullptr: none), each of max_mtiles entries.
struct RouteMaps {
  int32_t* map[2];
  int bm[2];
  int64_t max_mtiles;
};
// row_expert (optional, [T*k]): the expert of each row, E - 1 past the routed rows.
hipError_t launch_moe_route(const int32_t* ids, int64_t T, int k, int E, int32_t* offsets, int32_t* row_token,
                            int32_t* pos, int32_t* counts, const RouteMaps& maps, int32_t* row_expert,
                            hipStream_t stream);
hipError_t launch_moe_combine(const uint16_t* rows, int64_t H, const int32_t* pos, const float* w, int64_t T, int k,
                              void* y, bool y_bf16, int64_t ldy, hipStream_t stream);

// Measurement probes: back-to-back scaled-FP4 MFMAs on register operands
// (ops: 24576 bytes, out: workgroups * 256 floats) and a plain read of
// `bytes` at src (out: workgroups * 256 words).
hipError_t launch_mfma_probe(const void* ops, int workgroups, int iters, float* out, hipStream_t stream);
hipError_t launch_read_probe(const void* src, int64_t bytes, int workgroups, uint32_t* out, hipStream_t stream);

// Flip-Refinement: the Hessian of transformed calibration rows (xt: R x K fp32
// scratch) and the greedy code moves (E, G: N x K fp64 scratch, hdiag: K).
hipError_t launch_hessian(const void* xcal, int64_t R, int64_t K, int64_t ldx, const float* a, int b, float* xt,
                          double* H, hipStream_t stream);
hipError_t launch_flip_refine(const void* W, bool w_f32, int64_t N, int64_t K, int64_t ldw, const float* r, int b,
                              const double* H, int max_flips, uint8_t* codes, const uint8_t* scales, int32_t* flips,
                              double* E, double* G, double* hdiag, hipStream_t stream);

}  // namespace macaq
