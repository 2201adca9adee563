// Online activation transform and MXFP4 quantization (gfx950).
//
// Method: "MACaQ: Fast, Model Agnostic Calibrated Quantization for
// Low-Precision Weights and Activations" (paper card, Abstract) applies a
// per-channel scale and a block-Hadamard transform to each layer's
// activations at inference and quantizes to MXFP4; the same row transform with
// the weight-side multiplier produces the absorbed weights offline.
//
// The encode and nibble packing use the hardware scaled FP4 convert, which
// rounds to nearest-even, saturates at 6 and keeps the sign (it only reads
// the exponent of its fp32 scale operand).
#include "mx_lane.hpp"

namespace macaq {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Largest e in [0, E) with off[e] <= row (the expert that owns `row`).
__device__ __forceinline__ int expert_of_row(const int32_t* __restrict__ off, int E, int64_t row) {
  int lo = 0, hi = E;
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if ((int64_t)off[mid] <= row) lo = mid;
    else hi = mid;
  }
  return lo;
}

// One lane per MX group: a workgroup covers one block of the GEMM layout (32
// rows x 256 elements). Consecutive workgroups take consecutive k-blocks of
// the same 32 rows (a one-dimensional grid, k-block fastest), so neighbouring
// workgroups read consecutive pieces of each row and write consecutive blocks
// of the GEMM layout; with the row block fastest instead, the same kernel
// reads and writes 16-57 KB apart and runs 8-24% slower on 8192-row inputs.
// Lane (r, c) = (tid / 8, tid % 8) owns elements
// [32c, 32c + 32) of row r of the block. Butterflies of span 1 .. 16 stay in
// the lane; spans 32 and 64 (Hadamard blocks of 64 and 128) pair the lanes of
// chunks c ^ 1 and c ^ 2 of the same row. Eight lanes of a row load 512
// contiguous bytes; eight lanes of a chunk store 128 contiguous bytes of the
// GEMM layout (rows r .. r+7 of one chunk), or a row's 128 code bytes in the
// row-major layout.
// TILED: write the GEMM layout, including its zero padding; otherwise
// row-major [M, K/2] codes and [M, K/32] scales. The grouped GEMM-layout
// variants (the MoE inputs) are held to 8 waves per SIMD (59 VGPRs, no
// spills; left alone they take 68 and run at 7), which hides more of their
// gathered rows' latency.
template <bool F32_IN, int B, bool SCALE, bool GROUPED, bool TILED>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(GROUPED && TILED && !F32_IN ? 8 : 1))) void quant_rows_kernel(QuantArgs q) {
  const int tid = threadIdx.x;
  const int c = tid & 7;
  const int64_t nkb = q.kpad / kBlockK;
  const int64_t rb = (int64_t)blockIdx.x / nkb, kb = (int64_t)blockIdx.x - rb * nkb;
  const int64_t row = rb * kGroupRows + (tid >> 3);
  const int64_t k0 = kb * kBlockK + c * 32;
  const bool valid = row < q.M && k0 < q.K;

  // Load order matters: the vector-memory counter completes in issue order,
  // so a wait for a load also waits for every load issued before it. The
  // small loads that the block's barrier depends on (the MoE gather index,
  // the row experts, the multipliers) therefore go out before the rows'
  // values, and the barrier waits for them only, not for the rows.
  int64_t src = row < q.M ? row : q.M - 1;  // lanes past M read a row inside it
  if (q.gather) {  // MoE rows read their token's activations
    src = q.gather[src];
    src = src < 0 ? 0 : (src >= q.src_rows ? q.src_rows - 1 : src);
  }
  // The block's 256 multipliers are shared by its 32 rows: staged in LDS
  // once. Grouped rows take their expert's multipliers (the experts of the
  // block's first and last rows are uniform loads; a block whose rows span
  // two experts (rows are expert-major) has each lane read its own).
  __shared__ __attribute__((aligned(16))) float msh[kBlockK];
  bool staged = false;
  int e_lane = 0;  // grouped, not staged: this lane's expert
  float mval = 0.0f;
  if constexpr (SCALE) {
    const float* mrow = q.mult;
    staged = true;
    if constexpr (GROUPED) {
      const int64_t r0 = rb * kGroupRows;
      const int64_t r1 = (r0 + kGroupRows - 1 < q.M ? r0 + kGroupRows - 1 : q.M - 1);
      const int e0 = q.row_expert[r0 < q.M ? r0 : q.M - 1];
      staged = e0 == q.row_expert[r1];
      if (!staged) e_lane = q.row_expert[row < q.M ? row : q.M - 1];
      mrow += (int64_t)e0 * q.K;
    }
    if (staged) {
      const int64_t kk = kb * kBlockK + tid;
      mval = kk < q.K ? mrow[kk] : 0.0f;
    }
  }
  __builtin_amdgcn_sched_barrier(0);  // keep the rows' loads after these

  // every lane loads (a lane past K reads elements 0 .. 31 of its row and,
  // like a lane past M, takes zeros below), so the loads are branch-free and
  // the waits above count exactly the loads issued after theirs
  uint4 raw[F32_IN ? 8 : 4];
  {
    const int64_t kl = k0 < q.K ? k0 : 0;
    const uint4* p = F32_IN ? reinterpret_cast<const uint4*>(static_cast<const float*>(q.x) + src * q.ldx + kl)
                            : reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(q.x) + src * q.ldx + kl);
#pragma unroll
    for (int i = 0; i < (F32_IN ? 8 : 4); ++i) raw[i] = p[i];
  }
  if (SCALE && staged) {
    msh[tid] = mval;
    __syncthreads();
  }

  float v[32];
  if (valid) {
    if constexpr (F32_IN) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        v[4 * i] = __uint_as_float(raw[i].x);
        v[4 * i + 1] = __uint_as_float(raw[i].y);
        v[4 * i + 2] = __uint_as_float(raw[i].z);
        v[4 * i + 3] = __uint_as_float(raw[i].w);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint4 w = raw[i];
        v[8 * i] = bf16_lo(w.x);
        v[8 * i + 1] = bf16_hi(w.x);
        v[8 * i + 2] = bf16_lo(w.y);
        v[8 * i + 3] = bf16_hi(w.y);
        v[8 * i + 4] = bf16_lo(w.z);
        v[8 * i + 5] = bf16_hi(w.z);
        v[8 * i + 6] = bf16_lo(w.w);
        v[8 * i + 7] = bf16_hi(w.w);
      }
    }
    if constexpr (SCALE) {
      // the multipliers from LDS or (a block across two experts) from memory:
      // two paths, so each reads its own address space
      float4 u[8];
      if (staged) {
        const float4* mp = reinterpret_cast<const float4*>(msh + c * 32);
#pragma unroll
        for (int i = 0; i < 8; ++i) u[i] = mp[i];
      } else {
        const float4* mp = reinterpret_cast<const float4*>(q.mult + (int64_t)e_lane * q.K + k0);
#pragma unroll
        for (int i = 0; i < 8; ++i) u[i] = mp[i];
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        v[4 * i] *= u[i].x;
        v[4 * i + 1] *= u[i].y;
        v[4 * i + 2] *= u[i].z;
        v[4 * i + 3] *= u[i].w;
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 32; ++i) v[i] = 0.0f;
  }

  fwht_lane<B>(v, c);
  uint4 out;
  const int sc = mx_encode(v, out);

  if constexpr (TILED) {
    // every lane of the padded grid writes (zeros outside M x K)
    *reinterpret_cast<uint4*>(q.codes + tiled_code_offset(row, k0, q.kpad)) = out;
    q.scales[tiled_scale_offset(row, k0, q.kpad)] = (uint8_t)sc;
  } else if (valid) {
    *reinterpret_cast<uint4*>(q.codes + row * (q.K >> 1) + (k0 >> 1)) = out;
    q.scales[row * (q.K >> 5) + (k0 >> 5)] = (uint8_t)sc;
  }
}

// One thread per row: the expert offsets in LDS when they fit (one parallel
// load per workgroup), then a binary search.
__global__ __launch_bounds__(kThreads) void row_expert_kernel(const int32_t* __restrict__ off, int E, int64_t rows,
                                                              int32_t* __restrict__ out) {
  __shared__ int32_t offs[kMaxExperts + 1];
  const int tid = threadIdx.x;
  const int64_t r = (int64_t)blockIdx.x * kThreads + tid;
  if (E <= kMaxExperts) {  // uniform
    for (int i = tid; i <= E; i += kThreads) offs[i] = off[i];
    __syncthreads();
    if (r < rows) out[r] = expert_of_row(offs, E, r);
  } else if (r < rows) {
    out[r] = expert_of_row(off, E, r);
  }
}

// Correct rounding of a square root and a quotient of positive fp32 values.
// The device sqrt and divide may land one ulp off; the candidate and its two
// neighbours are told apart by the midpoint test: the rounded root y of x
// satisfies (y - ulp/2)^2 < x < (y + ulp/2)^2 (the rounded quotient y of c / s
// satisfies (y - ulp/2) s < c < (y + ulp/2) s). Midpoints have 25 significant
// bits, so their squares (and products with s) are exact in fp64, and no
// midpoint can be hit exactly by an fp32 x or c, so there are no ties.
__device__ __forceinline__ float next_up(float v) { return __uint_as_float(__float_as_uint(v) + 1u); }
__device__ __forceinline__ float next_down(float v) { return __uint_as_float(__float_as_uint(v) - 1u); }

__device__ float sqrt_rn(float x) {  // x > 0, finite
  float y = sqrtf(x);
  const double xd = x;
  for (int it = 0; it < 3; ++it) {
    const double hi = 0.5 * ((double)y + (double)next_up(y));
    const double lo = 0.5 * ((double)y + (double)next_down(y));
    if (xd > hi * hi) y = next_up(y);
    else if (xd < lo * lo) y = next_down(y);
    else break;
  }
  return y;
}

__device__ float div_rn(float c, float s) {  // c > 0, s > 0, finite
  float y = c / s;
  const double cd = c, sd = s;
  for (int it = 0; it < 3; ++it) {
    const double hi = 0.5 * ((double)y + (double)next_up(y));
    const double lo = 0.5 * ((double)y + (double)next_down(y));
    if (cd > hi * sd) y = next_up(y);
    else if (cd < lo * sd) y = next_down(y);
    else break;
  }
  return y;
}

// s[k] = (column max)^(quarters / 4): quarters 0 gives 1, 1 two correctly
// rounded square roots in turn, 2 one, 4 the maximum itself; an all-zero
// column gives 1.
__global__ __launch_bounds__(kThreads) void calibrate_kernel(const uint16_t* __restrict__ x, int64_t R, int64_t K,
                                                             int64_t ldx, int quarters, float* __restrict__ s) {
  const int64_t k = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (k >= K) return;
  float mx = 0.0f;
  for (int64_t r = 0; r < R; ++r) mx = fmaxf(mx, fabsf(__uint_as_float((uint32_t)x[r * ldx + k] << 16)));
  float v = 1.0f;
  if (mx != 0.0f) {
    if (quarters == 1) v = sqrt_rn(sqrt_rn(mx));
    else if (quarters == 2) v = sqrt_rn(mx);
    else if (quarters == 4) v = mx;
  }
  s[k] = v;
}

__global__ __launch_bounds__(kThreads) void multipliers_kernel(const float* __restrict__ s, int64_t K, float cb,
                                                               float* __restrict__ a, float* __restrict__ r) {
  const int64_t k = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (k >= K) return;
  const float sk = s[k];
  if (a) a[k] = div_rn(cb, sk);
  if (r) r[k] = cb * sk;
}

template <bool F32_IN, int B, bool SCALE, bool GROUPED, bool TILED>
hipError_t launch_one(const QuantArgs& q, hipStream_t stream) {
  // tiled: cover the padded rows and K; row-major: just M x K
  const int64_t rows = TILED ? pad_rows(q.M) : q.M;
  const int64_t gx = (rows + kGroupRows - 1) / kGroupRows, gy = q.kpad / kBlockK;
  if (gx * gy > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL((quant_rows_kernel<F32_IN, B, SCALE, GROUPED, TILED>), dim3((unsigned)(gx * gy)),
                     dim3(kThreads), 0, stream, q);
  return hipGetLastError();
}

template <bool F32_IN, bool SCALE, bool GROUPED, bool TILED>
hipError_t launch_b(const QuantArgs& q, int b, hipStream_t stream) {
  switch (b) {
    case 0: return launch_one<F32_IN, 0, SCALE, GROUPED, TILED>(q, stream);
    case 32: return launch_one<F32_IN, 32, SCALE, GROUPED, TILED>(q, stream);
    case 64: return launch_one<F32_IN, 64, SCALE, GROUPED, TILED>(q, stream);
    case 128: return launch_one<F32_IN, 128, SCALE, GROUPED, TILED>(q, stream);
    default: return hipErrorInvalidValue;
  }
}

template <bool TILED>
hipError_t launch_layout(const QuantArgs& q, int b, bool x_is_f32, hipStream_t stream) {
  const bool scale = q.mult != nullptr;
  const bool grouped = q.row_expert != nullptr;
  if (x_is_f32) {
    if (grouped) return hipErrorInvalidValue;
    return scale ? launch_b<true, true, false, TILED>(q, b, stream) : launch_b<true, false, false, TILED>(q, b, stream);
  }
  if (grouped)
    return scale ? launch_b<false, true, true, TILED>(q, b, stream) : launch_b<false, false, true, TILED>(q, b, stream);
  return scale ? launch_b<false, true, false, TILED>(q, b, stream) : launch_b<false, false, false, TILED>(q, b, stream);
}

}  // namespace

hipError_t launch_quant_rows(const QuantArgs& q, int b, bool x_is_f32, hipStream_t stream) {
  if (q.M == 0) return hipSuccess;
  return q.tiled ? launch_layout<true>(q, b, x_is_f32, stream) : launch_layout<false>(q, b, x_is_f32, stream);
}

hipError_t launch_row_expert(const int32_t* off, int E, int64_t rows, int32_t* out, hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  const int64_t blocks = (rows + kThreads - 1) / kThreads;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(row_expert_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, off, E, rows, out);
  return hipGetLastError();
}

hipError_t launch_calibrate(const void* xcal, int64_t R, int64_t K, int64_t ldx, int quarters, float* s,
                            hipStream_t stream) {
  const int64_t blocks = (K + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(calibrate_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream,
                     static_cast<const uint16_t*>(xcal), R, K, ldx, quarters, s);
  return hipGetLastError();
}

hipError_t launch_multipliers(const float* s, int64_t K, float cb, float* a, float* r, hipStream_t stream) {
  const int64_t blocks = (K + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(multipliers_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, s, K, cb, a, r);
  return hipGetLastError();
}

}  // namespace macaq
