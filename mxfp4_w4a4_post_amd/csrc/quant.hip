// Online activation transform and MXFP4 quantization (gfx950).
//
// Method: "MACaQ: Fast, Model Agnostic Calibrated Quantization for
// Low-Precision Weights and Activations" (paper card, Abstract) applies a
// per-channel scale and a block-Hadamard transform to each layer's
// activations at inference and quantizes to MXFP4; the same row transform with
// the weight-side multiplier produces the absorbed weights offline.
//
// Layout of the work: a workgroup of 256 lanes covers 16 rows x 128
// elements; each lane owns 8 consecutive
// elements of a row (one 16-byte bf16 load), 16 lanes a row. An MX group of 32
// is 4 adjacent lanes and a Hadamard block of b elements is b/8 adjacent
// lanes. Butterflies of span 1, 2, 4 stay inside the lane; spans 8 .. b/2 pair
// lanes 1 .. b/16 apart through cross-lane shuffles. The E2M1 encode and
// nibble packing use the hardware scaled FP4 convert, which rounds to
// nearest-even, saturates at 6 and keeps the sign (it only reads the exponent
// of its fp32 scale operand).
#include "common.hpp"

namespace macaq {
namespace {

constexpr int kThreads = 256;
constexpr int kTileRows = 16;   // rows per workgroup
constexpr int kTileK = 128;     // elements per workgroup along K

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

// TILED: write the GEMM layout (including its zero padding); otherwise
// row-major [M, K/2] codes and [M, K/32] scales.
template <bool F32_IN, int B, bool SCALE, bool GROUPED, bool TILED>
__global__ __launch_bounds__(kThreads) void quant_rows_kernel(QuantArgs q) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int64_t row = (int64_t)blockIdx.x * kTileRows + (tid >> 4);
  const int64_t k = (int64_t)blockIdx.y * kTileK + (tid & 15) * 8;
  const bool valid = row < q.M && k < q.K;

  float v[8];
  if (valid) {
    if constexpr (F32_IN) {
      const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(q.x) + row * q.ldx + k);
      const float4 u0 = p[0], u1 = p[1];
      v[0] = u0.x; v[1] = u0.y; v[2] = u0.z; v[3] = u0.w;
      v[4] = u1.x; v[5] = u1.y; v[6] = u1.z; v[7] = u1.w;
    } else {
      const uint4 w = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(q.x) + row * q.ldx + k);
      v[0] = bf16_lo(w.x); v[1] = bf16_hi(w.x);
      v[2] = bf16_lo(w.y); v[3] = bf16_hi(w.y);
      v[4] = bf16_lo(w.z); v[5] = bf16_hi(w.z);
      v[6] = bf16_lo(w.w); v[7] = bf16_hi(w.w);
    }
    if constexpr (SCALE) {
      const float* m = q.mult;
      if constexpr (GROUPED) m += (int64_t)expert_of_row(q.offsets, q.E, row) * q.K;
      const float4* mp = reinterpret_cast<const float4*>(m + k);
      const float4 m0 = mp[0], m1 = mp[1];
      v[0] *= m0.x; v[1] *= m0.y; v[2] *= m0.z; v[3] *= m0.w;
      v[4] *= m1.x; v[5] *= m1.y; v[6] *= m1.z; v[7] *= m1.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = 0.0f;
  }

  if constexpr (B > 0) {
    // spans 1, 2, 4 inside the lane
#pragma unroll
    for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (i & h) continue;
        const float u = v[i], w = v[i + h];
        v[i] = u + w;
        v[i + h] = u - w;
      }
    }
    // spans 8 .. B/2 across lanes d = span/8 apart: the lower lane keeps
    // u + w, the upper lane u - w. fma with +-1 rounds once, exactly as the
    // plain add or subtract would.
#pragma unroll
    for (int d = 1; d < B / 8; d <<= 1) {
      const float sgn = (lane & d) ? -1.0f : 1.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float p = __shfl_xor(v[i], d);
        v[i] = __builtin_fmaf(sgn, v[i], p);
      }
    }
  }

  // group maximum of |t| over the 4 lanes of the group
  float amax = fabsf(v[0]);
#pragma unroll
  for (int i = 1; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
  amax = fmaxf(amax, __shfl_xor(amax, 1));
  amax = fmaxf(amax, __shfl_xor(amax, 2));

  // E8M0: biased exponent of amax minus E2M1's largest exponent (2),
  // clamped at 0 (2^-127); covers amax == 0 and subnormal amax.
  const int ebits = (int)((__float_as_uint(amax) >> 23) & 0xFF);
  const int sc = ebits > 2 ? ebits - 2 : 0;
  const float scale = sc ? __uint_as_float((uint32_t)sc << 23) : __uint_as_float(0x00400000u);

  uint32_t packed = 0;
  packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, v[0], v[1], scale, 0);
  packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, v[2], v[3], scale, 1);
  packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, v[4], v[5], scale, 2);
  packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, v[6], v[7], scale, 3);

  if constexpr (TILED) {
    // every lane of the padded grid writes (zeros outside M x K)
    // a lane's 8 elements are 4 code bytes inside one 16-byte chunk
    *reinterpret_cast<uint32_t*>(q.codes + tiled_code_offset(row, k, q.kpad)) = packed;
    if ((k & 31) == 0) q.scales[tiled_scale_offset(row, k, q.kpad)] = (uint8_t)sc;
  } else if (valid) {
    *reinterpret_cast<uint32_t*>(q.codes + row * (q.K >> 1) + (k >> 1)) = packed;
    if ((k & 31) == 0) q.scales[row * (q.K >> 5) + (k >> 5)] = (uint8_t)sc;
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

__global__ __launch_bounds__(kThreads) void calibrate_kernel(const uint16_t* __restrict__ x, int64_t R, int64_t K,
                                                             int64_t ldx, float* __restrict__ s) {
  const int64_t k = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (k >= K) return;
  float mx = 0.0f;
  for (int64_t r = 0; r < R; ++r) mx = fmaxf(mx, fabsf(__uint_as_float((uint32_t)x[r * ldx + k] << 16)));
  s[k] = (mx == 0.0f) ? 1.0f : sqrt_rn(mx);
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
  const int64_t kk = TILED ? q.kpad : q.K;
  const int64_t gx = (rows + kTileRows - 1) / kTileRows, gy = (kk + kTileK - 1) / kTileK;
  if (gx > 0x7FFFFFFF || gy > 65535) return hipErrorInvalidValue;
  hipLaunchKernelGGL((quant_rows_kernel<F32_IN, B, SCALE, GROUPED, TILED>), dim3((unsigned)gx, (unsigned)gy),
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
  const bool grouped = q.offsets != nullptr;
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

hipError_t launch_calibrate(const void* xcal, int64_t R, int64_t K, int64_t ldx, float* s, hipStream_t stream) {
  const int64_t blocks = (K + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(calibrate_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream,
                     static_cast<const uint16_t*>(xcal), R, K, ldx, s);
  return hipGetLastError();
}

hipError_t launch_multipliers(const float* s, int64_t K, float cb, float* a, float* r, hipStream_t stream) {
  const int64_t blocks = (K + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(multipliers_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, s, K, cb, a, r);
  return hipGetLastError();
}

}  // namespace macaq
