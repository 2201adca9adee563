// The steps either side of the grouped layer in an MoE block (gfx950):
// routing of the (token, slot) entries to expert-major rows, and the
// weighted combine of each token's expert outputs.
//
// "MACaQ - Huawei open-sources a 4-bit quantizer ..." (What it is) lists MoE
// models among those the method covers; "Huawei's MACaQ-R beats Unsloth's
// ..." ("Changed tensors") names the routed experts' gate, up and down
// projections. Routing order and combine precision are readings: rows sorted
// by expert, ties by entry index t * k + j; the combine sums w[t, j] times
// the expert row over j = 0 .. k-1 in fp32.
#include "common.hpp"

namespace macaq {
namespace {

constexpr int kRouteThreads = 256;

// Exclusive prefix sum over the workgroup (Hillis-Steele in LDS); *total
// receives the sum of every thread's v.
__device__ int block_exclusive_scan(int v, int* sh, int* total) {
  const int tid = threadIdx.x;
  sh[tid] = v;
  __syncthreads();
  for (int d = 1; d < kRouteThreads; d <<= 1) {
    const int t = tid >= d ? sh[tid - d] : 0;
    __syncthreads();
    sh[tid] += t;
    __syncthreads();
  }
  const int incl = sh[tid];
  *total = sh[kRouteThreads - 1];
  __syncthreads();
  return incl - v;
}

// One workgroup per expert e. Every workgroup counts all n entries per expert
// (LDS histogram) to find where expert e's rows start; thread t owns the
// contiguous entries [t * chunk, (t + 1) * chunk), so a scan of the threads'
// counts of e gives each entry of e its rank in entry order. Workgroup 0 also
// writes the offsets, pos = -1 for ids outside [0, E), and token 0 for the
// rows past the routed ones (so every gather index stays in range).
__global__ __launch_bounds__(kRouteThreads) void moe_route_kernel(const int32_t* __restrict__ ids, int64_t n, int k,
                                                                 int E, int32_t* __restrict__ offsets,
                                                                 int32_t* __restrict__ row_token,
                                                                 int32_t* __restrict__ pos) {
  __shared__ int hist[kMaxExperts];
  __shared__ int sh[kRouteThreads];
  const int tid = threadIdx.x, e = blockIdx.x;
  for (int i = tid; i < E; i += kRouteThreads) hist[i] = 0;
  __syncthreads();
  const int64_t chunk = (n + kRouteThreads - 1) / kRouteThreads;
  const int64_t lo = tid * chunk < n ? tid * chunk : n;
  const int64_t hi = lo + chunk < n ? lo + chunk : n;
  int mine = 0;
  for (int64_t i = lo; i < hi; ++i) {
    const int id = ids[i];
    if (id >= 0 && id < E) {
      atomicAdd(&hist[id], 1);
      mine += id == e;
    }
  }
  __syncthreads();
  int part = 0;
  for (int i = tid; i < e; i += kRouteThreads) part += hist[i];
  int base = 0, unused = 0;
  block_exclusive_scan(part, sh, &base);
  const int start = block_exclusive_scan(mine, sh, &unused);
  int row = base + start;
  for (int64_t i = lo; i < hi; ++i) {
    if (ids[i] == e) {
      row_token[row] = (int32_t)(i / k);
      pos[i] = row;
      ++row;
    }
  }
  if (e != 0) return;
  // offsets: thread t covers experts [t * ce, (t + 1) * ce)
  const int ce = (E + kRouteThreads - 1) / kRouteThreads;
  const int e0 = tid * ce < E ? tid * ce : E, e1 = e0 + ce < E ? e0 + ce : E;
  int cnt = 0;
  for (int i = e0; i < e1; ++i) cnt += hist[i];
  int total = 0;
  int acc = block_exclusive_scan(cnt, sh, &total);
  for (int i = e0; i < e1; ++i) {
    offsets[i] = acc;
    acc += hist[i];
  }
  if (tid == 0) offsets[E] = total;
  for (int64_t i = lo; i < hi; ++i) {
    const int id = ids[i];
    if (id < 0 || id >= E) pos[i] = -1;
  }
  for (int64_t r = total + tid; r < n; r += kRouteThreads) row_token[r] = 0;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ uint32_t to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// y[t, c .. c+7] = sum_j w[t, j] * rows[pos[t*k + j], c .. c+7]: one thread
// per 8 outputs (one 16-byte load per expert row), one workgroup row per token.
// VEC: 16-byte output stores (aligned rows).
template <bool BF16, bool VEC>
__global__ __launch_bounds__(256) void moe_combine_kernel(const uint16_t* __restrict__ rows, int64_t H,
                                                          const int32_t* __restrict__ pos,
                                                          const float* __restrict__ w, int k, void* __restrict__ y,
                                                          int64_t ldy) {
  const int64_t t = blockIdx.y;
  const int64_t c = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
  if (c >= H) return;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < k; ++j) {
    const int32_t r = pos[t * k + j];
    if (r < 0) continue;
    const float wt = w[t * k + j];
    const uint4 u = *reinterpret_cast<const uint4*>(rows + (int64_t)r * H + c);
    const uint32_t q[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] = __builtin_fmaf(wt, bf16_lo(q[i]), acc[2 * i]);
      acc[2 * i + 1] = __builtin_fmaf(wt, bf16_hi(q[i]), acc[2 * i + 1]);
    }
  }
  if constexpr (BF16) {
    uint16_t* out = static_cast<uint16_t*>(y) + t * ldy + c;
    if constexpr (VEC) {
      uint4 v;
      v.x = to_bf16(acc[0]) | (to_bf16(acc[1]) << 16);
      v.y = to_bf16(acc[2]) | (to_bf16(acc[3]) << 16);
      v.z = to_bf16(acc[4]) | (to_bf16(acc[5]) << 16);
      v.w = to_bf16(acc[6]) | (to_bf16(acc[7]) << 16);
      *reinterpret_cast<uint4*>(out) = v;
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) out[i] = (uint16_t)to_bf16(acc[i]);
    }
  } else {
    float* out = static_cast<float*>(y) + t * ldy + c;
    if constexpr (VEC) {
      reinterpret_cast<float4*>(out)[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
      reinterpret_cast<float4*>(out)[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) out[i] = acc[i];
    }
  }
}

}  // namespace

hipError_t launch_moe_route(const int32_t* ids, int64_t T, int k, int E, int32_t* offsets, int32_t* row_token,
                            int32_t* pos, hipStream_t stream) {
  hipLaunchKernelGGL(moe_route_kernel, dim3((unsigned)E), dim3(kRouteThreads), 0, stream, ids, T * k, k, E, offsets,
                     row_token, pos);
  return hipGetLastError();
}

hipError_t launch_moe_combine(const uint16_t* rows, int64_t H, const int32_t* pos, const float* w, int64_t T, int k,
                              void* y, bool y_bf16, int64_t ldy, hipStream_t stream) {
  const dim3 grid((unsigned)((H + 2047) / 2048), (unsigned)T), block(256);
  const size_t es = y_bf16 ? 2 : 4;
  const bool vec = reinterpret_cast<uintptr_t>(y) % 16 == 0 && (ldy * es) % 16 == 0;
  if (y_bf16) {
    if (vec) hipLaunchKernelGGL((moe_combine_kernel<true, true>), grid, block, 0, stream, rows, H, pos, w, k, y, ldy);
    else hipLaunchKernelGGL((moe_combine_kernel<true, false>), grid, block, 0, stream, rows, H, pos, w, k, y, ldy);
  } else {
    if (vec) hipLaunchKernelGGL((moe_combine_kernel<false, true>), grid, block, 0, stream, rows, H, pos, w, k, y, ldy);
    else hipLaunchKernelGGL((moe_combine_kernel<false, false>), grid, block, 0, stream, rows, H, pos, w, k, y, ldy);
  }
  return hipGetLastError();
}

}  // namespace macaq
