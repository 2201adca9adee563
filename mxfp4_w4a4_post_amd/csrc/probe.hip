// Measurement probes (not part of the layer): the ceilings that the GEMM and
// the bandwidth-bound kernels are read against on this chip.
//
// mfma_probe_kernel: back-to-back scaled-FP4 MFMAs (32x32x64, E2M1 x E2M1)
// on register operands, with nothing else in the loop. Each wave keeps 8
// independent accumulators (4 activation x 2 weight operands, the fragment
// set of one wave of a 128 x 256 GEMM tile) and issues `iters` rounds of 8
// MFMAs. Thread t takes its 6 operands (16 bytes each) from ops[6t .. 6t+5],
// one 24 KiB block shared by every workgroup: random bytes make the matrix
// cores' inputs change from one MFMA to the next, constant bytes keep them
// still. Every scale is 2^0. 96 KiB of LDS per workgroup keep one workgroup
// (4 waves, one per SIMD) on a CU.
//
// read_probe_kernel: a plain read of device memory, each thread with 8 loads
// of 16 bytes in flight along a grid-stride walk, folding what it read into
// one word that it writes, so the loads cannot be dropped.
#include "common.hpp"

namespace macaq {
namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeLdsFloats = 24576;  // 96 KiB

__global__ __launch_bounds__(kProbeThreads) void mfma_probe_kernel(const v4i* __restrict__ ops, int iters,
                                                                  float* __restrict__ out) {
  __shared__ float pad[kProbeLdsFloats];
  const int t = threadIdx.x;
  v8i a[4], w[2];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const v4i v = ops[6 * t + i];
    a[i] = v8i{v[0], v[1], v[2], v[3], 0, 0, 0, 0};
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const v4i v = ops[6 * t + 4 + j];
    w[j] = v8i{v[0], v[1], v[2], v[3], 0, 0, 0, 0};
  }
  constexpr int kScaleOne = 0x7F7F7F7F;  // E8M0 127 in every byte: 2^0
  v16f acc[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[k] = v16f{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc[2 * i + j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(w[j], a[i], acc[2 * i + j], kFmtFp4, kFmtFp4,
                                                                         0, kScaleOne, 0, kScaleOne);
  }
  float s = 0.0f;
#pragma unroll
  for (int k = 0; k < 8; ++k)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[k][r];
  pad[t] = s;
  __syncthreads();
  out[(int64_t)blockIdx.x * kProbeThreads + t] = pad[kProbeThreads - 1 - t];
}

__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const v4i* __restrict__ p, int64_t n,
                                                                  uint32_t* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * kProbeThreads;
  int64_t i = (int64_t)blockIdx.x * kProbeThreads + threadIdx.x;
  uint32_t x = 0;
  for (; i + 7 * stride < n; i += 8 * stride) {
    v4i v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = p[i + u * stride];
#pragma unroll
    for (int u = 0; u < 8; ++u) x ^= (uint32_t)(v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3]);
  }
  for (; i < n; i += stride) {
    const v4i v = p[i];
    x ^= (uint32_t)(v[0] ^ v[1] ^ v[2] ^ v[3]);
  }
  out[(int64_t)blockIdx.x * kProbeThreads + threadIdx.x] = x;
}

}  // namespace

hipError_t launch_mfma_probe(const void* ops, int workgroups, int iters, float* out, hipStream_t stream) {
  hipLaunchKernelGGL(mfma_probe_kernel, dim3((unsigned)workgroups), dim3(kProbeThreads), 0, stream,
                     static_cast<const v4i*>(ops), iters, out);
  return hipGetLastError();
}

hipError_t launch_read_probe(const void* src, int64_t bytes, int workgroups, uint32_t* out, hipStream_t stream) {
  hipLaunchKernelGGL(read_probe_kernel, dim3((unsigned)workgroups), dim3(kProbeThreads), 0, stream,
                     static_cast<const v4i*>(src), bytes / 16, out);
  return hipGetLastError();
}

}  // namespace macaq
