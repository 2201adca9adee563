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

// Entries are read in rounds of 1024 (16 bytes per thread, one coalesced
// KiB per wave and round): entry i = 1024 j + 4 t + s lies in round j with
// thread t, slot s. In that order (round, wave, lane, slot) the entries keep
// their index order, so a rank among expert e's entries is the matches of
// earlier rounds, then of lower waves in the round, then of lower lanes of
// the wave (ballots), then of lower slots of the lane.
constexpr int kRouteRound = 4 * kRouteThreads;
constexpr int kRouteSegRounds = 1024;  // rounds whose wave counts sit in LDS at once

// Rounds are loaded kRouteBatch at a time, all loads of a batch in flight
// together (a full batch is unconditional 16-byte loads).
constexpr int kRouteBatch = 8;

__device__ __forceinline__ void load_batch(const int32_t* __restrict__ ids, int64_t n, int64_t j,
                                           int4 (&v)[kRouteBatch]) {
  const int64_t i = j * kRouteRound + 4 * threadIdx.x;
  if ((j + kRouteBatch) * kRouteRound <= n) {
#pragma unroll
    for (int b = 0; b < kRouteBatch; ++b) v[b] = *reinterpret_cast<const int4*>(ids + i + (int64_t)b * kRouteRound);
  } else {
#pragma unroll
    for (int b = 0; b < kRouteBatch; ++b) {
      const int64_t ib = i + (int64_t)b * kRouteRound;
      v[b].x = ib < n ? ids[ib] : -1;
      v[b].y = ib + 1 < n ? ids[ib + 1] : -1;
      v[b].z = ib + 2 < n ? ids[ib + 2] : -1;
      v[b].w = ib + 3 < n ? ids[ib + 3] : -1;
    }
  }
}

// Round j of this thread: from memory (batched loads) or from the LDS copy.
struct RouteSrcGlobal {
  const int32_t* ids;
  int64_t n;
  __device__ __forceinline__ void batch(int64_t j, int4 (&v)[kRouteBatch]) const { load_batch(ids, n, j, v); }
};
struct RouteSrcLds {
  const int* sh;
  __device__ __forceinline__ void batch(int64_t j, int4 (&v)[kRouteBatch]) const {
#pragma unroll
    for (int b = 0; b < kRouteBatch; ++b)
      v[b] = *reinterpret_cast<const int4*>(sh + (j + b) * kRouteRound + 4 * threadIdx.x);
  }
};

// One workgroup per expert e: the entries with an id below e give where
// expert e's rows start (offsets[e]); the entries with id e get their rows in
// index order. Workgroup 0 also writes pos = -1 for ids outside [0, E);
// workgroup E-1 writes offsets[E] and token 0 for the rows past the routed
// ones (so every gather index stays in range).
template <class Src>
__device__ __forceinline__ void route_expert(const Src& src, int64_t n, int k, int E, int32_t* __restrict__ offsets,
                                             int32_t* __restrict__ row_token, int32_t* __restrict__ pos, int* sh,
                                             int* cnt) {
  const int tid = threadIdx.x, e = blockIdx.x, wave = tid >> 6, lane = tid & 63;
  const uint64_t below_mask = (uint64_t(1) << lane) - 1;
  const int64_t rounds = (n + kRouteRound - 1) / kRouteRound;
  int below = 0;
  for (int64_t j = 0; j < rounds; j += kRouteBatch) {
    int4 v[kRouteBatch];
    src.batch(j, v);
#pragma unroll
    for (int b = 0; b < kRouteBatch; ++b)
      below += ((v[b].x >= 0) & (v[b].x < e)) + ((v[b].y >= 0) & (v[b].y < e)) + ((v[b].z >= 0) & (v[b].z < e)) +
               ((v[b].w >= 0) & (v[b].w < e));
  }
  int first = 0;
  block_exclusive_scan<kRouteThreads>(below, sh, &first);
  int row0 = first;  // first row of the current segment
  for (int64_t j0 = 0; j0 < rounds; j0 += kRouteSegRounds) {
    const int nr = (int)(rounds - j0 < kRouteSegRounds ? rounds - j0 : kRouteSegRounds);
    // matches of each (round, wave)
    for (int r0 = 0; r0 < nr; r0 += kRouteBatch) {
      int4 v[kRouteBatch];
      src.batch(j0 + r0, v);
#pragma unroll
      for (int b = 0; b < kRouteBatch; ++b) {
        const int c = __popcll(__ballot(v[b].x == e)) + __popcll(__ballot(v[b].y == e)) +
                      __popcll(__ballot(v[b].z == e)) + __popcll(__ballot(v[b].w == e));
        if (lane == 0 && r0 + b < nr) cnt[4 * (r0 + b) + wave] = c;
      }
    }
    __syncthreads();
    // exclusive prefix over (round, wave) in place: thread t scans a slice
    const int m = 4 * nr, per = (m + kRouteThreads - 1) / kRouteThreads;
    const int a0 = tid * per < m ? tid * per : m, a1 = a0 + per < m ? a0 + per : m;
    int part = 0;
    for (int i = a0; i < a1; ++i) part += cnt[i];
    int seg_total = 0;
    int acc = block_exclusive_scan<kRouteThreads>(part, sh, &seg_total);
    for (int i = a0; i < a1; ++i) {
      const int c = cnt[i];
      cnt[i] = acc;
      acc += c;
    }
    __syncthreads();
    for (int r0 = 0; r0 < nr; r0 += kRouteBatch) {
      int4 v[kRouteBatch];
      src.batch(j0 + r0, v);
#pragma unroll
      for (int b = 0; b < kRouteBatch; ++b) {
        if (r0 + b >= nr) break;
        const int vv[4] = {v[b].x, v[b].y, v[b].z, v[b].w};
        const int64_t i0 = (j0 + r0 + b) * kRouteRound + 4 * tid;
        const bool any = (vv[0] == e) | (vv[1] == e) | (vv[2] == e) | (vv[3] == e);
        int rank = row0 + cnt[4 * (r0 + b) + wave];
#pragma unroll
        for (int q = 0; q < 4; ++q) rank += __popcll(__ballot(vv[q] == e) & below_mask);
        if (any) {
          // token of entry i0 + q: one 32-bit division for the quad, then carries
          const uint32_t i32 = (uint32_t)i0;
          uint32_t tok = i32 / (uint32_t)k, rem = i32 - tok * (uint32_t)k;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            if (vv[q] == e) {
              row_token[rank] = (int32_t)tok;
              pos[i0 + q] = rank;
              ++rank;
            }
            if (++rem == (uint32_t)k) {
              rem = 0;
              ++tok;
            }
          }
        }
        if (e == 0) {
#pragma unroll
          for (int q = 0; q < 4; ++q)
            if (i0 + q < n && (vv[q] < 0 || vv[q] >= E)) pos[i0 + q] = -1;
        }
      }
    }
    row0 += seg_total;
    __syncthreads();  // cnt is rewritten by the next segment
  }
  if (tid == 0) offsets[e] = first;
  if (e == E - 1) {
    if (tid == 0) offsets[E] = row0;
    for (int64_t r = row0 + tid; r < n; r += kRouteThreads) row_token[r] = 0;
  }
}

__global__ __launch_bounds__(kRouteThreads) void moe_route_kernel(const int32_t* __restrict__ ids, int64_t n, int k,
                                                                 int E, int32_t* __restrict__ offsets,
                                                                 int32_t* __restrict__ row_token,
                                                                 int32_t* __restrict__ pos) {
  __shared__ int sh[kRouteThreads];
  __shared__ int cnt[kRouteSegRounds * 4];
  route_expert(RouteSrcGlobal{ids, n}, n, k, E, offsets, row_token, pos, sh, cnt);
}

// Up to kRouteLdsEntries entries: the workgroup first copies all of them to
// LDS with coalesced, unconditional loads (addresses clamped into the array,
// values past n replaced by -1), all in flight at once, so every pass after
// that reads LDS. QUAD: n is a multiple of 4, so the copy moves 16 bytes per
// load (entries 4t + 1024r .. +3 of round r); otherwise 4 bytes per load.
constexpr int kRouteLdsEntries = 32 * kRouteRound;  // 32768

template <bool QUAD>
__global__ __launch_bounds__(kRouteThreads) void moe_route_lds_kernel(const int32_t* __restrict__ ids, int64_t n,
                                                                     int k, int E, int32_t* __restrict__ offsets,
                                                                     int32_t* __restrict__ row_token,
                                                                     int32_t* __restrict__ pos) {
  __shared__ int sh[kRouteThreads];
  __shared__ int cnt[32 * 4];
  __shared__ __attribute__((aligned(16))) int all[kRouteLdsEntries];
  const int tid = threadIdx.x;
  const int rounds = (int)((n + kRouteRound - 1) / kRouteRound);
  const int padded = ((rounds + kRouteBatch - 1) / kRouteBatch) * kRouteBatch * kRouteRound;
  if constexpr (QUAD) {
    constexpr int R = kRouteLdsEntries / kRouteRound;  // 32 rounds
    int4 v[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int64_t q = (int64_t)r * kRouteRound + 4 * tid;
      v[r] = *reinterpret_cast<const int4*>(ids + (q < n ? q : n - 4));
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int q = r * kRouteRound + 4 * tid;
      if (q < padded) {
        const bool in = q < n;
        *reinterpret_cast<int4*>(all + q) =
            make_int4(in ? v[r].x : -1, in ? v[r].y : -1, in ? v[r].z : -1, in ? v[r].w : -1);
      }
    }
  } else {
    constexpr int PER = kRouteLdsEntries / kRouteThreads;  // 128
    int v[PER];
#pragma unroll
    for (int m = 0; m < PER; ++m) {
      const int64_t i = tid + (int64_t)m * kRouteThreads;
      v[m] = ids[i < n ? i : n - 1];
    }
#pragma unroll
    for (int m = 0; m < PER; ++m) {
      const int i = tid + m * kRouteThreads;
      if (i < padded) all[i] = i < n ? v[m] : -1;
    }
  }
  __syncthreads();
  route_expert(RouteSrcLds{all}, n, k, E, offsets, row_token, pos, sh, cnt);
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
  const int64_t n = T * k;
  if (n == 0) {
    hipLaunchKernelGGL(moe_route_kernel, dim3((unsigned)E), dim3(kRouteThreads), 0, stream, ids, n, k, E, offsets,
                       row_token, pos);
  } else if (n <= kRouteLdsEntries && n % 4 == 0) {
    hipLaunchKernelGGL(moe_route_lds_kernel<true>, dim3((unsigned)E), dim3(kRouteThreads), 0, stream, ids, n, k, E,
                       offsets, row_token, pos);
  } else if (n <= kRouteLdsEntries) {
    hipLaunchKernelGGL(moe_route_lds_kernel<false>, dim3((unsigned)E), dim3(kRouteThreads), 0, stream, ids, n, k, E,
                       offsets, row_token, pos);
  } else {
    hipLaunchKernelGGL(moe_route_kernel, dim3((unsigned)E), dim3(kRouteThreads), 0, stream, ids, n, k, E, offsets,
                       row_token, pos);
  }
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
