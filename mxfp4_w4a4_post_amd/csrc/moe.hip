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

// Routing works on chunks of kRouteChunk consecutive entries, 4 per thread
// (thread t holds entries 4t .. 4t+3 of its chunk), one workgroup per chunk.
// Pass one counts each chunk's entries per expert; pass two gives every
// chunk the rows of its entries: expert e's rows start at the entries of all
// chunks with an id below e, then come the chunk's predecessors' entries of
// e, then the chunk's own in index order (a stable sort of the chunk by id).
constexpr int kRouteChunk = 4 * kRouteThreads;
constexpr int kRouteIdxBits = 10;  // an entry's place in its chunk
static_assert(kRouteChunk == 1 << kRouteIdxBits, "chunk index bits");

__device__ __forceinline__ int wave_inclusive_scan(int v, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int t = __shfl_up(v, d, 64);
    if (lane >= d) v += t;
  }
  return v;
}

// Exclusive scan of one int per thread over the workgroup (4 waves); *total
// gets the sum. sh: 4 ints of LDS. Every thread must call it.
__device__ __forceinline__ int route_scan(int v, int* sh, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int incl = wave_inclusive_scan(v, lane);
  if (lane == 63) sh[wave] = incl;
  __syncthreads();
  int before = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) before += w < wave ? sh[w] : 0;
  *total = sh[0] + sh[1] + sh[2] + sh[3];
  __syncthreads();
  return before + incl - v;
}

// The 4 ids of this thread in chunk g: -2 past the end of the array.
__device__ __forceinline__ void chunk_ids(const int32_t* __restrict__ ids, int64_t n, int64_t g, int (&v)[4]) {
  const int64_t i = g * kRouteChunk + 4 * threadIdx.x;
  if (i + 3 < n) {
    const int4 q = *reinterpret_cast<const int4*>(ids + i);  // ids is 16-byte aligned
    v[0] = q.x;
    v[1] = q.y;
    v[2] = q.z;
    v[3] = q.w;
  } else {
#pragma unroll
    for (int s = 0; s < 4; ++s) v[s] = i + s < n ? ids[i + s] : -2;
  }
}

// counts[g * E + e] = entries of chunk g with id e.
__global__ __launch_bounds__(kRouteThreads) void route_count_kernel(const int32_t* __restrict__ ids, int64_t n, int E,
                                                                    int32_t* __restrict__ counts) {
  __shared__ int hist[kMaxExperts];
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += kRouteThreads) hist[e] = 0;
  __syncthreads();
  int v[4];
  chunk_ids(ids, n, blockIdx.x, v);
#pragma unroll
  for (int s = 0; s < 4; ++s)
    if (v[s] >= 0 && v[s] < E) atomicAdd(&hist[v[s]], 1);
  __syncthreads();
  for (int e = tid; e < E; e += kRouteThreads) counts[(int64_t)blockIdx.x * E + e] = hist[e];
}

// The tile map of a grouped GEMM with tiles of bm rows from the expert
// totals tot[] and first rows first_row[] (LDS, all E experts; this thread
// sums experts [e0, e1)): m-tile j of expert e gets entry (tiles of experts
// before e) + j, the remaining entries expert -1, and map[2 * max_mtiles] the
// number of used entries (the format build_tile_map_kernel writes). Each
// thread writes entries tid, tid + 256, ..., finding an entry's expert by
// binary search of the tile prefix tpre[] (LDS, E ints). Every thread of the
// workgroup calls it.
__device__ __forceinline__ void route_tile_map(int32_t* __restrict__ map, int bm, int64_t max_mtiles, int E, int e0,
                                               int e1, const int* tot, const int* first_row, int* tpre, int* sh) {
  int cnt = 0;
  for (int e = e0; e < e1; ++e) cnt += (tot[e] + bm - 1) / bm;
  int used = 0;
  int acc = route_scan(cnt, sh, &used);
  for (int e = e0; e < e1; ++e) {
    tpre[e] = acc;
    acc += (tot[e] + bm - 1) / bm;
  }
  __syncthreads();
  const int64_t n_used = used < max_mtiles ? used : max_mtiles;
  for (int64_t i = threadIdx.x; i < max_mtiles; i += kRouteThreads) {
    int e = -1, row = 0;
    if (i < n_used) {
      // the last expert whose tiles start at or before entry i (an expert
      // with no tiles shares its start with the next one, so it is skipped)
      int lo = 0, hi = E;
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (tpre[mid] <= i) lo = mid;
        else hi = mid;
      }
      e = lo;
      row = first_row[lo] + (int)(i - tpre[lo]) * bm;
    }
    map[2 * i] = e;
    map[2 * i + 1] = row;
  }
  if (threadIdx.x == 0) map[2 * max_mtiles] = (int32_t)n_used;
  __syncthreads();  // tpre is reused
}

// Rows of chunk g's entries (G chunks). Workgroup 0 writes offsets (and the
// tile maps m.map[i] of tiles of m.bm[i] rows, where given); ids outside
// [0, E) get pos = -1; rows past the routed ones get token 0.
__global__ __launch_bounds__(kRouteThreads) void route_scatter_kernel(const int32_t* __restrict__ ids, int64_t n,
                                                                      int k, int E, const int32_t* __restrict__ counts,
                                                                      int G, int32_t* __restrict__ offsets,
                                                                      int32_t* __restrict__ row_token,
                                                                      int32_t* __restrict__ pos, RouteMaps m,
                                                                      int32_t* __restrict__ row_expert) {
  __shared__ int base[kMaxExperts];   // first row of this chunk's entries of e
  __shared__ int first[kMaxExperts];  // expert totals, then the sorted place of e's first entry
  __shared__ int offs[kMaxExperts];   // offsets[e]
  __shared__ int tpre[kMaxExperts];   // tile maps: first entry of each expert
  __shared__ int buf[kRouteChunk];
  __shared__ int sh[4];
  const int tid = threadIdx.x, g = blockIdx.x;
  // entries of e in earlier chunks and in all chunks: the chunk counts are
  // loaded 16 at a time (a clamped index, so the loads are unconditional and
  // all in flight together) and summed in chunk order
  for (int e = tid; e < E; e += kRouteThreads) {
    int bef = 0, tot = 0;
    for (int c0 = 0; c0 < G; c0 += 16) {
      int v[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) v[j] = counts[(int64_t)(c0 + j < G ? c0 + j : G - 1) * E + e];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int c = c0 + j;
        const int x = c < G ? v[j] : 0;
        tot += x;
        bef += c < g ? x : 0;
      }
    }
    base[e] = bef;
    first[e] = tot;
  }
  __syncthreads();
  // offsets: exclusive scan of the totals, thread t over experts [t*EP, (t+1)*EP)
  const int EP = (E + kRouteThreads - 1) / kRouteThreads;
  const int e0 = tid * EP < E ? tid * EP : E, e1 = e0 + EP < E ? e0 + EP : E;
  int part = 0;
  for (int e = e0; e < e1; ++e) part += first[e];
  int routed = 0;
  int acc = route_scan(part, sh, &routed);
  for (int e = e0; e < e1; ++e) {
    const int c = first[e];
    if (g == 0) offsets[e] = acc;
    offs[e] = acc;
    base[e] += acc;
    acc += c;
  }
  if (g == 0 && tid == 0) offsets[E] = routed;
  // tile map i from workgroup i % G
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    if (m.map[i] && g == i % G) {
      __syncthreads();  // offs and the totals of every expert
      route_tile_map(m.map[i], m.bm[i], m.max_mtiles, E, e0, e1, first, offs, tpre, sh);
    }
  }
  // stable sort of the chunk by key (id; E for an id out of range, E + 1 past
  // the end), one key bit per pass; a key and the entry's place pack into one int
  int v[4], pk[4];
  chunk_ids(ids, n, g, v);
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int key = v[s] == -2 ? E + 1 : (v[s] >= 0 && v[s] < E ? v[s] : E);
    pk[s] = (key << kRouteIdxBits) | (4 * tid + s);
  }
  const int bits = 32 - __clz(E + 1);
  for (int bit = 0; bit < bits; ++bit) {
    bool zero[4];
    int z = 0;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      zero[s] = ((pk[s] >> (kRouteIdxBits + bit)) & 1) == 0;
      z += zero[s];
    }
    int zeros = 0;
    int zp = route_scan(z, sh, &zeros);
    int op = zeros + 4 * tid - zp;
#pragma unroll
    for (int s = 0; s < 4; ++s) buf[zero[s] ? zp++ : op++] = pk[s];
    __syncthreads();
#pragma unroll
    for (int s = 0; s < 4; ++s) pk[s] = buf[4 * tid + s];
    __syncthreads();
  }
  // sorted place p = 4t + s; the first place of each expert's run
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int p = 4 * tid + s, key = pk[s] >> kRouteIdxBits;
    const int prev = p == 0 ? -1 : (s > 0 ? pk[s - 1] : buf[p - 1]) >> kRouteIdxBits;
    if (key < E && key != prev) first[key] = p;
  }
  __syncthreads();
  const int64_t c0 = (int64_t)g * kRouteChunk;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int key = pk[s] >> kRouteIdxBits;
    const int64_t i = c0 + (pk[s] & (kRouteChunk - 1));
    if (key < E) {
      const int row = base[key] + (4 * tid + s - first[key]);
      pos[i] = row;
      row_token[row] = (int32_t)((uint32_t)i / (uint32_t)k);
      if (row_expert) row_expert[row] = key;
    } else if (key == E) {
      pos[i] = -1;
    }
  }
  // rows past the routed ones: token 0, and the expert a search of the
  // offsets gives them (the last)
  for (int64_t r = routed + (int64_t)g * kRouteThreads + tid; r < n; r += (int64_t)G * kRouteThreads) {
    row_token[r] = 0;
    if (row_expert) row_expert[r] = E - 1;
  }
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

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
  // the token's rows 8 at a time: every load issued before the first is
  // used (a dropped entry reads row 0 and is skipped), then summed in j order
  for (int j0 = 0; j0 < k; j0 += 8) {
    uint4 u[8];
    bool use[8];
    float wt[8];
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      const int j = j0 + jj < k ? j0 + jj : k - 1;
      const int32_t r = pos[t * k + j];
      use[jj] = j0 + jj < k && r >= 0;
      wt[jj] = w[t * k + j];
      u[jj] = *reinterpret_cast<const uint4*>(rows + (int64_t)(r >= 0 ? r : 0) * H + c);
    }
    __builtin_amdgcn_sched_barrier(0);  // all loads out before the first sum
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      const uint32_t q[4] = {u[jj].x, u[jj].y, u[jj].z, u[jj].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] = use[jj] ? __builtin_fmaf(wt[jj], bf16_lo(q[i]), acc[2 * i]) : acc[2 * i];
        acc[2 * i + 1] = use[jj] ? __builtin_fmaf(wt[jj], bf16_hi(q[i]), acc[2 * i + 1]) : acc[2 * i + 1];
      }
    }
  }
  if constexpr (BF16) {
    uint16_t* out = static_cast<uint16_t*>(y) + t * ldy + c;
    if constexpr (VEC) {
      uint4 v;
      v.x = bf16x2_rne(acc[0], acc[1]);
      v.y = bf16x2_rne(acc[2], acc[3]);
      v.z = bf16x2_rne(acc[4], acc[5]);
      v.w = bf16x2_rne(acc[6], acc[7]);
      *reinterpret_cast<uint4*>(out) = v;
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) out[i] = (uint16_t)bf16x2_rne(acc[i], 0.0f);
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

int64_t moe_route_chunks(int64_t n) { return n > 0 ? (n + kRouteChunk - 1) / kRouteChunk : 1; }

hipError_t launch_moe_route(const int32_t* ids, int64_t T, int k, int E, int32_t* offsets, int32_t* row_token,
                            int32_t* pos, int32_t* counts, const RouteMaps& maps, int32_t* row_expert,
                            hipStream_t stream) {
  const int64_t n = T * k, G = moe_route_chunks(n);
  hipLaunchKernelGGL(route_count_kernel, dim3((unsigned)G), dim3(kRouteThreads), 0, stream, ids, n, E, counts);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(route_scatter_kernel, dim3((unsigned)G), dim3(kRouteThreads), 0, stream, ids, n, k, E, counts,
                     (int)G, offsets, row_token, pos, maps, row_expert);
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
