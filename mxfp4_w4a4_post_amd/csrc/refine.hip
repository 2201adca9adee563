// Flip-Refinement of prepared MXFP4 weights (gfx950): the Hessian of the
// transformed calibration rows, and greedy single-code moves that lower each
// weight row's output error with the block scales kept.
//
// "MACaQ: Fast, Model Agnostic Calibrated Quantization for Low-Precision
// Weights and Activations" (paper card, Abstract) improves on round-to-nearest
// weights with a Hessian-aware coordinate descent that greedily moves single
// FP4 codes to adjacent representable values; "Huawei's MACaQ-R beats
// Unsloth's ..." (What we found when we compared the files) sees only codes
// change, never the block scales. The objective, move order and stopping
// rule are readings: row n minimises e^T H e, e = w~ - q in the transformed
// basis (w~ = S_b (r .* w) in fp32, q its dequantized codes), H = X~^T X~ of
// the transformed calibration rows; a step takes the adjacent move with the
// most negative change d^2 H[k][k] - 2 d g[k] (g = H e; ties: lowest k, then
// the downward move) until none is negative or max_flips moves are made.
// Every sum runs in index order in fp64, one fused multiply-add per term, so
// the decisions are reproducible bit for bit.
#include "mx_lane.hpp"

namespace macaq {
namespace {

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Signed index m in -7 .. 7 of a 4-bit code (the -0 code 8 is index 0) and back.
__device__ __forceinline__ int code_index(uint32_t c) { return (c & 8) ? -(int)(c & 7) : (int)(c & 7); }
__device__ __forceinline__ uint32_t index_code(int m) { return m < 0 ? (8u | (uint32_t)(-m)) : (uint32_t)m; }

// Rows through the multiplier and the block-Hadamard, one lane per 32-element
// chunk exactly as the quantizer does it (workgroup = 32 rows x 256 elements).
// OUT_E: write e = w~ - dequant(codes) in fp64 (codes and scales of the rows
// in the GEMM layout); otherwise write the fp32 transformed rows.
template <bool F32_IN, int B, bool OUT_E>
__global__ __launch_bounds__(256) void transform_kernel(const void* __restrict__ x, int64_t M, int64_t K, int64_t ldx,
                                                        const float* __restrict__ mult,
                                                        const uint8_t* __restrict__ codes,
                                                        const uint8_t* __restrict__ scales, float* __restrict__ out32,
                                                        double* __restrict__ out64) {
  const int tid = threadIdx.x;
  const int c = tid & 7;
  const int64_t row = (int64_t)blockIdx.x * kGroupRows + (tid >> 3);
  const int64_t k0 = (int64_t)blockIdx.y * kBlockK + c * 32;
  const bool valid = row < M && k0 < K;
  float v[32];
  if (valid) {
    if constexpr (F32_IN) {
      const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(x) + row * ldx + k0);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float4 u = p[i];
        v[4 * i] = u.x;
        v[4 * i + 1] = u.y;
        v[4 * i + 2] = u.z;
        v[4 * i + 3] = u.w;
      }
    } else {
      const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) + row * ldx + k0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint4 w = p[i];
        const uint32_t q[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          v[8 * i + 2 * j] = bf16_lo(q[j]);
          v[8 * i + 2 * j + 1] = bf16_hi(q[j]);
        }
      }
    }
    if (mult) {
      const float4* mp = reinterpret_cast<const float4*>(mult + k0);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float4 u = mp[i];
        v[4 * i] *= u.x;
        v[4 * i + 1] *= u.y;
        v[4 * i + 2] *= u.z;
        v[4 * i + 3] *= u.w;
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 32; ++i) v[i] = 0.0f;
  }
  fwht_lane<B>(v, c);
  if (!valid) return;
  if constexpr (OUT_E) {
    const int64_t kpad = pad_k(K);
    const uint4 cw = *reinterpret_cast<const uint4*>(codes + tiled_code_offset(row, k0, kpad));
    const int sc = scales[tiled_scale_offset(row, k0, kpad)];
    const uint32_t cb[4] = {cw.x, cw.y, cw.z, cw.w};
    // dequantized code, branch-free: magnitude code m < 2 is m / 2, else
    // (1 or 1.5) * 2^(m / 2 - 1); times 2^(scale - 127); every factor is exact
    double2* o = reinterpret_cast<double2*>(out64 + row * K + k0);
#pragma unroll
    for (int i = 0; i < 32; i += 2) {
      double q[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t nib = (cb[(i + h) >> 3] >> (4 * ((i + h) & 7))) & 0xF;
        const int m = (int)(nib & 7);
        const double mant = m < 2 ? 0.5 * (double)m : ((m & 1) ? 1.5 : 1.0);
        const double mag = ldexp(mant, (m < 2 ? 0 : (m >> 1) - 1) + sc - 127);
        q[h] = (double)v[i + h] - (((nib & 8) && m != 0) ? -mag : mag);  // the -0 code is +0
      }
      o[i >> 1] = make_double2(q[0], q[1]);
    }
  } else {
    float4* o = reinterpret_cast<float4*>(out32 + row * K + k0);
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
  }
}

// C[i][j] = sum over t (ascending) of A(t, i) * B(t, j) in fp64, one 128 x 128
// output tile per workgroup, on the fp64 matrix cores: each wave owns a 64 x 64
// quarter as 4 x 4 blocks of v_mfma_f64_16x16x4f64, which adds four products
// per output as fused multiply-adds in k order (checked bit for bit against
// the sequential chain, subnormals, signed zeros, overflow and NaN included),
// so chaining it over ascending t gives every output exactly the plain
// sequential sum of fused steps. t is staged 16 at a time through LDS (two
// buffers), the next chunk loaded into registers while the current one is
// multiplied; t past the end reads zeros, which leave a sum started at +0
// unchanged (it can never be -0). The two instances:
//   Hessian: A = B = the fp32 transformed rows [R, K]:  H[j][k] = sum_r x~[r][j] x~[r][k];
//   gradient: A = E^T (E [N, K] fp64), B = H:          G[n][j] = sum_k E[n][k] H[k][j].
constexpr int kTile = 128, kChunk = 16;
constexpr int kStage = kChunk * kTile / 256;    // staged values per thread and matrix
typedef double v4d __attribute__((ext_vector_type(4)));

template <bool HESSIAN>
__global__ __launch_bounds__(256) void gram_kernel(const float* __restrict__ xt, const double* __restrict__ e,
                                                   const double* __restrict__ h, int64_t rows_i, int64_t cols_j,
                                                   int64_t len_t, double* __restrict__ out) {
  // two buffers: chunk c is stored into buffer c % 2 while other waves may
  // still multiply chunk c - 1 out of the other one; the barrier after the
  // store then also orders the next reuse, so one barrier per chunk suffices
  __shared__ double as[2][kChunk][kTile + 1];  // padded: the gradient's A is written along t
  __shared__ double bs[2][kChunk][kTile];
  const int tid = threadIdx.x;
  // the Hessian is symmetric (x~[r][j] x~[r][k] and x~[r][k] x~[r][j] are the
  // same product, summed in the same order), so its launch covers only the
  // tiles with row tile <= column tile, one per workgroup of a 1-D grid, and
  // writes each off-diagonal tile twice
  int64_t i0, j0;
  if constexpr (HESSIAN) {
    const int64_t L = blockIdx.x;
    int64_t c = (int64_t)((sqrt(8.0 * (double)L + 1.0) - 1.0) * 0.5);
    while (c * (c + 1) / 2 > L) --c;
    while ((c + 1) * (c + 2) / 2 <= L) ++c;
    i0 = (L - c * (c + 1) / 2) * kTile;
    j0 = c * kTile;
  } else {
    i0 = (int64_t)blockIdx.y * kTile;
    j0 = (int64_t)blockIdx.x * kTile;
  }
  // this thread's staged values of a chunk: A then B, kStage each; loads run
  // along the contiguous dimension (i of the rows x~, t of E, j of H)
  double ra[kStage], rb[kStage];
  auto load = [&](int64_t t0) {
#pragma unroll
    for (int q = 0; q < kStage; ++q) {
      const int idx = tid + 256 * q;
      if constexpr (HESSIAN) {
        const int tt = idx / kTile, col = idx % kTile;
        const int64_t t = t0 + tt;
        ra[q] = (t < len_t && i0 + col < rows_i) ? (double)xt[t * rows_i + i0 + col] : 0.0;
        rb[q] = (t < len_t && j0 + col < cols_j) ? (double)xt[t * cols_j + j0 + col] : 0.0;
      } else {
        const int tt_a = idx % kChunk, col_a = idx / kChunk;
        const int64_t ta = t0 + tt_a;
        ra[q] = (ta < len_t && i0 + col_a < rows_i) ? e[(i0 + col_a) * len_t + ta] : 0.0;
        const int tt_b = idx / kTile, col_b = idx % kTile;
        const int64_t tb = t0 + tt_b;
        rb[q] = (tb < len_t && j0 + col_b < cols_j) ? h[tb * cols_j + j0 + col_b] : 0.0;
      }
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int q = 0; q < kStage; ++q) {
      const int idx = tid + 256 * q;
      if constexpr (HESSIAN) {
        as[buf][idx / kTile][idx % kTile] = ra[q];
      } else {
        as[buf][idx % kChunk][idx / kChunk] = ra[q];
      }
      bs[buf][idx / kTile][idx % kTile] = rb[q];
    }
  };
  // wave w owns rows i0 + 64 (w / 2) + [0, 64) and columns j0 + 64 (w % 2) +
  // [0, 64); block (mi, nj) is 16 x 16. Operand lane l holds row / column
  // l % 16 of its block at t offset l / 16; output lane l holds rows
  // 4 v + l / 16 (v = 0 .. 3) of column l % 16.
  const int lane = tid & 63, wave = tid >> 6;
  const int wi = 64 * (wave >> 1), wj = 64 * (wave & 1);
  const int lr = lane & 15, lk = lane >> 4;
  v4d acc[4][4];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int nj = 0; nj < 4; ++nj) acc[mi][nj] = v4d{0.0, 0.0, 0.0, 0.0};
  load(0);
  int buf = 0;
  for (int64_t t0 = 0; t0 < len_t; t0 += kChunk, buf ^= 1) {
    store(buf);
    __syncthreads();
    // the next chunk's loads are in flight during this chunk's products
    if (t0 + kChunk < len_t) load(t0 + kChunk);
    const int nt = (int)(len_t - t0 < kChunk ? len_t - t0 : kChunk);
    for (int s4 = 0; s4 < nt; s4 += 4) {
      double af[4], bf[4];
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) af[mi] = as[buf][s4 + lk][wi + 16 * mi + lr];
#pragma unroll
      for (int nj = 0; nj < 4; ++nj) bf[nj] = bs[buf][s4 + lk][wj + 16 * nj + lr];
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int nj = 0; nj < 4; ++nj)
          acc[mi][nj] = __builtin_amdgcn_mfma_f64_16x16x4f64(af[mi], bf[nj], acc[mi][nj], 0, 0, 0);
    }
  }
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t i = i0 + wi + 16 * mi + 4 * v + lk;
      if (i >= rows_i) continue;
#pragma unroll
      for (int nj = 0; nj < 4; ++nj) {
        const int64_t j = j0 + wj + 16 * nj + lr;
        if (j < cols_j) out[i * cols_j + j] = acc[mi][nj][v];
      }
    }
  if (HESSIAN && i0 != j0) {
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t i = i0 + wi + 16 * mi + 4 * v + lk;
        if (i >= rows_i) continue;
#pragma unroll
        for (int nj = 0; nj < 4; ++nj) {
          const int64_t j = j0 + wj + 16 * nj + lr;
          if (j < cols_j) out[j * rows_i + i] = acc[mi][nj][v];
        }
      }
  }
}

__global__ void hdiag_kernel(const double* __restrict__ h, int64_t K, double* __restrict__ d) {
  const int64_t k = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (k < K) d[k] = h[k * K + k];
}

// Exponent of the step from signed index m up to m + 1, per u = m + 7 in
// 0 .. 13 as two bits holding exponent + 1: the E2M1 grid spacing is 2 between
// magnitudes 4 and 6, 1 between 1 and 4 and 1/2 below 1. The step from m down
// to m - 1 is minus the step from m - 1 up. Every step is a power of two, so
// d = +-2^(e + scale - 127) is exactly the difference of the two dequantized
// values.
constexpr uint32_t kUpExp = (2u << 0) | (1u << 2) | (1u << 4) | (1u << 22) | (1u << 24) | (2u << 26);
__device__ __forceinline__ int up_exp(uint32_t u) { return (int)((kUpExp >> (2 * (u & 15u))) & 3u) - 1; }
// The step exponents of state u, each + 1: bits 0-1 upward, bits 2-3 downward.
__device__ __forceinline__ uint32_t step_bits(uint32_t u) {
  return (uint32_t)(up_exp(u) + 1) | ((uint32_t)(up_exp(u - 1) + 1) << 2);
}

// A candidate move: the change D of the objective, the element k, and the
// step d as (exponent + 512) * 2 + 1 for an upward move, + 0 for a downward one.
struct Cand {
  double D;
  int k, step;
};
// Candidates order by D, then by k. A thread scans its elements in ascending k,
// the downward move first, and keeps only a strictly lower D, so its winner is
// the first of its equals in index order; no two threads hold the same k.
__device__ __forceinline__ bool better(const Cand& a, const Cand& b) {
  return a.D < b.D || (a.D == b.D && a.k < b.k);
}
__device__ __forceinline__ Cand shfl_xor_cand(const Cand& c, int m) {
  Cand o;
  o.D = __shfl_xor(c.D, m);
  o.k = __shfl_xor(c.k, m);
  o.step = __shfl_xor(c.step, m);
  return o;
}
__device__ __forceinline__ double step_value(int step) {
  const double m = ldexp(1.0, (step >> 1) - 512);
  return (step & 1) ? m : -m;
}

// The greedy moves of one weight row per workgroup of T threads. Thread t owns
// the element pairs p = t + T i (elements 2p, 2p + 1, one code byte, one scale)
// for i < P and holds their g, H[k][k] (HD_REG) and signed indices in
// registers. Per move: the scan of every element's two moves (no branches), a
// wave argmin by shuffles, one barrier for the per-wave winners, the argmin of
// those in every wave, the owner's index update and the g update from one row
// of H.
template <int P, int T, bool HD_REG>
__global__ __launch_bounds__(T) void flip_kernel(const double* __restrict__ G, const double* __restrict__ H,
                                                 const double* __restrict__ hdiag, int64_t N, int64_t K,
                                                 int max_flips, uint8_t* __restrict__ codes,
                                                 const uint8_t* __restrict__ scales, int32_t* __restrict__ flips) {
  constexpr int kWaves = T / 64;
  __shared__ Cand slot[2][kWaves];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int64_t n = blockIdx.x;
  const int64_t kpad = pad_k(K);
  const int Ki = (int)K;  // K <= 32768: element indices fit 32 bits
  // per pair: g and H[k][k] of both elements, and one state word: bits 0-3 /
  // 4-7 the current signed indices + 7, bits 8-11 / 12-15 the original ones
  // + 7, bits 16-23 the scale byte, bits 24-27 / 28-31 the step bits of the
  // current indices. Elements past K get H[k][k] = +inf, so their moves never
  // lower the objective.
  double g[P][2], hd[HD_REG ? P : 1][2];
  uint32_t st[P];
#pragma unroll
  for (int i = 0; i < P; ++i) {
    const int k = 2 * (tid + T * i);
    double h0 = __builtin_inf(), h1 = __builtin_inf();
    if (k < Ki) {
      const double2 gv = *reinterpret_cast<const double2*>(G + n * K + k);
      g[i][0] = gv.x;
      g[i][1] = gv.y;
      const double2 hk = *reinterpret_cast<const double2*>(hdiag + k);
      h0 = hk.x;
      h1 = hk.y;
      const uint32_t byte = codes[tiled_code_offset(n, k, kpad)];
      const uint32_t lo = (uint32_t)(code_index(byte & 0xF) + 7), hi = (uint32_t)(code_index(byte >> 4) + 7);
      st[i] = lo | (hi << 4) | (lo << 8) | (hi << 12) | ((uint32_t)scales[tiled_scale_offset(n, k, kpad)] << 16) |
              (step_bits(lo) << 24) | (step_bits(hi) << 28);
    } else {
      g[i][0] = g[i][1] = 0.0;
      st[i] = 7u | (7u << 4) | (7u << 8) | (7u << 12) | (step_bits(7) << 24) | (step_bits(7) << 28);
    }
    if constexpr (HD_REG) {
      hd[i][0] = h0;
      hd[i][1] = h1;
    }
  }
  int moves = 0;
  for (int par = 0; moves < max_flips; par ^= 1) {
    // d = -2^ed (down) or 2^eu (up); (d d) H[k][k] and (2 d) g are products by
    // powers of two, each one rounding, so ldexp gives the same values
    double bD = 0.0;
    int bc = -1;  // 4 i + 2 s + (1 if upward) of the thread's best move
#pragma unroll
    for (int i = 0; i < P; ++i) {
      const int k = 2 * (tid + T * i);
      double hkk[2];
      if constexpr (HD_REG) {
        hkk[0] = hd[i][0];
        hkk[1] = hd[i][1];
      } else {
        const double2 hk = *reinterpret_cast<const double2*>(hdiag + (k < Ki ? k : 0));
        hkk[0] = k < Ki ? hk.x : __builtin_inf();
        hkk[1] = k < Ki ? hk.y : __builtin_inf();
      }
      const int sc1 = (int)((st[i] >> 16) & 0xFF) - 128;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const uint32_t u = (st[i] >> (4 * s)) & 0xF;
        const uint32_t sb = st[i] >> (24 + 4 * s);
        const int eu = (int)(sb & 3u) + sc1, ed = (int)((sb >> 2) & 3u) + sc1;
        const double Ddn = ldexp(hkk[s], 2 * ed) + ldexp(g[i][s], ed + 1);
        const double Dup = ldexp(hkk[s], 2 * eu) - ldexp(g[i][s], eu + 1);
        if (u > 0 && Ddn < bD) {
          bD = Ddn;
          bc = 4 * i + 2 * s;
        }
        if (u < 14 && Dup < bD) {
          bD = Dup;
          bc = 4 * i + 2 * s + 1;
        }
      }
      if constexpr (!HD_REG)
        if (i % 4 == 3) __builtin_amdgcn_sched_barrier(0);
    }
    Cand best{bD, Ki, 0};
    if (bc >= 0) {
      const int bi = bc >> 2, bs = (bc >> 1) & 1, bup = bc & 1;
      uint32_t w = st[0];
#pragma unroll
      for (int i = 1; i < P; ++i)
        if (bi == i) w = st[i];
      const uint32_t sb = w >> (24 + 4 * bs);
      const int e = (int)(bup ? (sb & 3u) : ((sb >> 2) & 3u)) + (int)((w >> 16) & 0xFF) - 128;
      best.k = 2 * (tid + T * bi) + bs;
      best.step = ((e + 512) << 1) | bup;
    }
#pragma unroll
    for (int msk = 32; msk >= 1; msk >>= 1) {
      const Cand o = shfl_xor_cand(best, msk);
      if (better(o, best)) best = o;
    }
    if (lane == 0) slot[par][wave] = best;
    __syncthreads();
    // every aligned group of kWaves lanes reduces the per-wave winners
    best = slot[par][lane % kWaves];
#pragma unroll
    for (int msk = kWaves / 2; msk >= 1; msk >>= 1) {
      const Cand o = shfl_xor_cand(best, msk);
      if (better(o, best)) best = o;
    }
    const int bk = __builtin_amdgcn_readfirstlane(best.k);
    const int bstep = __builtin_amdgcn_readfirstlane(best.step);
    if (bk >= Ki) break;  // no move lowers the objective
    // the owner of element bk applies the move to its signed index
    const int pidx = bk >> 1;
    if (pidx % T == tid) {
      const int i = pidx / T, sh = 4 * (bk & 1);
#pragma unroll
      for (int ii = 0; ii < P; ++ii)
        if (ii == i) {
          const uint32_t u = ((st[ii] >> sh) & 0xFu) + ((bstep & 1) ? 1u : 0xFFFFFFFFu);
          st[ii] = (st[ii] & ~((0xFu << sh) | (0xFu << (24 + sh)))) | ((u & 0xFu) << sh) | (step_bits(u) << (24 + sh));
        }
    }
    const double d = step_value(bstep);
    const double* hr = H + (int64_t)bk * K;
    // the row's loads are issued together, without branches (elements past K
    // read element 0; their g never matters), before any of them is used; with
    // more than 7 pairs per thread of 1024 the row (like H[k][k] in the scan
    // without HD_REG) is read in groups of 4 pairs, which bounds the registers
    // its loads hold
    constexpr int kGroup = (HD_REG && P * T <= 7 * 1024) ? P : 4;
#pragma unroll
    for (int i0 = 0; i0 < P; i0 += kGroup) {
      double2 hv[kGroup];
#pragma unroll
      for (int j = 0; j < kGroup; ++j) {
        const int k = 2 * (tid + T * (i0 + j));
        hv[j] = *reinterpret_cast<const double2*>(hr + (k < Ki ? k : 0));
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < kGroup; ++j) {
        g[i0 + j][0] = g[i0 + j][0] - d * hv[j].x;
        g[i0 + j][1] = g[i0 + j][1] - d * hv[j].y;
      }
    }
    ++moves;
  }
  // moved elements take the canonical code of their index; the rest keep their bits
#pragma unroll
  for (int i = 0; i < P; ++i) {
    const int k = 2 * (tid + T * i);
    const uint32_t cur = st[i] & 0xFF, orig = (st[i] >> 8) & 0xFF;
    if (k >= K || cur == orig) continue;
    uint8_t* bp = codes + tiled_code_offset(n, k, kpad);
    uint32_t byte = *bp;
    if ((cur & 0xF) != (orig & 0xF)) byte = (byte & 0xF0u) | index_code((int)(cur & 0xF) - 7);
    if ((cur >> 4) != (orig >> 4)) byte = (byte & 0x0Fu) | (index_code((int)(cur >> 4) - 7) << 4);
    *bp = (uint8_t)byte;
  }
  if (tid == 0 && flips) flips[n] = moves;
}

template <int P, int T>
void launch_flip(int64_t N, int64_t K, int max_flips, const double* G, const double* H, const double* hdiag,
                 uint8_t* codes, const uint8_t* scales, int32_t* flips, hipStream_t stream) {
  hipLaunchKernelGGL((flip_kernel<P, T, (P <= 8)>), dim3((unsigned)N), dim3(T), 0, stream, G, H, hdiag, N, K,
                     max_flips, codes, scales, flips);
}

template <bool F32_IN, bool OUT_E>
hipError_t launch_transform(const void* x, int64_t M, int64_t K, int64_t ldx, const float* mult, int b,
                            const uint8_t* codes, const uint8_t* scales, float* out32, double* out64,
                            hipStream_t stream) {
  const dim3 grid((unsigned)((M + kGroupRows - 1) / kGroupRows), (unsigned)((K + kBlockK - 1) / kBlockK));
  switch (b) {
    case 0: hipLaunchKernelGGL((transform_kernel<F32_IN, 0, OUT_E>), grid, dim3(256), 0, stream, x, M, K, ldx, mult,
                               codes, scales, out32, out64); break;
    case 32: hipLaunchKernelGGL((transform_kernel<F32_IN, 32, OUT_E>), grid, dim3(256), 0, stream, x, M, K, ldx, mult,
                                codes, scales, out32, out64); break;
    case 64: hipLaunchKernelGGL((transform_kernel<F32_IN, 64, OUT_E>), grid, dim3(256), 0, stream, x, M, K, ldx, mult,
                                codes, scales, out32, out64); break;
    default: hipLaunchKernelGGL((transform_kernel<F32_IN, 128, OUT_E>), grid, dim3(256), 0, stream, x, M, K, ldx,
                                mult, codes, scales, out32, out64); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_hessian(const void* xcal, int64_t R, int64_t K, int64_t ldx, const float* a, int b, float* xt,
                          double* H, hipStream_t stream) {
  hipError_t e = launch_transform<false, false>(xcal, R, K, ldx, a, b, nullptr, nullptr, xt, nullptr, stream);
  if (e != hipSuccess) return e;
  const int64_t tiles = (K + kTile - 1) / kTile;
  hipLaunchKernelGGL((gram_kernel<true>), dim3((unsigned)(tiles * (tiles + 1) / 2)), dim3(256), 0, stream, xt,
                     nullptr, nullptr, K, K, R, H);
  return hipGetLastError();
}

hipError_t launch_flip_refine(const void* W, bool w_f32, int64_t N, int64_t K, int64_t ldw, const float* r, int b,
                              const double* H, int max_flips, uint8_t* codes, const uint8_t* scales, int32_t* flips,
                              double* E, double* G, double* hdiag, hipStream_t stream) {
  hipError_t e = w_f32 ? launch_transform<true, true>(W, N, K, ldw, r, b, codes, scales, nullptr, E, stream)
                       : launch_transform<false, true>(W, N, K, ldw, r, b, codes, scales, nullptr, E, stream);
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)((K + kTile - 1) / kTile), (unsigned)((N + kTile - 1) / kTile));
  hipLaunchKernelGGL((gram_kernel<false>), grid, dim3(256), 0, stream, nullptr, E, H, N, K, K, G);
  hipLaunchKernelGGL(hdiag_kernel, dim3((unsigned)((K + 255) / 256)), dim3(256), 0, stream, H, K, hdiag);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // rows of up to 4096 elements: 256 threads (four rows a compute unit at a
  // time, each thread 8 pairs); longer rows: 1024 threads
  const int64_t half = K / 2;
  if (half <= 256 * 8) {
    if (half <= 256) launch_flip<1, 256>(N, K, max_flips, G, H, hdiag, codes, scales, flips, stream);
    else if (half <= 512) launch_flip<2, 256>(N, K, max_flips, G, H, hdiag, codes, scales, flips, stream);
    else if (half <= 1024) launch_flip<4, 256>(N, K, max_flips, G, H, hdiag, codes, scales, flips, stream);
    else launch_flip<8, 256>(N, K, max_flips, G, H, hdiag, codes, scales, flips, stream);
  } else if (half <= 1024 * 4) {
    launch_flip<4, 1024>(N, K, max_flips, G, H, hdiag, codes, scales, flips, stream);
  } else if (half <= 1024 * 6) {
    launch_flip<6, 1024>(N, K, max_flips, G, H, hdiag, codes, scales, flips, stream);
  } else if (half <= 1024 * 7) {
    launch_flip<7, 1024>(N, K, max_flips, G, H, hdiag, codes, scales, flips, stream);
  } else if (half <= 1024 * 8) {
    launch_flip<8, 1024>(N, K, max_flips, G, H, hdiag, codes, scales, flips, stream);
  } else {
    launch_flip<16, 1024>(N, K, max_flips, G, H, hdiag, codes, scales, flips, stream);
  }
  return hipGetLastError();
}

}  // namespace macaq
