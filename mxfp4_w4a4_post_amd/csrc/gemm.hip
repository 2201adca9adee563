// W4A4 GEMM on gfx950's scaled-FP4 matrix cores.
//
// Y[m, n] = sum_k dq(A[m, k]) dq(W'[n, k]): the contraction of the MACaQ
// layer ("MACaQ: Fast, Model Agnostic Calibrated Quantization for
// Low-Precision Weights and Activations", paper card, Abstract: MXFP4 W4A4).
// Both operands are K-major packed E2M1 with one E8M0 scale per 32 elements,
// which is exactly the operand layout of V_MFMA_SCALE_F32_*_F8F6F4 in FP4
// mode: each lane of an MFMA holds 32 consecutive K elements (16 bytes) of one
// row plus that row's E8M0 byte for those 32 elements.
//
//   32x32x64: lane l holds row l%32, K elements [32*(l/32), +32); output
//             register r of lane l is row 8*(r/4) + 4*(l/32) + r%4, col l%32.
//   16x16x128: lane l holds row l%16, K elements [32*(l/16), +32); output
//             register r of lane l is row 4*(l/16) + r, col l%16.
// A is the activation operand (output rows m), B the weights (output cols n),
// so consecutive lanes store consecutive n.
//
// Tiles of BM x BN outputs per workgroup walk K in steps of 256 elements
// (128 bytes per row). Code tiles go HBM -> registers -> LDS, double
// buffered, with the 16-byte chunks of each row XOR-swizzled by (row % 8) so
// that the 16-byte fragment reads of 8 consecutive rows hit disjoint banks.
// Scale tiles (8 bytes per row per step) are staged the same way and each
// lane gathers its bytes for the whole step into one dword whose byte s feeds
// the MFMA scale operand through op_sel.
#include "common.hpp"

namespace macaq {
namespace {

constexpr int BK = 256;       // K elements per step
constexpr int RB = BK / 2;    // code bytes per row per step
constexpr int SB = BK / 32;   // scale bytes per row per step

template <int BM_, int BN_, int WM_, int WN_, int MF_>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, MF = MF_;
  static constexpr int NT = WM * WN * 64;
  static constexpr int TM = BM / WM, TN = BN / WN;
  static constexpr int FM = TM / MF, FN = TN / MF;
  static constexpr int KSUB = (MF == 32) ? 64 : 128;  // K per MFMA
  static constexpr int NSUB = BK / KSUB;              // MFMAs along K per step
  static constexpr int A_CHUNKS = BM * (RB / 16);
  static constexpr int B_CHUNKS = BN * (RB / 16);
  static constexpr int A_PER_T = (A_CHUNKS + NT - 1) / NT;
  static constexpr int B_PER_T = (B_CHUNKS + NT - 1) / NT;
  static constexpr int A_SC_PER_T = (BM + NT - 1) / NT;
  static constexpr int B_SC_PER_T = (BN + NT - 1) / NT;
  static constexpr int LDS_A = BM * RB, LDS_B = BN * RB, LDS_AS = BM * SB, LDS_BS = BN * SB;
  static constexpr int LDS_STAGE = LDS_A + LDS_B + LDS_AS + LDS_BS;
  static constexpr int LDS_BYTES = 2 * LDS_STAGE;
  static_assert(TM % MF == 0 && TN % MF == 0, "wave tile must be a multiple of the MFMA tile");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget of a gfx950 workgroup");
};

// Which rows of A a tile covers. Plain GEMM: rows [m0, m_end) of A.
// Grouped: rows [m0, m_end) of expert e's range, with expert e's weights.
struct TileCoord {
  int64_t m0, m_end, n0;
  int64_t kt_begin, kt_end;  // k-steps of this split
  int split;
  int expert;
};

template <class C>
struct Stage {
  v4i a[C::A_PER_T];
  v4i b[C::B_PER_T];
  v2i as[C::A_SC_PER_T];
  v2i bs[C::B_SC_PER_T];
};

__device__ __forceinline__ int swz(int row, int chunk) { return row * RB + ((chunk ^ (row & 7)) << 4); }

template <class C>
__device__ __forceinline__ void load_stage(Stage<C>& st, const uint8_t* __restrict__ ac, const uint8_t* __restrict__ as,
                                           const uint8_t* __restrict__ bc, const uint8_t* __restrict__ bs,
                                           int64_t m0, int64_t m_end, int64_t n0, int64_t N, int64_t K, int64_t kt,
                                           bool scales_aligned) {
  const int tid = threadIdx.x;
  const int64_t lda = K >> 1, ldas = K >> 5;
  const int64_t kbyte0 = kt * RB;
#pragma unroll
  for (int i = 0; i < C::A_PER_T; ++i) {
    const int c = tid + i * C::NT;
    const int row = c >> 3, kc = c & 7;
    v4i v = {0, 0, 0, 0};
    const int64_t gm = m0 + row;
    if (c < C::A_CHUNKS && gm < m_end && kbyte0 + kc * 16 < lda)
      v = *reinterpret_cast<const v4i*>(ac + gm * lda + kbyte0 + kc * 16);
    st.a[i] = v;
  }
#pragma unroll
  for (int i = 0; i < C::B_PER_T; ++i) {
    const int c = tid + i * C::NT;
    const int row = c >> 3, kc = c & 7;
    v4i v = {0, 0, 0, 0};
    const int64_t gn = n0 + row;
    if (c < C::B_CHUNKS && gn < N && kbyte0 + kc * 16 < lda)
      v = *reinterpret_cast<const v4i*>(bc + gn * lda + kbyte0 + kc * 16);
    st.b[i] = v;
  }
  const int64_t ks0 = kt * SB;
#pragma unroll
  for (int i = 0; i < C::A_SC_PER_T; ++i) {
    const int row = tid + i * C::NT;
    v2i v = {0, 0};
    const int64_t gm = m0 + row;
    if (row < C::BM && gm < m_end) {
      const uint8_t* p = as + gm * ldas + ks0;
      if (scales_aligned) {
        v = *reinterpret_cast<const v2i*>(p);
      } else {
        uint32_t lo = 0, hi = 0;
        for (int j = 0; j < 4; ++j)
          if (ks0 + j < ldas) lo |= (uint32_t)p[j] << (8 * j);
        for (int j = 0; j < 4; ++j)
          if (ks0 + 4 + j < ldas) hi |= (uint32_t)p[4 + j] << (8 * j);
        v[0] = (int)lo;
        v[1] = (int)hi;
      }
    }
    st.as[i] = v;
  }
#pragma unroll
  for (int i = 0; i < C::B_SC_PER_T; ++i) {
    const int row = tid + i * C::NT;
    v2i v = {0, 0};
    const int64_t gn = n0 + row;
    if (row < C::BN && gn < N) {
      const uint8_t* p = bs + gn * ldas + ks0;
      if (scales_aligned) {
        v = *reinterpret_cast<const v2i*>(p);
      } else {
        uint32_t lo = 0, hi = 0;
        for (int j = 0; j < 4; ++j)
          if (ks0 + j < ldas) lo |= (uint32_t)p[j] << (8 * j);
        for (int j = 0; j < 4; ++j)
          if (ks0 + 4 + j < ldas) hi |= (uint32_t)p[4 + j] << (8 * j);
        v[0] = (int)lo;
        v[1] = (int)hi;
      }
    }
    st.bs[i] = v;
  }
}

template <class C>
__device__ __forceinline__ void store_stage(const Stage<C>& st, uint8_t* smem) {
  const int tid = threadIdx.x;
  uint8_t* sa = smem;
  uint8_t* sb = smem + C::LDS_A;
  uint8_t* ssa = sb + C::LDS_B;
  uint8_t* ssb = ssa + C::LDS_AS;
#pragma unroll
  for (int i = 0; i < C::A_PER_T; ++i) {
    const int c = tid + i * C::NT;
    if (c < C::A_CHUNKS) *reinterpret_cast<v4i*>(sa + swz(c >> 3, c & 7)) = st.a[i];
  }
#pragma unroll
  for (int i = 0; i < C::B_PER_T; ++i) {
    const int c = tid + i * C::NT;
    if (c < C::B_CHUNKS) *reinterpret_cast<v4i*>(sb + swz(c >> 3, c & 7)) = st.b[i];
  }
#pragma unroll
  for (int i = 0; i < C::A_SC_PER_T; ++i) {
    const int row = tid + i * C::NT;
    if (row < C::BM) *reinterpret_cast<v2i*>(ssa + row * SB) = st.as[i];
  }
#pragma unroll
  for (int i = 0; i < C::B_SC_PER_T; ++i) {
    const int row = tid + i * C::NT;
    if (row < C::BN) *reinterpret_cast<v2i*>(ssb + row * SB) = st.bs[i];
  }
}

template <int OPSEL>
__device__ __forceinline__ v16f mfma32(v4i a, v4i b, v16f c, int sa, int sb) {
  v8i a8 = {a[0], a[1], a[2], a[3], 0, 0, 0, 0};
  v8i b8 = {b[0], b[1], b[2], b[3], 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, c, kFmtFp4, kFmtFp4, OPSEL, sa, OPSEL, sb);
}

template <int OPSEL>
__device__ __forceinline__ v4f mfma16(v4i a, v4i b, v4f c, int sa, int sb) {
  v8i a8 = {a[0], a[1], a[2], a[3], 0, 0, 0, 0};
  v8i b8 = {b[0], b[1], b[2], b[3], 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, b8, c, kFmtFp4, kFmtFp4, OPSEL, sa, OPSEL, sb);
}

template <class C>
struct Acc;
template <int BM, int BN, int WM, int WN>
struct Acc<TileCfg<BM, BN, WM, WN, 32>> {
  using C = TileCfg<BM, BN, WM, WN, 32>;
  v16f v[C::FM][C::FN];
};
template <int BM, int BN, int WM, int WN>
struct Acc<TileCfg<BM, BN, WM, WN, 16>> {
  using C = TileCfg<BM, BN, WM, WN, 16>;
  v4f v[C::FM][C::FN];
};

// Gather this lane's scale bytes of one row for the whole step into a dword:
// byte s is the scale of the s-th MFMA along K.
template <int MF>
__device__ __forceinline__ int gather_scales(const uint8_t* row_scales, int lane) {
  const v2i w = *reinterpret_cast<const v2i*>(row_scales);
  uint32_t sel;
  if constexpr (MF == 32) {
    // MFMA s covers scale bytes 2s and 2s+1; this lane's is 2s + lane/32
    sel = (lane >> 5) ? 0x07050301u : 0x06040200u;
  } else {
    // MFMA s covers scale bytes 4s .. 4s+3; this lane's is 4s + lane/16
    const uint32_t q = (uint32_t)(lane >> 4);
    sel = 0x0C0C0000u | ((4u + q) << 8) | q;
  }
  return (int)__builtin_amdgcn_perm((uint32_t)w[1], (uint32_t)w[0], sel);
}

template <class C, int S>
__device__ __forceinline__ void mma_sub(Acc<C>& acc, const uint8_t* sa, const uint8_t* sb, const int (&sca)[C::FM],
                                        const int (&scb)[C::FN], int wm, int wn, int lane) {
  v4i af[C::FM], bf[C::FN];
  if constexpr (C::MF == 32) {
    const int chunk = S * 2 + (lane >> 5);
#pragma unroll
    for (int i = 0; i < C::FM; ++i) {
      const int row = wm * C::TM + i * 32 + (lane & 31);
      af[i] = *reinterpret_cast<const v4i*>(sa + swz(row, chunk));
    }
#pragma unroll
    for (int j = 0; j < C::FN; ++j) {
      const int row = wn * C::TN + j * 32 + (lane & 31);
      bf[j] = *reinterpret_cast<const v4i*>(sb + swz(row, chunk));
    }
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
      for (int j = 0; j < C::FN; ++j) acc.v[i][j] = mfma32<S>(af[i], bf[j], acc.v[i][j], sca[i], scb[j]);
  } else {
    const int chunk = S * 4 + (lane >> 4);
#pragma unroll
    for (int i = 0; i < C::FM; ++i) {
      const int row = wm * C::TM + i * 16 + (lane & 15);
      af[i] = *reinterpret_cast<const v4i*>(sa + swz(row, chunk));
    }
#pragma unroll
    for (int j = 0; j < C::FN; ++j) {
      const int row = wn * C::TN + j * 16 + (lane & 15);
      bf[j] = *reinterpret_cast<const v4i*>(sb + swz(row, chunk));
    }
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
      for (int j = 0; j < C::FN; ++j) acc.v[i][j] = mfma16<S>(af[i], bf[j], acc.v[i][j], sca[i], scb[j]);
  }
}

template <class C>
__device__ __forceinline__ void mma_stage(Acc<C>& acc, const uint8_t* smem, int wm, int wn, int lane) {
  const uint8_t* sa = smem;
  const uint8_t* sb = smem + C::LDS_A;
  const uint8_t* ssa = sb + C::LDS_B;
  const uint8_t* ssb = ssa + C::LDS_AS;
  int sca[C::FM], scb[C::FN];
  constexpr int LM = (C::MF == 32) ? 31 : 15;
#pragma unroll
  for (int i = 0; i < C::FM; ++i) sca[i] = gather_scales<C::MF>(ssa + (wm * C::TM + i * C::MF + (lane & LM)) * SB, lane);
#pragma unroll
  for (int j = 0; j < C::FN; ++j) scb[j] = gather_scales<C::MF>(ssb + (wn * C::TN + j * C::MF + (lane & LM)) * SB, lane);
  mma_sub<C, 0>(acc, sa, sb, sca, scb, wm, wn, lane);
  mma_sub<C, 1>(acc, sa, sb, sca, scb, wm, wn, lane);
  if constexpr (C::NSUB == 4) {
    mma_sub<C, 2>(acc, sa, sb, sca, scb, wm, wn, lane);
    mma_sub<C, 3>(acc, sa, sb, sca, scb, wm, wn, lane);
  }
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

template <class C>
__device__ __forceinline__ void store_out(const Acc<C>& acc, const GemmArgs& g, const TileCoord& tc, int wm, int wn,
                                          int lane, int64_t out_row0) {
  // out_row0: row of Y that tile row m0 maps to (m0 for plain; m0 for grouped
  // too since rows are global indices).
  const bool to_partial = g.splits > 1;
  float* pf = to_partial ? g.partial + (int64_t)tc.split * g.M * g.N : nullptr;
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j) {
      constexpr int NR = (C::MF == 32) ? 16 : 4;
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        int rr, cc;
        if constexpr (C::MF == 32) {
          rr = 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          cc = lane & 31;
        } else {
          rr = 4 * (lane >> 4) + r;
          cc = lane & 15;
        }
        const int64_t m = tc.m0 + wm * C::TM + i * C::MF + rr;
        const int64_t n = tc.n0 + wn * C::TN + j * C::MF + cc;
        if (m < tc.m_end && n < g.N) {
          const float val = acc.v[i][j][r];
          const int64_t ym = m - tc.m0 + out_row0;
          if (to_partial) {
            pf[ym * g.N + n] = val;
          } else if (g.y_bf16) {
            static_cast<uint16_t*>(g.y)[ym * g.ldy + n] = f32_to_bf16_rne(val);
          } else {
            static_cast<float*>(g.y)[ym * g.ldy + n] = val;
          }
        }
      }
    }
}

template <class C>
__device__ __forceinline__ void run_tile(const GemmArgs& g, const TileCoord& tc, const uint8_t* bc,
                                         const uint8_t* bs, uint8_t* smem) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave / C::WN, wn = wave % C::WN;
  const bool sc_al = ((g.K >> 5) % SB) == 0;
  Acc<C> acc;
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j)
#pragma unroll
      for (int r = 0; r < (C::MF == 32 ? 16 : 4); ++r) acc.v[i][j][r] = 0.0f;

  Stage<C> st;
  int64_t kt = tc.kt_begin;
  if (kt < tc.kt_end) {
    load_stage<C>(st, g.a_codes, g.a_scales, bc, bs, tc.m0, tc.m_end, tc.n0, g.N, g.K, kt, sc_al);
    store_stage<C>(st, smem);
  }
  __syncthreads();
  int buf = 0;
  for (; kt < tc.kt_end; ++kt) {
    const bool more = kt + 1 < tc.kt_end;
    if (more) load_stage<C>(st, g.a_codes, g.a_scales, bc, bs, tc.m0, tc.m_end, tc.n0, g.N, g.K, kt + 1, sc_al);
    mma_stage<C>(acc, smem + buf * C::LDS_STAGE, wm, wn, lane);
    if (more) store_stage<C>(st, smem + (buf ^ 1) * C::LDS_STAGE);
    __syncthreads();
    buf ^= 1;
  }
  store_out<C>(acc, g, tc, wm, wn, lane, tc.m0);
}

// Workgroup id -> (m tile, n tile, split), XCD-aware: ids are dispatched
// round-robin over the 8 XCDs, so id i runs on XCD i % 8. Renumber so that
// each XCD gets a contiguous run of tiles, and walk tiles in groups of
// GROUP_M m-tiles so that concurrently running tiles share A and B panels in
// that XCD's L2.
__device__ __forceinline__ int64_t xcd_remap(int64_t id, int64_t total) {
  if (total % kNumXcd != 0) return id;
  const int64_t per = total / kNumXcd;
  return (id % kNumXcd) * per + id / kNumXcd;
}

template <class C>
__global__ __launch_bounds__(C::NT) void gemm_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[C::LDS_BYTES];
  const int64_t mt = (g.M + C::BM - 1) / C::BM;
  const int64_t nt = (g.N + C::BN - 1) / C::BN;
  const int64_t tiles = mt * nt;
  const int64_t total = tiles * g.splits;
  const int64_t id = xcd_remap(blockIdx.x, total);
  const int split = (int)(id / tiles);
  const int64_t t = id - (int64_t)split * tiles;
  constexpr int64_t GROUP_M = 8;
  const int64_t group = t / (GROUP_M * nt);
  const int64_t first_m = group * GROUP_M;
  const int64_t gsize = (mt - first_m) < GROUP_M ? (mt - first_m) : GROUP_M;
  const int64_t in_group = t - group * GROUP_M * nt;
  const int64_t tm = first_m + in_group % gsize;
  const int64_t tn = in_group / gsize;
  const int64_t KT = (g.K + BK - 1) / BK;
  TileCoord tc;
  tc.m0 = tm * C::BM;
  tc.m_end = g.M;
  tc.n0 = tn * C::BN;
  tc.split = split;
  tc.kt_begin = KT * split / g.splits;
  tc.kt_end = KT * (split + 1) / g.splits;
  tc.expert = 0;
  run_tile<C>(g, tc, g.b_codes, g.b_scales, smem);
}

// Grouped: the tile map (built by build_tile_map) lists, per m-tile, the
// expert and the first row; tiles past the used count exit at once.
template <class C>
__global__ __launch_bounds__(C::NT) void gemm_grouped_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[C::LDS_BYTES];
  const int64_t nt = (g.N + C::BN - 1) / C::BN;
  const int64_t id = xcd_remap(blockIdx.x, g.max_mtiles * nt);
  const int64_t tm = id / nt;
  const int64_t tn = id - tm * nt;
  const int32_t expert = g.tile_map[2 * tm];
  if (expert < 0) return;
  const int64_t row0 = g.tile_map[2 * tm + 1];
  TileCoord tc;
  tc.m0 = row0;
  const int64_t e_end = g.offsets[expert + 1];
  tc.m_end = (row0 + C::BM < e_end) ? row0 + C::BM : e_end;
  tc.n0 = tn * C::BN;
  tc.split = 0;
  tc.kt_begin = 0;
  tc.kt_end = (g.K + BK - 1) / BK;
  tc.expert = expert;
  const int64_t lda = g.K >> 1, ldas = g.K >> 5;
  run_tile<C>(g, tc, g.b_codes + (int64_t)expert * g.N * lda, g.b_scales + (int64_t)expert * g.N * ldas, smem);
}

// One thread per expert slot: m-tile j of expert e gets entry
// (prefix of tile counts before e) + j. Unused entries get expert -1.
__global__ void build_tile_map_kernel(const int32_t* __restrict__ off, int E, int bm, int64_t max_mtiles,
                                      int32_t* __restrict__ map) {
  __shared__ int64_t base[1];
  if (threadIdx.x == 0) {
    int64_t acc = 0;
    for (int e = 0; e < E; ++e) {
      const int64_t rows = (int64_t)off[e + 1] - off[e];
      const int64_t tiles = rows > 0 ? (rows + bm - 1) / bm : 0;
      for (int64_t j = 0; j < tiles && acc < max_mtiles; ++j, ++acc) {
        map[2 * acc] = e;
        map[2 * acc + 1] = (int32_t)(off[e] + j * bm);
      }
    }
    base[0] = acc;
  }
  __syncthreads();
  for (int64_t i = base[0] + threadIdx.x; i < max_mtiles; i += blockDim.x) {
    map[2 * i] = -1;
    map[2 * i + 1] = 0;
  }
}

__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ part, int splits, int64_t M,
                                                            int64_t N, void* __restrict__ y, int64_t ldy, bool bf16) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= M * N) return;
  float s = 0.0f;
  for (int k = 0; k < splits; ++k) s += part[(int64_t)k * M * N + i];
  const int64_t m = i / N, n = i - m * N;
  if (bf16) static_cast<uint16_t*>(y)[m * ldy + n] = f32_to_bf16_rne(s);
  else static_cast<float*>(y)[m * ldy + n] = s;
}

using CfgL = TileCfg<256, 256, 2, 2, 32>;  // prefill
using CfgM = TileCfg<128, 256, 2, 2, 32>;
using CfgS64 = TileCfg<64, 256, 1, 4, 32>;
using CfgS32 = TileCfg<32, 256, 1, 4, 32>;
using CfgS16 = TileCfg<16, 256, 1, 4, 16>;

template <class C>
hipError_t launch_cfg(const GemmArgs& g, hipStream_t stream) {
  const int64_t mt = (g.M + C::BM - 1) / C::BM;
  const int64_t nt = (g.N + C::BN - 1) / C::BN;
  const int64_t total = mt * nt * g.splits;
  if (total > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(gemm_kernel<C>, dim3((unsigned)total), dim3(C::NT), 0, stream, g);
  return hipGetLastError();
}

template <class C>
hipError_t launch_grouped_cfg(const GemmArgs& g, hipStream_t stream) {
  hipLaunchKernelGGL(build_tile_map_kernel, dim3(1), dim3(256), 0, stream, g.offsets, g.E, C::BM, g.max_mtiles,
                     g.tile_map);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t nt = (g.N + C::BN - 1) / C::BN;
  const int64_t total = g.max_mtiles * nt;
  if (total > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(gemm_grouped_kernel<C>, dim3((unsigned)total), dim3(C::NT), 0, stream, g);
  return hipGetLastError();
}

constexpr int kNumCu = 256;

}  // namespace

GemmPlan plan_gemm(int64_t M, int64_t N, int64_t K) {
  GemmPlan p{};
  if (M <= 16) { p.cfg = 4; p.bm = 16; }
  else if (M <= 32) { p.cfg = 3; p.bm = 32; }
  else if (M <= 64) { p.cfg = 2; p.bm = 64; }
  else if (M <= 1024) { p.cfg = 1; p.bm = 128; }
  else { p.cfg = 0; p.bm = 256; }
  p.bn = 256;
  const int64_t tiles = ((M + p.bm - 1) / p.bm) * ((N + p.bn - 1) / p.bn);
  const int64_t KT = (K + BK - 1) / BK;
  int splits = 1;
  // split K when the tiles alone leave most of the chip idle
  while (tiles * splits * 2 <= 2 * kNumCu && KT / (splits * 2) >= 4 && splits < 16) splits *= 2;
  p.splits = splits;
  p.partial_bytes = splits > 1 ? (size_t)splits * (size_t)M * (size_t)N * sizeof(float) : 0;
  return p;
}

GemmPlan plan_gemm_grouped(int64_t T, int E, int64_t N, int64_t K) {
  (void)T;
  (void)E;
  (void)N;
  (void)K;
  GemmPlan p{};
  p.cfg = 1;
  p.bm = 128;
  p.bn = 256;
  p.splits = 1;
  p.partial_bytes = 0;
  return p;
}

hipError_t launch_gemm(const GemmArgs& g, const GemmPlan& p, hipStream_t stream) {
  if (g.M == 0) return hipSuccess;
  hipError_t e;
  switch (p.cfg) {
    case 0: e = launch_cfg<CfgL>(g, stream); break;
    case 1: e = launch_cfg<CfgM>(g, stream); break;
    case 2: e = launch_cfg<CfgS64>(g, stream); break;
    case 3: e = launch_cfg<CfgS32>(g, stream); break;
    default: e = launch_cfg<CfgS16>(g, stream); break;
  }
  if (e != hipSuccess || g.splits <= 1) return e;
  const int64_t n = g.M * g.N;
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, g.partial,
                     g.splits, g.M, g.N, g.y, g.ldy, g.y_bf16);
  return hipGetLastError();
}

hipError_t launch_gemm_grouped(const GemmArgs& g, const GemmPlan& p, hipStream_t stream) {
  (void)p;
  return launch_grouped_cfg<CfgM>(g, stream);
}

}  // namespace macaq
