// W4A4 GEMM on gfx950's scaled-FP4 matrix cores.
//
// Y[m, n] = sum_k dq(A[m, k]) dq(W'[n, k]): the contraction of the MACaQ
// layer ("MACaQ: Fast, Model Agnostic Calibrated Quantization for
// Low-Precision Weights and Activations", paper card, Abstract: MXFP4 W4A4).
// Both operands are packed E2M1 with one E8M0 scale per 32 elements along K,
// in the GEMM layout (common.hpp): every 1 KiB of codes is one operand of
// V_MFMA_SCALE_F32_32X32X64_F8F6F4 in FP4 mode (lane l = row l%32, 32 K
// elements), and one scale dword per lane serves the 4 MFMAs of a 256-element
// block through op_sel.
//
// The weights are the MFMA's first operand (output rows = n) and the
// activations its second (output columns = m), so output register r of lane l
// of a 32x32 tile is n = 8*(r/4) + 4*(l/32) + r%4, m = l%32: each lane holds
// runs of 4 consecutive n of one output row, stored as 8- or 16-byte vectors.
//
// A workgroup of 4 waves owns a BM x BN output tile and walks K in steps of
// one 256-element block. The waves split BN: each owns BN/4 weight rows and
// all BM activation rows. The weights of a wave are used by that wave only, so
// they go from memory straight into the registers the MFMAs read, PW steps
// ahead. The activation block of a step is shared by all 4 waves: it is loaded
// PA steps ahead into registers, written to one of three LDS buffers, and
// each wave reads its MFMA fragments back one half-step ahead of their use.
// LDS holds only the activations, with the layout's fragment order, so every
// LDS access of a wave is 64 consecutive 16-byte (or 4-byte) words.
#include "mx_lane.hpp"

#include <atomic>

namespace macaq {
namespace {

constexpr int NH = kBlockK / 64;  // MFMAs along K per step (4)
// epilogue staging: one wave's 32 rows of WN bf16, each padded by 16 bytes
constexpr int epi_pitch(int wn) { return wn * 2 + 16; }
constexpr int epi_region(int wn) { return 32 * epi_pitch(wn); }
constexpr int NT = 256;           // 4 waves
constexpr int kNumCu = 256;
// Deferred output keeps a tile's rows within 32-bit buffer offsets (128 rows
// of ldy bf16 below 2 GiB).
constexpr int64_t kDeferMaxLd = int64_t(1) << 22;

constexpr int lcm2(int a, int b) {
  int x = a, y = b;
  while (y) {
    const int t = x % y;
    x = y;
    y = t;
  }
  return a / x * b;
}

// OVERLAP: issue the next tile's loads before the current tile's epilogue
// (hides their latency; keeps both tiles' registers live at once).
// OCC: resident workgroups per CU (waves per SIMD) the register budget is
// sized for; the persistent grid is OCC workgroups per CU.
// DEFER: a tile's bf16 output goes to an LDS region of its own and is written
// to memory during the first steps of the workgroup's next tile, between its
// MFMAs, instead of in a store phase that every CU reaches at the same time.
template <int BM_, int BN_, int PW_, int PA_, bool OVERLAP_ = true, int OCC_ = 1, bool DEFER_ = false>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_, PW = PW_, PA = PA_, OCC = OCC_;
  static constexpr bool OVERLAP = OVERLAP_, DEFER = DEFER_;
  static constexpr int FM = BM / kGroupRows;  // activation fragments (32 rows each)
  static constexpr int WN = BN / 4;           // weight rows per wave
  static constexpr int FN = WN / kGroupRows;  // weight fragments per wave
  static constexpr int A_CODES = FM * kCodeBlock;
  static constexpr int A_SCALES = FM * kScaleBlock;
  static constexpr int A_SCALE_THREADS = FM * 64;  // one scale dword each
  // scale writes of threads without a scale dword land in a trash area, so
  // the stores of a step need no branches
  static constexpr int LDS_TRASH = NT * 4;
  static constexpr int STAGE = A_CODES + A_SCALES + LDS_TRASH;
  static constexpr int NBUF = 3;  // LDS buffers: compute s, read s+1, write s+2
  // deferred output: BM rows of BN bf16 (padded by 16 bytes) after the
  // buffers, written in 1 KiB pieces of PIECE_ROWS rows, PIECES_W per wave
  static constexpr int OUT_PITCH = BN * 2 + 16;
  static constexpr int OUT_OFF = NBUF * STAGE;
  static constexpr int OUT_BYTES = DEFER ? BM * OUT_PITCH : 0;
  static constexpr int PIECE_ROWS = 1024 / (BN * 2);
  static constexpr int PIECES_W = BM / PIECE_ROWS / 4;
  // the epilogue reuses the LDS: one staging region per wave
  static constexpr int LDS_BYTES =
      (NBUF * STAGE + OUT_BYTES > 4 * epi_region(WN)) ? NBUF * STAGE + OUT_BYTES : 4 * epi_region(WN);
  // main-loop unroll: register slots static
  static constexpr int U = lcm2(PW, PA);
  static_assert(!DEFER || (BN == 256 && OCC == 1 && (PIECES_W & (PIECES_W - 1)) == 0), "deferred output pieces");
  static constexpr int N_MFMA = FM * FN;  // per half step
  static_assert(BM % kGroupRows == 0 && BN % (4 * kGroupRows) == 0, "tile shape");
  static_assert(FM <= 4, "at most one scale dword per thread");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget of a gfx950 workgroup");
  static_assert(PW >= 2 && PA >= 2, "prefetch depths");
  // the leading zero steps that round the step count up to a multiple of U
  // must all be loaded by the prologue
  static_assert(U - 1 <= PW - 1 && U - 1 <= PA + 1, "prologue covers the padding steps");
};

// Rows [m0, m_end) of A against rows [n0, n0 + BN) of B over k-blocks
// [kt_begin, kt_end).
struct TileCoord {
  int64_t m0, m_end, n0;
  int64_t kt_begin, kt_end;
  int split;
};

// Buffer resources over the operand arrays: loads past num_records return 0.
typedef __amdgpu_buffer_rsrc_t Rsrc;
constexpr int kRsrcWord3 = 0x00020000;  // raw (untyped) buffer on gfx9
constexpr uint32_t kOob = 0x80000000u;  // an offset past every buffer (all are < 2 GiB)

__device__ __forceinline__ Rsrc make_rsrc(const void* p, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, kRsrcWord3);
}

// soff is the k-block's offset, uniform over the workgroup; readfirstlane
// states that, so it always travels in a scalar register.
__device__ __forceinline__ v4i load16(Rsrc r, uint32_t voff, int soff) {
  return __builtin_bit_cast(
      v4i, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, __builtin_amdgcn_readfirstlane(soff), 0));
}
__device__ __forceinline__ uint32_t load4(Rsrc r, uint32_t voff, int soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, __builtin_amdgcn_readfirstlane(soff), 0);
}

template <class C>
struct WStage {  // one step of this wave's weights
  v4i c[C::FN][NH];
  uint32_t s[C::FN];
};
template <class C>
struct AStage {  // this thread's share of one step of the activation block
  v4i c[C::FM];
  uint32_t s;
};
template <class C>
struct AFrag {  // activation MFMA operands of one half step
  v4i c[C::FM];
};

template <class T>
__device__ __forceinline__ T& lds_at(uint8_t* smem, int off) {
  return *reinterpret_cast<T*>(smem + off);
}

__device__ __forceinline__ v16f mfma(v4i a, v4i b, v16f c, int sa, int sb, int h) {
  v8i a8 = {a[0], a[1], a[2], a[3], 0, 0, 0, 0};
  v8i b8 = {b[0], b[1], b[2], b[3], 0, 0, 0, 0};
  switch (h) {  // op_sel picks the scale byte of the half step: an immediate
    case 0: return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, c, kFmtFp4, kFmtFp4, 0, sa, 0, sb);
    case 1: return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, c, kFmtFp4, kFmtFp4, 1, sa, 1, sb);
    case 2: return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, c, kFmtFp4, kFmtFp4, 2, sa, 2, sb);
    default: return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, c, kFmtFp4, kFmtFp4, 3, sa, 3, sb);
  }
}

// Scheduling hints: each MFMA is followed by a share of the half step's LDS
// reads, LDS writes and buffer loads, so the matrix core stays busy while the
// memory traffic is issued.
constexpr int kSchedMfma = 0x008, kSchedVmemRead = 0x020, kSchedVmemWrite = 0x040, kSchedDsRead = 0x100,
              kSchedDsWrite = 0x200;

template <int T, int NM, int NR, int NW, int NV, int NS = 0>
__device__ __forceinline__ void interleave() {
  if constexpr (T < NM) {
    constexpr int r0 = T * NR / NM, r1 = (T + 1) * NR / NM;
    constexpr int w0 = T * NW / NM, w1 = (T + 1) * NW / NM;
    constexpr int v0 = T * NV / NM, v1 = (T + 1) * NV / NM;
    constexpr int s0 = T * NS / NM, s1 = (T + 1) * NS / NM;
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
    if constexpr (r1 > r0) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, r1 - r0, 0);
    if constexpr (w1 > w0) __builtin_amdgcn_sched_group_barrier(kSchedDsWrite, w1 - w0, 0);
    if constexpr (v1 > v0) __builtin_amdgcn_sched_group_barrier(kSchedVmemRead, v1 - v0, 0);
    if constexpr (s1 > s0) __builtin_amdgcn_sched_group_barrier(kSchedVmemWrite, s1 - s0, 0);
    interleave<T + 1, NM, NR, NW, NV, NS>();
  }
}


template <class C>
struct Acc {
  v16f v[C::FM][C::FN];
};

// OUT: 0 fp32 to Y, 1 bf16 to Y, 2 fp32 to the split-K partial buffer.
// Fragment (i, jn), register 4q + e of lane l: m = 32i + l%32,
// n = 32jn + 8q + 4(l/32) + e. VEC: every run of 4 n may be stored as one
// vector (aligned rows, ld a multiple of 4); FULL: no bounds checks.
template <class C, int OUT, bool VEC, bool FULL>
__device__ __forceinline__ void store_frags(const Acc<C>& acc, void* base, int64_t ld, int64_t m_lim, int64_t n_lim,
                                            int lane) {
#pragma unroll
  for (int i = 0; i < C::FM; ++i) {
    const int m = i * 32 + (lane & 31);
    if (!FULL && m >= m_lim) continue;
#pragma unroll
    for (int jn = 0; jn < C::FN; ++jn)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = jn * 32 + 8 * q + 4 * (lane >> 5);
        const v16f& a = acc.v[i][jn];
        if (VEC && (FULL || n + 3 < n_lim)) {
          if constexpr (OUT == 1) {
            uint2 w;
            w.x = bf16x2_rne(a[4 * q], a[4 * q + 1]);
            w.y = bf16x2_rne(a[4 * q + 2], a[4 * q + 3]);
            *reinterpret_cast<uint2*>(static_cast<uint16_t*>(base) + m * ld + n) = w;
          } else {
            *reinterpret_cast<float4*>(static_cast<float*>(base) + m * ld + n) =
                make_float4(a[4 * q], a[4 * q + 1], a[4 * q + 2], a[4 * q + 3]);
          }
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if (!FULL && n + e >= n_lim) continue;
            if constexpr (OUT == 1) static_cast<uint16_t*>(base)[m * ld + n + e] = (uint16_t)bf16x2_rne(a[4 * q + e], 0.0f);
            else static_cast<float*>(base)[m * ld + n + e] = a[4 * q + e];
          }
        }
      }
  }
}

template <class C, int OUT>
__device__ __forceinline__ void store_sel(const Acc<C>& acc, void* p, int64_t ld, int64_t m_lim, int64_t n_lim,
                                          bool vec, int lane) {
  const bool full = m_lim >= C::BM && n_lim >= C::WN;
  if (vec) {
    if (full) store_frags<C, OUT, true, true>(acc, p, ld, m_lim, n_lim, lane);
    else store_frags<C, OUT, true, false>(acc, p, ld, m_lim, n_lim, lane);
  } else {
    store_frags<C, OUT, false, false>(acc, p, ld, m_lim, n_lim, lane);
  }
}

// bf16 output staged through a wave-private LDS region: per 32-row fragment
// the wave writes its 32 x WN tile in the MFMA layout and reads it back by
// rows, so each store instruction writes whole row segments of 2*WN bytes
// instead of 16-byte pieces of 32 rows.
template <class C>
__device__ __forceinline__ void store_bf16_staged(const Acc<C>& acc, uint16_t* y, int64_t ld, int64_t m_lim,
                                                  int64_t n_lim, uint8_t* region, int lane) {
  constexpr int PITCH = epi_pitch(C::WN);
  constexpr int LPR = C::WN / 8;       // lanes per row (16 bytes each)
  constexpr int RPP = 64 / LPR;        // rows per pass
  static_assert(C::WN == 32 || C::WN == 64, "row segment of one wave");
#pragma unroll
  for (int i = 0; i < C::FM; ++i) {
#pragma unroll
    for (int jn = 0; jn < C::FN; ++jn)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const v16f& a = acc.v[i][jn];
        const int n = jn * 32 + 8 * q + 4 * (lane >> 5);
        uint2 w;
        w.x = bf16x2_rne(a[4 * q], a[4 * q + 1]);
        w.y = bf16x2_rne(a[4 * q + 2], a[4 * q + 3]);
        lds_at<uint2>(region, (lane & 31) * PITCH + n * 2) = w;
      }
#pragma unroll
    for (int p = 0; p < 32 / RPP; ++p) {
      const int r = p * RPP + lane / LPR, c = (lane % LPR) * 8;
      const uint4 v = lds_at<uint4>(region, r * PITCH + c * 2);
      const int m = i * 32 + r;
      if (m < m_lim) {
        uint16_t* dst = y + m * ld + c;
        if (c + 8 <= n_lim) {
          // streaming store: the output is not read again by this kernel
          __builtin_nontemporal_store(v4i{(int)v.x, (int)v.y, (int)v.z, (int)v.w}, reinterpret_cast<v4i*>(dst));
        } else {
          const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (c + e < n_lim) dst[e] = (uint16_t)(u[e >> 1] >> (16 * (e & 1)));
        }
      }
    }
  }
}

// MoE gate/up epilogue: the tile's B rows alternate 32 gate and 32 up rows,
// so wave w holds, per 32-row group of A, gate and up of channels
// c0 + 32w .. c0 + 32w + 31 (c0 = n0 / 2) in matching registers. It writes
// h = SiLU(gate) * up (fp32) to LDS as [BM rows][BN/2 channels], then quads
// of lanes take the 4 channel groups of a row: multiply by the down
// projection's multipliers, block-Hadamard, MXFP4, and store the codes and
// scale in the GEMM layout of the down input. "MACaQ - Huawei open-sources a
// 4-bit quantizer ..." (What it is) covers MoE models; the gated form of the
// expert FFN is a reading.
constexpr int swiglu_pitch(int bn) { return (bn / 2) * 4 + 16; }
template <class C>
constexpr int swiglu_lds() {
  return C::BM * swiglu_pitch(C::BN) + (C::BN / 2) * 4;
}

template <class C, int B>
__device__ __forceinline__ void store_swiglu_quant(const Acc<C>& acc, const GemmArgs& g, const TileCoord& tc,
                                                   int expert, int wave, int lane, uint8_t* smem) {
  static_assert(C::FN == 2, "a wave holds 32 gate and 32 up rows");
  constexpr int CH = C::BN / 2;  // channels of the tile
  constexpr int GR = CH / 32;    // channel groups per row
  constexpr int PITCH = swiglu_pitch(C::BN);
  static_assert(GR == 4 && (C::BM * GR) % NT == 0, "a quad of lanes per row");
  float* mult = reinterpret_cast<float*>(smem + C::BM * PITCH);
  const int tid = threadIdx.x;
  const int64_t c0 = tc.n0 / 2;
  if (tid < CH) {
    const int64_t ch = c0 + tid;
    mult[tid] = (g.q_mult && ch < g.q_F) ? g.q_mult[(int64_t)expert * g.q_F + ch] : 1.0f;
  }
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float h[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float gt = acc.v[i][0][4 * q + e], up = acc.v[i][1][4 * q + e];
        // SiLU(g) = g / (1 + e^-g) through the hardware exp2 and reciprocal
        // (about 1 ulp each); e^-g overflowing to inf gives -0, as it should
        h[e] = gt * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(gt * -1.44269504f)) * up;
      }
      const int row = i * 32 + (lane & 31), ch = wave * 32 + 8 * q + 4 * (lane >> 5);
      lds_at<float4>(smem, row * PITCH + ch * 4) = make_float4(h[0], h[1], h[2], h[3]);
    }
  __syncthreads();
  const int64_t kpad = pad_k(g.q_F);
#pragma unroll
  for (int rd = 0; rd < C::BM * GR / NT; ++rd) {
    const int item = rd * NT + tid;
    const int row = item / GR, grp = item % GR;
    float v[32];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float4 hv = lds_at<float4>(smem, row * PITCH + (grp * 32 + 4 * j) * 4);
      const float4 mv = *reinterpret_cast<const float4*>(mult + grp * 32 + 4 * j);
      v[4 * j] = hv.x * mv.x;
      v[4 * j + 1] = hv.y * mv.y;
      v[4 * j + 2] = hv.z * mv.z;
      v[4 * j + 3] = hv.w * mv.w;
    }
    fwht_lane<B>(v, grp);
    uint4 codes;
    const int sc = mx_encode(v, codes);
    const int64_t m = tc.m0 + row, ch = c0 + grp * 32;
    if (m < tc.m_end && ch < g.q_F) {
      *reinterpret_cast<uint4*>(g.q_codes + tiled_code_offset(m, ch, kpad)) = codes;
      g.q_scales[tiled_scale_offset(m, ch, kpad)] = (uint8_t)sc;
    }
  }
  // the last tile along N also writes the zero padding of K up to kpad
  if (tc.n0 + C::BN >= g.N) {
    const int g0 = (int)(g.q_F / 32), g1 = (int)(kpad / 32);
    for (int item = tid; item < C::BM * (g1 - g0); item += NT) {
      const int row = item / (g1 - g0), grp = g0 + item % (g1 - g0);
      const int64_t m = tc.m0 + row;
      if (m < tc.m_end) {
        *reinterpret_cast<uint4*>(g.q_codes + tiled_code_offset(m, (int64_t)grp * 32, kpad)) = make_uint4(0, 0, 0, 0);
        g.q_scales[tiled_scale_offset(m, (int64_t)grp * 32, kpad)] = 0;
      }
    }
  }
}

// Output modes, chosen on the host per launch: fp32 to Y, bf16 to Y (plain
// stores), bf16 to Y staged through LDS (aligned rows), fp32 split-K partials,
// and the MoE gate/up epilogue with a Hadamard block of 0, 32, 64 or 128.
enum OutMode {
  kOutF32 = 0,
  kOutBf16 = 1,
  kOutBf16Staged = 2,
  kOutPartial = 3,
  kOutSwiGlu0 = 4,
  kOutSwiGlu32 = 5,
  kOutSwiGlu64 = 6,
  kOutSwiGlu128 = 7,
  kOutBf16Defer = 8
};
constexpr bool is_swiglu(int mode) { return mode >= kOutSwiGlu0 && mode <= kOutSwiGlu128; }

template <class C, int MODE>
__device__ __forceinline__ void store_out(const Acc<C>& acc, const GemmArgs& g, const TileCoord& tc, int expert,
                                          int wave, int lane, uint8_t* smem) {
  if constexpr (is_swiglu(MODE)) {
    constexpr int B = MODE == kOutSwiGlu0 ? 0 : (32 << (MODE - kOutSwiGlu32));
    store_swiglu_quant<C, B>(acc, g, tc, expert, wave, lane, smem);
    return;
  }
  const int64_t m0 = tc.m0, n0 = tc.n0 + wave * C::WN;
  const int64_t m_lim = tc.m_end - m0, n_lim = g.N - n0;
  if (n_lim <= 0) return;
  if constexpr (MODE == kOutPartial) {
    float* p = g.partial + (int64_t)tc.split * g.M * g.N + m0 * g.N + n0;
    store_sel<C, 2>(acc, p, g.N, m_lim, n_lim, g.vec_partial, lane);
  } else if constexpr (MODE == kOutBf16Staged) {
    store_bf16_staged<C>(acc, static_cast<uint16_t*>(g.y) + m0 * g.ldy + n0, g.ldy, m_lim, n_lim,
                         smem + wave * epi_region(C::WN), lane);
  } else if constexpr (MODE == kOutBf16) {
    store_sel<C, 1>(acc, static_cast<uint16_t*>(g.y) + m0 * g.ldy + n0, g.ldy, m_lim, n_lim, g.vec_y, lane);
  } else {
    store_sel<C, 0>(acc, static_cast<float*>(g.y) + m0 * g.ldy + n0, g.ldy, m_lim, n_lim, g.vec_y, lane);
  }
}

// The pipelined K loop over k-blocks [kt0, kt0 + nsteps). Per step s and
// half step h (one MFMA along K, 4 per step):
//   - the MFMAs of (s, h) read the weight registers of step s (slot s % PW)
//     and the activation fragments of (s, h), read from LDS during the
//     previous half step; meanwhile the fragments of the next half are read:
//     (s, h+1) from buffer s % 3, or (s+1, 0) and step s+1's scales from
//     buffer (s+1) % 3;
//   - after the MFMAs of (s, h), the weight registers of half h are refilled
//     with step s+PW (the scale dwords after the last half);
//   - in half 0, the activation block of step s+2 goes from its register
//     slot to LDS buffer (s+2) % 3; in half 1 the slot is refilled from
//     memory with step s+2+PA;
//   - one barrier ends the step.
// Buffer (s+2) % 3 held step s-1, whose reads all completed before the MFMAs
// of step s-1 were issued, that is before its closing barrier; buffer
// (s+1) % 3 was written during step s-1 and is visible after that barrier.
// Every load and LDS store is unconditional: the loads of steps past the range
// go through an empty buffer resource, so they return zeros without touching
// memory, and nothing uses what they bring. The loop is unrolled
// U = lcm(PW, PA) times so the register slots are static, and the step count
// is rounded up to a multiple of U by leading steps whose loads all return
// zero (a resource of zero bytes), so their MFMAs add nothing. The loop thus
// has one exit and no other branch, and each wait the compiler places covers
// only what it needs.
template <class C>
struct Pipe {
  Acc<C> acc;
  WStage<C> w[C::PW];
  AStage<C> a[C::PA];
  AFrag<C> af[2];
  uint32_t asc[C::FM], asc_next[C::FM];  // activation scale dwords, this / next step
  Rsrc ac, as, bc, bs;
  uint32_t a_off[C::FM], as_off;  // this thread's activation loads
  uint32_t w_off[C::FN], ws_off[C::FN];  // this wave's weight loads
  int la_w, la_ws;                // LDS: this thread's code / scale stores
  int lr, lrs;                    // LDS: this lane's fragment / scale reads
  int b_cur, b_next, b_fill;      // LDS byte offsets of the buffers of steps s, s+1, s+2
  int64_t kt0, nsteps;            // k-block of step 0 (a zero step if pad > 0), steps
  int pad;                        // leading zero steps
  uint8_t* smem;

  AStage<C> t0, t1;  // activation steps 0 and 1 on their way to LDS buffers 0 and 1
  int wave, lane;
  // deferred output of the previous tile (DEFER): rows [0, y_rows) of the
  // LDS output region go to the resource yr (its first row at offset 0);
  // lane offset yo of piece 0 (kOob for a column past N), y_step bytes
  // between a wave's successive pieces
  Rsrc yr;
  uint32_t yo;
  int y_rows, y_step;

  __device__ __forceinline__ Pipe(uint8_t* smem_, int wave_, int lane_) : smem(smem_), wave(wave_), lane(lane_) {
    const int tid = threadIdx.x;
    la_w = tid * 16;
    la_ws = tid < C::A_SCALE_THREADS ? C::A_CODES + tid * 4 : C::A_CODES + C::A_SCALES + tid * 4;
    lr = lane * 16;
    lrs = C::A_CODES + lane * 4;
  }

  // Offsets, resources and step count of one output tile.
  __device__ __forceinline__ void set_tile(const GemmArgs& g, const TileCoord& tc, int64_t a_rows,
                                           const uint8_t* bcodes, const uint8_t* bscales) {
    const int tid = threadIdx.x;
    const int64_t n = tc.kt_end - tc.kt_begin;
    pad = (int)((C::U - n % C::U) % C::U);
    kt0 = tc.kt_begin - pad;
    nsteps = n + pad;
    const int64_t kpad = pad_k(g.K), a_pad = pad_rows(a_rows), n_pad = pad_rows(g.N);
    ac = make_rsrc(g.a_codes, tiled_codes_bytes(a_rows, g.K));
    as = make_rsrc(g.a_scales, tiled_scales_bytes(a_rows, g.K));
    bc = make_rsrc(bcodes, tiled_codes_bytes(g.N, g.K));
    bs = make_rsrc(bscales, tiled_scales_bytes(g.N, g.K));
    // activations: thread t loads byte 16t of each 4 KiB fragment block, which
    // belongs to lane t%64 of half t/64; the row is per thread, so a tile may
    // start at any row (MoE experts)
    const int hl = tid >> 6, ln = tid & 63;
#pragma unroll
    for (int i = 0; i < C::FM; ++i) {
      const int64_t row = tc.m0 + i * kGroupRows + (ln & 31);
      a_off[i] = row < a_pad ? (uint32_t)(tiled_code_offset(row, (int64_t)(2 * hl + (ln >> 5)) * 32, kpad)) : kOob;
    }
    {
      const int64_t row = tc.m0 + hl * kGroupRows + (ln & 31);
      as_off = (tid < C::A_SCALE_THREADS && row < a_pad)
                   ? (uint32_t)(tiled_scale_offset(row, (int64_t)(ln >> 5) * 32, kpad))
                   : kOob;
    }
    // weights: wave-owned 32-row groups, aligned (n0 is a multiple of BN)
#pragma unroll
    for (int j = 0; j < C::FN; ++j) {
      const int64_t row = tc.n0 + wave * C::WN + j * kGroupRows;
      const int64_t blk = (row / kGroupRows) * (kpad / kBlockK);
      w_off[j] = row < n_pad ? (uint32_t)(blk * kCodeBlock + lane * 16) : kOob;
      ws_off[j] = row < n_pad ? (uint32_t)(blk * kScaleBlock + lane * 4) : kOob;
    }
  }

  // k-block of step s (past the range for the loads of the last steps).
  __device__ __forceinline__ int64_t kt_at(int64_t s) const { return kt0 + s; }
  // Resource for the loads of step s: empty (loads return zero and touch no
  // memory) for a leading padding step or a step past the range. A scalar
  // select, so the loop keeps its single basic block.
  __device__ __forceinline__ Rsrc pro(Rsrc r, int s) const { return s < pad ? make_rsrc(nullptr, 0) : r; }
  __device__ __forceinline__ Rsrc live(Rsrc r, int64_t s) const { return s < nsteps ? r : make_rsrc(nullptr, 0); }

  // Weights of k-block kt into a slot: half h only, or the scale dwords.
  __device__ __forceinline__ void load_w_half(WStage<C>& st, int64_t kt, int h, Rsrc rc) {
    const int kb = (int)(kt * kCodeBlock);
#pragma unroll
    for (int j = 0; j < C::FN; ++j) st.c[j][h] = load16(rc, w_off[j] + h * kCodeHalf, kb);
  }
  __device__ __forceinline__ void load_w_scales(WStage<C>& st, int64_t kt, Rsrc rs) {
    const int ks = (int)(kt * kScaleBlock);
#pragma unroll
    for (int j = 0; j < C::FN; ++j) st.s[j] = load4(rs, ws_off[j], ks);
  }
  __device__ __forceinline__ void load_w(WStage<C>& st, int64_t kt, Rsrc rc, Rsrc rs) {
#pragma unroll
    for (int h = 0; h < NH; ++h) load_w_half(st, kt, h, rc);
    load_w_scales(st, kt, rs);
  }
  __device__ __forceinline__ void load_a(AStage<C>& st, int64_t kt, Rsrc rc, Rsrc rs) {
    const int kb = (int)(kt * kCodeBlock), ks = (int)(kt * kScaleBlock);
#pragma unroll
    for (int i = 0; i < C::FM; ++i) st.c[i] = load16(rc, a_off[i], kb);
    st.s = load4(rs, as_off, ks);
  }
  __device__ __forceinline__ void store_a(const AStage<C>& st, int buf) {
#pragma unroll
    for (int i = 0; i < C::FM; ++i) lds_at<v4i>(smem, buf + la_w + i * kCodeBlock) = st.c[i];
    lds_at<uint32_t>(smem, buf + la_ws) = st.s;
  }
  __device__ __forceinline__ void read_frag(AFrag<C>& f, int buf, int h) {
#pragma unroll
    for (int i = 0; i < C::FM; ++i) f.c[i] = lds_at<v4i>(smem, buf + lr + i * kCodeBlock + h * kCodeHalf);
  }
  __device__ __forceinline__ void read_scales(uint32_t (&s)[C::FM], int buf) {
#pragma unroll
    for (int i = 0; i < C::FM; ++i) s[i] = lds_at<uint32_t>(smem, buf + lrs + i * kScaleBlock);
  }

  // Piece j of this wave's share of the deferred output: rows
  // PIECE_ROWS * (wave + 4 j) + lane / (64 / PIECE_ROWS), 16 bytes per lane.
  __device__ __forceinline__ int piece_row(int j) const {
    return C::PIECE_ROWS * (wave + 4 * j) + lane / (64 / C::PIECE_ROWS);
  }
  __device__ __forceinline__ v4i read_piece(int j) const {
    const int col = lane % (64 / C::PIECE_ROWS);
    return lds_at<v4i>(smem, C::OUT_OFF + piece_row(j) * C::OUT_PITCH + col * 16);
  }
  // live == false: the store goes through an empty resource (writes nothing).
  __device__ __forceinline__ void store_piece(int j, v4i d, bool live = true) const {
    const uint32_t off = piece_row(j) < y_rows ? yo + (uint32_t)(j * y_step) : kOob;
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned, d),
                                           live ? yr : make_rsrc(nullptr, 0), (int)off, 0, 0);
  }
  // Nothing pending (the first tile of the workgroup): the stores of the
  // first steps go through an empty resource and write nothing.
  __device__ __forceinline__ void clear_pending() {
    yr = make_rsrc(nullptr, 0);
    yo = kOob;
    y_rows = 0;
    y_step = 0;
  }
  // The tile's accumulators as bf16 into the LDS output region (the caller
  // makes it visible with a barrier), and the tile becomes the pending one.
  __device__ __forceinline__ void stage_out(const GemmArgs& g, const TileCoord& tc) {
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
      for (int jn = 0; jn < C::FN; ++jn)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const v16f& a = acc.v[i][jn];
          const int m = i * 32 + (lane & 31);
          const int n = wave * C::WN + jn * 32 + 8 * q + 4 * (lane >> 5);
          uint2 w;
          w.x = bf16x2_rne(a[4 * q], a[4 * q + 1]);
          w.y = bf16x2_rne(a[4 * q + 2], a[4 * q + 3]);
          lds_at<uint2>(smem, C::OUT_OFF + m * C::OUT_PITCH + n * 2) = w;
        }
    const int64_t m_lim = tc.m_end - tc.m0, n_lim = g.N - tc.n0;
    uint16_t* base = static_cast<uint16_t*>(g.y) + tc.m0 * g.ldy;
    yr = make_rsrc(base, ((m_lim - 1) * g.ldy + g.N) * 2);
    const int col = (lane % (64 / C::PIECE_ROWS)) * 8;
    yo = col < n_lim ? (uint32_t)((piece_row(0) * g.ldy + tc.n0 + col) * 2) : kOob;
    y_rows = (int)m_lim;
    y_step = (int)(4 * C::PIECE_ROWS * g.ldy * 2);
  }
  // Pieces [j0, PIECES_W) of the pending output.
  __device__ __forceinline__ void flush(int64_t j0 = 0) {
    for (int j = (int)j0; j < C::PIECES_W; ++j) store_piece(j, read_piece(j));
  }

  template <int H, int WS, int FS>
  __device__ __forceinline__ void mfma_half() {
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
      for (int j = 0; j < C::FN; ++j)
        acc.v[i][j] = mfma(w[WS].c[j][H], af[FS].c[i], acc.v[i][j], (int)w[WS].s[j], (int)asc[i], H);
  }

  // Half H of step s (J = s % U). DEF: half 0 also stores piece s of the
  // deferred output (none once s >= PIECES_W).
  template <int J, int H, bool DEF = false>
  __device__ __forceinline__ void half(int64_t s) {
    constexpr int WS = J % C::PW, AS = (J + 2) % C::PA;
    constexpr int FS = H & 1;
    constexpr int NR = (H < NH - 1) ? C::FM : 2 * C::FM;
    constexpr int NW = (H == 0) ? C::FM + 1 : 0;
    constexpr int NV = C::FN + ((H == NH - 1) ? C::FN : 0) + ((H == 1) ? C::FM + 1 : 0);
    if constexpr (H < NH - 1) {
      read_frag(af[FS ^ 1], b_cur, H + 1);
    } else {
      read_frag(af[FS ^ 1], b_next, 0);
      read_scales(asc_next, b_next);
    }
    if constexpr (H == 0) store_a(a[AS], b_fill);
    if constexpr (H == 1) load_a(a[AS], kt_at(s + 2 + C::PA), live(ac, s + 2 + C::PA), live(as, s + 2 + C::PA));
    constexpr bool PIECE = DEF && H == 0;
    mfma_half<H, WS, FS>();
    // read late so the piece does not hold registers across the MFMAs
    if constexpr (PIECE) store_piece((int)s & (C::PIECES_W - 1), read_piece((int)s & (C::PIECES_W - 1)), s < C::PIECES_W);
    load_w_half(w[WS], kt_at(s + C::PW), H, live(bc, s + C::PW));
    if constexpr (H == NH - 1) load_w_scales(w[WS], kt_at(s + C::PW), live(bs, s + C::PW));
    // the next half's LDS reads go first (they complete under this half's
    // MFMAs); the LDS writes and buffer loads are spread between the MFMAs
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, NR, 0);
    interleave<0, C::N_MFMA, 0, NW, NV>();
    if constexpr (PIECE) {
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedVmemWrite, 1, 0);
    }
    // keep this half's MFMAs on this side of the fence (they touch no memory,
    // so the scheduler would otherwise sink them and keep every half's
    // operands live at once)
    __builtin_amdgcn_sched_barrier(0);
  }

  template <int J, bool DEF = false>
  __device__ __forceinline__ void step(int64_t s) {
    half<J, 0, DEF>(s);
    half<J, 1, DEF>(s);
    half<J, 2, DEF>(s);
    half<J, 3, DEF>(s);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < C::FM; ++i) asc[i] = asc_next[i];
    const int t = b_cur;
    b_cur = b_next;
    b_next = b_fill;
    b_fill = t;
  }

  template <int J, bool DEF = false>
  __device__ __forceinline__ void steps(int64_t s0) {
    if constexpr (J < C::U) {
      step<J, DEF>(s0 + J);
      steps<J + 1, DEF>(s0);
    }
  }

  template <int P>
  __device__ __forceinline__ void prologue_a() {
    if constexpr (P < C::PA) {
      load_a(a[(2 + P) % C::PA], kt_at(2 + P), pro(ac, 2 + P), pro(as, 2 + P));
      prologue_a<P + 1>();
    }
  }
  template <int P>
  __device__ __forceinline__ void prologue_w() {
    if constexpr (P < C::PW) {
      load_w(w[P], kt_at(P), pro(bc, P), pro(bs, P));
      prologue_w<P + 1>();
    }
  }

  // Issue order: activation steps 0 and 1 (to LDS buffers 0 and 1 through
  // registers of their own) and the weight slot of step 0, which is all the
  // first step waits for, then the activation slots of steps 2 .. PA+1 and
  // the weight slots of steps 1 .. PW-1. The fences keep that order, so the
  // first step starts once its own operands are in, not behind the loads of
  // later steps (every CU issues its prologue at the same moment).
  __device__ __forceinline__ void prologue_loads() {
    load_a(t0, kt_at(0), pro(ac, 0), pro(as, 0));
    load_a(t1, kt_at(1), pro(ac, 1), pro(as, 1));
    __builtin_amdgcn_sched_barrier(0);
    load_w(w[0], kt_at(0), pro(bc, 0), pro(bs, 0));
    __builtin_amdgcn_sched_barrier(0);
    prologue_a<0>();
    __builtin_amdgcn_sched_barrier(0);
    prologue_w<1>();
    __builtin_amdgcn_sched_barrier(0);
  }

  // After prologue_loads, with the LDS idle in every wave.
  __device__ __forceinline__ void prologue_lds() {
    store_a(t0, 0);
    store_a(t1, C::STAGE);
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    b_cur = 0;
    b_next = C::STAGE;
    b_fill = 2 * C::STAGE;
    read_frag(af[0], 0, 0);
    read_scales(asc, 0);
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
      for (int j = 0; j < C::FN; ++j) acc.v[i][j] = {};
  }

  // The K loop; its last barrier leaves every LDS buffer idle. DEF: step s
  // also writes piece s of the pending output, and the pieces a short tile
  // did not reach follow the loop, fenced from the next staging by a barrier.
  // PEEL: the first iteration is its own code, so the loop keeps the steady
  // state's waits (the compiler's waits at a loop top otherwise also cover
  // the prologue's pending loads); nsteps is a positive multiple of U.
  template <bool DEF = false, bool PEEL = false>
  __device__ __forceinline__ void loop() {
    int64_t s0 = 0;
    if constexpr (PEEL) {
      steps<0, DEF>(0);
      s0 = C::U;
    }
    for (; s0 < nsteps; s0 += C::U) steps<0, DEF>(s0);
    if constexpr (DEF) {
      if (nsteps < C::PIECES_W) {
        flush(nsteps);
        __syncthreads();
      }
    }
  }
};

// Tile t of the launch: coordinates and this expert's weights (grouped), or
// false for an unused tile of the grouped launch.
struct TileRef {
  TileCoord tc;
  const uint8_t* bc;
  const uint8_t* bs;
  int expert;
};

template <class C, bool GROUPED>
__device__ __forceinline__ bool tile_at(const GemmArgs& g, int64_t t, TileRef& r) {
  const int64_t nt = (g.N + C::BN - 1) / C::BN;
  const int64_t KT = pad_k(g.K) / kBlockK;
  if constexpr (GROUPED) {
    const int64_t tm = t / nt, tn = t - tm * nt;
    const int32_t expert = g.tile_map[2 * tm];
    if (expert < 0) return false;
    const int64_t row0 = g.tile_map[2 * tm + 1];
    const int64_t e_end = g.offsets[expert + 1];
    r.tc.m0 = row0;
    r.tc.m_end = (row0 + C::BM < e_end) ? row0 + C::BM : e_end;
    r.tc.n0 = tn * C::BN;
    r.tc.split = 0;
    r.tc.kt_begin = 0;
    r.tc.kt_end = KT;
    r.expert = expert;
    r.bc = g.b_codes + (int64_t)expert * tiled_codes_bytes(g.N, g.K);
    r.bs = g.b_scales + (int64_t)expert * tiled_scales_bytes(g.N, g.K);
  } else {
    const int64_t mt = (g.M + C::BM - 1) / C::BM;
    const int64_t tiles = mt * nt;
    const int split = (int)(t / tiles);
    const int64_t u = t - (int64_t)split * tiles;
    // walk tiles in groups of GROUP_M m-tiles, n fastest within a group column
    constexpr int64_t GROUP_M = 8;
    const int64_t group = u / (GROUP_M * nt);
    const int64_t first_m = group * GROUP_M;
    const int64_t gsize = (mt - first_m) < GROUP_M ? (mt - first_m) : GROUP_M;
    const int64_t in_group = u - group * GROUP_M * nt;
    const int64_t tm = first_m + in_group % gsize;
    const int64_t tn = in_group / gsize;
    r.tc.m0 = tm * C::BM;
    r.tc.m_end = g.M;
    r.tc.n0 = tn * C::BN;
    r.tc.split = split;
    r.tc.kt_begin = KT * split / g.splits;
    r.tc.kt_end = KT * (split + 1) / g.splits;
    r.bc = g.b_codes;
    r.bs = g.b_scales;
    r.expert = 0;
  }
  return true;
}

// Workgroup ids are dispatched round-robin over the 8 XCDs (id i runs on XCD
// i % 8). Renumber so that each XCD works through a contiguous run of tiles
// (the first total % 8 XCDs one tile more), which the grouped order above
// makes share A and B panels in that XCD's L2.
__device__ __forceinline__ int64_t xcd_remap(int64_t id, int64_t total) {
  const int64_t x = id % kNumXcd, q = total / kNumXcd, r = total % kNumXcd;
  return x * q + (x < r ? x : r) + id / kNumXcd;
}

// Persistent workgroups: workgroup b takes tiles b, b + G, b + 2G, ... (G
// workgroups). The next tile's loads are issued before the current tile's
// epilogue, so its memory latency hides behind the output stores.
template <class C, bool GROUPED, int MODE>
__device__ __forceinline__ void gemm_tiles(const GemmArgs& g, int64_t total, uint8_t* smem) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  Pipe<C> p(smem, wave, lane);
  int64_t t = blockIdx.x;
  TileRef cur;
  while (t < total && !tile_at<C, GROUPED>(g, xcd_remap(t, total), cur)) t += gridDim.x;
  if (t >= total) return;
  p.set_tile(g, cur.tc, g.M, cur.bc, cur.bs);
  p.prologue_loads();
  constexpr bool DEF = MODE == kOutBf16Defer;
  if constexpr (DEF) p.clear_pending();
  for (;;) {
    p.prologue_lds();
    // (grouped kernels: the peeled copy spills registers, except with the
    // deferred output)
    p.template loop<DEF, !GROUPED || DEF>();
    TileRef nxt;
    int64_t tn = t + gridDim.x;
    while (tn < total && !tile_at<C, GROUPED>(g, xcd_remap(tn, total), nxt)) tn += gridDim.x;
    if (C::OVERLAP && tn < total) {
      p.set_tile(g, nxt.tc, g.M, nxt.bc, nxt.bs);
      p.prologue_loads();
    }
    if constexpr (DEF) {
      // the pending output was read from LDS during this tile's steps, whose
      // barriers every wave has passed
      p.stage_out(g, cur.tc);
      __syncthreads();
      if (tn >= total) {
        p.flush();
        break;
      }
    } else {
      store_out<C, MODE>(p.acc, g, cur.tc, cur.expert, wave, lane, smem);
      if (tn >= total) break;
    }
    if (!C::OVERLAP) {
      p.set_tile(g, nxt.tc, g.M, nxt.bc, nxt.bs);
      p.prologue_loads();
    }
    __syncthreads();  // every wave is done with its epilogue staging in LDS
    cur = nxt;
    t = tn;
  }
}

template <class C, int MODE>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(C::OCC, C::OCC))) void gemm_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[C::LDS_BYTES];
  const int64_t tiles = ((g.M + C::BM - 1) / C::BM) * ((g.N + C::BN - 1) / C::BN);
  gemm_tiles<C, false, MODE>(g, tiles * g.splits, smem);
}

// ---------------------------------------------------------------------------
// Wide tiles for large prefill shapes: 256 activation rows x 256 weight rows
// per workgroup of 4 waves. Wave w owns weight rows [64w, 64w + 64) of the
// tile and all 256 activation rows (8 x 2 fragments of 32 x 32, 256 fp32
// accumulators per lane). One 256-element step moves 34 KiB of activations
// and 34 KiB of weights for 33.5 MFLOP, two thirds of the bytes per flop of
// the 128 x 256 tile. The activation block goes from memory straight into LDS
// (buffer loads with the LDS flag, so no registers stage it) into one of four
// stages, each wave loading two of its eight row groups; the weights of a
// wave go into the registers its MFMAs read, two steps ahead, as in Pipe.
// Steps run on across tiles: the last steps of a tile already load the first
// steps of the workgroup's next tile, so only the epilogue separates them.
//
// Per step s (J = s % 4, stage J holds step s) and half step h:
//   h < 3: read the fragments of (s, h+1) from stage J;
//   h = 3: wait until this wave's loads of stage J+1 (step s+1) are done,
//          barrier (every wave's are), read the fragments and scales of
//          (s+1, 0) from stage J+1, then load step s+3 into stage J+3 = J-1
//          (last read during step s-1, before the barrier);
//   then the 16 MFMAs of (s, h), and the weight registers of half h are
//   refilled with step s+2 (in half 0 also the weight scale dwords of step
//   s+2, into one of four slots, so no MFMA of step s waits for them).
// The stage wait counts loads in issue order: after the loads of stage J+1
// (issued in half 3 of step s-2) come the 20 loads of step s-1 (10 weight,
// 10 of stage J+2) and the 8 weight loads of halves 0-2 of step s, each half
// fenced from the next, so vmcnt(28) covers stage J+1 and leaves the weights
// of steps s+1 and s+2 in flight (more operations after the stage only make
// the wait stricter). A tile's first two steps wait with the counter's
// maximum instead: the previous tile's output stores sit between their
// stages and the count, so they drain during those steps, and are waited
// for from step 2 on. Loads past a tile's range or of rows past the operand
// go through an empty buffer resource (zeros, no memory traffic) so that
// every step issues the same loads and the counts hold.
struct WideCfg {
  static constexpr int BM = 256, BN = 256, FM = 8, FN = 2, WN = 64;
  static constexpr int A_CODES = FM * kCodeBlock;    // 32 KiB
  static constexpr int A_SCALES = FM * kScaleBlock;  // 2 KiB
  // a stage holds the scales first, then the codes: every read of a stage
  // is within 64 KiB of its start (one base address, immediate offsets)
  static constexpr int CODES_AT = A_SCALES;
  static constexpr int STAGE = A_CODES + A_SCALES;
  static constexpr int GROUP_M = 8;                  // m-tiles that share n-tiles in the walk
  static constexpr int kStageWait = 28;              // vmcnt that covers the next stage (above)
};
static_assert(4 * WideCfg::STAGE <= 160 * 1024, "LDS budget of a gfx950 workgroup");

// Four LDS stages as distinct objects, so the compiler tells the loads into
// one stage from the reads of another and waits only for what a read needs.
__shared__ __attribute__((aligned(1024))) uint8_t wide_st0[WideCfg::STAGE];
__shared__ __attribute__((aligned(1024))) uint8_t wide_st1[WideCfg::STAGE];
__shared__ __attribute__((aligned(1024))) uint8_t wide_st2[WideCfg::STAGE];
__shared__ __attribute__((aligned(1024))) uint8_t wide_st3[WideCfg::STAGE];

template <int S>
__device__ __forceinline__ uint8_t* wide_stage() {
  if constexpr (S == 0) return wide_st0;
  else if constexpr (S == 1) return wide_st1;
  else if constexpr (S == 2) return wide_st2;
  else return wide_st3;
}

typedef __attribute__((address_space(3))) void* LdsPtr;

// 16 (or 4) bytes per lane from the buffer into LDS at lds + 16 * lane (4 *
// lane); lds is uniform over the wave.
__device__ __forceinline__ void dma16(Rsrc r, uint8_t* lds, uint32_t voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (LdsPtr)lds, 16, (int)voff, __builtin_amdgcn_readfirstlane(soff), 0, 0);
}
__device__ __forceinline__ void dma4(Rsrc r, uint8_t* lds, uint32_t voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (LdsPtr)lds, 4, (int)voff, __builtin_amdgcn_readfirstlane(soff), 0, 0);
}

// s_waitcnt immediates (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt
// 6:4, lgkmcnt 11:8); the counters not named keep their maximum.
constexpr int waitcnt_vm_lgkm0(int vm) { return (vm & 0xF) | ((vm >> 4) << 14) | (0x7 << 4); }
constexpr int kWaitAll = 0;

template <int MODE>
struct Wide {
  Acc<WideCfg> acc;
  WStage<WideCfg> w[2];             // weight codes of steps s, s+1 (slot s % 2)
  uint32_t wsc[4][WideCfg::FN];     // weight scale dwords of steps s .. s+2 (slot s % 4)
  AFrag<WideCfg> af;  // activation fragments of the current half step, refilled one by one
  uint32_t asc[WideCfg::FM], asc_next[WideCfg::FM];
  // The tile's operands as buffers that start at its first row group, so a
  // row group past the operand's end falls outside the buffer (loads of
  // zeros, no memory traffic).
  Rsrc ra, ras, rw, rws;
  // This wave's lane offsets into them: activation row groups 2w, 2w+1 by
  // quarter h of the k-block (codes) and their scales; weight row groups
  // 2w, 2w+1 (codes: the quarter is an instruction offset) and scales.
  uint32_t va[2][NH], vas[2], vw[2], vws[2];
  int wave, lane;
  int n;          // k-blocks per tile (a multiple of 4)

  __device__ __forceinline__ void set_tile(const GemmArgs& g, int64_t m0, int64_t n0) {
    const int64_t KB = n;
    const int64_t a0 = (m0 / kGroupRows) * KB, w0 = (n0 / kGroupRows) * KB;
    ra = make_rsrc(g.a_codes + a0 * kCodeBlock, tiled_codes_bytes(g.M, g.K) - a0 * kCodeBlock);
    ras = make_rsrc(g.a_scales + a0 * kScaleBlock, tiled_scales_bytes(g.M, g.K) - a0 * kScaleBlock);
    rw = make_rsrc(g.b_codes + w0 * kCodeBlock, tiled_codes_bytes(g.N, g.K) - w0 * kCodeBlock);
    rws = make_rsrc(g.b_scales + w0 * kScaleBlock, tiled_scales_bytes(g.N, g.K) - w0 * kScaleBlock);
  }

  __device__ __forceinline__ void set_lanes() {
    const uint32_t KB = (uint32_t)n;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint32_t grp = (uint32_t)(2 * wave + i) * KB;
#pragma unroll
      for (int h = 0; h < NH; ++h) va[i][h] = grp * kCodeBlock + h * kCodeHalf + lane * 16;
      vas[i] = grp * kScaleBlock + lane * 4;
      vw[i] = grp * kCodeBlock + lane * 16;
      vws[i] = grp * kScaleBlock + lane * 4;
    }
  }

  // The activation block of k-block kt into stage S (past the tile: zeros
  // through an empty buffer, so every step issues the same loads).
  template <int S>
  __device__ __forceinline__ void load_stage(int kt) {
    uint8_t* st = wide_stage<S>();
    const bool live = kt < n;
    const Rsrc rc = live ? ra : make_rsrc(nullptr, 0), rs = live ? ras : make_rsrc(nullptr, 0);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int h = 0; h < NH; ++h)
        dma16(rc, st + WideCfg::CODES_AT + (2 * wave + i) * kCodeBlock + h * kCodeHalf, va[i][h], kt * kCodeBlock);
#pragma unroll
    for (int i = 0; i < 2; ++i) dma4(rs, st + (2 * wave + i) * kScaleBlock, vas[i], kt * kScaleBlock);
  }

  // Quarter H of this wave's weights of k-block kt into slot st, or the
  // scale dwords.
  template <int H>
  __device__ __forceinline__ void load_w_half(WStage<WideCfg>& st, int kt) {
    const Rsrc r = kt < n ? rw : make_rsrc(nullptr, 0);
#pragma unroll
    for (int j = 0; j < WideCfg::FN; ++j) st.c[j][H] = load16(r, vw[j], kt * kCodeBlock + H * kCodeHalf);
  }
  __device__ __forceinline__ void load_w_scales(uint32_t (&sc)[WideCfg::FN], int kt) {
    const Rsrc r = kt < n ? rws : make_rsrc(nullptr, 0);
#pragma unroll
    for (int j = 0; j < WideCfg::FN; ++j) sc[j] = load4(r, vws[j], kt * kScaleBlock);
  }
  __device__ __forceinline__ void load_w(WStage<WideCfg>& st, uint32_t (&sc)[WideCfg::FN], int kt) {
    load_w_scales(sc, kt);
    load_w_half<0>(st, kt);
    load_w_half<1>(st, kt);
    load_w_half<2>(st, kt);
    load_w_half<3>(st, kt);
  }

  template <int S>
  __device__ __forceinline__ void read_frag(AFrag<WideCfg>& f, int h) {
    const uint8_t* st = wide_stage<S>();
#pragma unroll
    for (int i = 0; i < WideCfg::FM; ++i)
      f.c[i] = *reinterpret_cast<const v4i*>(st + WideCfg::CODES_AT + i * kCodeBlock + h * kCodeHalf + lane * 16);
  }
  template <int S>
  __device__ __forceinline__ void read_scales(uint32_t (&s)[WideCfg::FM]) {
    const uint8_t* st = wide_stage<S>();
#pragma unroll
    for (int i = 0; i < WideCfg::FM; ++i) s[i] = *reinterpret_cast<const uint32_t*>(st + i * kScaleBlock + lane * 4);
  }

  // Half H of step s (J = s % 4): fragment i feeds its two MFMAs, then is
  // refilled at once with fragment i of the next half step (read about 14
  // MFMAs ahead of its use), so one set of fragment registers serves.
  template <int J, int H, int WAIT, bool FIRST>
  __device__ __forceinline__ void half(int s) {
    constexpr int WS = J % 2;
    constexpr int N_MFMA = WideCfg::FM * WideCfg::FN;
    // the next half step: (s, H+1) from stage J, or (s+1, 0) from stage J+1
    constexpr int NS = H < NH - 1 ? J : (J + 1) % 4;
    constexpr int NHH = H < NH - 1 ? H + 1 : 0;
    if constexpr (H == NH - 1) {
      // stage J+1 complete in every wave, and every read of stage J+3 done
      __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(WAIT));
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      read_scales<NS>(asc_next);
      load_stage<(J + 3) % 4>(s + 3);
    }
    const uint8_t* nst = wide_stage<NS>() + WideCfg::CODES_AT + NHH * kCodeHalf + lane * 16;
#pragma unroll
    for (int i = 0; i < WideCfg::FM; ++i) {
#pragma unroll
      for (int j = 0; j < WideCfg::FN; ++j)
        acc.v[i][j] = mfma(w[WS].c[j][H], af.c[i], (FIRST && H == 0) ? v16f{} : acc.v[i][j], (int)wsc[J][j],
                           (int)asc[i], H);
      af.c[i] = *reinterpret_cast<const v4i*>(nst + i * kCodeBlock);
    }
    if constexpr (H == 0) load_w_scales(wsc[(J + 2) % 4], s + 2);
    load_w_half<H>(w[WS], s + 2);
    constexpr int NV = WideCfg::FN + ((H == 0) ? WideCfg::FN : 0) + ((H == NH - 1) ? 10 : 0);
    if constexpr (H == NH - 1) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, WideCfg::FM, 0);
    interleave<0, N_MFMA, WideCfg::FM, 0, NV>();
    __builtin_amdgcn_sched_barrier(0);
  }

  template <int J, int WAIT = WideCfg::kStageWait, bool FIRST = false>
  __device__ __forceinline__ void step(int s) {
    half<J, 0, WAIT, FIRST>(s);
    half<J, 1, WAIT, FIRST>(s);
    half<J, 2, WAIT, FIRST>(s);
    half<J, 3, WAIT, FIRST>(s);
#pragma unroll
    for (int i = 0; i < WideCfg::FM; ++i) asc[i] = asc_next[i];
  }

  // 32 stores into an empty buffer: before a workgroup's first tile they
  // stand in for an output, so that every tile starts with the same count
  // of operations between its stages.
  __device__ __forceinline__ void empty_stores() {
    const Rsrc nr = make_rsrc(nullptr, 0);
    const __attribute__((ext_vector_type(4))) unsigned z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 32; ++i) __builtin_amdgcn_raw_buffer_store_b128(z, nr, 0, 16 * i, 0);
  }

  // Stages 0-2 of a tile (issued before the previous tile's output: they
  // hold no registers).
  __device__ __forceinline__ void prologue_loads() {
    load_stage<0>(0);
    __builtin_amdgcn_sched_barrier(0);
    load_stage<1>(1);
    __builtin_amdgcn_sched_barrier(0);
    load_stage<2>(2);
    __builtin_amdgcn_sched_barrier(0);
  }

  // Weight steps 0 and 1 of a tile, issued right after its stages 0-2 and
  // before the previous tile's output, so that the first MFMAs, which wait
  // for these registers, do not also wait for that output's stores (the
  // counter is in order).
  __device__ __forceinline__ void first_weights() {
    load_w(w[0], wsc[0], 0);
    __builtin_amdgcn_sched_barrier(0);
    load_w(w[1], wsc[1], 1);
    __builtin_amdgcn_sched_barrier(0);
  }

  // Stage 0 visible to every wave, its first fragments and scales read.
  // After stage 0 come stages 1 and 2 and weight steps 0 and 1 (10 loads
  // each) and at least 32 stores (the previous tile's output, or
  // empty_stores): at least 72 operations, so the counter's maximum of 63
  // covers stage 0. The accumulators need no clearing: the tile's first
  // MFMAs take a zero input.
  __device__ __forceinline__ void stage0_ready() {
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(63));
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    read_frag<0>(af, 0);
    read_scales<0>(asc);
  }

  // The tile's output, wave w's 256 rows x 64 columns, through buffer
  // stores into a resource that spans rows [m0, M) from column n0w. A lane's
  // row and column are both in its VGPR offset (the scalar offset is 0), and
  // a lane whose row is past M or whose column run is past N takes an offset
  // past every buffer, so no store depends on whether the range check counts
  // the scalar offset. Needs N % 8 == 0 (bf16: 16-byte runs) or N % 4 == 0 (fp32:
  // 4 consecutive outputs per lane), ldy and Y aligned to match (the launcher
  // checks). Fenced per 32-row fragment so the compiler keeps only one
  // fragment's values in flight.
  __device__ __forceinline__ void epilogue(const GemmArgs& g, int64_t m0, int64_t n0w) {
    const int64_t m_lim = g.M - m0;
    const int m_rows = (int)(m_lim < WideCfg::BM ? m_lim : WideCfg::BM);  // rows of the tile inside M
    const int n_lim = (int)(g.N - n0w < WideCfg::WN ? g.N - n0w : WideCfg::WN);
    constexpr int ES = MODE == kOutBf16Staged ? 2 : 4;
    // a wave whose columns are all past N still issues its stores (into an
    // empty buffer), so every wave issues the same number of them
    const Rsrc yr = n_lim > 0 ? make_rsrc(static_cast<uint8_t*>(g.y) + (m0 * g.ldy + n0w) * ES,
                                          ((m_lim - 1) * g.ldy + n_lim) * ES)
                              : make_rsrc(nullptr, 0);
    // bytes per row (< 2^31: Y is within a 2 GiB buffer range), uniform
    const int ld = __builtin_amdgcn_readfirstlane((int)g.ldy * ES);
    // the lane index is recomputed here (mbcnt) where the compiler cannot
    // hoist it, so the lane's offsets are not held in registers across the
    // main loop
    int ln;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
    if constexpr (MODE == kOutBf16Staged) {
      // Lane l < 32 holds row l, columns 8q .. 8q+3 of each 32-column
      // fragment, lane l+32 columns 8q+4 .. 8q+7: one permlane32 swap per
      // dword of a q pair gives lane l columns 16p .. 16p+7 and lane l+32
      // columns 16p+8 .. 16p+15, so each lane stores 16 contiguous bytes.
      const int r = ln & 31, half = ln >> 5;
#pragma unroll
      for (int i = 0; i < WideCfg::FM; ++i) {
        __builtin_amdgcn_sched_barrier(0);
        // (32i + r) * ld < M * ldy * 2 < 2^31 for a row inside M
        const bool row_in = 32 * i + r < m_rows;
        const uint32_t vrow = (uint32_t)(32 * i + r) * (uint32_t)ld + (uint32_t)(half * 16);
        // keep the row's accumulators in their AGPRs until here, so the
        // conversion copies out one row at a time
#pragma unroll
        for (int jn = 0; jn < WideCfg::FN; ++jn) asm volatile("" : "+a"(acc.v[i][jn]));
#pragma unroll
        for (int jn = 0; jn < WideCfg::FN; ++jn) {
          const v16f& a = acc.v[i][jn];
#pragma unroll
          for (int p = 0; p < 2; ++p) {
            uint32_t lo[2], hi[2];  // q = 2p and q = 2p + 1, two dwords each
#pragma unroll
            for (int d = 0; d < 2; ++d) {
              lo[d] = bf16x2_rne(a[8 * p + 2 * d], a[8 * p + 2 * d + 1]);
              hi[d] = bf16x2_rne(a[8 * p + 4 + 2 * d], a[8 * p + 4 + 2 * d + 1]);
              const auto sw = __builtin_amdgcn_permlane32_swap(lo[d], hi[d], false, false);
              lo[d] = sw[0];
              hi[d] = sw[1];
            }
            const int col = jn * 32 + 16 * p + 8 * half;  // this lane's first column
            const uint32_t vo = row_in && col < n_lim ? vrow + (uint32_t)((jn * 32 + 16 * p) * 2) : kOob;
            const __attribute__((ext_vector_type(4))) unsigned v = {lo[0], lo[1], hi[0], hi[1]};
            __builtin_amdgcn_raw_buffer_store_b128(v, yr, (int)vo, 0, 0);
          }
        }
      }
    } else {
      const int r = ln & 31, c4 = 4 * (ln >> 5);
#pragma unroll
      for (int i = 0; i < WideCfg::FM; ++i) {
        __builtin_amdgcn_sched_barrier(0);
        // (32i + r) * ld < M * ldy * 4 < 2^31 for a row inside M
        const bool row_in = 32 * i + r < m_rows;
#pragma unroll
        for (int jn = 0; jn < WideCfg::FN; ++jn)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const v16f& a = acc.v[i][jn];
            const int n = jn * 32 + 8 * q + c4;
            const uint32_t vo = row_in && n < n_lim ? (uint32_t)(32 * i + r) * (uint32_t)ld + (uint32_t)(n * 4) : kOob;
            const v4f v = {a[4 * q], a[4 * q + 1], a[4 * q + 2], a[4 * q + 3]};
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned, v),
                                                   yr, (int)vo, 0, 0);
          }
      }
    }
  }

  // Tile t of the walk: groups of GROUP_M m-tiles share n-tiles, and each
  // XCD takes a contiguous run of the walk.
  __device__ __forceinline__ void tile_origin(const GemmArgs& g, uint32_t t, uint32_t tiles, int64_t& m0,
                                              int64_t& n0) const {
    const uint32_t x = t % kNumXcd, q = tiles / kNumXcd, r = tiles % kNumXcd;
    const uint32_t u = x * q + (x < r ? x : r) + t / kNumXcd;
    const uint32_t mt = (uint32_t)((g.M + WideCfg::BM - 1) / WideCfg::BM);
    const uint32_t nt = (uint32_t)((g.N + WideCfg::BN - 1) / WideCfg::BN);
    const uint32_t group = u / (WideCfg::GROUP_M * nt);
    const uint32_t first_m = group * WideCfg::GROUP_M;
    const uint32_t gsize = (mt - first_m) < WideCfg::GROUP_M ? (mt - first_m) : WideCfg::GROUP_M;
    const uint32_t in_group = u - group * WideCfg::GROUP_M * nt;
    m0 = (int64_t)(first_m + in_group % gsize) * WideCfg::BM;
    n0 = (int64_t)(in_group / gsize) * WideCfg::BN;
  }

  __device__ __forceinline__ void run(const GemmArgs& g) {
    lane = threadIdx.x & 63;
    wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t tiles =
        (uint32_t)(((g.M + WideCfg::BM - 1) / WideCfg::BM) * ((g.N + WideCfg::BN - 1) / WideCfg::BN));
    n = (int)(pad_k(g.K) / kBlockK);
    set_lanes();
    uint32_t t = blockIdx.x;
    int64_t m0, n0;
    tile_origin(g, t, tiles, m0, n0);
    set_tile(g, m0, n0);
    prologue_loads();
    first_weights();
    empty_stores();
    __builtin_amdgcn_sched_barrier(0);
    stage0_ready();
    for (;;) {
      // The first four steps are their own code, so the loop's waits are
      // those of the steady state. In steps 0 and 1 the stage wait is 63:
      // after stage 1 come stage 2, weight steps 0 and 1 (30), at least 32
      // stores and 8 loads of step 0 (at least 70 operations); after stage 2
      // come 20 + 32 + 20 (step 0) + 8 (at least 80). From step 2 on, the
      // next stage was issued after the stores and the usual count holds.
      step<0, 63, true>(0);
      step<1, 63>(1);
      step<2>(2);
      step<3>(3);
      for (int s0 = 4; s0 < n; s0 += 4) {
        step<0>(s0);
        step<1>(s0 + 1);
        step<2>(s0 + 2);
        step<3>(s0 + 3);
      }
      // every load still in flight is a zero load past the tile (the last
      // real ones fed its last steps): let them land, so that none holds a
      // register the output reuses; then the next tile's first activation
      // blocks and weight steps go out before this tile's output
      __builtin_amdgcn_s_waitcnt(kWaitAll);
      const uint32_t tn = t + gridDim.x;
      const int64_t pm0 = m0, pn0 = n0;
      if (tn < tiles) {
        tile_origin(g, tn, tiles, m0, n0);
        set_tile(g, m0, n0);
        prologue_loads();
        first_weights();
      }
      epilogue(g, pm0, pn0 + wave * WideCfg::WN);
      if (tn >= tiles) break;
      t = tn;
      stage0_ready();
    }
    // loads past the last tile write zeros into LDS: let them land before
    // the workgroup's LDS is released
    __builtin_amdgcn_s_waitcnt(kWaitAll);
  }
};

template <int MODE>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(1, 1))) void gemm_wide_kernel(GemmArgs g) {
  Wide<MODE> p;
  p.run(g);
}

// Grouped: the tile map (built by build_tile_map_kernel) lists, per m-tile,
// the expert and the first row; unused entries are skipped.
template <class C, int MODE>
constexpr int grouped_lds() {
  return (is_swiglu(MODE) && swiglu_lds<C>() > C::LDS_BYTES) ? swiglu_lds<C>() : C::LDS_BYTES;
}

template <class C, int MODE>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(C::OCC, C::OCC))) void gemm_grouped_kernel(
    GemmArgs g) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[grouped_lds<C, MODE>()];
  // the used m-tiles lead the map; the entry after the map holds their count
  const int64_t used = g.tile_map[2 * g.max_mtiles];
  gemm_tiles<C, true, MODE>(g, used * ((g.N + C::BN - 1) / C::BN), smem);
}

// Thread t takes experts [t * ce, (t + 1) * ce): it counts their m-tiles, a
// workgroup scan gives its first entry, and m-tile j of expert e gets entry
// (tiles of experts before e) + j; the remaining entries get expert -1, and
// map[2 * max_mtiles] the number of used entries.
__global__ __launch_bounds__(256) void build_tile_map_kernel(const int32_t* __restrict__ off, int E, int bm,
                                                             int64_t max_mtiles, int32_t* __restrict__ map) {
  __shared__ int sh[256];
  const int tid = threadIdx.x;
  const int ce = (E + 255) / 256;
  const int e0 = tid * ce < E ? tid * ce : E, e1 = e0 + ce < E ? e0 + ce : E;
  int cnt = 0;
  for (int e = e0; e < e1; ++e) {
    const int64_t rows = (int64_t)off[e + 1] - off[e];
    cnt += rows > 0 ? (int)((rows + bm - 1) / bm) : 0;
  }
  int used = 0;
  int64_t acc = block_exclusive_scan<256>(cnt, sh, &used);
  for (int e = e0; e < e1; ++e) {
    const int64_t rows = (int64_t)off[e + 1] - off[e];
    const int64_t tiles = rows > 0 ? (rows + bm - 1) / bm : 0;
    for (int64_t j = 0; j < tiles && acc < max_mtiles; ++j, ++acc) {
      map[2 * acc] = e;
      map[2 * acc + 1] = (int32_t)(off[e] + j * bm);
    }
  }
  const int64_t n_used = used < max_mtiles ? used : max_mtiles;
  for (int64_t i = n_used + tid; i < max_mtiles; i += 256) {
    map[2 * i] = -1;
    map[2 * i + 1] = 0;
  }
  if (tid == 0) map[2 * max_mtiles] = (int32_t)n_used;
}

__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ part, int splits, int64_t M,
                                                            int64_t N, void* __restrict__ y, int64_t ldy, bool bf16) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= M * N) return;
  float s = 0.0f;
  for (int k = 0; k < splits; ++k) s += part[(int64_t)k * M * N + i];
  const int64_t m = i / N, n = i - m * N;
  if (bf16) static_cast<uint16_t*>(y)[m * ldy + n] = (uint16_t)bf16x2_rne(s, 0.0f);
  else static_cast<float*>(y)[m * ldy + n] = s;
}

// The same sums for 4 consecutive outputs of a row per thread (N % 4 == 0,
// y and ldy aligned for 4-element stores): the split loads go out 8 at a time
// before any is added, then are summed in split order from 0, as above, so
// the results are the same bits; the one-element kernel waits for each
// split's load in turn.
__global__ __launch_bounds__(256) void splitk_reduce4_kernel(const float* __restrict__ part, int splits, int64_t M,
                                                             int64_t N, void* __restrict__ y, int64_t ldy, bool bf16) {
  const int64_t MN = M * N;
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= MN) return;
  float4 s = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  for (int k0 = 0; k0 < splits; k0 += 8) {
    float4 v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (k0 + j < splits) v[j] = *reinterpret_cast<const float4*>(part + (int64_t)(k0 + j) * MN + i);
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (k0 + j < splits) {
        s.x += v[j].x;
        s.y += v[j].y;
        s.z += v[j].z;
        s.w += v[j].w;
      }
  }
  const int64_t m = i / N, n = i - m * N;
  if (bf16) {
    uint2 w;
    w.x = bf16x2_rne(s.x, s.y);
    w.y = bf16x2_rne(s.z, s.w);
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(y) + m * ldy + n) = w;
  } else {
    *reinterpret_cast<float4*>(static_cast<float*>(y) + m * ldy + n) = s;
  }
}

// Persistent launches take at most g_workgroup_cap workgroups when it is
// positive. Every persistent kernel strides its tiles by gridDim.x, and the
// XCD renumbering is a bijection of the tiles for any grid, so a smaller
// grid only changes which workgroup computes a tile and in what order.
std::atomic<int32_t> g_workgroup_cap{0};

int64_t persistent_grid(int64_t tiles, int64_t resident) {
  int64_t grid = tiles < resident ? tiles : resident;
  const int32_t cap = g_workgroup_cap.load(std::memory_order_relaxed);
  return (cap > 0 && cap < grid) ? cap : grid;
}

using CfgM = TileCfg<128, 256, 2, 2>;  // prefill
using CfgS64 = TileCfg<64, 128, 4, 2, true, 2>;  // decode, M <= 64
using CfgS32 = TileCfg<32, 128, 4, 2, true, 2>;  // decode, M <= 32
using CfgG = TileCfg<128, 256, 2, 2, true, 1, true>;  // grouped (MoE experts), bf16 / fp32 output
using CfgGS = TileCfg<64, 256, 2, 2, true, 2>;  // grouped with the SwiGLU epilogue (MoE gate/up)

template <class C>
hipError_t launch_cfg(const GemmArgs& g, hipStream_t stream) {
  const int64_t mt = (g.M + C::BM - 1) / C::BM;
  const int64_t nt = (g.N + C::BN - 1) / C::BN;
  const int64_t total = mt * nt * g.splits;
  if (total > 0x7FFFFFFF) return hipErrorInvalidValue;
  const int64_t resident = (int64_t)kNumCu * C::OCC;
  const int64_t grid = persistent_grid(total, resident);
  const dim3 gd((unsigned)grid), bd(NT);
  if constexpr (C::DEFER) {
    if (g.splits == 1 && g.y_bf16 && g.vec16_y && g.N % 8 == 0 && g.ldy < kDeferMaxLd) {
      hipLaunchKernelGGL((gemm_kernel<C, kOutBf16Defer>), gd, bd, 0, stream, g);
      return hipGetLastError();
    }
  }
  if (g.splits > 1) hipLaunchKernelGGL((gemm_kernel<C, kOutPartial>), gd, bd, 0, stream, g);
  else if (g.y_bf16 && g.vec16_y) hipLaunchKernelGGL((gemm_kernel<C, kOutBf16Staged>), gd, bd, 0, stream, g);
  else if (g.y_bf16) hipLaunchKernelGGL((gemm_kernel<C, kOutBf16>), gd, bd, 0, stream, g);
  else hipLaunchKernelGGL((gemm_kernel<C, kOutF32>), gd, bd, 0, stream, g);
  return hipGetLastError();
}

template <class C, bool SWIGLU>
hipError_t launch_grouped_cfg(const GemmArgs& g, hipStream_t stream) {
  if (!g.map_ready) {
    hipLaunchKernelGGL(build_tile_map_kernel, dim3(1), dim3(256), 0, stream, g.offsets, g.E, C::BM, g.max_mtiles,
                       g.tile_map);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t nt = (g.N + C::BN - 1) / C::BN;
  const int64_t total = g.max_mtiles * nt;
  if (total > 0x7FFFFFFF) return hipErrorInvalidValue;
  const int64_t resident = (int64_t)kNumCu * C::OCC;
  const int64_t grid = persistent_grid(total, resident);
  const dim3 gd((unsigned)grid), bd(NT);
  if constexpr (SWIGLU) {
    switch (g.q_b) {
      case 0: hipLaunchKernelGGL((gemm_grouped_kernel<C, kOutSwiGlu0>), gd, bd, 0, stream, g); break;
      case 32: hipLaunchKernelGGL((gemm_grouped_kernel<C, kOutSwiGlu32>), gd, bd, 0, stream, g); break;
      case 64: hipLaunchKernelGGL((gemm_grouped_kernel<C, kOutSwiGlu64>), gd, bd, 0, stream, g); break;
      default: hipLaunchKernelGGL((gemm_grouped_kernel<C, kOutSwiGlu128>), gd, bd, 0, stream, g); break;
    }
  } else {
    if constexpr (C::DEFER) {
      if (g.y_bf16 && g.vec16_y && g.N % 8 == 0 && g.ldy < kDeferMaxLd) {
        hipLaunchKernelGGL((gemm_grouped_kernel<C, kOutBf16Defer>), gd, bd, 0, stream, g);
        return hipGetLastError();
      }
    }
    if (g.y_bf16 && g.vec16_y) hipLaunchKernelGGL((gemm_grouped_kernel<C, kOutBf16Staged>), gd, bd, 0, stream, g);
    else if (g.y_bf16) hipLaunchKernelGGL((gemm_grouped_kernel<C, kOutBf16>), gd, bd, 0, stream, g);
    else hipLaunchKernelGGL((gemm_grouped_kernel<C, kOutF32>), gd, bd, 0, stream, g);
  }
  return hipGetLastError();
}

// The wide kernel's output stores need whole 16-byte runs of a row (bf16
// with N % 8 == 0, fp32 with N % 4 == 0, row starts aligned to them) and
// address Y through a 32-bit buffer range.
bool wide_output_ok(const GemmArgs& g) {
  const int64_t es = g.y_bf16 ? 2 : 4;
  if (g.M * g.ldy * es >= (int64_t(1) << 31)) return false;
  return g.y_bf16 ? (g.vec16_y && g.N % 8 == 0) : (g.vec_y && g.N % 4 == 0);
}

hipError_t launch_wide(const GemmArgs& g, hipStream_t stream) {
  const int64_t tiles = ((g.M + WideCfg::BM - 1) / WideCfg::BM) * ((g.N + WideCfg::BN - 1) / WideCfg::BN);
  if (tiles > 0x7FFFFFFF || g.splits != 1 || !wide_output_ok(g)) return hipErrorInvalidValue;
  const dim3 gd((unsigned)persistent_grid(tiles, kNumCu)), bd(NT);
  if (g.y_bf16) hipLaunchKernelGGL(gemm_wide_kernel<kOutBf16Staged>, gd, bd, 0, stream, g);
  else hipLaunchKernelGGL(gemm_wide_kernel<kOutF32>, gd, bd, 0, stream, g);
  return hipGetLastError();
}

// Vector stores of 4 outputs need 4-element alignment of every row start.
void set_vec_flags(GemmArgs& g) {
  const size_t es = g.y_bf16 ? 2 : 4;
  g.vec_y = (reinterpret_cast<uintptr_t>(g.y) % (4 * es)) == 0 && g.ldy % 4 == 0;
  g.vec_partial = g.N % 4 == 0;  // the partial buffer is 256-byte aligned
  g.vec16_y = g.y_bf16 && (reinterpret_cast<uintptr_t>(g.y) % 16) == 0 && g.ldy % 8 == 0;
}

}  // namespace

void set_workgroup_cap(int32_t n) { g_workgroup_cap.store(n > 0 ? n : 0, std::memory_order_relaxed); }

// Bytes a CU would stream in the time a work unit spends starting its
// pipeline (first loads in flight, nothing consumed yet).
constexpr double kUnitStartBytes = 64.0 * 1024.0;

GemmPlan plan_gemm(int64_t M, int64_t N, int64_t K) {
  GemmPlan p{};
  int64_t resident;
  const int64_t wide_tiles = ((M + WideCfg::BM - 1) / WideCfg::BM) * ((N + WideCfg::BN - 1) / WideCfg::BN);
  if (M <= 32) { p.cfg = 3; p.bm = CfgS32::BM; p.bn = CfgS32::BN; resident = (int64_t)kNumCu * CfgS32::OCC; }
  else if (M <= 64) { p.cfg = 2; p.bm = CfgS64::BM; p.bn = CfgS64::BN; resident = (int64_t)kNumCu * CfgS64::OCC; }
  else if (wide_tiles >= kNumCu && (pad_k(K) / kBlockK) % 4 == 0) {
    p.cfg = 4;
    p.bm = WideCfg::BM;
    p.bn = WideCfg::BN;
    resident = kNumCu;
  }
  else { p.cfg = 1; p.bm = CfgM::BM; p.bn = CfgM::BN; resident = (int64_t)kNumCu * CfgM::OCC; }
  const int64_t nt = (N + p.bn - 1) / p.bn;
  const int64_t tiles = ((M + p.bm - 1) / p.bm) * nt;
  const int64_t KT = pad_k(K) / kBlockK;
  int64_t splits = 1;
  // Skinny (decode) shapes stream the weights. Split K (units of at least 4
  // k-blocks) to keep every CU streaming: the units spread evenly over the
  // CUs, so the time goes as the weight bytes of the busiest CU (units per
  // CU, rounded up, times the longest unit plus a pipeline start of about
  // kUnitStartBytes each), plus the fp32 partial sums written and read back.
  if (M <= 64 && tiles < resident) {
    const double row_block_bytes = (double)p.bn * kBlockK * 17.0 / 32.0;  // one tile's weights per k-block
    double best = 0.0;
    for (int64_t s = 1; s <= KT / 4 || s == 1; ++s) {
      const int64_t units = tiles * s;
      const int64_t per_cu = (units + kNumCu - 1) / kNumCu;
      const double unit_bytes = row_block_bytes * (double)((KT + s - 1) / s);
      const double partial = s > 1 ? 8.0 * (double)M * (double)N * (double)s : 0.0;
      const double cost = (double)kNumCu * (double)per_cu * (unit_bytes + kUnitStartBytes) + partial;
      if (s == 1 || cost < best) {
        best = cost;
        splits = s;
      }
    }
  }
  p.splits = (int)splits;
  p.partial_bytes = splits > 1 ? (size_t)splits * (size_t)M * (size_t)N * sizeof(float) : 0;
  return p;
}

GemmPlan plan_gemm_grouped(int64_t T, int E, int64_t N, int64_t K, bool swiglu) {
  (void)T;
  (void)E;
  (void)N;
  (void)K;
  GemmPlan p{};
  p.cfg = swiglu ? 2 : 1;
  p.bm = swiglu ? CfgGS::BM : CfgG::BM;
  p.bn = swiglu ? CfgGS::BN : CfgG::BN;
  p.splits = 1;
  p.partial_bytes = 0;
  return p;
}

hipError_t launch_gemm(const GemmArgs& g_in, const GemmPlan& p, hipStream_t stream) {
  if (g_in.M == 0) return hipSuccess;
  GemmArgs g = g_in;
  set_vec_flags(g);
  hipError_t e;
  switch (p.cfg) {
    case 4: e = wide_output_ok(g) ? launch_wide(g, stream) : launch_cfg<CfgM>(g, stream); break;
    case 1: e = launch_cfg<CfgM>(g, stream); break;
    case 2: e = launch_cfg<CfgS64>(g, stream); break;
    default: e = launch_cfg<CfgS32>(g, stream); break;
  }
  if (e != hipSuccess || g.splits <= 1) return e;
  const int64_t n = g.M * g.N;
  if (g.vec_partial && g.vec_y) {
    const int64_t threads = n / 4;
    hipLaunchKernelGGL(splitk_reduce4_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream,
                       g.partial, g.splits, g.M, g.N, g.y, g.ldy, g.y_bf16);
  } else {
    hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, g.partial,
                       g.splits, g.M, g.N, g.y, g.ldy, g.y_bf16);
  }
  return hipGetLastError();
}

hipError_t launch_gemm_grouped(const GemmArgs& g_in, const GemmPlan& p, hipStream_t stream) {
  (void)p;
  GemmArgs g = g_in;
  set_vec_flags(g);
  if (p.cfg == 2) {
    if (!g.swiglu) return hipErrorInvalidValue;
    return launch_grouped_cfg<CfgGS, true>(g, stream);
  }
  if (g.swiglu) return hipErrorInvalidValue;
  return launch_grouped_cfg<CfgG, false>(g, stream);
}

}  // namespace macaq
