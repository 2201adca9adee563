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
// Both operands come in the GEMM layout (16-row x 128-element blocks of 1 KiB,
// 64-row scale blocks of 256 bytes, zero padding). A workgroup owns a
// BM x BN output tile and walks K in steps of BK = 128 elements. Buffer loads,
// each one contiguous block per wave, run PD steps ahead of the matrix cores,
// held in registers; each step's codes and scales are then written to one of
// three LDS buffers, and its MFMA fragments are read back one step ahead of
// their use. The four 16-byte chunks of each LDS row are XOR-swizzled so that
// the fragment reads of 8 or 16 consecutive rows fall in distinct banks.
#include "common.hpp"

namespace macaq {
namespace {

constexpr int BK = 128;        // K elements per step
constexpr int RB = BK / 2;     // code bytes per row per step (4 chunks of 16)
constexpr int CPR = RB / 16;   // 16-byte chunks per row per step
constexpr int SB = BK / 32;    // scale bytes per row per step (one dword)
constexpr int kNumCu = 256;

template <int BM_, int BN_, int WM_, int WN_, int MF_, int PD_>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, MF = MF_, PD = PD_;
  static constexpr int NT = WM * WN * 64;
  static constexpr int TM = BM / WM, TN = BN / WN;
  static constexpr int FM = TM / MF, FN = TN / MF;
  static constexpr int KSUB = (MF == 32) ? 64 : 128;  // K per MFMA
  static constexpr int NSUB = BK / KSUB;              // MFMAs along K per step
  static constexpr int A_CHUNKS = BM * CPR;
  static constexpr int B_CHUNKS = BN * CPR;
  static constexpr int A_PER_T = (A_CHUNKS + NT - 1) / NT;
  static constexpr int B_PER_T = (B_CHUNKS + NT - 1) / NT;
  static constexpr int A_SC_PER_T = (BM + NT - 1) / NT;
  static constexpr int B_SC_PER_T = (BN + NT - 1) / NT;
  static constexpr int LDS_A = BM * RB, LDS_B = BN * RB, LDS_AS = BM * SB, LDS_BS = BN * SB;
  // writes of threads that have no chunk (small tiles) land in a trash area,
  // so the stores of a step need no branches
  static constexpr int LDS_TRASH = NT * 16;
  static constexpr int LDS_STAGE = LDS_A + LDS_B + LDS_AS + LDS_BS + LDS_TRASH;
  static constexpr int NBUF = 3;  // LDS buffers: compute s, read s+1, write s+2
  static constexpr int LDS_BYTES = NBUF * LDS_STAGE;
  static_assert(TM % MF == 0 && TN % MF == 0, "wave tile must be a multiple of the MFMA tile");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget of a gfx950 workgroup");
  static_assert(PD >= 2 && PD <= 4, "prefetch depth");
  // main-loop unroll: LDS buffer, register slot and fragment set all static
  static constexpr int U = (PD == 4) ? 12 : 6;
  // instructions per step, for the interleaving of the schedule
  static constexpr int N_MFMA = FM * FN;  // per half step
  static constexpr int N_DSR = FM + FN;
  static constexpr int N_DSW = A_PER_T + B_PER_T + A_SC_PER_T + B_SC_PER_T;
  static constexpr int N_VMEM = A_PER_T + B_PER_T + A_SC_PER_T + B_SC_PER_T;
};

// Rows [m0, m_end) of A against rows [n0, n0 + BN) of B over k-steps
// [kt_begin, kt_end).
struct TileCoord {
  int64_t m0, m_end, n0;
  int64_t kt_begin, kt_end;
  int split;
};

template <class C>
struct Stage {
  v4i a[C::A_PER_T];
  v4i b[C::B_PER_T];
  uint32_t as[C::A_SC_PER_T];
  uint32_t bs[C::B_SC_PER_T];
};

// Byte offset of 16-byte chunk `chunk` of LDS row `row`. The chunk slot is
// XORed with (r3 ^ r1, r2) of the row index: any 16 consecutive rows then
// cover all 16 bank groups of 16 bytes for one chunk, and any 8 consecutive
// rows cover all 8 groups of a 128-byte bank set.
__device__ __forceinline__ int swz(int row, int chunk) {
  const int f = ((((row >> 3) ^ (row >> 1)) & 1) << 1) | ((row >> 2) & 1);
  return row * RB + ((chunk ^ f) << 4);
}

// Buffer resources over the operand arrays (GEMM layout, zero padded to 64
// rows and a multiple of 128 in K): loads beyond num_records return zero.
typedef __amdgpu_buffer_rsrc_t Rsrc;
constexpr int kRsrcWord3 = 0x00020000;  // raw (untyped) buffer on gfx9
constexpr uint32_t kOob = 0x80000000u;  // an offset past every buffer (all are < 2 GiB)

__device__ __forceinline__ Rsrc make_rsrc(const void* p, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, kRsrcWord3);
}

struct Operands {
  Rsrc ac, as, bc, bs;  // A codes / scales, B codes / scales (this expert's)
  int64_t N, K;
};

// Per-thread byte offsets of the rows this thread loads, fixed for the tile
// (kOob for rows past the padded operand). In the GEMM layout a k-step of 16
// rows is one 1 KiB block and of 64 rows' scales one 256-byte block, so a
// wave's 16-byte loads of 16 rows read one contiguous block, and the step
// adds kt * 1024 (kt * 256) through the scalar offset.
template <class C>
struct LoadOffsets {
  uint32_t a[C::A_PER_T], b[C::B_PER_T], as[C::A_SC_PER_T], bs[C::B_SC_PER_T];
};

__device__ __forceinline__ uint32_t code_offset(int64_t row, int kc, int64_t ktp, int64_t rows_pad) {
  if (row >= rows_pad) return kOob;
  return (uint32_t)(((row / kTileRows) * ktp) * kCodeBlock + (row % kTileRows) * RB + kc * 16);
}
__device__ __forceinline__ uint32_t scale_offset(int64_t row, int64_t ktp, int64_t rows_pad) {
  if (row >= rows_pad) return kOob;
  return (uint32_t)(((row / kScaleRows) * ktp) * kScaleBlock + (row % kScaleRows) * 4);
}

template <class C>
__device__ __forceinline__ void make_offsets(LoadOffsets<C>& lo, const TileCoord& tc, int64_t a_rows, int64_t N,
                                             int64_t K) {
  const int tid = threadIdx.x;
  const int64_t ktp = pad_k(K) / BK, a_pad = pad_rows(a_rows), n_pad = pad_rows(N);
#pragma unroll
  for (int i = 0; i < C::A_PER_T; ++i) {
    const int c = tid + i * C::NT;
    lo.a[i] = c < C::A_CHUNKS ? code_offset(tc.m0 + c / CPR, c % CPR, ktp, a_pad) : kOob;
  }
#pragma unroll
  for (int i = 0; i < C::B_PER_T; ++i) {
    const int c = tid + i * C::NT;
    lo.b[i] = c < C::B_CHUNKS ? code_offset(tc.n0 + c / CPR, c % CPR, ktp, n_pad) : kOob;
  }
#pragma unroll
  for (int i = 0; i < C::A_SC_PER_T; ++i) {
    const int row = tid + i * C::NT;
    lo.as[i] = row < C::BM ? scale_offset(tc.m0 + row, ktp, a_pad) : kOob;
  }
#pragma unroll
  for (int i = 0; i < C::B_SC_PER_T; ++i) {
    const int row = tid + i * C::NT;
    lo.bs[i] = row < C::BN ? scale_offset(tc.n0 + row, ktp, n_pad) : kOob;
  }
}

// Loads of one k-step, branch-free.
template <class C>
__device__ __forceinline__ void load_stage(Stage<C>& st, const Operands& o, const LoadOffsets<C>& lo, int64_t kt) {
  const int kb = (int)(kt * kCodeBlock), ks = (int)(kt * kScaleBlock);
#pragma unroll
  for (int i = 0; i < C::A_PER_T; ++i)
    st.a[i] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(o.ac, (int)lo.a[i], kb, 0));
#pragma unroll
  for (int i = 0; i < C::B_PER_T; ++i)
    st.b[i] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(o.bc, (int)lo.b[i], kb, 0));
#pragma unroll
  for (int i = 0; i < C::A_SC_PER_T; ++i) st.as[i] = __builtin_amdgcn_raw_buffer_load_b32(o.as, (int)lo.as[i], ks, 0);
#pragma unroll
  for (int i = 0; i < C::B_SC_PER_T; ++i) st.bs[i] = __builtin_amdgcn_raw_buffer_load_b32(o.bs, (int)lo.bs[i], ks, 0);
}

// Per-lane LDS byte offsets, fixed for the kernel. The swizzle depends only
// on bits 1..3 of the row, and every other chunk, fragment or stage this lane
// touches sits a multiple of 16 rows (or a whole buffer) away, so one base
// offset plus a compile-time constant addresses each access.
template <class C>
struct LdsOffsets {
  int wa[C::A_PER_T], wb[C::B_PER_T];           // store_stage: code chunks of this thread
  int wsa[C::A_SC_PER_T], wsb[C::B_SC_PER_T];   // store_stage: scale words of this thread
  int ra[C::NSUB], rb[C::NSUB];  // fragment reads of MFMA s along K, fragment 0
  int rsa, rsb;                  // scale reads, fragment 0
};

template <class C>
__device__ __forceinline__ void make_lds_offsets(LdsOffsets<C>& l, int wm, int wn, int lane) {
  const int tid = threadIdx.x;
  const int trash = C::LDS_A + C::LDS_B + C::LDS_AS + C::LDS_BS + 16 * tid;
#pragma unroll
  for (int i = 0; i < C::A_PER_T; ++i) {
    const int c = tid + i * C::NT;
    l.wa[i] = c < C::A_CHUNKS ? swz(c / CPR, c % CPR) : trash;
  }
#pragma unroll
  for (int i = 0; i < C::B_PER_T; ++i) {
    const int c = tid + i * C::NT;
    l.wb[i] = c < C::B_CHUNKS ? C::LDS_A + swz(c / CPR, c % CPR) : trash;
  }
#pragma unroll
  for (int i = 0; i < C::A_SC_PER_T; ++i) {
    const int row = tid + i * C::NT;
    l.wsa[i] = row < C::BM ? C::LDS_A + C::LDS_B + 4 * row : trash;
  }
#pragma unroll
  for (int i = 0; i < C::B_SC_PER_T; ++i) {
    const int row = tid + i * C::NT;
    l.wsb[i] = row < C::BN ? C::LDS_A + C::LDS_B + C::LDS_AS + 4 * row : trash;
  }
  constexpr int LM = C::MF - 1;
#pragma unroll
  for (int s = 0; s < C::NSUB; ++s) {
    const int chunk = (C::MF == 32) ? s * 2 + (lane >> 5) : (lane >> 4);
    l.ra[s] = swz(wm * C::TM + (lane & LM), chunk);
    l.rb[s] = C::LDS_A + swz(wn * C::TN + (lane & LM), chunk);
  }
  l.rsa = C::LDS_A + C::LDS_B + 4 * (wm * C::TM + (lane & LM));
  l.rsb = C::LDS_A + C::LDS_B + C::LDS_AS + 4 * (wn * C::TN + (lane & LM));
}

template <class T>
__device__ __forceinline__ T& lds_at(uint8_t* smem, int off) {
  return *reinterpret_cast<T*>(smem + off);
}

template <class C, int BUF>
__device__ __forceinline__ void store_stage(const Stage<C>& st, uint8_t* smem, const LdsOffsets<C>& l) {
  constexpr int B0 = BUF * C::LDS_STAGE;
#pragma unroll
  for (int i = 0; i < C::A_PER_T; ++i) lds_at<v4i>(smem, l.wa[i] + B0) = st.a[i];
#pragma unroll
  for (int i = 0; i < C::B_PER_T; ++i) lds_at<v4i>(smem, l.wb[i] + B0) = st.b[i];
#pragma unroll
  for (int i = 0; i < C::A_SC_PER_T; ++i) lds_at<uint32_t>(smem, l.wsa[i] + B0) = st.as[i];
#pragma unroll
  for (int i = 0; i < C::B_SC_PER_T; ++i) lds_at<uint32_t>(smem, l.wsb[i] + B0) = st.bs[i];
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

template <class C, bool = (C::MF == 32)>
struct Acc {
  v16f v[C::FM][C::FN];
};
template <class C>
struct Acc<C, false> {
  v4f v[C::FM][C::FN];
};

// This lane's scale byte for each MFMA of the step, gathered into one dword
// (byte s feeds MFMA s through op_sel). The step's 4 scale bytes of a row are
// one dword; 32x32x64 MFMA s covers bytes 2s, 2s+1 and lane l uses byte
// 2s + l/32; 16x16x128 covers all 4 and lane l uses byte l/16.
template <int MF>
__device__ __forceinline__ int gather_scales(uint32_t w, int lane) {
  if constexpr (MF == 32) {
    const uint32_t h = (uint32_t)(lane >> 5);
    return (int)__builtin_amdgcn_perm(w, w, 0x0C0C0000u | ((2u + h) << 8) | h);
  } else {
    return (int)((w >> (8 * (lane >> 4))) & 0xFFu);
  }
}

// MFMA operands of this wave for one MFMA along K ("half" of a step when
// NSUB == 2, the whole step when NSUB == 1), and a step's scale dwords.
template <class C>
struct Half {
  v4i a[C::FM];
  v4i b[C::FN];
};
template <class C>
struct Scl {
  int sa[C::FM], sb[C::FN];
};

template <class C, int SUB, int BUF>
__device__ __forceinline__ void read_half(Half<C>& h, uint8_t* smem, const LdsOffsets<C>& l) {
  constexpr int B0 = BUF * C::LDS_STAGE;
#pragma unroll
  for (int i = 0; i < C::FM; ++i) h.a[i] = lds_at<v4i>(smem, l.ra[SUB] + B0 + i * C::MF * RB);
#pragma unroll
  for (int j = 0; j < C::FN; ++j) h.b[j] = lds_at<v4i>(smem, l.rb[SUB] + B0 + j * C::MF * RB);
}

template <class C, int BUF>
__device__ __forceinline__ void read_scales(Scl<C>& sc, uint8_t* smem, const LdsOffsets<C>& l, int lane) {
  constexpr int B0 = BUF * C::LDS_STAGE;
#pragma unroll
  for (int i = 0; i < C::FM; ++i) sc.sa[i] = gather_scales<C::MF>(lds_at<uint32_t>(smem, l.rsa + B0 + 4 * i * C::MF), lane);
#pragma unroll
  for (int j = 0; j < C::FN; ++j) sc.sb[j] = gather_scales<C::MF>(lds_at<uint32_t>(smem, l.rsb + B0 + 4 * j * C::MF), lane);
}

template <class C, int SUB>
__device__ __forceinline__ void mfma_half(Acc<C>& acc, const Half<C>& h, const Scl<C>& sc) {
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j) {
      if constexpr (C::MF == 32) acc.v[i][j] = mfma32<SUB>(h.a[i], h.b[j], acc.v[i][j], sc.sa[i], sc.sb[j]);
      else acc.v[i][j] = mfma16<SUB>(h.a[i], h.b[j], acc.v[i][j], sc.sa[i], sc.sb[j]);
    }
}

// Scheduling hints for one step: each MFMA is followed by a share of the
// step's LDS reads (next fragments), LDS writes (step s+2) and buffer loads,
// so the matrix core stays busy while the memory traffic is issued.
constexpr int kSchedMfma = 0x008, kSchedVmemRead = 0x020, kSchedDsRead = 0x100, kSchedDsWrite = 0x200;

template <int T, int NM, int NR, int NW, int NV>
__device__ __forceinline__ void interleave() {
  if constexpr (T < NM) {
    constexpr int r0 = T * NR / NM, r1 = (T + 1) * NR / NM;
    constexpr int w0 = T * NW / NM, w1 = (T + 1) * NW / NM;
    constexpr int v0 = T * NV / NM, v1 = (T + 1) * NV / NM;
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
    if constexpr (r1 > r0) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, r1 - r0, 0);
    if constexpr (w1 > w0) __builtin_amdgcn_sched_group_barrier(kSchedDsWrite, w1 - w0, 0);
    if constexpr (v1 > v0) __builtin_amdgcn_sched_group_barrier(kSchedVmemRead, v1 - v0, 0);
    interleave<T + 1, NM, NR, NW, NV>();
  }
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Tile-relative row / column of register r of fragment (i, j) of this lane.
template <class C>
__device__ __forceinline__ int frag_row(int i, int r, int lane) {
  if constexpr (C::MF == 32) return i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
  else return i * 16 + 4 * (lane >> 4) + r;
}
template <class C>
__device__ __forceinline__ int frag_col(int j, int lane) {
  if constexpr (C::MF == 32) return j * 32 + (lane & 31);
  else return j * 16 + (lane & 15);
}

// OUT: 0 fp32 to Y, 1 bf16 to Y, 2 fp32 to the split-K partial buffer.
template <class C, int OUT, bool FULL>
__device__ __forceinline__ void store_frags(const Acc<C>& acc, void* base, int64_t ld, int64_t m_lim, int64_t n_lim,
                                            int lane) {
  constexpr int NR = (C::MF == 32) ? 16 : 4;
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j) {
      const int n = frag_col<C>(j, lane);
      if (!FULL && n >= n_lim) continue;
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        const int m = frag_row<C>(i, r, lane);
        if (!FULL && m >= m_lim) continue;
        const float v = acc.v[i][j][r];
        if constexpr (OUT == 1) static_cast<uint16_t*>(base)[m * ld + n] = f32_to_bf16_rne(v);
        else static_cast<float*>(base)[m * ld + n] = v;
      }
    }
}

template <class C>
__device__ __forceinline__ void store_out(const Acc<C>& acc, const GemmArgs& g, const TileCoord& tc, int wm, int wn,
                                          int lane) {
  const int64_t m0 = tc.m0 + wm * C::TM, n0 = tc.n0 + wn * C::TN;
  const int64_t m_lim = tc.m_end - m0, n_lim = g.N - n0;
  const bool full = m_lim >= C::TM && n_lim >= C::TN;
  if (g.splits > 1) {
    float* p = g.partial + (int64_t)tc.split * g.M * g.N + m0 * g.N + n0;
    if (full) store_frags<C, 2, true>(acc, p, g.N, m_lim, n_lim, lane);
    else store_frags<C, 2, false>(acc, p, g.N, m_lim, n_lim, lane);
  } else if (g.y_bf16) {
    uint16_t* p = static_cast<uint16_t*>(g.y) + m0 * g.ldy + n0;
    if (full) store_frags<C, 1, true>(acc, p, g.ldy, m_lim, n_lim, lane);
    else store_frags<C, 1, false>(acc, p, g.ldy, m_lim, n_lim, lane);
  } else {
    float* p = static_cast<float*>(g.y) + m0 * g.ldy + n0;
    if (full) store_frags<C, 0, true>(acc, p, g.ldy, m_lim, n_lim, lane);
    else store_frags<C, 0, false>(acc, p, g.ldy, m_lim, n_lim, lane);
  }
}

// The pipelined K loop. Per step s (0-based from kt_begin) and per half h
// (one MFMA along K; NSUB halves per step):
//   - the MFMAs of (s, h) run on fragments already in registers while the
//     fragments of the next half are read from LDS into the other register
//     set: (s, 1) from buffer s % 3, or (s+1, 0) from buffer (s+1) % 3;
//   - in the last half, step s+2 goes from its register slot to LDS buffer
//     (s+2) % 3 and the slot is refilled from memory with step s+2+PD;
//   - one barrier ends the step.
// Buffer (s+2) % 3 held step s-1, whose last reads were issued in step s-1
// and completed at its barrier; buffer (s+1) % 3 was written during step s-1
// and is visible after that barrier. The loop is unrolled U times so the
// register slot (s+2) % PD, the fragment set and the scale set are static, and
// its steady state has no branches, so each wait covers only what it needs.
template <class C>
struct Pipe {
  Acc<C> acc;
  Stage<C> st[C::PD];
  Half<C> hf[2];
  Scl<C> sc[2];
  LoadOffsets<C> lo;
  LdsOffsets<C> lds;
  const Operands& o;
  int64_t kt0, nsteps;
  uint8_t* smem;
  int lane;

  __device__ __forceinline__ Pipe(const Operands& o_, const TileCoord& tc, int64_t a_rows, uint8_t* smem_, int wm,
                                  int wn, int lane_)
      : o(o_), kt0(tc.kt_begin), nsteps(tc.kt_end - tc.kt_begin), smem(smem_), lane(lane_) {
    make_offsets<C>(lo, tc, a_rows, o_.N, o_.K);
    make_lds_offsets<C>(lds, wm, wn, lane_);
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
      for (int j = 0; j < C::FN; ++j) acc.v[i][j] = {};
  }

  template <int P>
  __device__ __forceinline__ void prologue_loads() {
    if constexpr (P < C::PD) {
      if (P < nsteps) load_stage<C>(st[P], o, lo, kt0 + P);
      prologue_loads<P + 1>();
    }
  }

  // Step s = s0 + J with s0 a multiple of U: LDS buffer s % 3 = J % 3,
  // register slot (s+2) % PD, scale set s % 2, fragment set of half h
  // (s * NSUB + h) % 2. FULL: steps s+1, s+2 and s+2+PD exist, no checks.
  //
  // LDS operations complete in order and the wait counter only tracks 15 of
  // them, so the order is chosen so that no MFMA waits behind an LDS write:
  //   phase 1: reads of this step's second half, then the first half's MFMAs
  //            interleaved with the LDS writes of step s+2;
  //   phase 2: the second half's MFMAs interleaved with the reads of step
  //            s+1's first half and scales and with the buffer loads.
  template <int J, bool FULL>
  __device__ __forceinline__ void step(int64_t s) {
    constexpr int SLOT = (J + 2) % C::PD, SC = J % 2;
    constexpr int B_CUR = J % 3, B_NEXT = (J + 1) % 3, B_FILL = (J + 2) % 3;
    constexpr int F0 = (J * C::NSUB) % 2;
    constexpr int FL = (J * C::NSUB + C::NSUB - 1) % 2;  // set of the last half
    const bool has_fill = FULL || s + 2 < nsteps;
    if constexpr (C::NSUB == 2) {
      read_half<C, 1, B_CUR>(hf[F0 ^ 1], smem, lds);
      if (has_fill) store_stage<C, B_FILL>(st[SLOT], smem, lds);
      mfma_half<C, 0>(acc, hf[F0], sc[SC]);
      if constexpr (FULL) {
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, C::FM + C::FN, 0);
        interleave<0, C::N_MFMA, 0, C::N_DSW, 0>();
      }
      __builtin_amdgcn_sched_barrier(0);
    } else {
      if (has_fill) store_stage<C, B_FILL>(st[SLOT], smem, lds);
    }
    if (FULL || s + 1 < nsteps) {
      read_half<C, 0, B_NEXT>(hf[FL ^ 1], smem, lds);
      read_scales<C, B_NEXT>(sc[SC ^ 1], smem, lds, lane);
    }
    if (FULL || s + 2 + C::PD < nsteps) load_stage<C>(st[SLOT], o, lo, kt0 + s + 2 + C::PD);
    mfma_half<C, C::NSUB - 1>(acc, hf[FL], sc[SC]);
    if constexpr (FULL) {
      if constexpr (C::NSUB == 2) interleave<0, C::N_MFMA, C::N_DSR + C::FM + C::FN, 0, C::N_VMEM>();
      else interleave<0, C::N_MFMA, C::N_DSR + C::FM + C::FN, C::N_DSW, C::N_VMEM>();
    }
    // keep this step's MFMAs on this side of the barrier (they touch no memory,
    // so the scheduler would otherwise sink them and keep every step's
    // fragments live at once)
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
  }

  template <int J, bool FULL>
  __device__ __forceinline__ void steps(int64_t s0) {
    if constexpr (J < C::U) {
      if (!FULL && s0 + J >= nsteps) return;
      step<J, FULL>(s0 + J);
      steps<J + 1, FULL>(s0);
    }
  }

  __device__ __forceinline__ void run() {
    if (nsteps <= 0) return;
    prologue_loads<0>();                                  // steps 0 .. PD-1 in slots 0 .. PD-1
    store_stage<C, 0>(st[0], smem, lds);
    if (1 < nsteps) store_stage<C, 1>(st[1], smem, lds);
    if (C::PD < nsteps) load_stage<C>(st[0], o, lo, kt0 + C::PD);        // slot PD % PD
    if (C::PD + 1 < nsteps) load_stage<C>(st[1], o, lo, kt0 + C::PD + 1);  // slot (PD+1) % PD
    __syncthreads();
    read_half<C, 0, 0>(hf[0], smem, lds);
    read_scales<C, 0>(sc[0], smem, lds, lane);
    int64_t s0 = 0;
    for (; s0 + C::U + C::PD + 1 <= nsteps; s0 += C::U) steps<0, true>(s0);
    for (; s0 < nsteps; s0 += C::U) steps<0, false>(s0);
  }
};

template <class C>
__device__ __forceinline__ void run_tile(const GemmArgs& g, const TileCoord& tc, int64_t a_rows, const uint8_t* bc,
                                         const uint8_t* bs, uint8_t* smem) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave / C::WN, wn = wave % C::WN;
  Operands o{make_rsrc(g.a_codes, tiled_codes_bytes(a_rows, g.K)), make_rsrc(g.a_scales, tiled_scales_bytes(a_rows, g.K)),
             make_rsrc(bc, tiled_codes_bytes(g.N, g.K)), make_rsrc(bs, tiled_scales_bytes(g.N, g.K)), g.N, g.K};
  Pipe<C> p(o, tc, a_rows, smem, wm, wn, lane);
  p.run();
  store_out<C>(p.acc, g, tc, wm, wn, lane);
}

// Workgroup ids are dispatched round-robin over the 8 XCDs (id i runs on XCD
// i % 8). Renumber so that each XCD works through a contiguous run of tiles,
// which the grouped order below makes share A and B panels in that XCD's L2.
__device__ __forceinline__ int64_t xcd_remap(int64_t id, int64_t total) {
  if (total % kNumXcd != 0) return id;
  const int64_t per = total / kNumXcd;
  return (id % kNumXcd) * per + id / kNumXcd;
}

template <class C>
__global__ __launch_bounds__(C::NT) __attribute__((amdgpu_waves_per_eu(1, 1))) void gemm_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[C::LDS_BYTES];
  const int64_t mt = (g.M + C::BM - 1) / C::BM;
  const int64_t nt = (g.N + C::BN - 1) / C::BN;
  const int64_t tiles = mt * nt;
  const int64_t total = tiles * g.splits;
  const int64_t id = xcd_remap(blockIdx.x, total);
  const int split = (int)(id / tiles);
  const int64_t t = id - (int64_t)split * tiles;
  // walk tiles in groups of GROUP_M m-tiles, n fastest within a group column
  constexpr int64_t GROUP_M = 8;
  const int64_t group = t / (GROUP_M * nt);
  const int64_t first_m = group * GROUP_M;
  const int64_t gsize = (mt - first_m) < GROUP_M ? (mt - first_m) : GROUP_M;
  const int64_t in_group = t - group * GROUP_M * nt;
  const int64_t tm = first_m + in_group % gsize;
  const int64_t tn = in_group / gsize;
  const int64_t KT = pad_k(g.K) / BK;
  TileCoord tc;
  tc.m0 = tm * C::BM;
  tc.m_end = g.M;
  tc.n0 = tn * C::BN;
  tc.split = split;
  tc.kt_begin = KT * split / g.splits;
  tc.kt_end = KT * (split + 1) / g.splits;
  run_tile<C>(g, tc, g.M, g.b_codes, g.b_scales, smem);
}

// Grouped: the tile map (built by build_tile_map_kernel) lists, per m-tile,
// the expert and the first row; tiles past the used count exit at once.
template <class C>
__global__ __launch_bounds__(C::NT) __attribute__((amdgpu_waves_per_eu(1, 1))) void gemm_grouped_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[C::LDS_BYTES];
  const int64_t nt = (g.N + C::BN - 1) / C::BN;
  const int64_t id = xcd_remap(blockIdx.x, g.max_mtiles * nt);
  const int64_t tm = id / nt;
  const int64_t tn = id - tm * nt;
  const int32_t expert = g.tile_map[2 * tm];
  if (expert < 0) return;
  const int64_t row0 = g.tile_map[2 * tm + 1];
  const int64_t e_end = g.offsets[expert + 1];
  TileCoord tc;
  tc.m0 = row0;
  tc.m_end = (row0 + C::BM < e_end) ? row0 + C::BM : e_end;
  tc.n0 = tn * C::BN;
  tc.split = 0;
  tc.kt_begin = 0;
  tc.kt_end = pad_k(g.K) / BK;
  run_tile<C>(g, tc, g.M, g.b_codes + (int64_t)expert * tiled_codes_bytes(g.N, g.K),
              g.b_scales + (int64_t)expert * tiled_scales_bytes(g.N, g.K), smem);
}

// One thread walks the experts: m-tile j of expert e gets entry (tiles of
// experts before e) + j; the remaining entries get expert -1.
__global__ void build_tile_map_kernel(const int32_t* __restrict__ off, int E, int bm, int64_t max_mtiles,
                                      int32_t* __restrict__ map) {
  __shared__ int64_t used[1];
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
    used[0] = acc;
  }
  __syncthreads();
  for (int64_t i = used[0] + threadIdx.x; i < max_mtiles; i += blockDim.x) {
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

using CfgL = TileCfg<256, 256, 2, 2, 32, 2>;   // large prefill
using CfgM = TileCfg<128, 256, 2, 2, 32, 3>;   // prefill
using CfgS64 = TileCfg<64, 256, 1, 4, 32, 3>;  // decode, M <= 64
using CfgS32 = TileCfg<32, 256, 1, 4, 32, 3>;
using CfgS16 = TileCfg<16, 256, 1, 4, 16, 3>;

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

}  // namespace

GemmPlan plan_gemm(int64_t M, int64_t N, int64_t K) {
  GemmPlan p{};
  if (M <= 16) { p.cfg = 4; p.bm = 16; }
  else if (M <= 32) { p.cfg = 3; p.bm = 32; }
  else if (M <= 64) { p.cfg = 2; p.bm = 64; }
  else { p.cfg = 1; p.bm = 128; }
  p.bn = 256;
  const int64_t nt = (N + p.bn - 1) / p.bn;
  // the large tile only when it still gives every CU a tile
  if (false && M > 1024 && ((M + 255) / 256) * nt >= kNumCu) {
    p.cfg = 0;
    p.bm = 256;
  }
  const int64_t tiles = ((M + p.bm - 1) / p.bm) * nt;
  const int64_t KT = pad_k(K) / BK;
  int splits = 1;
  // split K only for skinny (decode) shapes whose tiles leave most CUs idle
  if (M <= 64)
    while (tiles * splits * 2 <= 2 * kNumCu && KT / (splits * 2) >= 8 && splits < 16) splits *= 2;
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
