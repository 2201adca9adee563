// One MX group of 32 values per lane: the block-Hadamard butterflies and the
// MXFP4 encode, shared by the activation quantizer and the GEMM epilogue that
// produces the next layer's quantized input (gfx950).
//
// Method: "MACaQ: Fast, Model Agnostic Calibrated Quantization for
// Low-Precision Weights and Activations" (paper card, Abstract) applies a
// block-Hadamard transform to the scaled activations and quantizes them to
// MXFP4 (OCP Microscaling Formats v1.0: 32 E2M1 codes share one E8M0 scale).
#pragma once

#include "common.hpp"

namespace macaq {

// The value of lane ^ d (d = 1 or 2, inside a quad of lanes) through a DPP
// quad permutation: [1,0,3,2] for d = 1, [2,3,0,1] for d = 2.
__device__ __forceinline__ float xor_lane(float x, int d) {
  return __int_as_float(d == 1 ? __builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, false)
                               : __builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, false));
}

// Sylvester butterflies of span 1 .. B/2 in ascending order over a lane's 32
// consecutive values: spans 1 .. 16 inside the lane, spans 32 and 64 (B = 64,
// 128) between the lanes of chunks c ^ 1 and c ^ 2 of the same row, which sit
// in one quad of lanes (c = the chunk's index in its quad). Each butterfly
// (u, v) -> (u + v, u - v) keeps the sum in the lower position.
template <int B>
__device__ __forceinline__ void fwht_lane(float (&v)[32], int c) {
  if constexpr (B > 0) {
#pragma unroll
    for (int h = 1; h < 32; h <<= 1) {
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        if (i & h) continue;
        const float u = v[i], w = v[i + h];
        v[i] = u + w;
        v[i + h] = u - w;
      }
    }
    // across lanes: the lower chunk keeps u + w, the upper one u - w. fma
    // with +-1 rounds once, exactly as the plain add or subtract would.
#pragma unroll
    for (int d = 1; d < B / 32; d <<= 1) {
      const float sgn = (c & d) ? -1.0f : 1.0f;
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const float p = xor_lane(v[i], d);
        v[i] = __builtin_fmaf(sgn, v[i], p);
      }
    }
  }
}

// MXFP4 of one group: E8M0 scale = biased exponent of amax minus E2M1's
// largest exponent (2), clamped at 0 (2^-127), which covers amax == 0 and
// subnormal amax; E2M1 codes by the hardware scaled convert (round to
// nearest even, saturating at 6, sign kept), element 2i in the low nibble of
// byte i. Returns the scale code.
__device__ __forceinline__ int mx_encode(const float (&v)[32], uint4& out) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const int ebits = (int)((__float_as_uint(amax) >> 23) & 0xFF);
  const int sc = ebits > 2 ? ebits - 2 : 0;
  const float scale = sc ? __uint_as_float((uint32_t)sc << 23) : __uint_as_float(0x00400000u);
  uint32_t packed[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    uint32_t w = 0;
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[8 * d], v[8 * d + 1], scale, 0);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[8 * d + 2], v[8 * d + 3], scale, 1);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[8 * d + 4], v[8 * d + 5], scale, 2);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[8 * d + 6], v[8 * d + 7], scale, 3);
    packed[d] = w;
  }
  out = make_uint4(packed[0], packed[1], packed[2], packed[3]);
  return sc;
}

}  // namespace macaq
