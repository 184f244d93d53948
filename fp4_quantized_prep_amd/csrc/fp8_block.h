// Device arithmetic of the packed-UE8M0 FP8 1x128 quantization, shared by the
// standalone quantizer and the one-launch small-batch indexer-Q kernel so that
// both produce the same bytes (tokenspeed PR "perf(deepseek-v4): accelerate
// indexer Q and packed FP8 quantization", Summary and Risk and fallback).
//
// A 128-element block is held by 8 consecutive lanes, 16 bf16 each.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace iqp {
namespace {
namespace fp8q {

typedef unsigned v4u __attribute__((ext_vector_type(4)));

// DPP controls (gfx9 encoding)
constexpr int DPP_QUAD_XOR1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int DPP_QUAD_XOR2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int DPP_ROW_HALF_MIRROR = 0x141;
constexpr int DPP_ROW_MIRROR = 0x140;

// maximum over each group of 8 lanes (a block)
__device__ __forceinline__ uint32_t lanes8_max(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, DPP_QUAD_XOR1, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, DPP_QUAD_XOR2, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, DPP_ROW_HALF_MIRROR, 0xF, 0xF, false));
  return v;
}

// Largest |bf16| of the two halves of a dword, as 15-bit magnitude codes.
__device__ __forceinline__ uint32_t mag2(uint32_t d) {
  return max(d & 0x7FFFu, (d >> 16) & 0x7FFFu);
}

// Largest magnitude code of a lane's 16 bf16 values.
__device__ __forceinline__ uint32_t mag16(v4u a, v4u b) {
  return max(max(max(mag2(a[0]), mag2(a[1])), max(mag2(a[2]), mag2(a[3]))),
             max(max(mag2(b[0]), mag2(b[1])), max(mag2(b[2]), mag2(b[3]))));
}

// Scale exponent from the bf16 magnitude code of the block amax:
// e = max(ceil(log2(amax / 448)), -22). With amax = (1 + f/128) 2^(E-127) and
// 448 = (1 + 96/128) 2^8, amax/448 <= 2^(E-135) exactly when f <= 96. E = 0
// (zero or subnormal amax) lands on the floor.
__device__ __forceinline__ int block_exponent(uint32_t amag) {
  const int E = (int)(amag >> 7);
  const int f = (int)(amag & 0x7F);
  const int e = E - 135 + (f > 96 ? 1 : 0);
  return max(e, -22);
}

// Four bf16 (two dwords) times 2^-e, rounded to E4M3 by v_cvt_pk_fp8_f32.
__device__ __forceinline__ uint32_t cvt4(uint32_t d0, uint32_t d1, float mul) {
  // bf16 -> f32 is a 16-bit shift; element 2k is the low half of dword k
  const float f0 = __uint_as_float(d0 << 16) * mul;
  const float f1 = __uint_as_float(d0 & 0xFFFF0000u) * mul;
  const float f2 = __uint_as_float(d1 << 16) * mul;
  const float f3 = __uint_as_float(d1 & 0xFFFF0000u) * mul;
  int r = __builtin_amdgcn_cvt_pk_fp8_f32(f0, f1, 0, false);
  r = __builtin_amdgcn_cvt_pk_fp8_f32(f2, f3, r, true);
  return (uint32_t)r;
}

// The lane's 16 E4M3 codes, given its 16 bf16 values (a, b) and the block
// exponent e (every lane of the block holds the same e).
__device__ __forceinline__ v4u codes16(v4u a, v4u b, int e) {
  const float mul = __uint_as_float((uint32_t)(127 - e) << 23);  // 2^-e, a normal float
  return v4u{cvt4(a[0], a[1], mul), cvt4(a[2], a[3], mul), cvt4(b[0], b[1], mul), cvt4(b[2], b[3], mul)};
}

typedef unsigned v2u __attribute__((ext_vector_type(2)));

// maximum over each row of 16 lanes (a block in the word layout below)
__device__ __forceinline__ uint32_t lanes16_max(uint32_t v) {
  v = lanes8_max(v);
  return max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, DPP_ROW_MIRROR, 0xF, 0xF, false));
}

// One wave's share of the packed quantization of a row-major [M, K] bf16
// matrix: packed words first and first + 1 (row-major over [M, nw], nw =
// ceil(K / 512), `words` = M nw in all). In load k lane l reads 16 bytes (8
// bf16) of word first + k at byte 16 l, so every load covers 1 KiB
// contiguously and 16 lanes hold one 128-element block; the block amax is a
// DPP maximum over that row of lanes; v_cvt_pk_fp8_f32 rounds x 2^-e to
// E4M3; lanes store 8 bytes each; the word's four block bytes (zero past
// the last block) are gathered by readlane and stored by lane 0. NT_STORE:
// non-temporal code stores. Used by the standalone quantizer and, beside
// the one-launch indexer-Q kernel, for an independent matrix.
template <bool NT_STORE>
__device__ __forceinline__ void quant_word_pair(const uint16_t* __restrict__ x, int64_t ldx, uint8_t* __restrict__ q,
                                                int64_t ldq, int32_t* __restrict__ scales, int64_t sm, int64_t sw,
                                                int32_t nw, int32_t nkb, int64_t words, int64_t first, int lane) {
  const int blk = lane >> 4;  // block of this lane within a word
  v4u d[2];
  int64_t row[2];
  int w[2];
  bool valid[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int64_t word = first + k;
    row[k] = word / nw;
    w[k] = (int)(word - row[k] * nw);
    valid[k] = word < words && 4 * w[k] + blk < nkb;
    d[k] = v4u{0u, 0u, 0u, 0u};
    if (valid[k])
      d[k] = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(x + row[k] * ldx + (int64_t)w[k] * 512 + lane * 8));
  }
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const uint32_t m = max(max(mag2(d[k][0]), mag2(d[k][1])), max(mag2(d[k][2]), mag2(d[k][3])));
    const int e = block_exponent(lanes16_max(m));
    const float mul = __uint_as_float((uint32_t)(127 - e) << 23);  // 2^-e, a normal float
    const v2u o = v2u{cvt4(d[k][0], d[k][1], mul), cvt4(d[k][2], d[k][3], mul)};
    if (valid[k]) {
      v2u* dst = reinterpret_cast<v2u*>(q + row[k] * ldq + (int64_t)w[k] * 512 + lane * 8);
      if constexpr (NT_STORE)
        __builtin_nontemporal_store(o, dst);
      else
        *dst = o;
    }
    // the word's four block bytes, from the first lane of each row
    const uint32_t byte = valid[k] ? (uint32_t)(e + 127) : 0u;
    const uint32_t wv = (uint32_t)__builtin_amdgcn_readlane((int)byte, 0) |
                        ((uint32_t)__builtin_amdgcn_readlane((int)byte, 16) << 8) |
                        ((uint32_t)__builtin_amdgcn_readlane((int)byte, 32) << 16) |
                        ((uint32_t)__builtin_amdgcn_readlane((int)byte, 48) << 24);
    if (lane == 0 && first + k < words) scales[row[k] * sm + (int64_t)w[k] * sw] = (int32_t)wv;
  }
}

}  // namespace fp8q
}  // namespace
}  // namespace iqp
