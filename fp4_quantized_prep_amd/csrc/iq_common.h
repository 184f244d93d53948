// Device helpers shared by the fused indexer-Q kernels: operand and
// accumulator types, cross-half lane exchange, the FP4 block exponent, the
// RoPE table rows, the per-sub-tile epilogue (RoPE, Hadamard-128, FP4) and
// the buffer / barrier / wait-count primitives.
#pragma once

#include "iqp_internal.h"

namespace iqp {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int HEAD_DIM = 128;
constexpr int KB = 128;              // K block (one activation / weight scale)
constexpr float INV_SQRT_128 = 0.08838834764831845f;

__device__ __forceinline__ v8i make_v8i(v4u a, v4u b) {
  v8i r;
  r[0] = (int)a[0]; r[1] = (int)a[1]; r[2] = (int)a[2]; r[3] = (int)a[3];
  r[4] = (int)b[0]; r[5] = (int)b[1]; r[6] = (int)b[2]; r[7] = (int)b[3];
  return r;
}

// Exchange with the partner lane l^32: returns {value of lane l&31, value of lane l|32}
// for the pair (x, y): lanes < 32 receive x's two halves, lanes >= 32 receive y's.
__device__ __forceinline__ void swap32(float x, float y, float& r0, float& r1) {
  auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  r0 = __uint_as_float(s[0]);
  r1 = __uint_as_float(s[1]);
}

__device__ __forceinline__ uint32_t swap32_u(uint32_t x, uint32_t y, uint32_t& r1) {
  auto s = __builtin_amdgcn_permlane32_swap(x, y, false, false);
  r1 = s[1];
  return s[0];
}

// FP4 block exponent: e = max(ceil(log2(amax / 6)), -15) from the float bits of
// amax >= 0. With amax = (1 + f 2^-23) 2^(E-127) and 6 = 1.5 * 2^2,
// amax / 6 <= 2^(E-129) exactly when f <= 2^22.
__device__ __forceinline__ int fp4_exponent(float amax) {
  const uint32_t b = __float_as_uint(amax);
  const int E = (int)(b >> 23);
  const int e = E - 129 + ((b & 0x7FFFFFu) > 0x400000u ? 1 : 0);
  return max(e, -15);
}

// FP4 block exponent by the OCP MX rule, e = max(floor(log2 amax), floor(log2 1e-4)) - 2,
// from the float bits of amax >= 0 (floor(log2 1e-4) = -14)
__device__ __forceinline__ int fp4_exponent_floor(float amax) {
  return max((int)(__float_as_uint(amax) >> 23) - 129, -16);
}

// Convention variants of the FP4-output kernels ride on the STAGE template
// argument: STAGE = -1 - v with v bit 0 = interleaved RoPE pairs (2i, 2i+1),
// bit 1 = OCP floor-rule FP4 scales, bit 2 = one weight scale per row and K
// block; the diagnostic stages (>= 0) and STAGE = -1 take the defaults (pairs
// (i, i+32), e = ceil(log2(amax / 6)), one weight scale per 128x128 tile).
constexpr int stage_of_variant(int v) { return -1 - v; }
constexpr bool stage_interleaved(int stage) { return stage < 0 && ((-1 - stage) & 1); }
constexpr bool stage_floor(int stage) { return stage < 0 && ((-1 - stage) & 2); }
constexpr bool stage_row_scales(int stage) { return stage < 0 && ((-1 - stage) & 4); }

// ---------------------------------------------------------------------------
// Epilogue for one 32-token column tile of one head: acc[tn][r] holds head dim
//   d = 32 tn + 8 (r >> 2) + 4 half + (r & 3)
// of token t (lane % 32 of the tile). RoPE, the seven Hadamard stages and the
// FP4 quantization all run on these registers.
// cos / sin of the RoPE pairs one lane rotates (its 16 of the 32 pairs), from
// the table row of its token's position (clamped to the table).
struct RopeCS {
  v4f c[4], s[4];
};

__device__ __forceinline__ int64_t load_position(int64_t t, const IndexerQArgs& p) {
  return p.positions[t < p.M ? t : p.M - 1];
}

// Half-split: c[g][s] is the cosine of pair 8g + 4half + s. Interleaved: the
// lane's pairs are i = 16tn + 4g + 2half + k (dims 2i, 2i+1 in registers
// 4g + 2k, 4g + 2k + 1 of acc[tn], tn < 2), held as c[2tn + (g >> 1)][2(g & 1) + k],
// i.e. table entries 8j + 2half + {0, 1} and 8j + 2half + {4, 5} of c[j].
template <bool INTERLEAVED = false>
__device__ __forceinline__ RopeCS load_rope(int64_t pos, int half, const IndexerQArgs& p) {
  pos = pos < 0 ? 0 : (pos >= p.max_pos ? p.max_pos - 1 : pos);
  const float* cs = p.cos_sin + pos * 64;
  RopeCS r;
  if constexpr (!INTERLEAVED) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      r.c[g] = *reinterpret_cast<const v4f*>(cs + 8 * g + 4 * half);
      r.s[g] = *reinterpret_cast<const v4f*>(cs + 32 + 8 * g + 4 * half);
    }
  } else {
    typedef float v2f __attribute__((ext_vector_type(2)));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float* b = cs + 8 * j + 2 * half;
      const v2f c0 = *reinterpret_cast<const v2f*>(b), c1 = *reinterpret_cast<const v2f*>(b + 4);
      const v2f s0 = *reinterpret_cast<const v2f*>(b + 32), s1 = *reinterpret_cast<const v2f*>(b + 36);
      r.c[j] = v4f{c0[0], c0[1], c1[0], c1[1]};
      r.s[j] = v4f{s0[0], s0[1], s1[0], s1[1]};
    }
  }
  return r;
}

template <int STAGE>
__device__ __forceinline__ void epilogue_tile(const v16f (&acc)[4], int64_t t, int head, bool store,
                                              int half, const IndexerQArgs& p, const RopeCS& rcs) {
  const int64_t tc = t < p.M ? t : p.M - 1;
  const bool live = store && t < p.M;
  float v[4][16];
#pragma unroll
  for (int tn = 0; tn < 4; ++tn)
#pragma unroll
    for (int r = 0; r < 16; ++r) v[tn][r] = acc[tn][r];

  float* dbg_row = nullptr;
  if (STAGE >= 0) dbg_row = p.dbg + (tc * p.H + (head < p.H ? head : 0)) * HEAD_DIM;

  if (STAGE == 0) {
    if (live)
#pragma unroll
      for (int tn = 0; tn < 4; ++tn)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *reinterpret_cast<v4f*>(dbg_row + 32 * tn + 8 * g + 4 * half) =
              v4f{v[tn][4 * g], v[tn][4 * g + 1], v[tn][4 * g + 2], v[tn][4 * g + 3]};
    return;
  }

  if constexpr (!stage_interleaved(STAGE)) {
    // RoPE on dims 0..63: the pair (i, i + 32), i = 8 g + 4 half + s, lives in
    // v[0][4g+s] and v[1][4g+s].
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const v4f cc = rcs.c[g];
      const v4f ss = rcs.s[g];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const float x = v[0][4 * g + s], y = v[1][4 * g + s];
        v[0][4 * g + s] = x * cc[s] - y * ss[s];
        v[1][4 * g + s] = y * cc[s] + x * ss[s];
      }
    }
  } else {
    // interleaved: pair i = 16tn + 4g + 2half + k is (v[tn][4g+2k], v[tn][4g+2k+1]), tn < 2
#pragma unroll
    for (int tn = 0; tn < 2; ++tn)
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const float cc = rcs.c[2 * tn + (g >> 1)][2 * (g & 1) + k];
          const float ss = rcs.s[2 * tn + (g >> 1)][2 * (g & 1) + k];
          const float x = v[tn][4 * g + 2 * k], y = v[tn][4 * g + 2 * k + 1];
          v[tn][4 * g + 2 * k] = x * cc - y * ss;
          v[tn][4 * g + 2 * k + 1] = y * cc + x * ss;
        }
  }

  if (STAGE == 1) {
    if (live)
#pragma unroll
      for (int tn = 0; tn < 4; ++tn)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *reinterpret_cast<v4f*>(dbg_row + 32 * tn + 8 * g + 4 * half) =
              v4f{v[tn][4 * g], v[tn][4 * g + 1], v[tn][4 * g + 2], v[tn][4 * g + 3]};
    return;
  }

  // Unnormalised Hadamard butterflies inside the lane: dim bits 0, 1 (r bits
  // 0, 1), bits 3, 4 (r bits 2, 3) and bits 5, 6 (tn bits 0, 1).
#pragma unroll
  for (int rb = 1; rb < 16; rb <<= 1)
#pragma unroll
    for (int tn = 0; tn < 4; ++tn)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (!(r & rb)) {
          const float a = v[tn][r], b = v[tn][r | rb];
          v[tn][r] = a + b;
          v[tn][r | rb] = a - b;
        }
#pragma unroll
  for (int tb = 1; tb < 4; tb <<= 1)
#pragma unroll
    for (int tn = 0; tn < 4; ++tn)
      if (!(tn & tb))
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float a = v[tn][r], b = v[tn | tb][r];
          v[tn][r] = a + b;
          v[tn | tb][r] = a - b;
        }
  // Dim bit 2 lives in the lane half. Swapping the pair (r, r|4) (dims that
  // differ in bit 3) hands lanes < 32 both bit-2 halves of the bit3=0 dims
  // and lanes >= 32 those of the bit3=1 dims; after the butterfly the lane
  // half holds dim bit 3 and r bit 2 holds dim bit 2:
  //   d = 32 tn + 16 ((r >> 3) & 1) + 8 half + 4 ((r >> 2) & 1) + (r & 3).
#pragma unroll
  for (int tn = 0; tn < 4; ++tn)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (!(r & 4)) {
        float r0, r1;
        swap32(v[tn][r], v[tn][r | 4], r0, r1);
        v[tn][r] = r0 + r1;
        v[tn][r | 4] = r0 - r1;
      }

  if (STAGE == 2) {
    if (live)
#pragma unroll
      for (int tn = 0; tn < 4; ++tn)
#pragma unroll
        for (int r = 0; r < 16; r += 4)
          *reinterpret_cast<v4f*>(dbg_row + 32 * tn + 16 * ((r >> 3) & 1) + 8 * half + 4 * ((r >> 2) & 1)) =
              v4f{v[tn][r] * INV_SQRT_128, v[tn][r + 1] * INV_SQRT_128, v[tn][r + 2] * INV_SQRT_128,
                  v[tn][r + 3] * INV_SQRT_128};
    return;
  }

  // FP4 over 32-dim block b = tn: this lane holds 16 of its values, the
  // partner lane the other 16. z = u / sqrt(128) is formed explicitly (the
  // conversion's scale operand only carries a power of two).
#pragma unroll
  for (int tn = 0; tn < 4; ++tn)
#pragma unroll
    for (int r = 0; r < 16; ++r) v[tn][r] *= INV_SQRT_128;
  uint32_t sbytes = 0;
  uint32_t dw[4][2];
#pragma unroll
  for (int tn = 0; tn < 4; ++tn) {
    float m = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) m = fmaxf(m, fabsf(v[tn][r]));
    float m0, m1;
    swap32(m, m, m0, m1);
    const int e = stage_floor(STAGE) ? fp4_exponent_floor(fmaxf(m0, m1)) : fp4_exponent(fmaxf(m0, m1));
    sbytes |= (uint32_t)(e + 127) << (8 * tn);
    const float scale = __uint_as_float((uint32_t)(e + 127) << 23);  // 2^e: codes are RNE(z / 2^e)
    // dword (tn, r3) holds the packed codes of dims 32tn + 16r3 + 8half + [0, 8)
#pragma unroll
    for (int r3 = 0; r3 < 2; ++r3) {
      const float* x = &v[tn][8 * r3];
      uint32_t d = 0;
      d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, x[0], x[1], scale, 0);
      d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, x[2], x[3], scale, 1);
      d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, x[4], x[5], scale, 2);
      d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, x[6], x[7], scale, 3);
      dw[tn][r3] = d;
    }
  }
  // dword (tn, r3) sits at position 4tn + 2r3 + half of the 16-dword row.
  // Lanes < 32 collect positions 0..7 (blocks 0, 1), lanes >= 32 positions
  // 8..15 (blocks 2, 3); each then writes 32 contiguous bytes.
  uint32_t out[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int tn = i >> 1, r3 = i & 1;
    uint32_t r1;
    const uint32_t r0 = swap32_u(dw[tn][r3], dw[tn + 2][r3], r1);
    out[2 * i] = r0;
    out[2 * i + 1] = r1;
  }
  if (live) {
    uint8_t* dst = p.q_fp4 + (t * p.H + head) * (HEAD_DIM / 2) + 32 * half;
    *reinterpret_cast<v4u*>(dst) = v4u{out[0], out[1], out[2], out[3]};
    *reinterpret_cast<v4u*>(dst + 16) = v4u{out[4], out[5], out[6], out[7]};
    if (half == 0) *reinterpret_cast<uint32_t*>(p.q_scales + (t * p.H + head) * 4) = sbytes;
  }
}

// s_waitcnt immediates (gfx9 encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] << 14)
constexpr int WAITCNT_VM0 = 0 | (7 << 4) | (15 << 8) | (0 << 14);
constexpr int WAITCNT_LGKM0 = 15 | (7 << 4) | (0 << 8) | (3 << 14);
constexpr int BUFFER_FLAGS = 0x00020000;   // raw untyped buffer, 32-bit data format

__device__ __forceinline__ void block_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

typedef __attribute__((address_space(3))) void lds_void;
typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint64_t bytes) {
  const uint32_t n = bytes > 0xFFFFFFF0ull ? 0xFFFFFFF0u : (uint32_t)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)n, BUFFER_FLAGS);
}

}  // namespace
}  // namespace iqp
