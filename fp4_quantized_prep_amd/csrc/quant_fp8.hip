// Packed-UE8M0 FP8 1x128 activation quantizer for gfx950.
//
// tokenspeed PR "perf(deepseek-v4): accelerate indexer Q and packed FP8
// quantization", Summary (online FP8 activation quantization whose UE8M0 scale
// exponents are packed four to an int32) and Risk and fallback (BF16 input with
// K divisible by 128; the tiny-scale floor is kept).
//
// The work is HBM-bound (2 bytes in, 1 + 1/128 bytes out per element), so the
// kernel is organised around wide, coalesced memory operations:
//   * one wave64 owns two packed scale words = 8 blocks = 1024 bf16 (2 KiB of
//     input), one word per load: in load k lane l reads 16 B (8 bf16) of word
//     k at byte 16 l, so each load instruction covers 1 KiB contiguous, every
//     cache line whole, and 16 lanes hold one 128-element block;
//   * the block amax is reduced with four DPP max steps inside each row of
//     16 lanes, on the bf16 magnitude bits as integers (order-free and
//     exact), with no LDS;
//   * the scale exponent comes from the amax bits with integer arithmetic;
//   * v_cvt_pk_fp8_f32 rounds x * 2^-e to E4M3 (OCP "fn", round to nearest
//     even, subnormals kept); lanes store 8 B each, 512 B per word
//     contiguous;
//   * the four block bytes of each word are gathered with readlane and stored
//     as one dword;
//   * loads are non-temporal (the input is read once); so are the stores of
//     outputs too large to stay in the caches (see the launcher).
// Measured on MI355X at [4632, 7168]: 18.4 us, against 18.7 us when each
// lane held 16 consecutive values (two 16-byte loads 32 bytes apart: every
// line fetched by two instructions) and 19.4 us for a copy with no
// arithmetic in that older pattern; four words per wave instead of two ran
// slower.
#include "fp8_block.h"
#include "iqp_internal.h"

namespace iqp {
namespace {

constexpr int QWAVES = 4;  // waves per workgroup, two scale words each
using namespace fp8q;
typedef unsigned v2u __attribute__((ext_vector_type(2)));

// maximum over each row of 16 lanes (a block)
__device__ __forceinline__ uint32_t lanes16_max(uint32_t v) {
  v = lanes8_max(v);
  return max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, DPP_ROW_MIRROR, 0xF, 0xF, false));
}

// Words 2 i and 2 i + 1 (row-major over [M, nw]) of the whole tensor go to
// wave i.
template <bool NT_STORE>
__global__ __launch_bounds__(QWAVES * 64)
void fp8_quant_1x128_kernel(const uint16_t* __restrict__ x, int64_t ldx,
                            uint8_t* __restrict__ q, int64_t ldq,
                            int32_t* __restrict__ scales, int64_t sm, int64_t sw,
                            int32_t nw, int32_t nkb, int64_t words) {
  const int lane = threadIdx.x & 63;
  const int blk = lane >> 4;  // block of this lane within a word
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t first = 2 * ((int64_t)blockIdx.x * QWAVES + wave);
  if (first >= words) return;   // uniform across the wave

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

}  // namespace

hipError_t launch_fp8_quant(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                            uint8_t* q, int64_t ldq, int32_t* scales,
                            int64_t s_stride_m, int64_t s_stride_w, hipStream_t stream) {
  const int32_t nkb = (int32_t)(K / 128);
  const int32_t nw = (nkb + 3) / 4;
  const int64_t words = M * nw;
  const int64_t per_block = (int64_t)QWAVES * 2;
  const int64_t blocks = (words + per_block - 1) / per_block;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  // Up to 16 MiB of codes are stored through the caches, so that the
  // projection that reads them next finds them there; larger outputs are
  // streamed past them. Measured on MI355X: the 4632-token chain (7 MB of
  // codes) steps in 69.1 us against 71.9 us with streamed codes (the fused
  // kernel alone: 62.4 us), while streaming keeps the standalone [4632,
  // 7168] quantization at 18.6 us against 19.0 us cached.
  const bool nt = M * ldq > ((int64_t)16 << 20);
  hipLaunchKernelGGL(nt ? fp8_quant_1x128_kernel<true> : fp8_quant_1x128_kernel<false>, dim3((unsigned)blocks),
                     dim3(QWAVES * 64), 0, stream,
                     x, ldx, q, ldq, scales, s_stride_m, s_stride_w, nw, nkb, words);
  return hipGetLastError();
}

}  // namespace iqp
