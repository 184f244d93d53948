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
// slower. Workgroups of 8 waves instead of 4 took it to 17.8 us (and
// [32768, 7168] from 115.7 to 112.1 us) but slowed the small cached
// quantization of [4632, 1536] (5.9 against 5.6 us), so the launcher picks
// the shape with the store policy.
#include "fp8_block.h"
#include "iqp_internal.h"

namespace iqp {
namespace {

// waves per workgroup (two scale words each): outputs streamed past the
// caches, and outputs kept in them
constexpr int QWAVES_STREAM = 8;
constexpr int QWAVES_CACHED = 4;

// Words 2 i and 2 i + 1 (row-major over [M, nw]) of the whole tensor go to
// wave i (the arithmetic: fp8q::quant_word_pair).
template <bool NT_STORE, int QWAVES>
__global__ __launch_bounds__(QWAVES * 64)
void fp8_quant_1x128_kernel(const uint16_t* __restrict__ x, int64_t ldx,
                            uint8_t* __restrict__ q, int64_t ldq,
                            int32_t* __restrict__ scales, int64_t sm, int64_t sw,
                            int32_t nw, int32_t nkb, int64_t words) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t first = 2 * ((int64_t)blockIdx.x * QWAVES + wave);
  if (first >= words) return;   // uniform across the wave
  fp8q::quant_word_pair<NT_STORE>(x, ldx, q, ldq, scales, sm, sw, nw, nkb, words, first, lane);
}

}  // namespace

hipError_t launch_fp8_quant(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                            uint8_t* q, int64_t ldq, int32_t* scales,
                            int64_t s_stride_m, int64_t s_stride_w, hipStream_t stream) {
  const int32_t nkb = (int32_t)(K / 128);
  const int32_t nw = (nkb + 3) / 4;
  const int64_t words = M * nw;
  // Up to 16 MiB of codes are stored through the caches, so that the
  // projection that reads them next finds them there; larger outputs are
  // streamed past them. Measured on MI355X: the 4632-token chain (7 MB of
  // codes) steps in 69.1 us against 71.9 us with streamed codes (the fused
  // kernel alone: 62.4 us), while streaming keeps the standalone [4632,
  // 7168] quantization at 18.6 us against 19.0 us cached.
  const bool nt = M * ldq > ((int64_t)16 << 20);
  const int qwaves = nt ? QWAVES_STREAM : QWAVES_CACHED;
  const int64_t per_block = (int64_t)qwaves * 2;
  const int64_t blocks = (words + per_block - 1) / per_block;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  auto kern = nt ? fp8_quant_1x128_kernel<true, QWAVES_STREAM> : fp8_quant_1x128_kernel<false, QWAVES_CACHED>;
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(qwaves * 64), 0, stream,
                     x, ldx, q, ldq, scales, s_stride_m, s_stride_w, nw, nkb, words);
  return hipGetLastError();
}

}  // namespace iqp
