// Weight preparation for gfx950: bf16 weights to E4M3 codes with one UE8M0
// scale per 128x128 tile, the format the fused indexer-Q kernels consume.
//
// The pages only say the Q projection is a block-scaled FP8 GEMM (tokenspeed
// PR "perf(deepseek-v4): accelerate indexer Q and packed FP8 quantization",
// Summary; TensorRT-LLM PR "Fuse DeepSeek-V4 Indexer Q projection with CuTe
// DSL", sequence diagram). The tile's scale follows the activation rule: amax
// over the tile floored at 1e-4, e = ceil(log2(amax / 448)) exactly, codes
// E4M3 round-to-nearest-even of w * 2^-e.
//
// Not on the per-token path (weights change only when they are loaded or
// updated), so the kernel is plain: one workgroup of 256 threads per tile,
// each thread holding 8 of the tile's 2048 16-byte chunks (16 threads cover a
// row's 256 bytes, so loads are coalesced); the tile amax is an integer
// maximum over bf16 magnitude codes (exact, order-free): a butterfly across
// the wave, then the four waves' values through LDS.
#include "fp8_block.h"
#include "iqp_internal.h"

namespace iqp {
namespace {

constexpr int WQ_THREADS = 256;
constexpr int WQ_TILE = 128;
constexpr int WQ_CHUNKS = WQ_TILE * WQ_TILE / 8 / WQ_THREADS;   // 16-byte chunks per thread: 8

__global__ __launch_bounds__(WQ_THREADS)
void fp8_quant_weight_kernel(const uint16_t* __restrict__ w, int64_t ldw, uint8_t* __restrict__ q, int64_t ldq,
                             uint8_t* __restrict__ scales, int64_t ld_scales) {
  __shared__ uint32_t wave_max[WQ_THREADS / 64];
  const int t = threadIdx.x;
  const int64_t r0 = (int64_t)blockIdx.y * WQ_TILE, c0 = (int64_t)blockIdx.x * WQ_TILE;
  fp8q::v4u x[WQ_CHUNKS];
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < WQ_CHUNKS; ++i) {
    const int c = t + WQ_THREADS * i;   // chunk c: row c / 16, elements 8 (c % 16) .. +7
    x[i] = *reinterpret_cast<const fp8q::v4u*>(w + (r0 + (c >> 4)) * ldw + c0 + 8 * (c & 15));
  }
#pragma unroll
  for (int i = 0; i < WQ_CHUNKS; ++i)
    m = max(m, max(max(fp8q::mag2(x[i][0]), fp8q::mag2(x[i][1])), max(fp8q::mag2(x[i][2]), fp8q::mag2(x[i][3]))));
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off));
  if ((t & 63) == 0) wave_max[t >> 6] = m;
  __syncthreads();
  m = max(max(wave_max[0], wave_max[1]), max(wave_max[2], wave_max[3]));
  const int e = fp8q::block_exponent(m);
  const float mul = __uint_as_float((uint32_t)(127 - e) << 23);  // 2^-e, a normal float
#pragma unroll
  for (int i = 0; i < WQ_CHUNKS; ++i) {
    const int c = t + WQ_THREADS * i;
    const uint2 codes = make_uint2(fp8q::cvt4(x[i][0], x[i][1], mul), fp8q::cvt4(x[i][2], x[i][3], mul));
    *reinterpret_cast<uint2*>(q + (r0 + (c >> 4)) * ldq + c0 + 8 * (c & 15)) = codes;
  }
  if (t == 0) scales[(int64_t)blockIdx.y * ld_scales + blockIdx.x] = (uint8_t)(e + 127);
}

}  // namespace

hipError_t launch_fp8_quant_weight(const uint16_t* w, int64_t N, int64_t K, int64_t ldw, uint8_t* q, int64_t ldq,
                                   uint8_t* scales, int64_t ld_scales, hipStream_t stream) {
  const int64_t tn = N / WQ_TILE, tk = K / WQ_TILE;
  if (tn > 65535 || tk > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(fp8_quant_weight_kernel, dim3((unsigned)tk, (unsigned)tn), dim3(WQ_THREADS), 0, stream,
                     w, ldw, q, ldq, scales, ld_scales);
  return hipGetLastError();
}

}  // namespace iqp
