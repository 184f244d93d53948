// RoPE cos/sin table: cos_sin[p, i] = cos(p * theta^(-2i/rope_dim)) and
// cos_sin[p, rope_dim/2 + i] = sin(...), evaluated in float64 and rounded to
// float32 once (tokenspeed PR "perf(deepseek-v4): accelerate indexer Q and
// packed FP8 quantization", Summary: RoPE on the indexer Q). Built once per
// model, not per call; float64 keeps the angle exact enough for positions up
// to 2^17 and beyond, which float32 angles would not.
#include "iqp_internal.h"

namespace iqp {
namespace {

__global__ void rope_table_kernel(double theta, int64_t max_pos, int32_t rope_dim, float* __restrict__ out) {
  const int half = rope_dim / 2;
  const int64_t n = max_pos * half;
  for (int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; k < n; k += (int64_t)gridDim.x * blockDim.x) {
    const int64_t p = k / half;
    const int i = (int)(k - p * half);
    const double inv_freq = pow(theta, -2.0 * (double)i / (double)rope_dim);
    const double ang = (double)p * inv_freq;
    double s, c;
    sincos(ang, &s, &c);
    out[p * rope_dim + i] = (float)c;
    out[p * rope_dim + half + i] = (float)s;
  }
}

// Lane-ordered copy of a [max_pos, 64] table for the split-role fused kernel.
// There a lane holds one token (lane % 32 of a 32-token sub-tile) and one half
// h = lane / 32 of its RoPE pairs, and fetches that token's row as eight
// 16-byte loads: load L reads columns 32 (L % 2) + 8 (L / 2) + 4 h .. + 3
// (cosines for even L, sines for odd). From the table itself each such load
// gathers 32 rows, 32 cache lines for 1 KiB. The copy puts load L of position
// p, half h at float 2048 (p / 32) + 256 L + 4 (2 (p % 32) + h): the 32
// consecutive positions of a prefill sub-tile then read one 1 KiB segment per
// load (8 lines; 16 when they straddle two 32-position blocks). Positions past
// max_pos in the last block hold zeros.
__global__ void rope_table_lanes_kernel(const float* __restrict__ cs, int64_t max_pos, float* __restrict__ out) {
  typedef float v4f __attribute__((ext_vector_type(4)));
  const int64_t n = (max_pos + 31) / 32 * 512;   // 16-byte pieces
  for (int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; k < n; k += (int64_t)gridDim.x * blockDim.x) {
    const int64_t b = k >> 9;
    const int L = (int)(k >> 6) & 7, slot = (int)k & 63;
    const int64_t p = 32 * b + (slot >> 1);
    v4f v = v4f{0.f, 0.f, 0.f, 0.f};
    if (p < max_pos) v = *reinterpret_cast<const v4f*>(cs + p * 64 + 32 * (L & 1) + 8 * (L >> 1) + 4 * (slot & 1));
    *reinterpret_cast<v4f*>(out + 4 * k) = v;
  }
}

}  // namespace

hipError_t launch_rope_table_lanes(const float* cos_sin, int64_t max_pos, float* out, hipStream_t stream) {
  const int64_t n = (max_pos + 31) / 32 * 512;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(rope_table_lanes_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, cos_sin, max_pos, out);
  return hipGetLastError();
}

hipError_t launch_rope_table(double theta, int64_t max_pos, int32_t rope_dim, float* cos_sin,
                             hipStream_t stream) {
  const int64_t n = max_pos * (rope_dim / 2);
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     theta, max_pos, rope_dim, cos_sin);
  return hipGetLastError();
}

}  // namespace iqp
