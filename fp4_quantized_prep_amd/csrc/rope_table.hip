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

}  // namespace

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
