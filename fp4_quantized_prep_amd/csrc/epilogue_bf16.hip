// Standalone indexer-Q epilogue for gfx950: bf16 Q in, RoPE on each head's
// rope slice, Hadamard-128, FP4 e2m1 with UE8M0 block scales out.
//
// This is the second half of the unfused chain the pages compare against:
// TensorRT-LLM PR "Fuse DeepSeek-V4 Indexer Q projection with CuTe DSL",
// Description / Paths compared (the Q GEMM writes a bf16 Q, then a RoPE
// kernel and an FP4 quantization kernel run on it), and tokenspeed PR
// "perf(deepseek-v4): accelerate indexer Q and packed FP8 quantization",
// Summary (the MLA RoPE kernel, the Hadamard transform and the fused FP4 cat
// kernel of the Q preparation). Here the three run as one launch.
//
// The work is HBM-bound: 256 bytes of bf16 in and 68 bytes out per
// (token, head), plus a table row per token that stays in cache. Layout:
//   * a workgroup takes one token and up to 64 of its heads (grid: tokens x
//     head chunks), so token and head need no division;
//   * four lanes (a quad) own one (token, head) vector of 128 dims; lane j
//     holds dims d = 8 j + t + 32 u (t < 8, u < 4), loaded as four 16-byte
//     loads (one per u);
//   * the RoPE pairs (i, i + 32), i < 32, are (u = 0, u = 1) of the same t in
//     the same lane;
//   * Hadamard butterflies over dim bits 0-2 (t) and 5-6 (u) run in the lane,
//     those over bits 3 and 4 (lane bits 0 and 1) exchange with the quad
//     neighbours by DPP;
//   * FP4 block b = u (dims 32u .. 32u+31) is 8 values in each lane of the
//     quad: an in-lane maximum, then two DPP maxima;
//   * the packed codes (one dword per lane and block) are transposed within
//     the quad through LDS so that lane j stores block j's 16 bytes: a wave
//     writes 1 KiB of whole lines per store; lane 0 stores the scale bytes.
// Measured on MI355X at 4632 tokens x 64 heads (four rotating buffer sets):
// 18.5 us; a copy of the kernel with the arithmetic removed (same loads and
// stores) takes 17.4 us. Storing one dword per block from each lane, or
// non-temporal loads, cost 20.0-21.6 us.
#include "iq_common.h"

namespace iqp {
namespace {

constexpr int EPI_THREADS = 256;
constexpr int DPP_QUAD_XOR1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int DPP_QUAD_XOR2 = 0x4E;  // quad_perm [2,3,0,1]

template <int CTRL>
__device__ __forceinline__ float quad_xchg(float v) {
  // quad permutes read a valid lane everywhere, so no "old" value is needed
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}

// INTERLEAVED: RoPE pairs (2i, 2i + 1) instead of (i, i + 32); FLOOR: FP4
// scales by the OCP MX rule (codes saturate at 6) instead of the ceil rule.
template <bool INTERLEAVED, bool FLOOR>
__global__ __launch_bounds__(EPI_THREADS)
void indexer_q_epilogue_kernel(const uint16_t* __restrict__ q, int64_t ldq, int32_t H,
                               const int64_t* __restrict__ positions,
                               const float* __restrict__ cos_sin, int64_t max_pos,
                               uint8_t* __restrict__ q_fp4, uint8_t* __restrict__ q_scales) {
  // workgroup (m, c): token m, heads 64c .. 64c + 63, one quad per head
  const int j = threadIdx.x & 3;
  const int64_t m = blockIdx.x;
  const int hh = (int)blockIdx.y * (EPI_THREADS / 4) + (int)(threadIdx.x >> 2);
  const bool live = hh < H;
  const int h = live ? hh : H - 1;   // past the last head: read the last head, store nothing
  const int64_t v = m * H + h;       // (token, head) vector index of the outputs

  const uint16_t* src = q + m * ldq + (int64_t)h * HEAD_DIM + 8 * j;
  v4u x[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) x[u] = *reinterpret_cast<const v4u*>(src + 32 * u);

  int64_t pos = positions[m];
  pos = pos < 0 ? 0 : (pos >= max_pos ? max_pos - 1 : pos);
  // half-split: pairs i = 8j + t (t < 8); interleaved: pairs i = 4j + k (dims
  // (2k, 2k + 1) of u = 0) and 16 + 4j + k (u = 1), k < 4
  const float* cs = cos_sin + pos * 64 + (INTERLEAVED ? 4 * j : 8 * j);
  const v4f c0 = *reinterpret_cast<const v4f*>(cs), c1 = *reinterpret_cast<const v4f*>(cs + (INTERLEAVED ? 16 : 4));
  const v4f s0 = *reinterpret_cast<const v4f*>(cs + 32), s1 = *reinterpret_cast<const v4f*>(cs + (INTERLEAVED ? 48 : 36));

  // bf16 -> float32: element 2k is the low half of dword k
  float f[4][8];
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      f[u][2 * k] = __uint_as_float(x[u][k] << 16);
      f[u][2 * k + 1] = __uint_as_float(x[u][k] & 0xFFFF0000u);
    }

  if (!INTERLEAVED) {
    // RoPE: pair i = 8j + t is (f[0][t], f[1][t])
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const float c = t < 4 ? c0[t] : c1[t - 4];
      const float s = t < 4 ? s0[t] : s1[t - 4];
      const float a = f[0][t], b = f[1][t];
      f[0][t] = a * c - b * s;
      f[1][t] = b * c + a * s;
    }
  } else {
    // RoPE: pair 16u + 4j + k is (f[u][2k], f[u][2k + 1]), u < 2
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float c = u ? c1[k] : c0[k];
        const float s = u ? s1[k] : s0[k];
        const float a = f[u][2 * k], b = f[u][2 * k + 1];
        f[u][2 * k] = a * c - b * s;
        f[u][2 * k + 1] = b * c + a * s;
      }
  }

  // Unnormalised Hadamard butterflies: dim bits 0-2 (t) and 5-6 (u) in the lane
#pragma unroll
  for (int tb = 1; tb < 8; tb <<= 1)
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int t = 0; t < 8; ++t)
        if (!(t & tb)) {
          const float a = f[u][t], b = f[u][t | tb];
          f[u][t] = a + b;
          f[u][t | tb] = a - b;
        }
#pragma unroll
  for (int ub = 1; ub < 4; ub <<= 1)
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (!(u & ub))
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const float a = f[u][t], b = f[u | ub][t];
          f[u][t] = a + b;
          f[u | ub][t] = a - b;
        }
  // dim bit 3 = lane bit 0, dim bit 4 = lane bit 1: the lane with the bit
  // clear keeps mine + partner, the other partner - mine
  {
    const float sg = (j & 1) ? -1.f : 1.f;
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int t = 0; t < 8; ++t) f[u][t] = quad_xchg<DPP_QUAD_XOR1>(f[u][t]) + sg * f[u][t];
  }
  {
    const float sg = (j & 2) ? -1.f : 1.f;
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int t = 0; t < 8; ++t) f[u][t] = quad_xchg<DPP_QUAD_XOR2>(f[u][t]) + sg * f[u][t];
  }

  // FP4: z = butterfly sum / sqrt(128), formed explicitly (the conversion's
  // scale operand carries only a power of two)
  uint32_t sbytes = 0;
  uint32_t dw[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    float mx = 0.f;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      f[u][t] *= INV_SQRT_128;
      mx = fmaxf(mx, fabsf(f[u][t]));
    }
    mx = fmaxf(mx, quad_xchg<DPP_QUAD_XOR1>(mx));
    mx = fmaxf(mx, quad_xchg<DPP_QUAD_XOR2>(mx));
    const int e = FLOOR ? fp4_exponent_floor(mx) : fp4_exponent(mx);
    sbytes |= (uint32_t)(e + 127) << (8 * u);
    const float scale = __uint_as_float((uint32_t)(e + 127) << 23);  // 2^e: codes are RNE(z / 2^e)
    uint32_t d = 0;
    d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, f[u][0], f[u][1], scale, 0);
    d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, f[u][2], f[u][3], scale, 1);
    d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, f[u][4], f[u][5], scale, 2);
    d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, f[u][6], f[u][7], scale, 3);
    dw[u] = d;
  }
  // The codes of dims 32u + 8j .. 32u + 8j + 7 belong at bytes 16u + 4j .. +3
  // of the vector's 64-byte row. Each quad's row goes through 16 dwords of LDS
  // (rows 20 dwords apart, so the 64 lanes of a write hit 64 distinct banks);
  // lane j reads back dwords 4j .. 4j + 3. Only the lanes of one wave touch a
  // row, so a wave-level barrier orders the writes before the reads.
  __shared__ __attribute__((aligned(16))) uint32_t rows[EPI_THREADS / 64][16 * 20];
  uint32_t* row = rows[threadIdx.x >> 6] + 20 * ((threadIdx.x >> 2) & 15);
#pragma unroll
  for (int u = 0; u < 4; ++u) row[4 * u + j] = dw[u];
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const v4u codes = *reinterpret_cast<const v4u*>(row + 4 * j);
  if (live) {
    __builtin_nontemporal_store(codes, reinterpret_cast<v4u*>(q_fp4 + v * (HEAD_DIM / 2) + 16 * j));
    if (j == 0) __builtin_nontemporal_store(sbytes, reinterpret_cast<uint32_t*>(q_scales + v * 4));
  }
}

}  // namespace

hipError_t launch_indexer_q_epilogue(const uint16_t* q, int64_t ldq, int64_t M, int32_t H,
                                     const int64_t* positions, const float* cos_sin, int64_t max_pos,
                                     uint8_t* q_fp4, uint8_t* q_scales, bool interleaved, bool floor_rule,
                                     hipStream_t stream) {
  const int64_t chunks = ((int64_t)H + EPI_THREADS / 4 - 1) / (EPI_THREADS / 4);
  if (M > 0x7FFFFFFF || chunks > 65535) return hipErrorInvalidValue;
  auto kern = interleaved ? (floor_rule ? indexer_q_epilogue_kernel<true, true> : indexer_q_epilogue_kernel<true, false>)
                          : (floor_rule ? indexer_q_epilogue_kernel<false, true> : indexer_q_epilogue_kernel<false, false>);
  hipLaunchKernelGGL(kern, dim3((unsigned)M, (unsigned)chunks), dim3(EPI_THREADS), 0,
                     stream, q, ldq, H, positions, cos_sin, max_pos, q_fp4, q_scales);
  return hipGetLastError();
}

}  // namespace iqp
