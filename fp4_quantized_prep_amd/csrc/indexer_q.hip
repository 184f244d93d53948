// Fused indexer-Q preparation for gfx950: block-scaled FP8 Q projection on the
// matrix cores, then RoPE, a 128-point Hadamard rotation and FP4 e2m1
// quantization with UE8M0 block scales, all on the accumulators in registers.
//
// TensorRT-LLM PR "Fuse DeepSeek-V4 Indexer Q projection with CuTe DSL",
// sequence diagram (one GEMM whose epilogue applies RoPE and writes packed FP4
// Q and scales) and Description / Paths compared (it replaces the Q GEMM, a
// RoPE kernel, an FP4 quantization kernel and scale copies); tokenspeed PR
// "perf(deepseek-v4): accelerate indexer Q and packed FP8 quantization",
// Summary (RoPE, the Hadamard transform and FP4 quantization of Q).
//
// Design (MI355X-first, not the pages' SM100 design):
//   * The product is computed transposed, Q^T = W A^T, on
//     v_mfma_scale_f32_32x32x64_f8f6f4: MFMA rows are weight rows (head dims),
//     MFMA columns are tokens. The 32x32 accumulator layout then gives lane l
//     the token l%32 and 16 head dims per 32-dim tile, so one lane holds 64 of
//     its token's 128 dims (all dims whose bit 2 equals l/32) and its partner
//     lane l^32 holds the rest. RoPE pairs (i, i+32), six of the seven
//     Hadamard butterfly stages and the FP4 block maxima stay inside a lane;
//     the seventh stage and the block maxima use v_permlane32_swap.
//   * The UE8M0 block scales are applied by the MFMA itself: scale byte 127
//     means 1.0, every lane passes the scale of its own row / column, and one
//     scale covers a whole 128-deep K block.
//   * A workgroup owns one head (128 weight rows) and NWAVES*MT*32 tokens. The
//     weight tile of each 128-deep K block is staged through LDS (XOR-swizzled
//     16-byte chunks, double buffered) and shared by all waves; each wave loads
//     its own tokens' activation bytes straight into MFMA operand registers.
//   * Workgroups are mapped so that one XCD works on H/8 heads: their weights
//     (1.5 MiB at K = 1536) stay in that XCD's L2 while tokens stream.
//   * Q never leaves registers; each lane writes 32 contiguous bytes of packed
//     codes per token and head, and one lane per pair writes the 4 scale bytes.
#include "iqp_internal.h"

namespace iqp {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int HEAD_DIM = 128;
constexpr int KB = 128;              // K block (one activation / weight scale)
constexpr int WTILE = HEAD_DIM * KB; // bytes of one weight tile in LDS
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

// Global -> registers: this thread's 16-byte chunks of the 128x128 weight tile
// of K block j (chunk q covers row q/8, bytes 16 (q%8) of the block).
template <int CHUNKS, int NT>
__device__ __forceinline__ void load_w_tile(v4u (&wst)[CHUNKS], const uint8_t* wbase, int64_t ldw,
                                            int j, int tid) {
#pragma unroll
  for (int i = 0; i < CHUNKS; ++i) {
    const int q = tid + i * NT;
    const int row = q >> 3, c = q & 7;
    wst[i] = *reinterpret_cast<const v4u*>(wbase + (int64_t)row * ldw + (int64_t)KB * j + 16 * c);
  }
}

// Registers -> LDS, with the 16-byte chunks of row r XOR-swizzled by r % 8 so
// that eight consecutive rows read at one column offset hit distinct banks.
template <int CHUNKS, int NT>
__device__ __forceinline__ void store_w_tile(const v4u (&wst)[CHUNKS], uint8_t* tile, int tid) {
#pragma unroll
  for (int i = 0; i < CHUNKS; ++i) {
    const int q = tid + i * NT;
    const int row = q >> 3, c = q & 7;
    *reinterpret_cast<v4u*>(tile + row * KB + 16 * (c ^ (row & 7))) = wst[i];
  }
}

// Activation operands of K block j: for each 32-token column tile, the lane's
// 32 bytes of each 64-deep half (bytes 64 kh + 32 (lane / 32) of the block), and
// the token's UE8M0 scale byte of the block.
template <int MT>
__device__ __forceinline__ void load_a_frags(v8i (&f)[MT][2], int (&sc)[MT], const uint8_t* const (&arow)[MT],
                                             const uint8_t* const (&srow)[MT], int64_t as_sw, int j) {
#pragma unroll
  for (int tm = 0; tm < MT; ++tm) {
    const uint8_t* src = arow[tm] + (int64_t)KB * j;
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      const v4u lo = *reinterpret_cast<const v4u*>(src + 64 * kh);
      const v4u hi = *reinterpret_cast<const v4u*>(src + 64 * kh + 16);
      f[tm][kh] = make_v8i(lo, hi);
    }
    sc[tm] = srow[tm][4 * (int64_t)(j >> 2) * as_sw + (j & 3)];
  }
}

template <int NWAVES, int MT, int STAGE>
__global__ __launch_bounds__(NWAVES * 64)
void indexer_q_kernel(IndexerQArgs p) {
  constexpr int NT = NWAVES * 64;
  constexpr int TOK_WAVE = 32 * MT;
  constexpr int TOK_WG = NWAVES * TOK_WAVE;
  constexpr int CHUNKS = WTILE / 16 / NT;  // 16-byte weight chunks per thread per K block
  static_assert(WTILE / 16 % NT == 0, "weight tile must split evenly");

  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * WTILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int half = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // ---- workgroup -> (head, token tile); XCD-aware when H % 8 == 0
  const int bid = blockIdx.x;
  int head, mtile;
  if ((p.H & 7) == 0) {
    const int hpx = p.H >> 3;
    const int s = bid >> 3;
    head = (bid & 7) * hpx + s % hpx;
    mtile = s / hpx;
  } else {
    head = bid % p.H;
    mtile = bid / p.H;
  }
  const int64_t mbase = (int64_t)mtile * TOK_WG + (int64_t)wave * TOK_WAVE;
  const int nkb = p.nkb;

  // ---- per-lane token rows (clamped: rows past M are computed, never stored)
  const uint8_t* arow[MT];
  const uint8_t* srow[MT];  // scale words of the token, viewed as bytes
#pragma unroll
  for (int tm = 0; tm < MT; ++tm) {
    int64_t t = mbase + 32 * tm + (lane & 31);
    t = t < p.M ? t : p.M - 1;
    arow[tm] = p.a + t * p.lda + 32 * half;
    srow[tm] = p.a_scale_bytes + 4 * t * p.as_sm;
  }
  const uint8_t* wbase = p.w + (int64_t)head * HEAD_DIM * p.ldw;
  const uint8_t* wsc = p.w_scales + (int64_t)head * nkb;

  v4u wst[CHUNKS];
  v8i afrag[MT][2], anext[MT][2];
  int asc[MT], anext_sc[MT];

  v16f acc[MT][4];
#pragma unroll
  for (int tm = 0; tm < MT; ++tm)
#pragma unroll
    for (int tn = 0; tn < 4; ++tn)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[tm][tn][r] = 0.f;

  load_w_tile<CHUNKS, NT>(wst, wbase, p.ldw, 0, tid);
  load_a_frags<MT>(afrag, asc, arow, srow, p.as_sw, 0);
  store_w_tile<CHUNKS, NT>(wst, lds, tid);
  __syncthreads();

  for (int j = 0; j < nkb; ++j) {
    const int buf = j & 1;
    const bool more = j + 1 < nkb;
    if (more) {
      load_w_tile<CHUNKS, NT>(wst, wbase, p.ldw, j + 1, tid);
      load_a_frags<MT>(anext, anext_sc, arow, srow, p.as_sw, j + 1);
    }
    const int wscale = wsc[j];
    const uint8_t* tile = lds + buf * WTILE;
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
#pragma unroll
      for (int tn = 0; tn < 4; ++tn) {
        const int row = 32 * tn + (lane & 31);
        const int c0 = 4 * kh + 2 * half;
        const v4u lo = *reinterpret_cast<const v4u*>(tile + row * KB + 16 * (c0 ^ (row & 7)));
        const v4u hi = *reinterpret_cast<const v4u*>(tile + row * KB + 16 * ((c0 + 1) ^ (row & 7)));
        const v8i wf = make_v8i(lo, hi);
#pragma unroll
        for (int tm = 0; tm < MT; ++tm)
          acc[tm][tn] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              wf, afrag[tm][kh], acc[tm][tn], 0, 0, 0, wscale, 0, asc[tm]);
      }
    }
    if (more) store_w_tile<CHUNKS, NT>(wst, lds + (buf ^ 1) * WTILE, tid);
    __syncthreads();
    if (more) {
#pragma unroll
      for (int tm = 0; tm < MT; ++tm) {
        afrag[tm][0] = anext[tm][0];
        afrag[tm][1] = anext[tm][1];
        asc[tm] = anext_sc[tm];
      }
    }
  }

  // ---- epilogue, one 32-token column tile at a time.
  // Before the cross-lane stage, acc[tm][tn][r] holds head dim
  //   d = 32 tn + 8 (r >> 2) + 4 half + (r & 3)   of token mbase + 32 tm + lane%32.
#pragma unroll
  for (int tm = 0; tm < MT; ++tm) {
    const int64_t t = mbase + 32 * tm + (lane & 31);
    const bool live = t < p.M;
    const int64_t tc = live ? t : p.M - 1;
    float v[4][16];
#pragma unroll
    for (int tn = 0; tn < 4; ++tn)
#pragma unroll
      for (int r = 0; r < 16; ++r) v[tn][r] = acc[tm][tn][r];

    float* dbg_row = nullptr;
    if (STAGE >= 0) dbg_row = p.dbg + (tc * p.H + head) * HEAD_DIM;

    if (STAGE == 0) {
      if (live)
#pragma unroll
        for (int tn = 0; tn < 4; ++tn)
#pragma unroll
          for (int g = 0; g < 4; ++g)
            *reinterpret_cast<v4f*>(dbg_row + 32 * tn + 8 * g + 4 * half) =
                v4f{v[tn][4 * g], v[tn][4 * g + 1], v[tn][4 * g + 2], v[tn][4 * g + 3]};
      continue;
    }

    // RoPE on dims 0..63: pair (i, i + 32) with i = 8 g + 4 half + s lives in
    // v[0][4g+s] and v[1][4g+s].
    int64_t pos = p.positions[tc];
    pos = pos < 0 ? 0 : (pos >= p.max_pos ? p.max_pos - 1 : pos);
    const float* cs = p.cos_sin + pos * 64;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const v4f cc = *reinterpret_cast<const v4f*>(cs + 8 * g + 4 * half);
      const v4f ss = *reinterpret_cast<const v4f*>(cs + 32 + 8 * g + 4 * half);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const float x = v[0][4 * g + s], y = v[1][4 * g + s];
        v[0][4 * g + s] = x * cc[s] - y * ss[s];
        v[1][4 * g + s] = y * cc[s] + x * ss[s];
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
      continue;
    }

    // Hadamard butterflies inside the lane: dim bits 0, 1 (r bits 0, 1),
    // bits 3, 4 (r bits 2, 3) and bits 5, 6 (tn bits 0, 1).
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
          v[tn][r] = (r0 + r1) * INV_SQRT_128;
          v[tn][r | 4] = (r0 - r1) * INV_SQRT_128;
        }

    if (STAGE == 2) {
      if (live)
#pragma unroll
        for (int tn = 0; tn < 4; ++tn)
#pragma unroll
          for (int r = 0; r < 16; r += 4)
            *reinterpret_cast<v4f*>(dbg_row + 32 * tn + 16 * ((r >> 3) & 1) + 8 * half + 4 * ((r >> 2) & 1)) =
                v4f{v[tn][r], v[tn][r + 1], v[tn][r + 2], v[tn][r + 3]};
      continue;
    }

    // FP4: 32-dim block b = tn; this lane holds 16 of its values, the partner
    // lane the other 16.
    uint32_t sbytes = 0;
    uint32_t dw[4][2];
#pragma unroll
    for (int tn = 0; tn < 4; ++tn) {
      float m = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) m = fmaxf(m, fabsf(v[tn][r]));
      float m0, m1;
      swap32(m, m, m0, m1);
      const int e = fp4_exponent(fmaxf(m0, m1));
      sbytes |= (uint32_t)(e + 127) << (8 * tn);
      const float scale = __uint_as_float((uint32_t)(e + 127) << 23);  // 2^e
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
    // 8..15 (blocks 2, 3), then each writes 32 contiguous bytes.
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
      if (half == 0)
        *reinterpret_cast<uint32_t*>(p.q_scales + (t * p.H + head) * 4) = sbytes;
    }
  }
}

template <int NWAVES, int MT>
hipError_t launch_cfg(const IndexerQArgs& a, int stage, hipStream_t stream) {
  constexpr int TOK_WG = NWAVES * 32 * MT;
  const int64_t n_mt = (a.M + TOK_WG - 1) / TOK_WG;
  const int64_t blocks = n_mt * a.H;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  const dim3 grid((unsigned)blocks), block(NWAVES * 64);
  switch (stage) {
    case -1: hipLaunchKernelGGL((indexer_q_kernel<NWAVES, MT, -1>), grid, block, 0, stream, a); break;
    case 0: hipLaunchKernelGGL((indexer_q_kernel<NWAVES, MT, 0>), grid, block, 0, stream, a); break;
    case 1: hipLaunchKernelGGL((indexer_q_kernel<NWAVES, MT, 1>), grid, block, 0, stream, a); break;
    case 2: hipLaunchKernelGGL((indexer_q_kernel<NWAVES, MT, 2>), grid, block, 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_indexer_q(const IndexerQArgs& a, int stage, hipStream_t stream) {
  // token tile per workgroup: 4 waves x 2 column tiles x 32 tokens = 256
  return launch_cfg<4, 2>(a, stage, stream);
}

}  // namespace iqp
