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

// ---------------------------------------------------------------------------
// Epilogue for one 32-token column tile of one head: acc[tn][r] holds head dim
//   d = 32 tn + 8 (r >> 2) + 4 half + (r & 3)
// of token t (lane % 32 of the tile). RoPE, the seven Hadamard stages and the
// FP4 quantization all run on these registers.
template <int STAGE>
__device__ __forceinline__ void epilogue_tile(const v16f (&acc)[4], int64_t t, int head, bool store,
                                              int half, const IndexerQArgs& p) {
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

  // RoPE on dims 0..63: the pair (i, i + 32), i = 8 g + 4 half + s, lives in
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
    const int e = fp4_exponent(fmaxf(m0, m1));
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

// ---------------------------------------------------------------------------
// Main kernel. Workgroup tile: 256 weight rows (a pair of heads) x 256 tokens,
// 8 waves; wave w owns head 2*pair + (w & 1) and tokens 64 (w >> 1) .. +63,
// i.e. a 128 x 64 sub-tile held as 4 x 2 accumulators of 32 x 32.
//
// Per 128-deep K block both operand tiles (W 256 x 128 B and A 256 x 128 B)
// are copied global -> LDS by global_load_lds_dwordx4 (no staging registers):
// one instruction moves 1 KiB = 8 rows, lane i writing bytes 16 i of it. Row
// r's 16-byte chunks are stored XOR-swizzled (chunk c at slot c ^ (r % 8)),
// so a lane loads the global chunk whose swizzled slot is its own, and the
// MFMA operand reads (8 consecutive rows, one chunk column) hit distinct banks.
// Two stages double-buffer the K loop; the barrier is a bare s_barrier with
// explicit wait counts so the next stage's copies stay in flight.
constexpr int NWAVES = 8;
constexpr int NTHREADS = NWAVES * 64;
constexpr int TILE_ROWS = 256;                    // weight rows (2 heads) and tokens per workgroup
constexpr int TILE_BYTES = TILE_ROWS * KB;        // one operand tile of one K block: 32 KiB
constexpr int SLAB = 1024;                        // bytes written by one wave-wide LDS copy
constexpr int COPIES = TILE_BYTES / SLAB / NWAVES;  // per operand per wave per stage: 4
constexpr int VM_PER_STAGE = 2 * COPIES + 1;       // operand copies + the scale-word copy
constexpr int SCALE_OFF = 2 * TILE_BYTES;           // scale words after the two operand tiles
constexpr int STAGE_BYTES = SCALE_OFF + NWAVES * 256;

// s_waitcnt immediates (gfx9 encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] << 14)
constexpr int waitcnt_vm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }
constexpr int WAITCNT_LGKM0 = 15 | (7 << 4) | (0 << 8) | (3 << 14);

__device__ __forceinline__ void block_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

typedef __attribute__((address_space(3))) void lds_void;

template <int STAGE>
__global__ __launch_bounds__(NTHREADS, 1)
void indexer_q_kernel(IndexerQArgs p) {
  // per stage: W tile, A tile, then the scale words [wave][64 tokens]
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][STAGE_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int half = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hn = wave & 1;          // head of the pair
  const int q = wave >> 1;          // token quarter (64 tokens)

  // ---- workgroup -> (head pair, token tile); XCD-aware when the pair count
  // is a multiple of 8 (consecutive workgroup ids go to consecutive XCDs)
  const int bid = blockIdx.x;
  const int npairs = (p.H + 1) >> 1;
  int pair, mtile;
  if ((npairs & 7) == 0) {
    const int ppx = npairs >> 3;
    const int s = bid >> 3;
    pair = (bid & 7) * ppx + s % ppx;
    mtile = s / ppx;
  } else {
    pair = bid % npairs;
    mtile = bid / npairs;
  }
  const int head = 2 * pair + hn;
  const int head_c = head < p.H ? head : p.H - 1;   // odd H: the last pair's second head is a clamped copy, never stored
  const int64_t mbase = (int64_t)mtile * TILE_ROWS;
  const int nkb = p.nkb;

  // ---- LDS-copy sources: for copy i this lane lands in row r = 8 slab + lane/8,
  // slot lane%8, which holds the row's chunk c = (lane%8) ^ (r%8).
  const int chunk = (lane & 7) ^ ((lane >> 3) & 7);
  const uint8_t* wsrc[COPIES];
  const uint8_t* asrc[COPIES];
  const int64_t wrow_max = (int64_t)p.H * HEAD_DIM - 1;
#pragma unroll
  for (int i = 0; i < COPIES; ++i) {
    const int r = 8 * (wave + NWAVES * i) + (lane >> 3);
    int64_t wr = (int64_t)2 * pair * HEAD_DIM + r;
    wr = wr < wrow_max ? wr : wrow_max;
    wsrc[i] = p.w + wr * p.ldw + 16 * chunk;
    int64_t t = mbase + r;
    t = t < p.M ? t : p.M - 1;
    asrc[i] = p.a + t * p.lda + 16 * chunk;
  }
  // ---- scale-word copies: lane l fetches the packed UE8M0 word of token
  // mbase + 64 q + l (one 256-byte LDS copy per wave per stage); a lane's two
  // MFMA tokens are entries 32 tm + lane%32 of its wave's copy.
  const uint8_t* ssrc;
  {
    int64_t t = mbase + 64 * q + lane;
    t = t < p.M ? t : p.M - 1;
    ssrc = p.a_scale_bytes + 4 * t * p.as_sm;
  }
  // ---- the head's weight-scale bytes, lane j holding K block 64 c + j of
  // chunk c; read back per K block with readlane (a scalar, no memory op)
  const uint8_t* wsc = p.w_scales + (int64_t)head_c * nkb;
  uint32_t wsc_lane = lane < nkb ? wsc[lane] : 0u;

  auto issue_stage = [&](int j, int st) {
#pragma unroll
    for (int i = 0; i < COPIES; ++i) {
      __builtin_amdgcn_global_load_lds((const void*)(wsrc[i] + (int64_t)KB * j),
                                       (lds_void*)(&lds[st][SLAB * (wave + NWAVES * i)]), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void*)(asrc[i] + (int64_t)KB * j),
                                       (lds_void*)(&lds[st][TILE_BYTES + SLAB * (wave + NWAVES * i)]), 16, 0, 0);
    }
    __builtin_amdgcn_global_load_lds((const void*)(ssrc + 4 * (int64_t)(j >> 2) * p.as_sw),
                                     (lds_void*)(&lds[st][SCALE_OFF + 256 * wave]), 4, 0, 0);
  };

  v16f acc[2][4];
#pragma unroll
  for (int tm = 0; tm < 2; ++tm)
#pragma unroll
    for (int tn = 0; tn < 4; ++tn)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[tm][tn][r] = 0.f;

  issue_stage(0, 0);

  for (int j = 0; j < nkb; ++j) {
    const int st = j & 1;
    if ((j & 63) == 0 && j > 0) {   // next 64 weight-scale bytes (only for K > 8192)
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
      wsc_lane = j + lane < nkb ? wsc[j + lane] : 0u;
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    }
    if (j + 1 < nkb) {
      issue_stage(j + 1, st ^ 1);
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(VM_PER_STAGE));   // stage j's copies have landed
    } else {
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    }
    block_barrier();                                          // ... for every wave

    const int wscale = __builtin_amdgcn_readlane((int)wsc_lane, j & 63);
    const int sshift = 8 * (j & 3);
    int asc[2];
#pragma unroll
    for (int tm = 0; tm < 2; ++tm)
      asc[tm] = (int)(*reinterpret_cast<const uint32_t*>(&lds[st][SCALE_OFF + 256 * wave + 4 * (32 * tm + (lane & 31))]) >> sshift);
    const uint8_t* wt = &lds[st][0];
    const uint8_t* at = &lds[st][TILE_BYTES];
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      const int c0 = 4 * kh + 2 * half;
      v8i af[2];
#pragma unroll
      for (int tm = 0; tm < 2; ++tm) {
        const int row = 64 * q + 32 * tm + (lane & 31);
        const v4u lo = *reinterpret_cast<const v4u*>(at + row * KB + 16 * (c0 ^ (row & 7)));
        const v4u hi = *reinterpret_cast<const v4u*>(at + row * KB + 16 * ((c0 + 1) ^ (row & 7)));
        af[tm] = make_v8i(lo, hi);
      }
#pragma unroll
      for (int tn = 0; tn < 4; ++tn) {
        const int row = HEAD_DIM * hn + 32 * tn + (lane & 31);
        const v4u lo = *reinterpret_cast<const v4u*>(wt + row * KB + 16 * (c0 ^ (row & 7)));
        const v4u hi = *reinterpret_cast<const v4u*>(wt + row * KB + 16 * ((c0 + 1) ^ (row & 7)));
        const v8i wf = make_v8i(lo, hi);
#pragma unroll
        for (int tm = 0; tm < 2; ++tm)
          acc[tm][tn] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              wf, af[tm], acc[tm][tn], 0, 0, 0, wscale, 0, asc[tm]);
      }
    }
    __builtin_amdgcn_s_waitcnt(WAITCNT_LGKM0);               // this wave's LDS reads are done
    block_barrier();                                          // stage st may be overwritten
  }

#pragma unroll
  for (int tm = 0; tm < 2; ++tm)
    epilogue_tile<STAGE>(acc[tm], mbase + 64 * q + 32 * tm + (lane & 31), head, head < p.H, half, p);
}

hipError_t launch_kernel(const IndexerQArgs& a, int stage, hipStream_t stream) {
  const int64_t n_mt = (a.M + TILE_ROWS - 1) / TILE_ROWS;
  const int64_t blocks = n_mt * ((a.H + 1) / 2);
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  const dim3 grid((unsigned)blocks), block(NTHREADS);
  switch (stage) {
    case -1: hipLaunchKernelGGL(indexer_q_kernel<-1>, grid, block, 0, stream, a); break;
    case 0: hipLaunchKernelGGL(indexer_q_kernel<0>, grid, block, 0, stream, a); break;
    case 1: hipLaunchKernelGGL(indexer_q_kernel<1>, grid, block, 0, stream, a); break;
    case 2: hipLaunchKernelGGL(indexer_q_kernel<2>, grid, block, 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_indexer_q(const IndexerQArgs& a, int stage, hipStream_t stream) {
  return launch_kernel(a, stage, stream);
}

}  // namespace iqp
