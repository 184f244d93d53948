// Small-batch variant of the fused indexer-Q kernel (decode-sized token
// counts, K = 12 blocks of 128): the same computation as indexer_q.hip
// (block-scaled FP8 GEMM on the matrix cores, RoPE, Hadamard-128, FP4 with
// UE8M0 scales), laid out for few tokens.
//
// tokenspeed PR "perf(deepseek-v4): accelerate indexer Q and packed FP8
// quantization", Summary and Perf (small shapes are kept off the multi-launch
// path); TensorRT-LLM PR "Fuse DeepSeek-V4 Indexer Q projection with CuTe
// DSL", kernel routing (a separate small-M route with swapped operands).
//
// With at most 64 tokens the projection is a read of the 12.6 MB weight
// matrix: the MFMA work is a few percent of the large-batch kernel's, so the
// layout is chosen for streaming the weights through as many CUs as there
// are heads and for latency, not for operand reuse:
//   * one workgroup per head (4 waves); wave w owns the head's weight rows
//     32 w .. 32 w + 31 (48 KiB) and streams them through a ring of LDS
//     stages of its own (7 or 4 K blocks deep), with coalesced buffer-to-LDS
//     copies of 8 rows x 128 bytes; no other wave reads them, so the ring
//     needs no barrier, only the wave's own wait counts. (Loading the
//     fragments straight into registers touches 32 rows per instruction and
//     ran at a third of the rate.)
//   * the activation rows of the batch (at most 64 x 1536 bytes) are copied
//     once into LDS by the same path, 16-byte chunks permuted per row so
//     that the operand reads of 32 rows hit distinct banks;
//   * 32-token column tiles (NT = 1, 2) on the 32x32x64 scaled FP8 MFMA,
//     weight rows as the first operand, as in the other kernels, so the
//     accumulators have their layout;
//   * the four waves' 32-row slices of each column tile meet in LDS, and
//     wave tm runs the shared epilogue (RoPE, Hadamard, FP4, stores) of
//     column tile tm.
// Tokens past M: their LDS rows are never written (no copy reaches them) and
// their results are never stored; an MFMA column depends on its own token's
// row only, so whatever those rows hold stays in columns that are dropped.
#include <type_traits>

#include "iq_common.h"

namespace iqp {
namespace {
namespace small {

constexpr int NWAVES = 4;
constexpr int NTHREADS = NWAVES * 64;
constexpr int NKB = 12;                     // K blocks (K = 1536)
constexpr int KROW = NKB * KB;              // bytes of one activation row in LDS
constexpr int MAX_NT = 2;                   // 32-token column tiles
constexpr int SLAB = 1024;                  // one wave-wide LDS copy
constexpr int LDS_BYTES = 160 * 1024;
constexpr int XTILE = 4 * 4 * SLAB;         // one column tile's accumulators (4 slices x 16 floats x 64 lanes)
constexpr int WSTAGE = 32 * KB;             // one K block of a wave's 32 weight rows: 4 KiB

// Activation rows first, then the four weight rings. A weight copy's LDS
// address is given as its destination minus its column offset in the row
// (at most 11 K blocks), which must not go below zero.
template <int NT>
struct Layout {
  static constexpr int W_OFF = 32 * NT * KROW;
  static constexpr int NST = (LDS_BYTES - W_OFF) / (NWAVES * WSTAGE);   // 7 or 4
  static_assert(NT * XTILE <= W_OFF, "the accumulator exchange reuses the activation rows' LDS");
  static_assert(W_OFF >= KB * (NKB - 1), "copy LDS bases must stay non-negative");
};

__device__ __forceinline__ constexpr int waitcnt_vm(int n) {
  return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14);
}

template <int I, int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// LDS byte of 16-byte chunk c (0..95) of activation row r
__device__ __forceinline__ uint32_t a_slot(int r, int c) { return (uint32_t)(r * KROW + 16 * (c ^ (r & 15))); }

template <int NT>
__global__ __launch_bounds__(NTHREADS, 1)
void indexer_q_small_kernel(IndexerQArgs p) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[LDS_BYTES];
  const int head = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63, half = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int M = (int)p.M;   // at most 32 NT

  // RoPE rows of the column tile this wave finishes (first: their latency
  // then hides under everything else)
  RopeCS rope;
  if (wave < NT) rope = load_rope(load_position(32 * wave + (lane & 31), p), half, p);

  // 1. the activation rows into LDS: slab k covers LDS bytes [1 KiB k, 1 KiB
  //    (k + 1)); its lane i fills byte 1 KiB k + 16 i, which is slot
  //    (1 KiB k + 16 i) % 1536 / 16 of row (1 KiB k + 16 i) / 1536 and holds
  //    that row's chunk slot ^ (row % 16). Slabs past the batch's rows are
  //    skipped; rows past M inside the last one read zeros (bounds check).
  {
    const rsrc_t ra = make_rsrc(p.a, (uint64_t)M * p.lda);
    const int nslab = (M * KROW + SLAB - 1) / SLAB;
    for (int k = wave; k < nslab; k += NWAVES) {
      const int b = SLAB * k + 16 * lane;
      const int r = b / KROW, s = (b % KROW) / 16;
      const uint32_t voff = (uint32_t)(r * (int)p.lda + 16 * (s ^ (r & 15)));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void*)(lds + SLAB * k), 16, voff, 0, 0, 0);
    }
  }
  __builtin_amdgcn_sched_barrier(0);

  // 2. the lane's token scale words (token 32 tm + lane % 32, clamped into the batch)
  uint32_t asw[NT][3];
#pragma unroll
  for (int tm = 0; tm < NT; ++tm) {
    int t = 32 * tm + (lane & 31);
    t = t < M ? t : M - 1;
    const uint32_t* w = reinterpret_cast<const uint32_t*>(p.a_scale_bytes) + (int64_t)t * p.as_sm;
#pragma unroll
    for (int k = 0; k < 3; ++k) asw[tm][k] = w[k * p.as_sw];
  }
  // the head's weight scales, one byte per K block
  const uint32_t* wsp = reinterpret_cast<const uint32_t*>(p.w_scales + (int64_t)head * NKB);
  uint32_t wsw[3];
#pragma unroll
  for (int k = 0; k < 3; ++k) wsw[k] = __builtin_amdgcn_readfirstlane(wsp[k]);
  __builtin_amdgcn_sched_barrier(0);

  // 3. the wave's weight ring. Copy c (0..3) of K block j moves rows
  //    8 c + l / 8 (of the wave's 32) into stage j % NST, LDS row 8 c + l / 8
  //    slot l % 8, which holds the row's 16-byte chunk (l % 8) ^ (row / 2 % 8);
  //    the column 128 j is the instruction offset (added to the LDS address too).
  constexpr int NST = Layout<NT>::NST;
  const rsrc_t rw = make_rsrc(p.w + (int64_t)head * HEAD_DIM * p.ldw, (uint64_t)HEAD_DIM * p.ldw);
  uint32_t wv[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int r = 8 * c + (lane >> 3);
    wv[c] = (uint32_t)((32 * wave + r) * (int)p.ldw + 16 * ((lane & 7) ^ ((r >> 1) & 7)));
  }
  uint8_t* const ring = lds + Layout<NT>::W_OFF + NST * WSTAGE * wave;
  auto copies = [&](auto jc) __attribute__((always_inline)) {
    constexpr int j = decltype(jc)::value;
#pragma unroll
    for (int c = 0; c < 4; ++c)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void*)(ring + (j % NST) * WSTAGE + SLAB * c - KB * j), 16,
                                               wv[c], 0, KB * j, 0);
  };
  static_for<0, NST>([&](auto jc) __attribute__((always_inline)) { copies(jc); });
  __builtin_amdgcn_sched_barrier(0);
  // the activation copies were issued before the ring's first copies: once
  // only those may be outstanding, they have landed
  {
    constexpr int WAIT = waitcnt_vm(4 * NST);
    __builtin_amdgcn_s_waitcnt(WAIT);
  }
  block_barrier();

  // 4. the K loop: block j's weights are in stage j % NST once only the
  //    copies of the blocks after it may be outstanding; the stage is refilled
  //    with block j + NST once its fragments are read
  v16f acc[NT];
#pragma unroll
  for (int tm = 0; tm < NT; ++tm)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[tm][r] = 0.f;
  const int arow = lane & 31;
  const int wswz = (arow >> 1) & 7;
  static_for<0, NKB>([&](auto jc) __attribute__((always_inline)) {
    constexpr int j = decltype(jc)::value;
    constexpr int last = j + NST - 1 < NKB - 1 ? j + NST - 1 : NKB - 1;
    constexpr int WAIT = waitcnt_vm(4 * (last - j));
    __builtin_amdgcn_s_waitcnt(WAIT);
    const uint8_t* st = ring + (j % NST) * WSTAGE + KB * arow;
    v8i wfr[2];
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      const v4u w0 = *reinterpret_cast<const v4u*>(st + 16 * ((4 * kh + 2 * half) ^ wswz));
      const v4u w1 = *reinterpret_cast<const v4u*>(st + 16 * ((4 * kh + 2 * half + 1) ^ wswz));
      wfr[kh] = make_v8i(w0, w1);
    }
    v8i afr[2][NT];
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
      for (int tm = 0; tm < NT; ++tm) {
        const int r = 32 * tm + arow, c0 = 8 * j + 4 * kh + 2 * half;
        afr[kh][tm] = make_v8i(*reinterpret_cast<const v4u*>(lds + a_slot(r, c0)),
                               *reinterpret_cast<const v4u*>(lds + a_slot(r, c0 + 1)));
      }
    if constexpr (j + NST < NKB) {
      __builtin_amdgcn_s_waitcnt(WAITCNT_LGKM0);   // the stage's fragments are in registers
      copies(std::integral_constant<int, j + NST>{});
    }
    const int ws = (int)(wsw[j >> 2] >> (8 * (j & 3)));
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
      for (int tm = 0; tm < NT; ++tm) {
        const int as = (int)(asw[tm][j >> 2] >> (8 * (j & 3)));
        acc[tm] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wfr[kh], afr[kh][tm], acc[tm], 0, 0, 0, ws, 0, as);
      }
    __builtin_amdgcn_sched_barrier(0);
  });

  // 5. the column tiles' four 32-row slices meet in LDS (over the activation
  //    rows, once every wave is done reading them): slice tn of tile tm, group
  //    g of 4 accumulators at ((tm * 4 + tn) * 4 + g) KiB + 16 lane
  block_barrier();
#pragma unroll
  for (int tm = 0; tm < NT; ++tm)
#pragma unroll
    for (int g = 0; g < 4; ++g)
      *reinterpret_cast<v4f*>(lds + XTILE * tm + SLAB * (4 * wave + g) + 16 * lane) =
          v4f{acc[tm][4 * g], acc[tm][4 * g + 1], acc[tm][4 * g + 2], acc[tm][4 * g + 3]};
  block_barrier();
  if (wave < NT) {
    v16f full[4];
#pragma unroll
    for (int tn = 0; tn < 4; ++tn)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const v4f x = *reinterpret_cast<const v4f*>(lds + XTILE * wave + SLAB * (4 * tn + g) + 16 * lane);
#pragma unroll
        for (int q = 0; q < 4; ++q) full[tn][4 * g + q] = x[q];
      }
    epilogue_tile<-1>(full, 32 * wave + (lane & 31), head, true, half, p, rope);
  }
}

}  // namespace small
}  // namespace

// activation and weight row offsets are formed in 32 bits; the weight scales
// are read four at a time
bool indexer_q_small_supported(const IndexerQArgs& a) {
  return a.nkb == small::NKB && a.M >= 1 && a.M <= 32 * small::MAX_NT && a.lda <= (1 << 24) &&
         a.ldw <= (1 << 22) && (reinterpret_cast<uintptr_t>(a.w_scales) & 3) == 0;
}

hipError_t launch_indexer_q_small(const IndexerQArgs& a, hipStream_t stream) {
  const dim3 grid((unsigned)a.H), block(small::NTHREADS);
  if (a.M <= 32)
    hipLaunchKernelGGL(small::indexer_q_small_kernel<1>, grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL(small::indexer_q_small_kernel<2>, grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace iqp
