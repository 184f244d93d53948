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
// Up to 256 tokens the projection is mostly a read of the 12.6 MB weight
// matrix and the MFMA work is a few percent of the large-batch kernel's, so
// the layout is chosen for streaming the weights through many CUs and for
// latency rather than for operand reuse:
//   * one workgroup per head and 32-token column tile, 4 waves. The tiles of
//     a head are H workgroups apart, so with 64 heads they land on one XCD
//     and share its L2 for the head's weights.
//   * wave w owns the head's weight rows 32 w .. 32 w + 31 (48 KiB) and
//     streams them through a ring of 7 LDS stages of its own, with coalesced
//     buffer-to-LDS copies of 8 rows x 128 bytes. No other wave reads them,
//     so the ring needs no barrier, only the wave's own wait counts. (Loading
//     the fragments straight into registers touches 32 rows per instruction
//     and ran at a third of the rate.)
//   * the tile's activation rows (32 x 1536 bytes) are copied once into LDS
//     by the same path, 16-byte chunks permuted per row so that the operand
//     reads of 32 rows hit distinct banks.
//   * the 32x32x64 scaled FP8 MFMA, weight rows as the first operand as in
//     the other kernels, so the accumulators have their layout.
//   * the four waves' 32-row slices meet in LDS as token rows of 128 floats,
//     and the epilogue (RoPE, Hadamard-128, FP4, stores) is split over all
//     four waves, 8 tokens each: lane l takes token 8 w + l % 8 and 16 of its
//     dims, d = 64 b6 + 32 b5 + 16 b4 + 8 b3 + k with (b3, b4, b6) the lane
//     bits 3..5 and (b5, k) in the lane. The RoPE pairs (d, d + 32) and the
//     FP4 blocks' 8-dim runs are then in the lane, and the Hadamard stages
//     over dim bits 3, 4, 6 are exchanges with lane l ^ 8 (DPP), l ^ 16 and
//     l ^ 32 (permlane swaps).
// Tokens past M: their LDS rows are never written (no copy reaches them) and
// their results are never stored; an MFMA column depends on its own token's
// row only, so whatever those rows hold stays in columns that are dropped.
//
// Split-K build of the one-launch variant below (S > 1; 12 to 64 tokens,
// given a workspace): with one or two tiles the grid above fills 64 or 128
// CUs, and each of them quantizes the tile's whole 32 x 1536 activations
// before its K loop can start. Here S workgroups share a head and tile, each
// taking 12 / S consecutive K blocks (it quantizes only those, and has all of
// its weight blocks in flight at once, no ring refills). Each stores its float32 sums (4 KiB a wave, in the
// accumulators' register order) to the workspace, then takes a ticket from
// the head and tile's counter; the one that draws the last ticket adds the S
// partial sums in split order (so the result does not depend on which one
// that is), resets the counter and runs the epilogue; the others exit. No
// workgroup waits for another.
//
// One-launch variant (XIN): the workgroup takes bf16 activations and
// quantizes its own rows (the packed-UE8M0 FP8 1x128 rule, with the
// standalone quantizer's arithmetic) straight into the LDS layout above,
// while the weight ring fills: the rows are loaded into registers first,
// then the ring's copies are issued, then the blocks are quantized (8 lanes a
// block). The blocks' scale bytes cross waves through LDS; all 160 KiB are
// in use, so the ring's seventh block is issued after that exchange and the
// exchange borrows its stage (the blocks keep their issue order, so the K
// loop's wait counts hold).
#include <type_traits>

#include "fp8_block.h"
#include "iq_common.h"

// Convention variant compiled into this translation unit (bit 0: interleaved
// RoPE pairs, bit 1: OCP floor-rule FP4 scales, bit 2: one weight scale per
// row and K block; 0: the defaults). The variant units define it and the
// names of the FP8-input and bf16-input launchers before including this file.
#ifndef IQP_SMALL_VARIANT
#define IQP_SMALL_VARIANT 0
#define IQP_SMALL_KERNEL indexer_q_small_kernel
#endif

namespace iqp {
namespace {
namespace small {

constexpr bool VAR_IL = (IQP_SMALL_VARIANT & 1) != 0;
constexpr bool VAR_FLOOR = (IQP_SMALL_VARIANT & 2) != 0;
constexpr bool VAR_ROWS = (IQP_SMALL_VARIANT & 4) != 0;

constexpr int NWAVES = 4;
constexpr int NTHREADS = NWAVES * 64;
constexpr int NKB = 12;                     // K blocks (K = 1536)
constexpr int TILE = 32;                    // tokens per workgroup
constexpr int MAX_TILES = 8;                // column tiles per head: up to 256 tokens
constexpr int KROW = NKB * KB;              // bytes of one activation row in LDS
constexpr int SLAB = 1024;                  // one wave-wide LDS copy
constexpr int LDS_BYTES = 160 * 1024;
constexpr int XROW = 4 * (HEAD_DIM + 4);    // one token's 128 floats in LDS, padded against bank conflicts
constexpr int WSTAGE = 32 * KB;             // one K block of a wave's 32 weight rows: 4 KiB
// Activation rows first, then the four weight rings. A weight copy's LDS
// address is given as its destination minus its column offset in the row
// (at most 11 K blocks), which must not go below zero.
constexpr int W_OFF = TILE * KROW;                                  // 48 KiB
constexpr int NST = (LDS_BYTES - W_OFF) / (NWAVES * WSTAGE);        // 7 stages per wave
static_assert(TILE * XROW <= W_OFF, "the accumulator exchange reuses the activation rows' LDS");
static_assert(W_OFF >= KB * (NKB - 1), "copy LDS bases must stay non-negative");

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

// byte i (0 .. 11) of the 12 held in w[0..2]; i is uniform, so the selects
// are scalar where w is
__device__ __forceinline__ uint32_t byte12(const uint32_t (&w)[3], int i) {
  const uint32_t x = i < 4 ? w[0] : (i < 8 ? w[1] : w[2]);
  return x >> (8 * (i & 3));
}

// DUMP (diagnostic build, default configuration only): the float32 GEMM
// sums (Q before RoPE) go to pa.dbg [M, H*128] in place of the epilogue.
// S: workgroups per head and tile, each over NKB / S K blocks (split-K
// build, default configuration only; grid rows are tile-major, split-minor).
template <bool XIN, bool DUMP = false, int S = 1>
__global__ __launch_bounds__(NTHREADS, 1)
void IQP_SMALL_KERNEL(IndexerQArgs pa) {
  constexpr int KBS = NKB / S;                  // K blocks of this workgroup
  constexpr int XSTEPS = TILE * KBS / 32;       // one-launch variant: 32 blocks per step
  static_assert(NKB % S == 0 && (S == 1 || KBS <= NST - 1), "a split's blocks fit the ring, its last stage spare");
  static_assert(S == 1 || (XIN && IQP_SMALL_VARIANT == 0), "the split-K build is the default one-launch kernel's");
  __shared__ __attribute__((aligned(16))) uint8_t lds[LDS_BYTES];
  const int tid = threadIdx.x;
  const int ntiles = (int)((pa.M + TILE - 1) / TILE);
  if constexpr (XIN && !DUMP) {
    // grid rows past the heads' token tiles: the independent quantization run
    // beside this kernel, two packed words per wave as the standalone
    // quantizer's workgroups take them (its codes stay in cache: decode-sized)
    const int main_rows = ntiles * S;
    if ((int)blockIdx.y >= main_rows) {
      const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
      const int64_t g = (int64_t)(blockIdx.y - main_rows) * gridDim.x + blockIdx.x;
      const int64_t first = 2 * (g * NWAVES + w);
      if (first < pa.side_words)
        fp8q::quant_word_pair<false>(pa.side_x, pa.side_ldx, pa.side_q, pa.side_ldq, pa.side_scales, pa.side_sm,
                                     pa.side_sw, pa.side_nw, pa.side_nkb, pa.side_words, first, tid & 63);
      return;
    }
  }
  const int head = blockIdx.x;
  const int lane = tid & 63, half = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tile = (int)blockIdx.y / S;
  const int split = (int)blockIdx.y - S * tile;
  const int kb0 = S == 1 ? 0 : KBS * split;   // the first K block of this workgroup
  // the column tile's tokens: the batch seen from token t0 on (and, split,
  // from K block kb0 on)
  const int64_t t0 = TILE * (int64_t)tile;
  IndexerQArgs p = pa;
  if constexpr (XIN) {
    p.x += t0 * p.ldx + KB * kb0;
  } else {
    p.a += t0 * p.lda;
    p.a_scale_bytes += 4 * t0 * p.as_sm;
  }
  p.positions += t0;
  p.q_fp4 += t0 * p.H * (HEAD_DIM / 2);
  p.q_scales += t0 * p.H * 4;
  p.M = pa.M - t0 < TILE ? pa.M - t0 : TILE;
  const int M = (int)p.M;   // 1 .. 32

  // 1x. (one-launch variant) the tile's bf16 rows into registers: block
  //     b = KBS r + j (row r, K block j of the workgroup's KBS) is step
  //     b / 32, wave b / 8 % 4, lanes 8 (b % 8) .. +7 of it, 16 values a
  //     lane; steps past the tile's KBS M blocks are not loaded, lanes past
  //     them reload the last block.
  fp8q::v4u xa[XSTEPS], xb[XSTEPS];
  const int nblk = KBS * M;
  const int nsteps = (nblk + 31) / 32;
  if constexpr (XIN) {
#pragma unroll
    for (int s = 0; s < XSTEPS; ++s) {
      if (s < nsteps) {
        const int b = min(32 * s + 8 * wave + (lane >> 3), nblk - 1);
        const int r = b / KBS, j = b - KBS * r;
        const fp8q::v4u* src = reinterpret_cast<const fp8q::v4u*>(p.x + (int64_t)r * p.ldx + KB * j + 16 * (lane & 7));
        xa[s] = src[0];
        xb[s] = src[1];
      }
    }
  }
  __builtin_amdgcn_sched_barrier(0);

  // 1. the activation rows into LDS: slab k covers LDS bytes [1 KiB k, 1 KiB
  //    (k + 1)); its lane i fills byte 1 KiB k + 16 i, which is slot
  //    (1 KiB k + 16 i) % 1536 / 16 of row (1 KiB k + 16 i) / 1536 and holds
  //    that row's chunk slot ^ (row % 16). Slabs past the tile's rows are
  //    skipped; rows past M inside the last one read zeros (bounds check).
  if constexpr (!XIN) {
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

  // 2. the lane's token scale words (token lane % 32, clamped into the tile);
  //    the one-launch variant forms them from its own blocks below
  uint32_t asw[3];
  if constexpr (!XIN) {
    const int t = (lane & 31) < M ? (lane & 31) : M - 1;
    const uint32_t* w = reinterpret_cast<const uint32_t*>(p.a_scale_bytes) + (int64_t)t * p.as_sm;
#pragma unroll
    for (int k = 0; k < 3; ++k) asw[k] = w[k * p.as_sw];
  }
  // the head's weight scales, one byte per K block (per-row variant: the
  // 12 bytes of this lane's MFMA row 32 wave + lane % 32, 4-byte aligned
  // since the array is and 12 divides by 4)
  const uint32_t* wsp = reinterpret_cast<const uint32_t*>(
      p.w_scales + (VAR_ROWS ? ((int64_t)head * HEAD_DIM + 32 * wave + (lane & 31)) * NKB : (int64_t)head * NKB));
  uint32_t wsw[3];
#pragma unroll
  for (int k = 0; k < 3; ++k) wsw[k] = VAR_ROWS ? wsp[k] : __builtin_amdgcn_readfirstlane(wsp[k]);
  // Epilogue lanes: token 8 wave + l % 8 and the dims
  // 64 b6 + 32 b5 + 8 (b3 + 2 b4) + k, (b3, b4, b6) = lane bits 3, 4, 5.
  // The token's position now; its RoPE table row (the pairs
  // i = 8 (b3 + 2 b4) + k) once the K loop runs, so that no load waits for
  // another before the weight stream starts.
  const int sub = lane >> 3;
  const int eoff = 8 * (sub & 3) + 64 * (sub >> 2);   // the lane's dims: eoff + 32 b5 + k
  const int et = 8 * wave + (lane & 7);                // the lane's epilogue token
  const int64_t posv = load_position(et, p);
  __builtin_amdgcn_sched_barrier(0);

  // 3. the wave's weight ring. Copy c (0..3) of K block j moves rows
  //    8 c + l / 8 (of the wave's 32) into stage j % NST, LDS row 8 c + l / 8
  //    slot l % 8, which holds the row's 16-byte chunk (l % 8) ^ (row / 2 % 8);
  //    the column 128 j is the instruction offset (added to the LDS address too).
  //    Split build: blocks kb0 .. kb0 + KBS - 1, all issued at once.
  const rsrc_t rw = make_rsrc(p.w + (int64_t)head * HEAD_DIM * p.ldw + KB * kb0,
                              (uint64_t)HEAD_DIM * p.ldw - KB * kb0);
  uint32_t wv[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int r = 8 * c + (lane >> 3);
    wv[c] = (uint32_t)((32 * wave + r) * (int)p.ldw + 16 * ((lane & 7) ^ ((r >> 1) & 7)));
  }
  uint8_t* const ring = lds + W_OFF + NST * WSTAGE * wave;
  auto copies = [&](auto jc) __attribute__((always_inline)) {
    constexpr int j = decltype(jc)::value;
#pragma unroll
    for (int c = 0; c < 4; ++c)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void*)(ring + (j % NST) * WSTAGE + SLAB * c - KB * j), 16,
                                               wv[c], 0, KB * j, 0);
  };
  if constexpr (!XIN) {
    static_for<0, NST>([&](auto jc) __attribute__((always_inline)) { copies(jc); });
    __builtin_amdgcn_sched_barrier(0);
    // the activation copies, scale words and position were issued before the
    // ring's first copies: once only those may be outstanding, they have landed
    constexpr int WAIT = waitcnt_vm(4 * NST);
    __builtin_amdgcn_s_waitcnt(WAIT);
    block_barrier();
  } else {
    // the ring's first NST - 1 blocks; the last stage of wave 0's ring holds
    // the scale-byte exchange (byte 12 r + j: row r, block j) until its block
    // is issued (split build: all KBS blocks, the last stage stays spare)
    constexpr int FIRST = S > 1 ? KBS : NST - 1;
    static_for<0, FIRST>([&](auto jc) __attribute__((always_inline)) { copies(jc); });
    __builtin_amdgcn_sched_barrier(0);
    uint8_t* const xch = lds + W_OFF + (NST - 1) * WSTAGE;
    {
      constexpr int WAIT = waitcnt_vm(4 * FIRST);   // the rows and the position have landed
      __builtin_amdgcn_s_waitcnt(WAIT);
    }
#pragma unroll
    for (int s = 0; s < XSTEPS; ++s) {
      if (s < nsteps) {
        const int b = 32 * s + 8 * wave + (lane >> 3);
        const int e = fp8q::block_exponent(fp8q::lanes8_max(fp8q::mag16(xa[s], xb[s])));
        const fp8q::v4u codes = fp8q::codes16(xa[s], xb[s], e);
        if (b < nblk) {
          const int r = b / KBS, j = b - KBS * r;
          *reinterpret_cast<fp8q::v4u*>(lds + a_slot(r, 8 * j + (lane & 7))) = codes;
          if ((lane & 7) == 0) xch[NKB * r + j] = (uint8_t)(e + 127);
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(WAITCNT_LGKM0);   // this wave's LDS writes are done
    block_barrier();
    // token lane % 32's twelve bytes (rows past M: never written, columns dropped)
    const uint32_t* xw = reinterpret_cast<const uint32_t*>(xch + NKB * (lane & 31));
#pragma unroll
    for (int k = 0; k < 3; ++k) asw[k] = xw[k];
    __builtin_amdgcn_s_waitcnt(WAITCNT_LGKM0);
    if constexpr (S == 1) {
      block_barrier();   // every wave has its words: the stage may be refilled
      copies(std::integral_constant<int, NST - 1>{});
    }
    __builtin_amdgcn_sched_barrier(0);
  }

  // 4. the K loop: block j's weights are in stage j % NST once only the
  //    copies of the blocks after it may be outstanding (and the 4 RoPE row
  //    loads issued after block NST's copies); the stage is refilled with
  //    block j + NST once its fragments are read (split build: the KBS
  //    blocks of the workgroup, none refilled)
  v4f rc[2], rs[2];
  v16f acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
  const int arow = lane & 31;
  const int wswz = (arow >> 1) & 7;
  static_for<0, KBS>([&](auto jc) __attribute__((always_inline)) {
    constexpr int j = decltype(jc)::value;
    constexpr int last = j + NST - 1 < KBS - 1 ? j + NST - 1 : KBS - 1;
    constexpr int WAIT = waitcnt_vm(4 * (last - j) + (j >= 1 && j <= NST ? 4 : 0));
    __builtin_amdgcn_s_waitcnt(WAIT);
    const uint8_t* st = ring + (j % NST) * WSTAGE + KB * arow;
    v8i wfr[2], afr[2];
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      const int c0 = 4 * kh + 2 * half;
      wfr[kh] = make_v8i(*reinterpret_cast<const v4u*>(st + 16 * (c0 ^ wswz)),
                         *reinterpret_cast<const v4u*>(st + 16 * ((c0 + 1) ^ wswz)));
      afr[kh] = make_v8i(*reinterpret_cast<const v4u*>(lds + a_slot(arow, 8 * j + c0)),
                         *reinterpret_cast<const v4u*>(lds + a_slot(arow, 8 * j + c0 + 1)));
    }
    if constexpr (j + NST < KBS) {
      __builtin_amdgcn_s_waitcnt(WAITCNT_LGKM0);   // the stage's fragments are in registers
      copies(std::integral_constant<int, j + NST>{});
    }
    if constexpr (j == 0) {
      int64_t pos = posv;
      pos = pos < 0 ? 0 : (pos >= p.max_pos ? p.max_pos - 1 : pos);
      // half-split: rc[h][s] is pair 8 (sub & 3) + 4 h + s; interleaved: pair
      // 4 (sub & 3) + 16 h + s (dims (2i, 2i + 1) = v[h][2s], v[h][2s + 1])
      const float* row = p.cos_sin + pos * 64 + (VAR_IL ? 4 : 8) * (sub & 3);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        rc[h] = *reinterpret_cast<const v4f*>(row + (VAR_IL ? 16 : 4) * h);
        rs[h] = *reinterpret_cast<const v4f*>(row + 32 + (VAR_IL ? 16 : 4) * h);
      }
    }
    // the weight bytes are the head's 12 (from the workgroup's first K
    // block); the activation bytes the token's 12 (split build: its KBS)
    const int ws = (int)byte12(wsw, kb0 + j);
    const int as = (int)byte12(asw, j);
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
      acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wfr[kh], afr[kh], acc, 0, 0, 0, ws, 0, as);
    __builtin_amdgcn_sched_barrier(0);
  });

  // 4s. split build: the sums to the workspace (split s, head and tile u:
  //     4 KiB a wave, register group g of lane l at byte 16 (64 g + l), so
  //     that each store writes 1 KiB), a ticket from u's counter, and only
  //     the last of u's workgroups goes on, with the S sums added in split
  //     order. The sums are stored and loaded device-coherent (the sc1 cache
  //     policy of relaxed device-scope atomics), and each workgroup's stores
  //     have completed before its ticket is taken; the counter is a
  //     device-scope atomic. No fence is needed beyond that, so no cache is
  //     written back or invalidated.
  if constexpr (S > 1) {
    constexpr int CPOL_DEVICE = 0x10;   // sc1
    const int64_t nunits = (int64_t)pa.H * ntiles;
    const int64_t unit = (int64_t)head * ntiles + tile;
    int32_t* const cnt = reinterpret_cast<int32_t*>(pa.splitk_ws) + unit;
    const rsrc_t rp = make_rsrc(pa.splitk_ws + splitk_counter_region(pa.splitk_ws_bytes), (uint64_t)65536 * pa.H);
    const uint32_t off0 = (uint32_t)((unit * NWAVES + wave) * 4096 + 16 * lane);
    const uint32_t split_stride = (uint32_t)(nunits * NWAVES * 4096);
#pragma unroll
    for (int g = 0; g < 4; ++g)
      __builtin_amdgcn_raw_buffer_store_b128(
          v4u{__float_as_uint(acc[4 * g]), __float_as_uint(acc[4 * g + 1]), __float_as_uint(acc[4 * g + 2]),
              __float_as_uint(acc[4 * g + 3])},
          rp, off0 + split * split_stride + 1024 * g, 0, CPOL_DEVICE);
    __builtin_amdgcn_s_waitcnt(WAITCNT_VM0);   // this wave's sums have been written
    __syncthreads();
    // wave 0's spare ring stage (the scale exchange before it ended with the K loop)
    int32_t* const flag = reinterpret_cast<int32_t*>(lds + W_OFF + NST * WSTAGE - 4);
    if (tid == 0) {
      const int32_t ticket = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const bool last_one = ticket == S - 1;
      if (last_one) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);   // for the next call
      *flag = last_one ? 1 : 0;
    }
    __syncthreads();
    if (*flag == 0) return;   // uniform over the workgroup
#pragma unroll
    for (int s2 = 0; s2 < S; ++s2) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const v4u x = __builtin_amdgcn_raw_buffer_load_b128(rp, off0 + s2 * split_stride + 1024 * g, 0, CPOL_DEVICE);
#pragma unroll
        for (int q = 0; q < 4; ++q)
          acc[4 * g + q] = s2 == 0 ? __uint_as_float(x[q]) : acc[4 * g + q] + __uint_as_float(x[q]);
      }
    }
  }

  // 5. the four 32-row slices meet in LDS (over the activation rows, once
  //    every wave is done reading them) as token rows: accumulator group g
  //    of slice w holds dims 32 w + 8 g + 4 half + 0..3 of token lane % 32
  block_barrier();
#pragma unroll
  for (int g = 0; g < 4; ++g)
    *reinterpret_cast<v4f*>(lds + XROW * (lane & 31) + 4 * (32 * wave + 8 * g + 4 * half)) =
        v4f{acc[4 * g], acc[4 * g + 1], acc[4 * g + 2], acc[4 * g + 3]};
  block_barrier();

  // 6. the epilogue of token et
  float v[2][8];   // v[b5][k]: dim eoff + 32 b5 + k
  {
    const uint8_t* xr = lds + XROW * et + 4 * eoff;
#pragma unroll
    for (int b5 = 0; b5 < 2; ++b5)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const v4f x = *reinterpret_cast<const v4f*>(xr + 128 * b5 + 16 * h);
#pragma unroll
        for (int q = 0; q < 4; ++q) v[b5][4 * h + q] = x[q];
      }
  }
  if constexpr (DUMP) {
    if (et < M) {
      float* row = pa.dbg + ((t0 + et) * p.H + head) * HEAD_DIM + eoff;
#pragma unroll
      for (int b5 = 0; b5 < 2; ++b5)
#pragma unroll
        for (int h = 0; h < 2; ++h)
          *reinterpret_cast<v4f*>(row + 32 * b5 + 4 * h) =
              v4f{v[b5][4 * h], v[b5][4 * h + 1], v[b5][4 * h + 2], v[b5][4 * h + 3]};
    }
    return;
  }
  // RoPE on dims 0..63 (b6 = 0): the pair (i, i + 32) is (v[0][k], v[1][k])
  if (!(sub & 4) && !VAR_IL) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float x = v[0][k], y = v[1][k];
      const float c = rc[k >> 2][k & 3], sn = rs[k >> 2][k & 3];
      v[0][k] = x * c - y * sn;
      v[1][k] = y * c + x * sn;
    }
  } else if (!(sub & 4)) {   // interleaved: the pair (v[b5][2m], v[b5][2m + 1])
#pragma unroll
    for (int b5 = 0; b5 < 2; ++b5)
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const float x = v[b5][2 * m], y = v[b5][2 * m + 1];
        const float c = rc[b5][m], sn = rs[b5][m];
        v[b5][2 * m] = x * c - y * sn;
        v[b5][2 * m + 1] = y * c + x * sn;
      }
  }
  // Hadamard: dim bits 0, 1, 2 (k) and 5 (b5) in the lane ...
#pragma unroll
  for (int kb = 1; kb < 8; kb <<= 1)
#pragma unroll
    for (int b5 = 0; b5 < 2; ++b5)
#pragma unroll
      for (int k = 0; k < 8; ++k)
        if (!(k & kb)) {
          const float a = v[b5][k], b = v[b5][k | kb];
          v[b5][k] = a + b;
          v[b5][k | kb] = a - b;
        }
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const float a = v[0][k], b = v[1][k];
    v[0][k] = a + b;
    v[1][k] = a - b;
  }
  // ... and dim bits 3, 4, 6 across lanes l ^ 8, l ^ 16, l ^ 32: with a and
  // b the values of the lanes with the bit clear and set, the first becomes
  // a + b and the second a - b, i.e. partner + sign * own with sign -1 where
  // the bit is set (one stage over all 16 values at a time, so that
  // independent exchanges are in flight)
  const float sg3 = (sub & 1) ? -1.f : 1.f, sg4 = (sub & 2) ? -1.f : 1.f, sg6 = (sub & 4) ? -1.f : 1.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    float& x = v[i >> 3][i & 7];
    x = fmaf(sg3, x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x128, 0xF, 0xF, false)));
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    float& x = v[i >> 3][i & 7];
    const auto s16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaf(sg4, __uint_as_float(s16[1]), __uint_as_float(s16[0]));
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    float& x = v[i >> 3][i & 7];
    const auto s32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaf(sg6, __uint_as_float(s32[1]), __uint_as_float(s32[0])) * INV_SQRT_128;
  }
  // FP4 blocks q = 2 b6 + b5: 8 of the block's 32 values here, the rest in
  // lanes l ^ 8, l ^ 16
  uint32_t code[2], sb = 0;
#pragma unroll
  for (int b5 = 0; b5 < 2; ++b5) {
    float m = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) m = fmaxf(m, fabsf(v[b5][k]));
    m = fmaxf(m, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(m), 0x128, 0xF, 0xF, false)));
    const auto s16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(m), __float_as_uint(m), false, false);
    m = fmaxf(__uint_as_float(s16[0]), __uint_as_float(s16[1]));
    const int e = VAR_FLOOR ? fp4_exponent_floor(m) : fp4_exponent(m);
    sb |= (uint32_t)(e + 127) << (8 * b5);
    const float scale = __uint_as_float((uint32_t)(e + 127) << 23);   // codes are RNE(z / 2^e)
    const float* x = v[b5];
    uint32_t d = 0;
    d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, x[0], x[1], scale, 0);
    d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, x[2], x[3], scale, 1);
    d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, x[4], x[5], scale, 2);
    d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, x[6], x[7], scale, 3);
    code[b5] = d;
  }
  // the scale bytes of blocks 2, 3 come from lane l ^ 32
  const auto ss = __builtin_amdgcn_permlane32_swap(sb, sb, false, false);
  const uint32_t sbytes = ss[0] | (ss[1] << 16);
  if (et < M) {
    // codes of dims 32 q + 8 (b3 + 2 b4) + k: bytes 16 q + 4 (b3 + 2 b4) + k / 2
    uint8_t* dst = p.q_fp4 + ((int64_t)et * p.H + head) * (HEAD_DIM / 2) + eoff / 2;
    *reinterpret_cast<uint32_t*>(dst) = code[0];
    *reinterpret_cast<uint32_t*>(dst + 16) = code[1];
    if (sub == 0) *reinterpret_cast<uint32_t*>(p.q_scales + ((int64_t)et * p.H + head) * 4) = sbytes;
  }
}

}  // namespace small
}  // namespace

#if IQP_SMALL_VARIANT == 0
// activation and weight row offsets are formed in 32 bits; the weight scales
// are read four at a time
bool indexer_q_small_supported(const IndexerQArgs& a) {
  return a.nkb == small::NKB && a.M >= 1 && a.M <= small::TILE * small::MAX_TILES && a.lda <= (1 << 24) &&
         a.ldw <= (1 << 22) && (reinterpret_cast<uintptr_t>(a.w_scales) & 3) == 0;
}

// workgroups per head and tile of the one-launch kernel: with a workspace,
// 3 from 12 to 32 tokens and 2 from 33 to 64 (at most 4 partial-sum sets a
// head, the workspace's), else 1. Measured on MI355X with an [M, 7168]
// quantization beside it, split against unsplit, weights hot in the
// Infinity Cache / cold in HBM: 8 tokens 7.3 / 8.7 against 6.7 / 8.9, 12
// tokens 7.5 / 8.7 against 7.3 / 9.5, 16 tokens 7.6 / 8.7 against 7.6 / 9.9,
// 24 tokens 7.9 / 8.8 against 8.6 / 10.8, 32 tokens 8.2 / 9.1 against
// 9.5 / 11.6, 48 tokens 8.7 against 9.6, 64 tokens 9.6 against 9.8 (hot);
// with one token the split's extra round trip costs 1.1 / 0.3 us. Hot
// weights would start the split at 17 tokens, cold ones at 8.
static int splitk_splits(const IndexerQArgs& a) {
  if (a.splitk_ws == nullptr || a.M < SPLITK_MIN_TOKENS || a.M > SPLITK_MAX_TOKENS) return 1;
  return a.M <= small::TILE ? 3 : 2;
}


hipError_t launch_indexer_q_small(const IndexerQArgs& a, hipStream_t stream) {
  const dim3 grid((unsigned)a.H, (unsigned)((a.M + small::TILE - 1) / small::TILE)), block(small::NTHREADS);
  hipLaunchKernelGGL(small::IQP_SMALL_KERNEL<false>, grid, block, 0, stream, a);
  return hipGetLastError();
}

// bf16 rows are addressed through 64-bit pointers (16-byte loads)
bool indexer_q_small_bf16_supported(const IndexerQArgs& a) {
  return a.nkb == small::NKB && a.M >= 1 && a.M <= small::TILE * small::MAX_TILES && a.x != nullptr &&
         (reinterpret_cast<uintptr_t>(a.x) & 15) == 0 && a.ldx % 8 == 0 && a.ldw <= (1 << 22) &&
         (reinterpret_cast<uintptr_t>(a.w_scales) & 3) == 0;
}

hipError_t launch_indexer_q_small_bf16(const IndexerQArgs& a, hipStream_t stream) {
  // extra grid rows for the quantization beside it: two words per wave
  const int64_t side_wgs = (a.side_words + 2 * small::NWAVES - 1) / (2 * small::NWAVES);
  const int64_t side_rows = (side_wgs + a.H - 1) / a.H;
  const int S = splitk_splits(a);
  const int64_t rows = S * ((a.M + small::TILE - 1) / small::TILE) + side_rows;
  if (rows > 65535) return hipErrorInvalidValue;
  const dim3 grid((unsigned)a.H, (unsigned)rows), block(small::NTHREADS);
  if (S == 3)
    hipLaunchKernelGGL((small::IQP_SMALL_KERNEL<true, false, 3>), grid, block, 0, stream, a);
  else if (S == 2)
    hipLaunchKernelGGL((small::IQP_SMALL_KERNEL<true, false, 2>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((small::IQP_SMALL_KERNEL<true, false, 1>), grid, block, 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_indexer_q_small_dump(const IndexerQArgs& a, hipStream_t stream) {
  const dim3 grid((unsigned)a.H, (unsigned)((a.M + small::TILE - 1) / small::TILE)), block(small::NTHREADS);
  if (a.x != nullptr)
    hipLaunchKernelGGL((small::IQP_SMALL_KERNEL<true, true>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((small::IQP_SMALL_KERNEL<false, true>), grid, block, 0, stream, a);
  return hipGetLastError();
}
#else
hipError_t IQP_SMALL_LAUNCH(const IndexerQArgs& a, hipStream_t stream) {
  const dim3 grid((unsigned)a.H, (unsigned)((a.M + small::TILE - 1) / small::TILE)), block(small::NTHREADS);
  hipLaunchKernelGGL(small::IQP_SMALL_KERNEL<false>, grid, block, 0, stream, a);
  return hipGetLastError();
}

hipError_t IQP_SMALL_LAUNCH_BF16(const IndexerQArgs& a, hipStream_t stream) {
  const dim3 grid((unsigned)a.H, (unsigned)((a.M + small::TILE - 1) / small::TILE)), block(small::NTHREADS);
  hipLaunchKernelGGL(small::IQP_SMALL_KERNEL<true>, grid, block, 0, stream, a);
  return hipGetLastError();
}
#endif

}  // namespace iqp
