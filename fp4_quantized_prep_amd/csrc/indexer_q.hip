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
#include <atomic>

#include "iq_common.h"

namespace iqp {
namespace {

// ---------------------------------------------------------------------------
// Main kernel. One workgroup of 4 waves (one per SIMD) owns a pair of heads
// (256 weight rows) and a contiguous range of tokens, which it walks in tiles
// of up to 256 tokens (8 sub-tiles of 32). Wave w computes head 2 pair + (w&1)
// for the sub-tiles s of the tile with s % 2 == w >> 1 (up to 4 of them), as
// 4 x NTM accumulators of 32 x 32 (up to 256 registers, the matrix-core
// accumulator file).
//
// Per 128-deep K block both operand tiles (W 256 x 128 B, A 256 x 128 B) and
// the tokens' scale words are copied global -> LDS by buffer loads that write
// LDS directly (no staging registers): one dwordx4 copy moves 8 full 128-byte
// rows, lane i writing bytes 16 i. Buffer bounds return zeros for rows past
// the last token or head. Row r's 16-byte chunks are stored XOR-swizzled
// (chunk c at slot c ^ ((r / 2) % 8)): a 128-byte row covers half of the 64
// LDS banks, rows 2i and 2i+1 the two halves, so the 16 lanes of one read
// cycle (16 consecutive rows, one chunk column) hit 64 distinct banks. Two
// stages double-buffer the K
// loop with one barrier per block, placed between the block's two 64-deep
// halves:
//
//   read (j, second half) -> MFMAs (j, first half) -> barrier -> copies of
//   block j+2 into j's stage, reads of (j+1, first half), MFMAs (j, second half)
//
// so every wave's MFMAs run on operands read one half-step earlier, and the
// copies are spread among the MFMAs instead of stalling them. The last block
// of a tile starts the copies of the next tile's first two blocks, which land
// while the epilogue runs.
#ifndef IQP_NWAVES
#define IQP_NWAVES 4
#endif
constexpr int NWAVES = IQP_NWAVES;
constexpr int TGROUPS = NWAVES / 2;                  // waves per head (token groups)
constexpr int NTHREADS = NWAVES * 64;
constexpr int TILE_ROWS = 256;                       // weight rows (2 heads) and most tokens per tile
constexpr int SUB = 32;                              // tokens per MFMA column tile
constexpr int MAX_SUB = TILE_ROWS / SUB;             // sub-tiles per tile
constexpr int MAX_TM = MAX_SUB / TGROUPS;            // sub-tiles per wave
constexpr int TM_STRIDE = SUB * TGROUPS;             // tokens between a wave's sub-tiles
constexpr int TILE_BYTES = TILE_ROWS * KB;           // one operand tile of one K block: 32 KiB
constexpr int SLAB = 1024;                           // bytes written by one wave-wide LDS copy
constexpr int COPIES = TILE_BYTES / SLAB / NWAVES;   // per operand per wave per block: 8
// LDS: W stages at [0, 64K), A stages at [64K, 128K), then two stages of the
// tile's 256 token scale words; every operand read is a lane base + immediate.
constexpr int W_OFF = 0;
constexpr int A_OFF = 2 * TILE_BYTES;
constexpr int S_OFF = 4 * TILE_BYTES;
constexpr int LDS_BYTES = S_OFF + 2 * TILE_ROWS * 4;

template <int NTM>
struct Frags {
  v8i a[NTM > 0 ? NTM : 1];
  v8i w[4];
};

struct Ctx {
  const IndexerQArgs& p;
  uint8_t* lds;
  int lane, half, wave, hn, th;
  int nkb;
  int head;
  uint32_t wsc_lane;   // weight-scale bytes 4 lane .. 4 lane + 3 of the head (K blocks)
  // per-row weight scales [H*128, nkb] (that variant only): the bytes of W row
  // 32 tn + lane % 32 of the head are at wsr_row + tn * wsr_tn_stride
  const uint8_t* wsr_row;
  int64_t wsr_tn_stride;
  rsrc_t rw, ra, rs;                 // weights of the pair; activations and scale words of the tile
  uint32_t vw, va, vs;               // this lane's byte offsets into them
  uint32_t rd_w[2][2], rd_a[2][2];   // LDS operand-read bases [kh][lo/hi]
  uint32_t rd_s;

  __device__ Ctx(const IndexerQArgs& p_, uint8_t* lds_, int pair) : p(p_), lds(lds_) {
    const int tid = threadIdx.x;
    lane = tid & 63;
    half = lane >> 5;
    wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    hn = wave & 1;
    th = wave >> 1;   // token group: sub-tiles s with s % TGROUPS == th
    nkb = p.nkb;
    head = 2 * pair + hn;
    const int head_c = head < p.H ? head : p.H - 1;   // odd H: the missing head reads zeros, never stored
    const uint8_t* wsc = p.w_scales + (int64_t)head_c * nkb;
    wsc_lane = 0;
    uint8_t wsc_b[4];
#pragma unroll
    for (int b = 0; b < 4; ++b)   // all four loads in flight before the first use
      wsc_b[b] = wsc[4 * lane + b < nkb ? 4 * lane + b : 0];
#pragma unroll
    for (int b = 0; b < 4; ++b)
      if (4 * lane + b < nkb) wsc_lane |= (uint32_t)wsc_b[b] << (8 * b);
    wsr_row = p.w_scales + ((int64_t)head_c * HEAD_DIM + (lane & 31)) * nkb;
    wsr_tn_stride = (int64_t)32 * nkb;
    // copy i of this wave lands in rows 8 (wave + 4 i) + lane / 8, slot lane % 8,
    // which holds the row's chunk (lane % 8) ^ ((row / 2) % 8); as the slab
    // index wave + 4 i has the parity of wave, that is the same for every copy
    const int chunk = (lane & 7) ^ ((4 * (wave & 1) + (lane >> 4)) & 7);
    const int64_t row0 = (int64_t)2 * pair * HEAD_DIM;
    const int64_t wrows = (int64_t)p.H * HEAD_DIM - row0;
    rw = make_rsrc(p.w + row0 * p.ldw, (uint64_t)(wrows < TILE_ROWS ? wrows : TILE_ROWS) * p.ldw);
    vw = (uint32_t)((8 * wave + (lane >> 3)) * p.ldw + 16 * chunk);
    va = (uint32_t)((8 * wave + (lane >> 3)) * p.lda + 16 * chunk);
    vs = (uint32_t)(4 * (64 * (wave & 3) + lane) * p.as_sm);   // with 8 waves, pairs copy the same words
    // operand reads: A row 64 tm + 32 th + lane % 32, W row 128 hn + 32 tn + lane % 32;
    // all row bases are multiples of 32, so the swizzle term (row / 2) % 8 is
    // (lane / 2) % 8
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const uint32_t col = 16 * ((4 * kh + 2 * half + e) ^ ((lane >> 1) & 7));
        rd_w[kh][e] = W_OFF + KB * (HEAD_DIM * hn + (lane & 31)) + col;
        rd_a[kh][e] = A_OFF + KB * (32 * th + (lane & 31)) + col;
      }
    rd_s = S_OFF + 4 * (32 * th + (lane & 31));
  }

  // buffers of the tile whose first token is tbase
  // (tbase = M: an empty range, every copy reads zeros)
  __device__ __forceinline__ void set_tile(int64_t tbase) {
    const int64_t rows = p.M - tbase;
    const int64_t nw = (nkb + 3) / 4;
    ra = make_rsrc(p.a + tbase * p.lda, rows > 0 ? (uint64_t)rows * p.lda : 0);
    rs = make_rsrc(p.a_scale_bytes + 4 * tbase * p.as_sm,
                   rows > 0 ? 4 * (uint64_t)((rows - 1) * p.as_sm + (nw - 1) * p.as_sw + 1) : 0);
  }

  // One of the 2 COPIES + 1 copies of K block j of the current tile into stage
  // ST: w < COPIES a W slab, w < 2 COPIES an A slab, else the scale words.
  // The whole offset goes in the lane offset, which the buffer bounds check
  // covers (the scalar offset is not checked): a row past the buffer's last
  // valid row starts at or beyond its size, so it reads zeros. The uniform
  // part passes through readfirstlane so it is formed here, not hoisted.
  template <int ST>
  __device__ __forceinline__ void copy(int w, int j) {
    if (w < COPIES) {
      const uint32_t u = __builtin_amdgcn_readfirstlane((int)(32 * w * p.ldw + KB * j));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void*)(lds + W_OFF + ST * TILE_BYTES + SLAB * (wave + NWAVES * w)),
                                               16, vw + u, 0, 0, 0);
    } else if (w < 2 * COPIES) {
      const int i = w - COPIES;
      const uint32_t u = __builtin_amdgcn_readfirstlane((int)(32 * i * p.lda + KB * j));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void*)(lds + A_OFF + ST * TILE_BYTES + SLAB * (wave + NWAVES * i)),
                                               16, va + u, 0, 0, 0);
    } else {
      const uint32_t u = __builtin_amdgcn_readfirstlane((int)(4 * (j >> 2) * p.as_sw));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(lds + S_OFF + ST * TILE_ROWS * 4 + 256 * (wave & 3)), 4,
                                               vs + u, 0, 0, 0);
    }
  }

  // 16 operand bytes of half kh, column e (lo / hi 16 bytes of the lane's 32)
  // of the A row 64 tm + 32 th + lane % 32 (rowoff = 64 tm) or the W row
  // 128 hn + 32 tn + lane % 32 (rowoff = 32 tn), in stage ST
  template <int ST>
  __device__ __forceinline__ v4u read16(bool is_a, int kh, int e, int rowoff) const {
    const uint32_t base = is_a ? rd_a[kh][e] : rd_w[kh][e];
    return *reinterpret_cast<const v4u*>(lds + base + ST * TILE_BYTES + KB * rowoff);
  }

  // packed scale word (K blocks 4 (j / 4) .. + 3) of sub-tile tm's token
  template <int ST>
  __device__ __forceinline__ int read_scale(int tm) const {
    return (int)*reinterpret_cast<const uint32_t*>(lds + rd_s + ST * TILE_ROWS * 4 + 4 * TM_STRIDE * tm);
  }
};

// One half-step of the K loop, scheduled by hand: slot s issues MFMA s of the
// 4 x NTM on the operands F (W tile tn = s / NTM, token tile tm = s % NTM),
// then its share of the copies and of the LDS reads that fill N, the operands
// of the next half-step. A scheduling fence closes every slot, so the order
// below is the issue order: no copy or read waits behind a run of MFMAs, and
// every MFMA's operands were read one half-step earlier.
//   RKH >= 0: read the 64-deep half RKH of the block in stage RST into N;
//   RSC: also the packed scale words of the block in stage RST into asn;
//   NBLK copy blocks: block jd + b into stage (DST + b) & 1.
//   ROW: the weight scale of MFMA tn is this lane's row's byte wsr[tn], not ws
template <int NTM, int RST, int RKH, bool RSC, int NBLK, int DST, bool ROW>
__device__ __forceinline__ void half_step(Ctx& c, v16f (&acc)[MAX_TM][4], const Frags<NTM>& F,
                                          const int (&as)[MAX_TM], int ws, const int (&wsr)[4], Frags<NTM>& N,
                                          int (&asn)[MAX_TM], int jr, int jd) {
  constexpr int NM = 4 * NTM;
  constexpr int NS = NM > 0 ? NM : 1;
  constexpr int NCOPY = NBLK * (2 * COPIES + 1);
  constexpr int NREAD = RKH >= 0 ? (RSC ? NTM : 0) + NTM + 4 : 0;   // scale words, then whole fragments
  // front-loaded: copies in the first half of the slots, reads in the first
  // three quarters, so both have landed by the waits that follow
  constexpr int NSC = NS / 2 > 0 ? NS / 2 : 1;
  constexpr int NSR = 3 * NS / 4 > 0 ? 3 * NS / 4 : 1;
  constexpr int NSCALE = RSC ? NTM : 0;
#pragma unroll
  for (int slot = 0; slot < NS; ++slot) {
    if (slot < NM) {
      const int tn = slot / (NTM > 0 ? NTM : 1), tm = slot % (NTM > 0 ? NTM : 1);
      acc[tm][tn] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(F.w[tn], F.a[tm], acc[tm][tn], 0, 0, 0,
                                                                    ROW ? wsr[tn] : ws, 0, as[tm]);
      asm volatile("" : "+a"(acc[tm][tn]));   // the MFMA stays in its slot (no sinking past this)
    }
#pragma unroll
    for (int k = NCOPY * slot / NSC; k < (slot < NSC ? NCOPY * (slot + 1) / NSC : 0); ++k) {
      const int b = k / (2 * COPIES + 1), w = k % (2 * COPIES + 1);
      if ((DST + b) & 1)
        c.copy<1>(w, jd + b);
      else
        c.copy<0>(w, jd + b);
    }
#pragma unroll
    for (int r = NREAD * slot / NSR; r < (slot < NSR ? NREAD * (slot + 1) / NSR : 0); ++r) {
      // a fragment is replaced whole: a partial update would keep the
      // previous one (the operands of the half-step before) alive
      if (r < NSCALE) {
        asn[r] = c.read_scale<RST>(r);
      } else if (r < NSCALE + NTM) {
        const int tm = r - NSCALE;
        N.a[tm] = make_v8i(c.read16<RST>(true, RKH, 0, TM_STRIDE * tm), c.read16<RST>(true, RKH, 1, TM_STRIDE * tm));
      } else {
        const int tn = r - NSCALE - NTM;
        N.w[tn] = make_v8i(c.read16<RST>(false, RKH, 0, 32 * tn), c.read16<RST>(false, RKH, 1, 32 * tn));
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

enum { MODE_STEADY, MODE_PENULT, MODE_LAST, MODE_ONLY };

// One K block j in stage ST: the first half's MFMAs (reading the second
// half), the block barrier, then the second half's MFMAs with the copies and
// reads the mode asks for. Block b of the next tile goes to stage b, copied
// as soon as that stage is free:
//   STEADY: copy block j+2 into stage ST, read block j+1's first half;
//   PENULT (last but one): switch the copy buffers to the next tile, copy its
//           block ST into stage ST, read block j+1's first half;
//   LAST:   copy the next tile's block ST into stage ST;
//   ONLY (a single K block): switch buffers, copy next blocks 0 and 1.
// LAST and ONLY fetch the RoPE rows of the epilogue's first sub-tile before
// the barrier.
// ROW (per-row weight scales): wsr holds block j's bytes on entry and block
// j+1's on exit, loaded here one block ahead so the barrier's wait covers them.
template <int NTM, int MODE, int ST, bool IL, bool ROW>
__device__ __forceinline__ void k_block(Ctx& c, int j, v16f (&acc)[MAX_TM][4], Frags<NTM>& f0, Frags<NTM>& f1,
                                        int (&as0)[MAX_TM], int (&as1)[MAX_TM], int64_t next_tbase,
                                        RopeCS& rope0, int64_t pos0, int (&wsr)[4]) {
  // a branch here would let the compiler sink the MFMAs out of their slots:
  // the block's weight-scale byte comes from a register, its activation
  // scale bytes from the words read one half-step earlier
  const int ws = (int)((uint32_t)__builtin_amdgcn_readlane((int)c.wsc_lane, j >> 2) >> (8 * (j & 3)));
  int as[MAX_TM];
#pragma unroll
  for (int tm = 0; tm < MAX_TM; ++tm) as[tm] = (int)((uint32_t)as0[tm] >> (8 * (j & 3)));
  if constexpr (MODE == MODE_LAST || MODE == MODE_ONLY) {
    if constexpr (NTM > 0) rope0 = load_rope<IL>(pos0, c.half, c.p);
  }
  constexpr bool PREFETCH = ROW && (MODE == MODE_STEADY || MODE == MODE_PENULT);
  int wsn[4] = {0, 0, 0, 0};
  if constexpr (PREFETCH) {
#pragma unroll
    for (int tn = 0; tn < 4; ++tn) wsn[tn] = c.wsr_row[tn * c.wsr_tn_stride + j + 1];
  }
  __builtin_amdgcn_sched_barrier(0);
  half_step<NTM, ST, 1, false, 0, 0, ROW>(c, acc, f0, as, ws, wsr, f1, as1, j, 0);
  __builtin_amdgcn_s_waitcnt(WAITCNT_LGKM0);
  // block j+1 must have landed, except after the last block: there only the
  // next tile's copies are in flight, and the next tile's start waits for them
  if constexpr (MODE == MODE_STEADY || MODE == MODE_PENULT) __builtin_amdgcn_s_waitcnt(WAITCNT_VM0);
  block_barrier();   // all of block j read by every wave (and block j+1 landed)
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (MODE == MODE_STEADY)
    half_step<NTM, ST ^ 1, 0, true, 1, ST, ROW>(c, acc, f1, as, ws, wsr, f0, as1, j + 1, j + 2);
  if constexpr (MODE == MODE_PENULT) {
    c.set_tile(next_tbase);
    half_step<NTM, ST ^ 1, 0, true, 1, ST, ROW>(c, acc, f1, as, ws, wsr, f0, as1, j + 1, ST);
  }
  if constexpr (MODE == MODE_LAST)
    half_step<NTM, 0, -1, false, 1, ST, ROW>(c, acc, f1, as, ws, wsr, f0, as1, 0, ST);
  if constexpr (MODE == MODE_ONLY) {
    c.set_tile(next_tbase);
    half_step<NTM, 0, -1, false, 2, 0, ROW>(c, acc, f1, as, ws, wsr, f0, as1, 0, 0);
  }
#pragma unroll
  for (int tm = 0; tm < MAX_TM; ++tm) as0[tm] = as1[tm];
  if constexpr (PREFETCH) {
#pragma unroll
    for (int tn = 0; tn < 4; ++tn) wsr[tn] = wsn[tn];
  }
}

// Shapes of the K loop: 1 block, 2 blocks, an even count >= 4, an odd count >= 3.
enum { SHAPE_ONE, SHAPE_TWO, SHAPE_EVEN, SHAPE_ODD };

// The K loop of one tile for a wave owning NTM sub-tiles, then its epilogue.
// On entry the copies of blocks 0 and 1 of this tile are in flight. Block j
// sits in stage j % 2 and the schedule for the block count's SHAPE is
// straight-line code around one loop: the accumulators never pass a branch.
// The last block always starts the copies of the next tile (past the
// workgroup's last tile they read zeros into stages nobody reads again).
template <int STAGE, int NTM, int SHAPE>
__device__ __forceinline__ void run_tile(Ctx& c, int64_t tbase, int64_t next_tbase) {
  v16f acc[MAX_TM][4];
#pragma unroll
  for (int tm = 0; tm < MAX_TM; ++tm)
#pragma unroll
    for (int tn = 0; tn < 4; ++tn)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[tm][tn][r] = 0.f;

  Frags<NTM> f0, f1;
  int as0[MAX_TM] = {}, as1[MAX_TM] = {};
  RopeCS rope;
  const int64_t t_lane = tbase + 32 * c.th + (c.lane & 31);   // token of sub-tile tm: t_lane + TM_STRIDE tm
  // the epilogue's positions, fetched now so its RoPE-row prefetches never
  // wait on a dependent load
  int64_t pos[MAX_TM > 0 ? MAX_TM : 1];
#pragma unroll
  for (int tm = 0; tm < NTM; ++tm) pos[tm] = load_position(t_lane + TM_STRIDE * tm, c.p);
  int wsr[4] = {0, 0, 0, 0};   // per-row weight scales of block 0 (that variant only)
  if constexpr (stage_row_scales(STAGE)) {
#pragma unroll
    for (int tn = 0; tn < 4; ++tn) wsr[tn] = c.wsr_row[tn * c.wsr_tn_stride];
  }
  __builtin_amdgcn_s_waitcnt(WAITCNT_VM0);
  block_barrier();
#pragma unroll
  for (int tm = 0; tm < NTM; ++tm) as0[tm] = c.read_scale<0>(tm);
#pragma unroll
  for (int tm = 0; tm < NTM; ++tm)
    f0.a[tm] = make_v8i(c.read16<0>(true, 0, 0, TM_STRIDE * tm), c.read16<0>(true, 0, 1, TM_STRIDE * tm));
#pragma unroll
  for (int tn = 0; tn < 4; ++tn)
    f0.w[tn] = make_v8i(c.read16<0>(false, 0, 0, 32 * tn), c.read16<0>(false, 0, 1, 32 * tn));
  // Block 0 is peeled (its MFMAs start from zero accumulators); blocks
  // 1, 2, ... run in (stage 1, stage 0) pairs while both are STEADY; the
  // remaining two or three blocks follow from the parity of the block count.
  const int nkb = c.nkb;
  const int64_t p0 = NTM > 0 ? pos[0] : 0;
  if constexpr (SHAPE == SHAPE_ONE) {
    k_block<NTM, MODE_ONLY, 0, stage_interleaved(STAGE), stage_row_scales(STAGE)>(c, 0, acc, f0, f1, as0, as1, next_tbase, rope, p0, wsr);
  } else if constexpr (SHAPE == SHAPE_TWO) {
    k_block<NTM, MODE_PENULT, 0, stage_interleaved(STAGE), stage_row_scales(STAGE)>(c, 0, acc, f0, f1, as0, as1, next_tbase, rope, 0, wsr);
    k_block<NTM, MODE_LAST, 1, stage_interleaved(STAGE), stage_row_scales(STAGE)>(c, 1, acc, f0, f1, as0, as1, next_tbase, rope, p0, wsr);
  } else {
    k_block<NTM, MODE_STEADY, 0, stage_interleaved(STAGE), stage_row_scales(STAGE)>(c, 0, acc, f0, f1, as0, as1, 0, rope, 0, wsr);
    int j = 1;
    for (; j + 3 < nkb; j += 2) {
      k_block<NTM, MODE_STEADY, 1, stage_interleaved(STAGE), stage_row_scales(STAGE)>(c, j, acc, f0, f1, as0, as1, 0, rope, 0, wsr);
      k_block<NTM, MODE_STEADY, 0, stage_interleaved(STAGE), stage_row_scales(STAGE)>(c, j + 1, acc, f0, f1, as0, as1, 0, rope, 0, wsr);
    }
    if constexpr (SHAPE == SHAPE_EVEN) {   // three left: j (stage 1), j+1, j+2
      k_block<NTM, MODE_STEADY, 1, stage_interleaved(STAGE), stage_row_scales(STAGE)>(c, j, acc, f0, f1, as0, as1, 0, rope, 0, wsr);
      k_block<NTM, MODE_PENULT, 0, stage_interleaved(STAGE), stage_row_scales(STAGE)>(c, j + 1, acc, f0, f1, as0, as1, next_tbase, rope, 0, wsr);
      k_block<NTM, MODE_LAST, 1, stage_interleaved(STAGE), stage_row_scales(STAGE)>(c, j + 2, acc, f0, f1, as0, as1, next_tbase, rope, p0, wsr);
    } else {                               // two left: j (stage 1), j+1
      k_block<NTM, MODE_PENULT, 1, stage_interleaved(STAGE), stage_row_scales(STAGE)>(c, j, acc, f0, f1, as0, as1, next_tbase, rope, 0, wsr);
      k_block<NTM, MODE_LAST, 0, stage_interleaved(STAGE), stage_row_scales(STAGE)>(c, j + 1, acc, f0, f1, as0, as1, next_tbase, rope, p0, wsr);
    }
  }

  // every MFMA of the tile completes here: none is sunk into the epilogue,
  // whose branches would then hold the operand registers live
#pragma unroll
  for (int tm = 0; tm < NTM; ++tm)
#pragma unroll
    for (int tn = 0; tn < 4; ++tn) asm volatile("" : "+a"(acc[tm][tn]));
  // one sub-tile's epilogue at a time keeps register use flat; the next
  // sub-tile's RoPE rows are fetched while this one computes
#pragma unroll
  for (int tm = 0; tm < NTM; ++tm) {
    __builtin_amdgcn_sched_barrier(0);
    RopeCS next;
    if (tm + 1 < NTM) next = load_rope<stage_interleaved(STAGE)>(pos[tm + 1], c.half, c.p);
    epilogue_tile<STAGE>(acc[tm], t_lane + TM_STRIDE * tm, c.head, c.head < c.p.H, c.half, c.p, rope);
    if (tm + 1 < NTM) rope = next;
  }
}

template <int STAGE, int SHAPE>
__device__ __forceinline__ void run_tiles(Ctx& c, int64_t s_begin, int64_t s_end) {
  for (int64_t s0 = s_begin; s0 < s_end; s0 += MAX_SUB) {
    const int nsub = (int)(s_end - s0 < MAX_SUB ? s_end - s0 : MAX_SUB);
    const int ntm = (nsub + TGROUPS - 1 - c.th) / TGROUPS;
    const int64_t tbase = SUB * s0;
    // past the chunk's last tile, an empty token range: its copies read zeros
    const int64_t next_tbase = s0 + MAX_SUB < s_end ? SUB * (s0 + MAX_SUB) : c.p.M;
    switch (ntm) {
      case 4: if constexpr (MAX_TM >= 4) run_tile<STAGE, 4, SHAPE>(c, tbase, next_tbase); break;
      case 3: if constexpr (MAX_TM >= 3) run_tile<STAGE, 3, SHAPE>(c, tbase, next_tbase); break;
      case 2: run_tile<STAGE, 2, SHAPE>(c, tbase, next_tbase); break;
      case 1: run_tile<STAGE, 1, SHAPE>(c, tbase, next_tbase); break;
      default: run_tile<STAGE, 0, SHAPE>(c, tbase, next_tbase); break;
    }
  }
}

template <int STAGE>
__global__ __launch_bounds__(NTHREADS, 1)
void indexer_q_kernel(IndexerQArgs p) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[LDS_BYTES];

  // ---- workgroup -> (head pair, token chunk). Consecutive workgroup ids go
  // to consecutive XCDs; when the pair count is a multiple of 8 each XCD
  // works on pairs/8 head pairs, whose weights then stay in its L2.
  const int bid = blockIdx.x;
  const int npairs = (p.H + 1) >> 1;
  const int cpp = p.chunks;
  int pair, chunk;
  if ((npairs & 7) == 0) {
    const int ppx = npairs >> 3;
    const int s = bid >> 3;
    pair = (bid & 7) * ppx + s % ppx;
    chunk = s / ppx;
  } else {
    pair = bid % npairs;
    chunk = bid / npairs;
  }
  // the chunk's sub-tiles [s_begin, s_end) of the ceil(M / 32) token sub-tiles
  const int64_t nsub_all = (p.M + SUB - 1) / SUB;
  const int64_t s_begin = nsub_all * chunk / cpp;
  const int64_t s_end = nsub_all * (chunk + 1) / cpp;
  if (s_begin >= s_end) return;   // uniform over the workgroup

  Ctx c(p, lds, pair);
  c.set_tile(SUB * s_begin);
  for (int w = 0; w < 2 * COPIES + 1; ++w) c.copy<0>(w, 0);
  for (int w = 0; w < 2 * COPIES + 1; ++w) c.copy<1>(w, 1);   // with a single K block stage 1 is never read
  if (c.nkb == 1)
    run_tiles<STAGE, SHAPE_ONE>(c, s_begin, s_end);
  else if (c.nkb == 2)
    run_tiles<STAGE, SHAPE_TWO>(c, s_begin, s_end);
  else if (c.nkb & 1)
    run_tiles<STAGE, SHAPE_ODD>(c, s_begin, s_end);
  else
    run_tiles<STAGE, SHAPE_EVEN>(c, s_begin, s_end);
  __builtin_amdgcn_s_waitcnt(WAITCNT_VM0);   // no LDS copy may outlive the workgroup
}

constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];

}  // namespace

int cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  int n = g_cu_count[dev].load(std::memory_order_acquire);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    g_cu_count[dev].store(n, std::memory_order_release);
  }
  return n;
}

namespace {

hipError_t launch_kernel(const IndexerQArgs& a_in, int stage, hipStream_t stream) {
  IndexerQArgs a = a_in;
  const int64_t npairs = (a.H + 1) / 2;
  const int64_t nsub_all = (a.M + SUB - 1) / SUB;
  // one workgroup per CU: each head pair gets CUs / pairs token chunks
  int64_t cpp = cu_count() / npairs;
  cpp = cpp < 1 ? 1 : cpp;
  cpp = cpp < nsub_all ? cpp : nsub_all;
  const int64_t blocks = npairs * cpp;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  a.chunks = (int32_t)cpp;
  const dim3 grid((unsigned)blocks), block(NTHREADS);
  switch (stage) {
    case -1: hipLaunchKernelGGL(indexer_q_kernel<-1>, grid, block, 0, stream, a); break;
    case 0: hipLaunchKernelGGL(indexer_q_kernel<0>, grid, block, 0, stream, a); break;
    case 1: hipLaunchKernelGGL(indexer_q_kernel<1>, grid, block, 0, stream, a); break;
    case 2: hipLaunchKernelGGL(indexer_q_kernel<2>, grid, block, 0, stream, a); break;
    case stage_of_variant(1): hipLaunchKernelGGL(indexer_q_kernel<stage_of_variant(1)>, grid, block, 0, stream, a); break;
    case stage_of_variant(2): hipLaunchKernelGGL(indexer_q_kernel<stage_of_variant(2)>, grid, block, 0, stream, a); break;
    case stage_of_variant(3): hipLaunchKernelGGL(indexer_q_kernel<stage_of_variant(3)>, grid, block, 0, stream, a); break;
    case stage_of_variant(4): hipLaunchKernelGGL(indexer_q_kernel<stage_of_variant(4)>, grid, block, 0, stream, a); break;
    case stage_of_variant(5): hipLaunchKernelGGL(indexer_q_kernel<stage_of_variant(5)>, grid, block, 0, stream, a); break;
    case stage_of_variant(6): hipLaunchKernelGGL(indexer_q_kernel<stage_of_variant(6)>, grid, block, 0, stream, a); break;
    case stage_of_variant(7): hipLaunchKernelGGL(indexer_q_kernel<stage_of_variant(7)>, grid, block, 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

// token count from which the fused FP4 call runs the split-role build of the
// pipelined kernel: right above the small-batch kernel's range (measured,
// byte-identical: 3-10 % faster than the one-role build from 384 to 1023
// tokens, which keeps the per-row weight-scale builds and tables beyond
// 2^31 positions)
constexpr int64_t SPLIT_MIN_TOKENS = 257;

// the pipelined kernel's launch arguments: one workgroup per CU, each head
// pair gets CUs / pairs chunks of whole 128-token tiles
static bool pipe_args(const IndexerQArgs& a_in, IndexerQArgs& a) {
  a = a_in;
  const int64_t npairs = (a.H + 1) / 2;
  const int64_t ntiles = (a.M + 127) / 128;
  int64_t cpp = cu_count() / npairs;
  cpp = cpp < 1 ? 1 : cpp;
  cpp = cpp < ntiles ? cpp : ntiles;
  if (npairs * cpp > 0x7FFFFFFF) return false;
  a.chunks = (int32_t)cpp;
  return true;
}

hipError_t launch_indexer_q_gemm_dump(const IndexerQArgs& a_in, hipStream_t stream) {
  if (indexer_q_small_supported(a_in)) return launch_indexer_q_small_dump(a_in, stream);
  if (indexer_q_pipe_supported(a_in)) {
    IndexerQArgs a;
    if (!pipe_args(a_in, a)) return hipErrorInvalidValue;
    if (a.M >= SPLIT_MIN_TOKENS && indexer_q_split_supported(a)) return launch_indexer_q_split_dump(a, stream);
    return launch_indexer_q_pipe_dump(a, stream);
  }
  return launch_kernel(a_in, 0, stream);
}

hipError_t launch_indexer_q_clock(const IndexerQArgs& a_in, int64_t stamp_capacity, int64_t* workgroups,
                                  hipStream_t stream) {
  *workgroups = 0;
  if (indexer_q_small_supported(a_in) || !indexer_q_pipe_supported(a_in)) return hipErrorNotSupported;
  IndexerQArgs a;
  if (!pipe_args(a_in, a)) return hipErrorInvalidValue;
  if (a.M < SPLIT_MIN_TOKENS || !indexer_q_split_supported(a)) return hipErrorNotSupported;
  *workgroups = (int64_t)((a.H + 1) / 2) * a.chunks;
  if (stamp_capacity < 4 * *workgroups) return hipErrorInvalidValue;
  return a.cos_sin_lanes ? launch_indexer_q_split_lanes_clock(a, stream) : launch_indexer_q_split_clock(a, stream);
}

hipError_t launch_indexer_q_small_bf16_variant(const IndexerQArgs& a, int variant, hipStream_t stream) {
  switch (variant) {
    case 0: return launch_indexer_q_small_bf16(a, stream);
    case 1: return launch_indexer_q_small_bf16_v1(a, stream);
    case 2: return launch_indexer_q_small_bf16_v2(a, stream);
    case 3: return launch_indexer_q_small_bf16_v3(a, stream);
    case 4: return launch_indexer_q_small_bf16_v4(a, stream);
    case 5: return launch_indexer_q_small_bf16_v5(a, stream);
    case 6: return launch_indexer_q_small_bf16_v6(a, stream);
    case 7: return launch_indexer_q_small_bf16_v7(a, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_indexer_q_variant(const IndexerQArgs& a_in, int variant, hipStream_t stream) {
  if (variant == 0) return launch_indexer_q(a_in, -1, stream);
  if (variant < 0 || variant > 7) return hipErrorInvalidValue;
  if (indexer_q_small_supported(a_in)) {
    switch (variant) {
      case 1: return launch_indexer_q_small_v1(a_in, stream);
      case 2: return launch_indexer_q_small_v2(a_in, stream);
      case 3: return launch_indexer_q_small_v3(a_in, stream);
      case 4: return launch_indexer_q_small_v4(a_in, stream);
      case 5: return launch_indexer_q_small_v5(a_in, stream);
      case 6: return launch_indexer_q_small_v6(a_in, stream);
      default: return launch_indexer_q_small_v7(a_in, stream);
    }
  }
  if (indexer_q_pipe_supported(a_in) &&
      (variant <= 3 || (reinterpret_cast<uintptr_t>(a_in.w_scales) & 3) == 0)) {
    IndexerQArgs a;
    if (!pipe_args(a_in, a)) return hipErrorInvalidValue;
    // the variants without per-row weight scales have split-role builds
    if (variant <= 3 && a.M >= SPLIT_MIN_TOKENS && indexer_q_split_supported(a)) {
      switch (variant) {
        case 1: return launch_indexer_q_split_v1(a, stream);
        case 2: return launch_indexer_q_split_v2(a, stream);
        default: return launch_indexer_q_split_v3(a, stream);
      }
    }
    switch (variant) {
      case 1: return launch_indexer_q_pipe_v1(a, stream);
      case 2: return launch_indexer_q_pipe_v2(a, stream);
      case 3: return launch_indexer_q_pipe_v3(a, stream);
      case 4: return launch_indexer_q_pipe_v4(a, stream);
      case 5: return launch_indexer_q_pipe_v5(a, stream);
      case 6: return launch_indexer_q_pipe_v6(a, stream);
      default: return launch_indexer_q_pipe_v7(a, stream);
    }
  }
  return launch_kernel(a_in, stage_of_variant(variant), stream);
}

hipError_t launch_indexer_q(const IndexerQArgs& a_in, int stage, hipStream_t stream) {
  if (stage == -1 && indexer_q_small_supported(a_in)) return launch_indexer_q_small(a_in, stream);
  if (stage == -1 && indexer_q_pipe_supported(a_in)) {
    IndexerQArgs a;
    if (!pipe_args(a_in, a)) return hipErrorInvalidValue;
    // from SPLIT_MIN_TOKENS on, the split-role build: its epilogue runs in
    // its own waves, which pays once most workgroups hold two tiles or more
    if (a.M >= SPLIT_MIN_TOKENS && indexer_q_split_supported(a))
      return a.cos_sin_lanes ? launch_indexer_q_split_lanes(a, stream) : launch_indexer_q_split(a, stream);
    return launch_indexer_q_pipe(a, stream);
  }
  return launch_kernel(a_in, stage, stream);
}

}  // namespace iqp
