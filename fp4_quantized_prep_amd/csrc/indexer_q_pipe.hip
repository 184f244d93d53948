// Pipelined variant of the fused indexer-Q kernel for K = 12 blocks of 128
// (the 1536-wide input of the indexer's Q projection): the same computation
// as indexer_q.hip (block-scaled FP8 GEMM on the matrix cores, RoPE,
// Hadamard-128, FP4 with UE8M0 scales, all in registers), scheduled so that
// the vector-ALU epilogue of one tile runs underneath the MFMAs of the next.
//
// TensorRT-LLM PR "Fuse DeepSeek-V4 Indexer Q projection with CuTe DSL",
// sequence diagram (one GEMM whose epilogue applies RoPE and writes packed FP4
// Q and scales); tokenspeed PR "perf(deepseek-v4): accelerate indexer Q and
// packed FP8 quantization", Summary (RoPE, the Hadamard transform and FP4
// quantization of Q).
//
// Why a second schedule. On gfx950 a wave that issues back-to-back MFMAs can
// still issue about eight independent VALU instructions per 64-cycle MFMA for
// free, but the epilogue (about 800 VALU instructions per 32-token sub-tile)
// otherwise runs alone after each tile's K loop and costs about a third of
// the kernel. Overlapping it needs two accumulator sets, so the tile shrinks:
//   * 4 waves (one per SIMD); a workgroup owns a head pair (256 weight rows)
//     and walks a contiguous range of 128-token tiles (4 sub-tiles of 32).
//     Wave w computes head 2 pair + (w & 1) for the sub-tiles s of the tile
//     with s % 2 == w >> 1: 2 sub-tiles, 128 accumulator registers (acc); the
//     previous tile's 128 (accp) are read by its epilogue meanwhile.
//   * The sets never swap roles: the epilogue has copied all of accp into
//     VGPRs by the middle of the next K loop, and the MFMAs of a tile's last
//     half-step write their sums into accp instead of acc. The tile loop is
//     one body with no accumulator moves.
//   * Three LDS stages of one 128-deep K block each (W 32 KiB + A 16 KiB + the
//     tokens' scale words), 146 KiB in all. The copies of block b (13 per wave,
//     bounds-checked buffer loads that write LDS directly) are split over the
//     half-step after block b-3 is consumed and the half-step after it, so
//     they have two blocks to land and never arrive as one burst; the block
//     sequence runs straight across tile boundaries, so the next tile's first
//     blocks stream in during the current tile's last ones. A copy costs one
//     scalar add (its LDS address) and the load itself: row offsets are
//     per-lane registers or per-slab scalars, the column within the K block
//     is the instruction offset (added to the LDS address as well).
//   * Each K block is two 64-deep half-steps with one barrier between them.
//     A half-step issues one MFMA per slot and, in the same slot, its share
//     of: the next half-step's LDS operand reads, the copies, and the
//     previous tile's epilogue. The epilogue is cut into 24 phases (12 per
//     sub-tile: loads from the accumulators, RoPE, seven butterfly stages,
//     scaling, block maxima and FP4 conversion, stores), one phase per
//     half-step of the 12-block loop.
//   * The last tile's epilogue runs alone after its K loop.
//   * The operand layout, scale handling, swizzle and epilogue arithmetic are
//     those of indexer_q.hip (shared through iq_common.h).
#include <type_traits>

#include "iq_common.h"

// Convention variant compiled into this translation unit (bit 0: interleaved
// RoPE pairs, bit 1: OCP floor-rule FP4 scales, bit 2: one weight scale per
// row and K block; 0: the defaults). The variant units define it and the
// launcher's name before including this file.
#ifndef IQP_PIPE_VARIANT
#define IQP_PIPE_VARIANT 0
#define IQP_PIPE_LAUNCH launch_indexer_q_pipe
#define IQP_PIPE_KERNEL indexer_q_pipe_kernel
#endif
// Split-role build (IQP_PIPE_SPLIT 1): eight waves, two per SIMD. The two
// accumulator sets of one schedule live in two waves instead of one: tile t
// is computed by wave group t % 2 (K loop: MFMAs and operand reads only)
// while the other group runs the epilogue of the tile it computed before and
// issues the weight and scale-word copies (the computing group issues the
// activation copies, which balances the two). Measured on gfx950: a wave's VALU and memory
// instructions cost a co-resident wave's MFMAs almost nothing, while the same
// instructions in the MFMA wave itself cost it issue cycles.
#ifndef IQP_PIPE_SPLIT
#define IQP_PIPE_SPLIT 0
#endif
// Diagnostic builds (default configuration only):
//   IQP_PIPE_DUMP 1: the same K loop, but each tile's float32 sums (Q before
//     RoPE) are written to args.dbg [M, H*128] and no epilogue runs;
//   IQP_PIPE_STAMP 1: the FP4 kernel unchanged, plus four 64-bit stamps per
//     workgroup in args.dbg: s_memtime (shader clock cycles) and
//     s_memrealtime (constant-rate counter) at its start and end.
#ifndef IQP_PIPE_DUMP
#define IQP_PIPE_DUMP 0
#endif
// Split build reading the RoPE rows from the table's lane-ordered copy
// (args.cos_sin_lanes, rope_table.hip): IQP_PIPE_LANES 1.
#ifndef IQP_PIPE_LANES
#define IQP_PIPE_LANES 0
#endif
#ifndef IQP_PIPE_STAMP
#define IQP_PIPE_STAMP 0
#endif

namespace iqp {
namespace {
namespace pipe {

constexpr bool VAR_IL = (IQP_PIPE_VARIANT & 1) != 0;
constexpr bool VAR_FLOOR = (IQP_PIPE_VARIANT & 2) != 0;
constexpr bool VAR_ROWS = (IQP_PIPE_VARIANT & 4) != 0;

constexpr bool SPLIT = IQP_PIPE_SPLIT != 0;
constexpr bool DUMP = IQP_PIPE_DUMP != 0;
constexpr bool STAMP = IQP_PIPE_STAMP != 0;
constexpr bool LANES = IQP_PIPE_LANES != 0;
static_assert(!LANES || (SPLIT && IQP_PIPE_VARIANT == 0 && !DUMP), "the lane-ordered table: split FP4 build only");
static_assert(IQP_PIPE_VARIANT == 0 || !(DUMP || STAMP), "diagnostic builds of the default configuration only");
constexpr int NWAVES = 4;                           // waves of one role (one per SIMD)
constexpr int NTHREADS = (SPLIT ? 2 : 1) * NWAVES * 64;
// the parts of a half-step a wave issues
enum Role { ROLE_ALL, ROLE_MFMA, ROLE_EPI };
constexpr int WROWS = 256;                          // weight rows: two heads
constexpr int TOKS = 128;                           // tokens per tile
constexpr int SUB = 32;                             // tokens per MFMA column tile
constexpr int MAX_SUB = TOKS / SUB;                 // 4 sub-tiles per tile
constexpr int MAX_TM = 2;                           // sub-tiles per wave
constexpr int TM_STRIDE = 64;                       // tokens between a wave's two sub-tiles
constexpr int NKB = 12;                             // K blocks (K = 1536)
constexpr int NST = 3;                              // LDS stages
constexpr int W_BYTES = WROWS * KB;                 // 32 KiB
constexpr int A_BYTES = TOKS * KB;                  // 16 KiB
constexpr int S_BYTES = TOKS * 4;                   // token scale words of one block
constexpr int SLAB = 1024;                          // one wave-wide LDS copy
constexpr int WCOPIES = W_BYTES / SLAB / NWAVES;    // 8
constexpr int ACOPIES = A_BYTES / SLAB / NWAVES;    // 4
constexpr int NCOPY = WCOPIES + ACOPIES + 1;        // 13 copies per wave per block
constexpr int PART1 = 7;                            // copies issued in the first half-step of a block's window
// scale words first: a copy's LDS address is given as (destination - its
// column offset in the K block), which must not go below zero
constexpr int S_OFF = 0;
constexpr int W_OFF = S_OFF + NST * S_BYTES;
constexpr int A_OFF = W_OFF + NST * W_BYTES;
// split build: the K-loop tile's token positions (int64), two tiles' worth
constexpr int P_OFF = A_OFF + NST * A_BYTES;
constexpr int P_BYTES = TOKS * 8;
constexpr int LDS_BYTES = P_OFF + (SPLIT ? 2 * P_BYTES : 0);   // 148,992 (split: 151,040)
static_assert(W_OFF >= KB * (NKB - 1), "copy LDS bases must stay non-negative");
// at a block barrier the copies of the block after next (13 per wave) may
// still be in flight: s_waitcnt vmcnt(13)
constexpr int WAITCNT_VM13 = (13 & 15) | (7 << 4) | (15 << 8) | ((13 >> 4) << 14);
// Split build: RoPE rows are fetched where no copy is waited for behind them
// (vmcnt counts in issue order, so a load queued behind copies lands only as
// late as they do): the first sub-tile's by the MFMA role right after its
// last barrier, the second's by the epilogue role at the start of block
// ROPE1_BLOCK (its first sub-tile's RoPE is done by then), ahead of that
// half-step's copies, whose barrier then leaves ROPE_LOADS more outstanding.
constexpr int ROPE1_BLOCK = 2;
// load_rope: 8 loads of 16 bytes; interleaved pairs, 16 of 8 bytes
constexpr int ROPE_LOADS = VAR_IL ? 16 : 8;
// s_waitcnt vmcnt(n), n < 64
constexpr int waitcnt_vm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }

// A lane value the compiler must treat as new at each use: addresses built
// from it are then computed where they are used instead of being hoisted out
// of the tile loop, where each would hold a register pair for the whole loop.
__device__ __forceinline__ int fresh(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// operands of one 64-deep half-step (a wave with NTM < 2 sub-tiles uses the first NTM)
template <int I, int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

struct Frags {
  v8i a[MAX_TM];
  v8i w[4];
};

// The previous tile's epilogue in flight: values of the sub-tile being
// processed, its FP4 dwords and scale bytes, the RoPE rows of the next one.
struct Epi {
  float v[4][16];
  uint32_t dw[4][2];
  uint32_t sbytes;
  RopeCS rope;      // RoPE rows of the sub-tile whose phase 0 comes next
  int tlane;        // the epilogue tile's token of sub-tile 0 (sub-tile tm: + TM_STRIDE tm)
  // positions as loaded (clamped into the table where the RoPE rows are
  // fetched, so no load is waited for before then); the split build keeps
  // pos1 only, clamped, and reads the K-loop tile's from LDS
  std::conditional_t<SPLIT, int32_t, int64_t> pos1;    // the epilogue tile's sub-tile 1
  std::conditional_t<SPLIT, int32_t, int64_t> npos0;   // the K-loop tile's (its epilogue comes next)
  int64_t npos1;
};

struct Ctx {
  const IndexerQArgs& p;
  uint8_t* lds;
  int lane, half, wave, hn, th, head;
  uint32_t wsc_lane;             // the head's weight-scale bytes, 4 per lane
  uint32_t wsr[4][3];            // per-row variant: the 12 bytes of W row 32 tn + lane % 32 of the head
  rsrc_t rw, ra, rs, ra_n, rs_n; // weights; activations / scale words of this and the next tile
  rsrc_t rw_n;                   // the weights for the next tile's copies (empty past the chunk's last tile)
  // Copy addressing. A copy's row part is a lane offset (bounds-checked:
  // rows past the tokens read zeros) or, for the weights, a scalar offset per
  // slab (rows that always exist); its column part within the K block is the
  // instruction offset, which the hardware adds to the LDS address as well.
  uint32_t vw;                   // weight lane offset (row within an 8-row slab, chunk)
  uint32_t va[SPLIT ? 1 : ACOPIES];   // activation lane offsets of the four slabs (split: slab 0, the
                                      // others a scalar stride on)
  uint32_t vs;                   // scale-word lane offset
  int wrow[WCOPIES];             // weight slab row offsets (bytes)
  int wave_lds;                  // 1 KiB per wave: this wave's part of each group of four slabs
  int words_lds;                 // 256 bytes per wave pair: its half of the scale words
  uint32_t rd_w[2][2], rd_a[2][2], rd_s;
  rsrc_t rp;                     // split build: the K-loop tile's positions
  int pos_lds;                   // split build: their LDS area (by tile parity)

  __device__ Ctx(const IndexerQArgs& p_, uint8_t* lds_, int pair) : p(p_), lds(lds_) {
    const int tid = threadIdx.x;
    lane = tid & 63;
    half = lane >> 5;
    wave = __builtin_amdgcn_readfirstlane(tid >> 6) & (NWAVES - 1);   // within its group
    hn = wave & 1;
    th = wave >> 1;
    head = 2 * pair + hn;
    const int head_c = head < p.H ? head : p.H - 1;   // odd H: the missing head reads zeros, never stored
    const uint8_t* wsc = p.w_scales + (int64_t)head_c * NKB;
    wsc_lane = 0;
    uint8_t wsc_b[4];
#pragma unroll
    for (int b = 0; b < 4; ++b)   // all four loads in flight before the first use
      wsc_b[b] = wsc[4 * lane + b < NKB ? 4 * lane + b : 0];
#pragma unroll
    for (int b = 0; b < 4; ++b)
      if (4 * lane + b < NKB) wsc_lane |= (uint32_t)wsc_b[b] << (8 * b);
    if constexpr (VAR_ROWS) {
      // [H*128, 12] bytes, 4-byte aligned (the launcher checks): three words a row
#pragma unroll
      for (int tn = 0; tn < 4; ++tn) {
        const uint32_t* row = reinterpret_cast<const uint32_t*>(
            p.w_scales + ((int64_t)head_c * HEAD_DIM + 32 * tn + (lane & 31)) * NKB);
#pragma unroll
        for (int k = 0; k < 3; ++k) wsr[tn][k] = row[k];
      }
    }
    const int64_t row0 = (int64_t)2 * pair * HEAD_DIM;
    const int64_t wrows = (int64_t)p.H * HEAD_DIM - row0;
    rw = make_rsrc(p.w + row0 * p.ldw, (uint64_t)(wrows < WROWS ? wrows : WROWS) * p.ldw);
    copy_offsets(lane);
    // slabs 4..7 hold the pair's second head; with an odd head count the last
    // pair has none and they re-read the first head's rows (never stored)
    const int hi = 2 * pair + 1 < p.H ? 128 * (int)p.ldw : 0;
#pragma unroll
    for (int w = 0; w < WCOPIES; ++w) wrow[w] = (w < 4 ? 0 : hi) + 32 * (w & 3) * (int)p.ldw;
    wave_lds = SLAB * wave;
    words_lds = 256 * (wave & 1);
    read_bases(lane);
  }

  // Lane offsets of the copies. copy i of this wave lands in rows 8 (wave +
  // 4 i) + lane / 8, slot lane % 8, which holds the row's chunk (lane % 8) ^
  // ((row / 2) % 8): the slab index wave + 4 i has the parity of wave, so that
  // is the same for every copy. (The split build re-forms them from a fresh
  // lane id at every epilogue role.)
  __device__ __forceinline__ void copy_offsets(int ln) {
    const int chunk = (ln & 7) ^ ((4 * (wave & 1) + (ln >> 4)) & 7);
    vw = (uint32_t)((8 * wave + (ln >> 3)) * p.ldw + 16 * chunk);
#pragma unroll
    for (int i = 0; i < (SPLIT ? 1 : ACOPIES); ++i)
      va[i] = (uint32_t)((8 * wave + (ln >> 3) + 32 * i) * p.lda + 16 * chunk);
    vs = (uint32_t)(4 * (64 * (wave & 1) + ln) * p.as_sm);   // waves w and w + 2 copy the same words
  }

  // LDS bases of the operand reads (the split build re-forms them at every
  // MFMA role); whole bases: the stage and row offsets fold into the reads'
  // offset field
  __device__ __forceinline__ void read_bases(int ln) {
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const uint32_t col = 16 * ((4 * kh + 2 * (ln >> 5) + e) ^ ((ln >> 1) & 7));
        rd_w[kh][e] = (uint32_t)fresh((int)(W_OFF + KB * (HEAD_DIM * hn + (ln & 31)) + col));
        rd_a[kh][e] = (uint32_t)fresh((int)(A_OFF + KB * (32 * th + (ln & 31)) + col));
      }
    rd_s = (uint32_t)fresh((int)(S_OFF + 4 * (32 * th + (ln & 31))));
  }

  __device__ __forceinline__ void buffers(int64_t tbase, rsrc_t& a, rsrc_t& s) const {
    const int64_t rows = p.M - tbase;
    constexpr int64_t nw = (NKB + 3) / 4;
    a = make_rsrc(p.a + tbase * p.lda, rows > 0 ? (uint64_t)rows * p.lda : 0);
    s = make_rsrc(p.a_scale_bytes + 4 * tbase * p.as_sm,
                  rows > 0 ? 4 * (uint64_t)((rows - 1) * p.as_sm + (nw - 1) * p.as_sw + 1) : 0);
  }

  // copy w (0..12) of K block j of this (NEXT: the next) tile into stage ST;
  // w < 8: a W slab, w < 12: an A slab, 12: the scale words. The whole offset
  // is in the lane offset, which the buffer bounds check covers.
  // Copy WI (0..12) of K block J of this (NEXT: the next) tile into stage ST;
  // WI < 8: a weight slab, < 12: an activation slab, 12: the scale words.
  // The LDS address is formed by a scalar add in an asm statement: one per
  // copy, at the copy (the compiler would otherwise keep all 39 per tile live).
  template <int C>
  __device__ __forceinline__ uint8_t* lds_at(int base) const {
    int m;
    asm volatile("s_add_u32 %0, %1, %2" : "=s"(m) : "s"(base), "i"(C) : "scc");
    return lds + m;
  }

  template <int ST, bool NEXT, int WI, int J>
  __device__ __forceinline__ void copy() const {
    if constexpr (WI < WCOPIES) {
      uint8_t* d = lds_at<W_OFF + ST * W_BYTES + SLAB * NWAVES * WI - KB * J>(wave_lds);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(NEXT ? rw_n : rw, (lds_void*)d, 16, vw, wrow[WI], KB * J, 0);
    } else if constexpr (WI < WCOPIES + ACOPIES) {
      constexpr int i = WI - WCOPIES;
      uint8_t* d = lds_at<A_OFF + ST * A_BYTES + SLAB * NWAVES * i - KB * J>(wave_lds);
      const uint32_t vo = SPLIT ? va[0] + (uint32_t)(32 * i) * (uint32_t)p.lda : va[SPLIT ? 0 : i];
      __builtin_amdgcn_raw_ptr_buffer_load_lds(NEXT ? ra_n : ra, (lds_void*)d, 16, vo, 0, KB * J, 0);
    } else {
      // the word offset stays in the lane offset, under the bounds check
      const uint32_t u = (uint32_t)(4 * (J >> 2) * (int)p.as_sw);
      uint8_t* d = lds_at<S_OFF + ST * S_BYTES>(words_lds);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(NEXT ? rs_n : rs, (lds_void*)d, 4, vs + u, 0, 0, 0);
    }
  }

  template <int ST>
  __device__ __forceinline__ v4u read16(bool is_a, int kh, int e, int rowoff) const {
    const uint32_t base = is_a ? rd_a[kh][e] + ST * A_BYTES : rd_w[kh][e] + ST * W_BYTES;
    return *reinterpret_cast<const v4u*>(lds + base + KB * rowoff);
  }

  template <int ST>
  __device__ __forceinline__ int read_scale(int tm) const {
    return (int)*reinterpret_cast<const uint32_t*>(lds + rd_s + ST * S_BYTES + 4 * TM_STRIDE * tm);
  }
};

// ---------------------------------------------------------------------------
// The epilogue of one sub-tile as 12 phases of items that run in order. Phase
// 0: the 64 dims past the RoPE slice out of the accumulators, then their
// butterfly stage r-bit 0; 1: RoPE pairs (reading the accumulators), then
// their r-bit 0; 2-4: r-bits 1-3; 5, 6: tn bits 0, 1; 7, 8: the cross-half
// stage (v_permlane32_swap); 9: the 1/sqrt(128) scaling; 10, 11: block maxima,
// exponents and FP4 conversion, 10 of dims 0-63 and 11 of dims 64-127. Once
// dims 0-63 are converted, the RoPE rows of the next sub-tile are fetched
// into their registers' worth of room, four loads in each of phases 10 and
// 11 (the copies keep the memory pipeline busy, so loads come a few at a
// time); 11 ends with the stores.
constexpr int phase_items(int h) {
  return h == 0 ? 48 : h == 1 ? 32 : h <= 6 ? 32 : h <= 8 ? 16 : h == 9 ? 64 : h == 10 ? 6 : 7;
}

// index of the k-th r in 0..15 with bit rb clear
__device__ __forceinline__ constexpr int r_clear(int k, int rb) { return (k & (rb - 1)) | ((k & ~(rb - 1)) << 1); }

// load L (0..7) of the RoPE rows of position pos: cosines (even L) or sines
// of angle group L / 2, this lane's half of it
// (interleaved: group j is table entries 8j + 2half + {0, 1, 4, 5}, the
// layout load_rope<true> gives)
__device__ __forceinline__ void rope_part(Epi& es, int64_t pos, int L, const Ctx& c) {
  pos = pos < 0 ? 0 : (pos >= c.p.max_pos ? c.p.max_pos - 1 : pos);
  if constexpr (!VAR_IL) {
    const float* cs = c.p.cos_sin + pos * 64 + 8 * (L >> 1) + 4 * fresh(c.half);
    if (L & 1)
      es.rope.s[L >> 1] = *reinterpret_cast<const v4f*>(cs + 32);
    else
      es.rope.c[L >> 1] = *reinterpret_cast<const v4f*>(cs);
  } else {
    typedef float v2f __attribute__((ext_vector_type(2)));
    const float* cs = c.p.cos_sin + pos * 64 + 8 * (L >> 1) + 2 * fresh(c.half) + ((L & 1) ? 32 : 0);
    const v2f lo = *reinterpret_cast<const v2f*>(cs), hi = *reinterpret_cast<const v2f*>(cs + 4);
    const v4f r = v4f{lo[0], lo[1], hi[0], hi[1]};
    if (L & 1)
      es.rope.s[L >> 1] = r;
    else
      es.rope.c[L >> 1] = r;
  }
}

// LAST: no tile follows (the sub-tile after the last one has no RoPE rows to fetch)
template <int H, int NTMP, bool LAST>
__device__ __forceinline__ void epi_item(Epi& es, v16f (&accp)[MAX_TM][4], int i, const Ctx& c) {
  constexpr int tm = H / 12, h = H % 12;
  if constexpr (tm >= NTMP) {
    return;
  } else if constexpr (h == 0) {
    // The accumulators are named in AGPRs right where the phase starts reading
    // them: copies into VGPRs cannot be placed any earlier (a whole set
    // copied out at the top of the K loop would not fit beside its operands).
    if (i == 0) asm volatile("" : "+a"(accp[tm][2]), "+a"(accp[tm][3]));
    if (i < 32) {
      es.v[2 + (i >> 4)][i & 15] = accp[tm][2 + (i >> 4)][i & 15];
    } else {
      const int k = i - 32, tn = 2 + (k >> 3), r = r_clear(k & 7, 1);
      const float a = es.v[tn][r], b = es.v[tn][r | 1];
      es.v[tn][r] = a + b;
      es.v[tn][r | 1] = a - b;
    }
  } else if constexpr (h == 1) {
    if (i == 0) asm volatile("" : "+a"(accp[tm][0]), "+a"(accp[tm][1]));
    if (i < 16 && !VAR_IL) {       // RoPE pair (i, i + 32), i = 8 g + 4 half + s
      const int g = i >> 2, s = i & 3;
      const float x = accp[tm][0][4 * g + s], y = accp[tm][1][4 * g + s];
      // split build, second sub-tile: its rows sit in the first sub-tile's
      // accumulators 0 (cosines) and 1 (sines)
      const float cc = (SPLIT && tm == 1) ? accp[0][0][4 * g + s] : es.rope.c[g][s];
      const float ss = (SPLIT && tm == 1) ? accp[0][1][4 * g + s] : es.rope.s[g][s];
      es.v[0][4 * g + s] = x * cc - y * ss;
      es.v[1][4 * g + s] = y * cc + x * ss;
    } else if (i < 16) {           // interleaved pair 16 tn + 4 g + 2 half + k: registers 4g + 2k, 4g + 2k + 1
      const int tn = i >> 3, g = (i >> 1) & 3, k = i & 1, r = 4 * g + 2 * k;
      const float x = accp[tm][tn][r], y = accp[tm][tn][r + 1];
      const int cj = 2 * tn + (g >> 1), ce = 2 * (g & 1) + k;   // entry ce of group cj
      const float cc = (SPLIT && tm == 1) ? accp[0][0][4 * cj + ce] : es.rope.c[cj][ce];
      const float ss = (SPLIT && tm == 1) ? accp[0][1][4 * cj + ce] : es.rope.s[cj][ce];
      es.v[tn][r] = x * cc - y * ss;
      es.v[tn][r + 1] = y * cc + x * ss;
    } else {
      const int k = i - 16, tn = k >> 3, r = r_clear(k & 7, 1);
      const float a = es.v[tn][r], b = es.v[tn][r | 1];
      es.v[tn][r] = a + b;
      es.v[tn][r | 1] = a - b;
    }
  } else if constexpr (h <= 4) {   // r bits 1..3
    constexpr int rb = 1 << (h - 1);
    const int tn = i >> 3, r = r_clear(i & 7, rb);
    const float a = es.v[tn][r], b = es.v[tn][r | rb];
    es.v[tn][r] = a + b;
    es.v[tn][r | rb] = a - b;
  } else if constexpr (h <= 6) {   // tn bits 0, 1
    constexpr int tb = 1 << (h - 5);
    const int tnp = i >> 4, r = i & 15;
    const int tn = (tnp & (tb - 1)) | ((tnp & ~(tb - 1)) << 1);
    const float a = es.v[tn][r], b = es.v[tn | tb][r];
    es.v[tn][r] = a + b;
    es.v[tn | tb][r] = a - b;
  } else if constexpr (h <= 8) {   // dim bit 2, across the lane halves (see epilogue_tile)
    const int k = (h - 7) * 16 + i, tn = k >> 3, r = r_clear(k & 7, 4);
    float r0, r1;
    swap32(es.v[tn][r], es.v[tn][r | 4], r0, r1);
    if constexpr (SPLIT) {
      // the 1/sqrt(128) scaling folded in: (r0 +- r1) / sqrt(128)
      const float t = r1 * INV_SQRT_128;
      es.v[tn][r] = __builtin_fmaf(r0, INV_SQRT_128, t);
      es.v[tn][r | 4] = __builtin_fmaf(r0, INV_SQRT_128, -t);
    } else {
      es.v[tn][r] = r0 + r1;
      es.v[tn][r | 4] = r0 - r1;
    }
  } else if constexpr (h == 9) {
    if constexpr (!SPLIT) es.v[i >> 4][i & 15] *= INV_SQRT_128;
  } else {
    // item roles: phase 10: 0, 1 convert dims 0-63 (block tn = item), 2-5 RoPE
    // loads 0-3; phase 11: 0-3 RoPE loads 4-7, 4, 5 convert dims 64-127, 6 stores
    const int load = h == 10 ? i - 2 : i + 4;
    if ((h == 10 && i >= 2) || (h == 11 && i < 4)) {
      // RoPE rows of the next sub-tile: this tile's second, or the next tile's first
      if (tm == 0 && !SPLIT)
        rope_part(es, es.pos1, load, c);
      else if (tm != 0 && !LAST)
        rope_part(es, es.npos0, load, c);
      return;
    }
    if (h == 11 && i == 6) {       // assemble and store (dword (tn, r3) at 4 tn + 2 r3 + half)
      const int64_t t = (int64_t)es.tlane + TM_STRIDE * tm;
      uint32_t out[8];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int tn = q >> 1, r3 = q & 1;
        uint32_t r1;
        const uint32_t r0 = swap32_u(es.dw[tn][r3], es.dw[tn + 2][r3], r1);
        out[2 * q] = r0;
        out[2 * q + 1] = r1;
      }
      if (c.head < c.p.H && t < c.p.M) {
        const int half = fresh(c.half);
        uint8_t* dst = c.p.q_fp4 + (t * c.p.H + c.head) * (HEAD_DIM / 2) + 32 * half;
        *reinterpret_cast<v4u*>(dst) = v4u{out[0], out[1], out[2], out[3]};
        *reinterpret_cast<v4u*>(dst + 16) = v4u{out[4], out[5], out[6], out[7]};
        if (half == 0) *reinterpret_cast<uint32_t*>(c.p.q_scales + (t * c.p.H + c.head) * 4) = es.sbytes;
      }
      return;
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) {  // FP4 block tn over dims 32 tn .. 32 tn + 31 (16 here, 16 in the partner lane)
      const int tn = 2 * (h - 10) + q;
      if (q != (h == 11 ? i - 4 : i)) continue;
      float m = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) m = fmaxf(m, fabsf(es.v[tn][r]));
      float m0, m1;
      swap32(m, m, m0, m1);
      const int e = VAR_FLOOR ? fp4_exponent_floor(fmaxf(m0, m1)) : fp4_exponent(fmaxf(m0, m1));
      if (tn == 0) es.sbytes = 0;
      es.sbytes |= (uint32_t)(e + 127) << (8 * tn);
      const float scale = __uint_as_float((uint32_t)(e + 127) << 23);
#pragma unroll
      for (int r3 = 0; r3 < 2; ++r3) {
        const float* x = &es.v[tn][8 * r3];
        uint32_t d = 0;
        d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, x[0], x[1], scale, 0);
        d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, x[2], x[3], scale, 1);
        d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, x[4], x[5], scale, 2);
        d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, x[6], x[7], scale, 3);
        es.dw[tn][r3] = d;
      }
    }
  }
}

// slot s of NS runs items [n s / NS, n (s + 1) / NS) of epilogue half-step H
// (LAST: no tile's rows follow this one's in the same wave)
template <int H, int NTMP, int NS, bool LAST = false>
__device__ __forceinline__ void epi_slot(Epi& es, v16f (&accp)[MAX_TM][4], int slot, const Ctx& c) {
  if constexpr (H < 24 && NTMP > 0) {
    constexpr int n = phase_items(H % 12);
#pragma unroll
    for (int i = n * slot / NS; i < n * (slot + 1) / NS; ++i) epi_item<H, NTMP, LAST>(es, accp, i, c);
  }
}

// Split build: the epilogue of a tile (both sub-tiles' 24 phases, in order)
// is cut into 24 pieces of about equal cost, one per half-step, by a
// compile-time estimate of each item's instructions; only the cut points
// move, so the items keep their order. (In one wave the phase cut of
// phase_items is fine: there the MFMAs set the pace.)
constexpr int UNITS_SUB = 349;   // items of one sub-tile's 12 phases
static_assert(UNITS_SUB == 48 + 32 + 5 * 32 + 2 * 16 + 64 + 6 + 7, "phase_items");
constexpr int unit_phase(int k) {
  int h = 0;
  while (k >= phase_items(h)) k -= phase_items(h++);
  return h;
}
constexpr int unit_item(int k) {
  int h = 0;
  while (k >= phase_items(h)) k -= phase_items(h++);
  return k;
}
// instructions of item i of phase h of sub-tile tm (the split build's roles:
// no RoPE rows fetched in phases 10, 11)
constexpr int unit_cost(int tm, int h, int i) {
  if (h == 0) return i < 32 ? 1 : 2;
  if (h == 1) return i < 16 ? 6 : 2;
  if (h <= 6) return 2;
  if (h <= 8) return 4;
  if (h == 9) return 0;
  if (h == 10) return i < 2 ? 31 : 0;
  return i < 4 ? 0 : (i < 6 ? 31 : 13);
}
constexpr int unit_cost_flat(int u) { return unit_cost(u / UNITS_SUB, unit_phase(u % UNITS_SUB), unit_item(u % UNITS_SUB)); }
constexpr int cost_before(int u) {
  int c = 0;
  for (int k = 0; k < u; ++k) c += unit_cost_flat(k);
  return c;
}
constexpr int TOTAL_COST = cost_before(2 * UNITS_SUB);
// first unit of half-step H: the first whose cost starts at or after H / 24 of the total
constexpr int unit_begin(int H) {
  int u = 0, c = 0;
  while (u < 2 * UNITS_SUB && c < (int64_t)TOTAL_COST * H / 24) c += unit_cost_flat(u++);
  return u;
}

template <int U>
__device__ __forceinline__ void epi_unit(Epi& es, v16f (&accp)[MAX_TM][4], const Ctx& c) {
  constexpr int tm = U / UNITS_SUB, k = U % UNITS_SUB;
  constexpr int item = unit_item(k);   // a constant before any pass looks at the indexing
  epi_item<12 * tm + unit_phase(k), MAX_TM, true>(es, accp, item, c);
}

// slot s of NS runs units [b + (e - b) s / NS, b + (e - b) (s + 1) / NS) of half-step H's share
template <int H, int NS, int SLOT>
__device__ __forceinline__ void epi_slot_even(Epi& es, v16f (&accp)[MAX_TM][4], const Ctx& c) {
  constexpr int b = unit_begin(H), e = unit_begin(H + 1);
  static_for<b + (e - b) * SLOT / NS, b + (e - b) * (SLOT + 1) / NS>([&](auto uc) __attribute__((always_inline)) {
    epi_unit<decltype(uc)::value>(es, accp, c);
  });
}

// split build: the RoPE rows of a position clamped into the table, from the
// table or (LANES) its lane-ordered copy, where load L of position p, half h
// sits at float 2048 (p / 32) + 256 L + 4 (2 (p % 32) + h): for a sub-tile of
// consecutive positions each load reads one 1 KiB segment instead of 32 rows
__device__ __forceinline__ RopeCS rope_rows(int pos, const Ctx& c) {
  if constexpr (LANES) {
    const float* tl = c.p.cos_sin_lanes + (int64_t)(pos >> 5) * 2048 + 4 * (2 * (pos & 31) + c.half);
    RopeCS r;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      r.c[g] = *reinterpret_cast<const v4f*>(tl + 256 * (2 * g));
      r.s[g] = *reinterpret_cast<const v4f*>(tl + 256 * (2 * g + 1));
    }
    return r;
  } else {
    return load_rope<VAR_IL>(pos, c.half, c.p);
  }
}

// split build: the second sub-tile's RoPE rows into the first sub-tile's
// accumulators 0 (cosines) and 1 (sines), whose values its RoPE has used
__device__ __forceinline__ void rope_into_acc(const RopeCS& r, v16f (&accp)[MAX_TM][4]) {
#pragma unroll
  for (int g = 0; g < 4; ++g)
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      accp[0][0][4 * g + s] = r.c[g][s];
      accp[0][1][4 * g + s] = r.s[g][s];
    }
}

// the whole epilogue of a tile, alone (after the chunk's last K loop)
template <int NTMP>
__device__ __forceinline__ void epilogue_alone(Epi& es, v16f (&accp)[MAX_TM][4], const Ctx& c) {
  auto run = [&](auto hc) __attribute__((always_inline)) {
    constexpr int H = decltype(hc)::value;
    constexpr int n = phase_items(H % 12);
#pragma unroll
    for (int i = 0; i < n; ++i) epi_item<H, NTMP, true>(es, accp, i, c);
  };
#define IQP_EPI_H(H) run(std::integral_constant<int, H>{});
  IQP_EPI_H(0) IQP_EPI_H(1)
  // split build: the second sub-tile's RoPE rows (no copies in flight here)
  if constexpr (SPLIT && NTMP > 1) {
    rope_into_acc(rope_rows(es.pos1, c), accp);
    asm volatile("" : "+a"(accp[0][0]), "+a"(accp[0][1]));
  }
  IQP_EPI_H(2) IQP_EPI_H(3) IQP_EPI_H(4) IQP_EPI_H(5)
  IQP_EPI_H(6) IQP_EPI_H(7) IQP_EPI_H(8) IQP_EPI_H(9) IQP_EPI_H(10) IQP_EPI_H(11)
  IQP_EPI_H(12) IQP_EPI_H(13) IQP_EPI_H(14) IQP_EPI_H(15) IQP_EPI_H(16) IQP_EPI_H(17)
  IQP_EPI_H(18) IQP_EPI_H(19) IQP_EPI_H(20) IQP_EPI_H(21) IQP_EPI_H(22) IQP_EPI_H(23)
#undef IQP_EPI_H
}

// Split build, the chunk's last tile: no K loop runs under its epilogue, and
// the other group's waves are idle, so the wave that computed the tile runs
// the first sub-tile's epilogue and hands the second sub-tile's sums to the
// other group's wave on its SIMD (same head and tokens) through LDS, 16 KiB a
// wave: group-major 16-byte pieces, piece q = 4 tn + g of lane l at 1 KiB q +
// 16 l. The areas are weight stage 0 (waves 0, 1) and activation stages 0
// and 2 (waves 2, 3): the copies into them were those of blocks 11 and 12,
// landed by the tile's last barrier, and no later copy goes there (the
// chunk's last copies, zero-byte reads past it, fill weight stages 1 and 2
// and activation stage 1, and may still be in flight). One barrier, which
// both groups take, separates the writes from the reads.
__device__ __forceinline__ uint8_t* handoff_at(const Ctx& c) {
  const int off = c.wave < 2 ? W_OFF + 16384 * c.wave : A_OFF + 2 * A_BYTES * (c.wave - 2);
  return c.lds + off + 16 * fresh(c.lane);
}
static_assert(NST == 3 && W_BYTES >= 2 * 16384 && A_BYTES == 16384, "the hand-over areas");

template <int NTMP>
__device__ __forceinline__ void epilogue_owner(Epi& es, v16f (&accp)[MAX_TM][4], const Ctx& c) {
  static_assert(SPLIT && NTMP == 2, "the split build's two sub-tiles");
  {
    uint8_t* const b = handoff_at(c);
#pragma unroll
    for (int tn = 0; tn < 4; ++tn)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<v4f*>(b + 1024 * (4 * tn + g)) =
            v4f{accp[1][tn][4 * g], accp[1][tn][4 * g + 1], accp[1][tn][4 * g + 2], accp[1][tn][4 * g + 3]};
  }
  __builtin_amdgcn_s_waitcnt(WAITCNT_LGKM0);
  block_barrier();   // the second sub-tile's sums are in LDS
  es.rope = rope_rows(es.npos0, c);
  auto run = [&](auto hc) __attribute__((always_inline)) {
    constexpr int H = decltype(hc)::value;
    constexpr int n = phase_items(H % 12);
#pragma unroll
    for (int i = 0; i < n; ++i) epi_item<H, NTMP, true>(es, accp, i, c);
  };
#define IQP_EPI_H(H) run(std::integral_constant<int, H>{});
  IQP_EPI_H(0) IQP_EPI_H(1) IQP_EPI_H(2) IQP_EPI_H(3) IQP_EPI_H(4) IQP_EPI_H(5)
  IQP_EPI_H(6) IQP_EPI_H(7) IQP_EPI_H(8) IQP_EPI_H(9) IQP_EPI_H(10) IQP_EPI_H(11)
#undef IQP_EPI_H
}

// the other group's wave: the second sub-tile of the chunk's last tile (tile
// `last`, whose positions are still in LDS), from the sums handed over
template <int NTMP>
__device__ __forceinline__ void epilogue_helper(Epi& es, v16f (&accp)[MAX_TM][4], const Ctx& c, int64_t last) {
  static_assert(SPLIT && NTMP == 2, "the split build's two sub-tiles");
  const int64_t tbase = TOKS * last;
  es.tlane = (int)(tbase + 32 * c.th + (fresh(c.lane) & 31));
  {
    const int64_t* pl = reinterpret_cast<const int64_t*>(c.lds + P_OFF + P_BYTES * (int)(last & 1)) + 32 * c.th +
                        (fresh(c.lane) & 31);
    const int64_t v = pl[TM_STRIDE];
    es.pos1 = (int32_t)(v < 0 ? 0 : (v >= c.p.max_pos ? c.p.max_pos - 1 : v));
  }
  // its RoPE rows into the first sub-tile's accumulators 0 and 1, where the
  // second sub-tile's RoPE reads them
  rope_into_acc(rope_rows(es.pos1, c), accp);
  block_barrier();   // the owner's sums are in LDS
  {
    const uint8_t* const b = handoff_at(c);
#pragma unroll
    for (int tn = 0; tn < 4; ++tn)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const v4f x = *reinterpret_cast<const v4f*>(b + 1024 * (4 * tn + g));
#pragma unroll
        for (int q = 0; q < 4; ++q) accp[1][tn][4 * g + q] = x[q];
      }
  }
  asm volatile("" : "+a"(accp[0][0]), "+a"(accp[0][1]));
  auto run = [&](auto hc) __attribute__((always_inline)) {
    constexpr int H = decltype(hc)::value;
    constexpr int n = phase_items(H % 12);
#pragma unroll
    for (int i = 0; i < n; ++i) epi_item<H, NTMP, true>(es, accp, i, c);
  };
#define IQP_EPI_H(H) run(std::integral_constant<int, H>{});
  IQP_EPI_H(12) IQP_EPI_H(13) IQP_EPI_H(14) IQP_EPI_H(15) IQP_EPI_H(16) IQP_EPI_H(17)
  IQP_EPI_H(18) IQP_EPI_H(19) IQP_EPI_H(20) IQP_EPI_H(21) IQP_EPI_H(22) IQP_EPI_H(23)
#undef IQP_EPI_H
}

// ---------------------------------------------------------------------------
// One half-step: slot s issues MFMA s of 4 NTM on the operands F, then its
// share of the LDS reads filling N (the next half-step's operands), of the
// copies (COPY_LO .. COPY_HI of K block JD of this or the NEXT tile into stage
// DST) and of epilogue half-step EH, then a scheduling fence.
//   RKH >= 0: read half RKH of the block in stage RST; RSC: also its scale words
//   TO_P: the tile's last half-step, whose MFMAs write the finished sums into
//         accp (read by this tile's epilogue during the next K loop)
//   ROLE: ROLE_ALL issues everything; ROLE_MFMA only the MFMAs and the
//         operand reads; ROLE_EPI only the copies and the epilogue (of the
//         tile this wave computed before: no prefetch of a following tile's
//         RoPE rows)
template <int ROLE, int NTM, int RST, int RKH, bool RSC, int COPY_LO, int COPY_HI, int DST, bool NEXT, int JD,
          int EH, int NTMP, bool TO_P>
__device__ __forceinline__ void half_step(Ctx& c, v16f (&acc)[MAX_TM][4], const Frags& F, const int (&as)[MAX_TM],
                                          int ws, const int (&ws4)[4], Frags& N, int (&asn)[MAX_TM], Epi& es,
                                          v16f (&accp)[MAX_TM][4]) {
  constexpr int NM = ROLE == ROLE_EPI ? 0 : 4 * NTM;
  // the epilogue role keeps the fenced slots too (they bound how far the
  // scheduler moves its items, and so its register use)
  constexpr int NS = ROLE == ROLE_EPI ? 4 * MAX_TM : (NM > 0 ? NM : 1);
  constexpr int NCP = COPY_HI - COPY_LO;
  constexpr int NSCALE = RSC ? NTM : 0;
  constexpr int NSR = 3 * NS / 4 > 0 ? 3 * NS / 4 : 1;   // scale words and A fragments: first three quarters
  static_for<0, NS>([&](auto sc) __attribute__((always_inline)) {
    constexpr int slot = decltype(sc)::value;
    if (slot < NM) {
      const int tn = slot / (NTM > 0 ? NTM : 1), tm = slot % (NTM > 0 ? NTM : 1);
      v16f& dst = TO_P ? accp[tm][tn] : acc[tm][tn];
      dst = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(F.w[tn], F.a[tm], acc[tm][tn], 0, 0, 0,
                                                            VAR_ROWS ? ws4[tn] : ws, 0, as[tm]);
      asm volatile("" : "+a"(dst));   // the MFMA stays in its slot
      // acc stays live past the MFMA writing accp, so accp cannot take acc's
      // registers (it would have to move back into its own at the tile's end)
      if constexpr (TO_P) asm volatile("" ::"a"(acc[tm][tn]));
    }
    static_for<NCP * slot / NS, NCP * (slot + 1) / NS>([&](auto kc) __attribute__((always_inline)) {
      constexpr int WI = COPY_LO + decltype(kc)::value;
      // split roles: the MFMA role copies the activation slabs, the epilogue
      // role the weight slabs and the scale words
      constexpr bool A_SLAB = WI >= WCOPIES && WI < WCOPIES + ACOPIES;
      if constexpr (ROLE == ROLE_ALL || (ROLE == ROLE_MFMA) == A_SLAB) c.template copy<DST, NEXT, WI, JD>();
    });
    constexpr int NRA = (RKH >= 0 && ROLE != ROLE_EPI) ? NSCALE + NTM : 0;
#pragma unroll
    for (int r = NRA * slot / NSR; r < (slot < NSR ? NRA * (slot + 1) / NSR : 0); ++r) {
      if (r < NSCALE) {
        asn[r] = c.read_scale<RST>(r);
      } else {
        const int tm = r - NSCALE;
        N.a[tm] = make_v8i(c.read16<RST>(true, RKH, 0, TM_STRIDE * tm), c.read16<RST>(true, RKH, 1, TM_STRIDE * tm));
      }
    }
    // W fragment tn right after its last use in this half-step (slot NTM (tn + 1) - 1),
    // so the next one takes over its registers
    if constexpr (RKH >= 0 && ROLE != ROLE_EPI) {
#pragma unroll
      for (int tn = 0; tn < 4; ++tn)
        if (slot == (NTM > 0 ? NTM * (tn + 1) - 1 : 0))
          N.w[tn] = make_v8i(c.read16<RST>(false, RKH, 0, 32 * tn), c.read16<RST>(false, RKH, 1, 32 * tn));
    }
    if constexpr (ROLE == ROLE_ALL) epi_slot<EH, NTMP, NS>(es, accp, slot, c);
    if constexpr (ROLE == ROLE_EPI && NTMP > 0 && EH < 24)
      epi_slot_even<EH, NS, slot>(es, accp, c);
    __builtin_amdgcn_sched_barrier(0);
  });
}

// K block j (compile time, stage j % 3) of a tile:
//   half A: MFMAs on block j's first half, reads of its second half, copies
//           PART1.. of block j+2, epilogue half-step 2j;
//   barrier (block j+1 has landed, all of block j has been read);
//   half B: MFMAs on block j's second half, reads of block j+1's first half
//           and scale words, copies ..PART1 of block j+3 into stage j % 3,
//           epilogue half-step 2j+1.
// Blocks past the tile's 12 are the next tile's (the copies use its buffers).
// Split roles: block b's weight slabs 0-6 are copied by the epilogue role in
// the half-step after block b-3's barrier, its weight slab 7 and scale words
// by the epilogue role and its activation slabs by the MFMA role in the
// half-step before block b-2's barrier. At block j's barrier block j+1 must
// have landed, so each wave may leave outstanding only what it issued after
// its own copies of block j+1: the MFMA role block j+2's activation slabs
// (4); the epilogue role block j+2's weight slabs and words (7 + 2). At block
// 0 the copies of block 1 came from the other role of the previous tile:
// the MFMA role (then in the epilogue role) has issued 7 + 4 after them, the
// epilogue role (then the MFMA role) 2. The MFMA role reads no operands of
// the following tile (the other group computes it).
template <int ROLE, int NTM, int J, int NTMP, bool FIRST>
__device__ __forceinline__ void k_block(Ctx& c, v16f (&acc)[MAX_TM][4], Frags& f0, Frags& f1,
                                        int (&as0)[MAX_TM], int (&as1)[MAX_TM], Epi& es,
                                        v16f (&accp)[MAX_TM][4]) {
  constexpr int ST = J % NST;
  const int ws = (int)((uint32_t)__builtin_amdgcn_readlane((int)c.wsc_lane, J >> 2) >> (8 * (J & 3)));
  int ws4[4] = {0, 0, 0, 0};   // per-row variant: this lane's rows' bytes of block J
  if constexpr (VAR_ROWS) {
#pragma unroll
    for (int tn = 0; tn < 4; ++tn) ws4[tn] = (int)(c.wsr[tn][J >> 2] >> (8 * (J & 3)));
  }
  int as[MAX_TM];
#pragma unroll
  for (int tm = 0; tm < MAX_TM; ++tm) as[tm] = (int)((uint32_t)as0[tm] >> (8 * (J & 3)));
  __builtin_amdgcn_sched_barrier(0);
  // split epilogue role: the second sub-tile's RoPE rows, ahead of this
  // half-step's copies (see above)
  // (held in the first sub-tile's accumulators 0 and 1, which its RoPE has
  // read by then, so the rows take no registers of their own; pinned there
  // a block later, once landed)
  if constexpr (ROLE == ROLE_EPI && NTMP > 1 && J == ROPE1_BLOCK) {
    rope_into_acc(rope_rows(es.pos1, c), accp);
    __builtin_amdgcn_sched_barrier(0);
  }
  if constexpr (ROLE == ROLE_EPI && NTMP > 1 && J == ROPE1_BLOCK + 1) {
    asm volatile("" : "+a"(accp[0][0]), "+a"(accp[0][1]));
    __builtin_amdgcn_sched_barrier(0);
  }
  // in a chunk's first tile the prologue copied blocks 0 and 1 whole and block 2's first part
  constexpr int J2 = J + 2;
  half_step<ROLE, NTM, ST, 1, false, PART1, NCOPY, J2 % NST, (J2 >= NKB), J2 % NKB, 2 * J, NTMP, false>(
      c, acc, f0, as, ws, ws4, f1, as1, es, accp);
  if constexpr (ROLE != ROLE_EPI) __builtin_amdgcn_s_waitcnt(WAITCNT_LGKM0);
  if constexpr (ROLE == ROLE_ALL) __builtin_amdgcn_s_waitcnt(WAITCNT_VM13);
  if constexpr (ROLE == ROLE_MFMA) __builtin_amdgcn_s_waitcnt(J == 0 ? waitcnt_vm(PART1 + 1 + ACOPIES) : waitcnt_vm(ACOPIES));
  if constexpr (ROLE == ROLE_EPI)
    __builtin_amdgcn_s_waitcnt(J == 0 ? waitcnt_vm(NCOPY - PART1 - ACOPIES + (NTMP > 0 ? ROPE_LOADS : 0))
                                      : waitcnt_vm(NCOPY - ACOPIES + (J == ROPE1_BLOCK && NTMP > 1 ? ROPE_LOADS : 0)));
  block_barrier();   // all of block j read by every wave; block j+1 has landed
  __builtin_amdgcn_sched_barrier(0);
  // split MFMA role, last block: this wave's positions of the tile (clamped
  // into the table; max_pos < 2^31), for the epilogue it runs next
  if constexpr (ROLE == ROLE_MFMA && J == NKB - 1) {
    const int64_t* pl = reinterpret_cast<const int64_t*>(c.lds + c.pos_lds) + 32 * c.th + (fresh(c.lane) & 31);
    auto clamp = [&](int64_t v) __attribute__((always_inline)) {
      return (int32_t)(v < 0 ? 0 : (v >= c.p.max_pos ? c.p.max_pos - 1 : v));
    };
    es.npos0 = clamp(pl[0]);
    es.pos1 = clamp(pl[TM_STRIDE]);
    __builtin_amdgcn_sched_barrier(0);
  }
  constexpr int J3 = J + 3;
  // the split MFMA role reads no operands of the following tile (another group computes it)
  constexpr int RKH_B = (ROLE == ROLE_MFMA && J == NKB - 1) ? -1 : 0;
  half_step<ROLE, NTM, (J + 1) % NST, RKH_B, true, 0, PART1, ST, (J3 >= NKB), J3 % NKB, 2 * J + 1, NTMP,
            ROLE == ROLE_ALL && J == NKB - 1>(c, acc, f1, as, ws, ws4, f0, as1, es, accp);
#pragma unroll
  for (int tm = 0; tm < MAX_TM; ++tm) as0[tm] = as1[tm];
  (void)FIRST;
}

// The K loop of one tile (acc, zeroed here) with the previous tile's epilogue
// (accp, NTMP sub-tiles per wave; 0: none) running underneath; the epilogue
// has read all of accp by block 7, and the last half-step's MFMAs write this
// tile's sums there (so the sets never swap roles). On entry the
// operands of block 0's first half are in f0 / as0 and blocks 0, 1 (and part
// of 2) are in flight or landed; on exit the same holds for the next tile.
// The epilogue fetches the RoPE rows of its next sub-tile itself; with no
// epilogue running, this tile's first ones are fetched after block 9.
// Split roles: the MFMA role starts by reading block 0's first half (it
// landed before the previous tile's last barrier) and its sums stay in acc;
// the epilogue role runs the epilogue of accp (this wave's previous tile),
// fetching its first sub-tile's RoPE rows as it starts.
template <int ROLE, int NTM, int NTMP>
__device__ __forceinline__ void k_loop(Ctx& c, v16f (&acc)[MAX_TM][4], Frags& f0, Frags& f1,
                                       int (&as0)[MAX_TM], int (&as1)[MAX_TM], Epi& es,
                                       v16f (&accp)[MAX_TM][4]) {
  if constexpr (ROLE != ROLE_EPI) {
#pragma unroll
    for (int tm = 0; tm < MAX_TM; ++tm)
#pragma unroll
      for (int tn = 0; tn < 4; ++tn)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[tm][tn][r] = 0.f;
  }
  if constexpr (ROLE == ROLE_EPI && NTMP > 0) es.rope = rope_rows(es.npos0, c);
  if constexpr (ROLE == ROLE_MFMA) {
    // the tile's 128 positions into LDS, 16 bytes a lane (every wave of the
    // group issues the same copy, so that the wait counts are the group's);
    // landed by block 1's barrier, read after block 11's
    __builtin_amdgcn_raw_ptr_buffer_load_lds(c.rp, (lds_void*)(c.lds + c.pos_lds), 16,
                                             (uint32_t)(16 * fresh(c.lane)), 0, 0, 0);
#pragma unroll
    for (int tm = 0; tm < MAX_TM; ++tm) as0[tm] = c.read_scale<0>(tm);
#pragma unroll
    for (int tm = 0; tm < MAX_TM; ++tm)
      f0.a[tm] = make_v8i(c.read16<0>(true, 0, 0, TM_STRIDE * tm), c.read16<0>(true, 0, 1, TM_STRIDE * tm));
#pragma unroll
    for (int tn = 0; tn < 4; ++tn)
      f0.w[tn] = make_v8i(c.read16<0>(false, 0, 0, 32 * tn), c.read16<0>(false, 0, 1, 32 * tn));
  }
#define IQP_KB(J) k_block<ROLE, NTM, J, NTMP, false>(c, acc, f0, f1, as0, as1, es, accp);
  IQP_KB(0) IQP_KB(1) IQP_KB(2) IQP_KB(3) IQP_KB(4) IQP_KB(5) IQP_KB(6) IQP_KB(7) IQP_KB(8) IQP_KB(9)
  if constexpr (ROLE == ROLE_ALL && NTMP == 0) es.rope = load_rope<VAR_IL>(es.npos0, c.half, c.p);
  IQP_KB(10) IQP_KB(11)
#undef IQP_KB
  // every MFMA of the tile completes here
  if constexpr (ROLE == ROLE_ALL) {
#pragma unroll
    for (int tm = 0; tm < NTM; ++tm)
#pragma unroll
      for (int tn = 0; tn < 4; ++tn) asm volatile("" : "+a"(accp[tm][tn]));
  }
  if constexpr (ROLE == ROLE_MFMA) {
#pragma unroll
    for (int tm = 0; tm < NTM; ++tm)
#pragma unroll
      for (int tn = 0; tn < 4; ++tn) asm volatile("" : "+a"(acc[tm][tn]));
  }
}

// Before a tile's K loop: fetch its positions (the K loop fetches RoPE rows
// from them near its end). After it: the tile becomes the epilogue's.
__device__ __forceinline__ void tile_positions(Ctx& c, Epi& es, int64_t tbase) {
  const int64_t tl = tbase + 32 * c.th + (fresh(c.lane) & 31);
  es.npos0 = load_position(tl, c.p);
  es.npos1 = load_position(tl + TM_STRIDE, c.p);
}

__device__ __forceinline__ void hand_over(Ctx& c, Epi& es, int64_t tbase) {
  es.tlane = (int)(tbase + 32 * c.th + (fresh(c.lane) & 31));
  if constexpr (!SPLIT) es.pos1 = es.npos1;   // the split build set it at block 11
}

// Diagnostic build: a tile's float32 sums to dbg [M, H*128]. Sub-tile tm of
// this wave holds tokens tbase + 32 th + TM_STRIDE tm + lane % 32; its
// accumulator tn, registers 4 g .. 4 g + 3, holds dims 32 tn + 8 g + 4 half
// + 0..3 of the head (the layout the epilogue starts from).
__device__ __forceinline__ void dump_sums(const v16f (&s)[MAX_TM][4], const Ctx& c, int64_t tbase) {
  if (c.head >= c.p.H) return;   // odd head count: the pair's missing head
#pragma unroll
  for (int tm = 0; tm < MAX_TM; ++tm) {
    const int64_t t = tbase + 32 * c.th + TM_STRIDE * tm + (c.lane & 31);
    if (t >= c.p.M) continue;
    float* row = c.p.dbg + (t * c.p.H + c.head) * HEAD_DIM + 4 * c.half;
#pragma unroll
    for (int tn = 0; tn < 4; ++tn)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<v4f*>(row + 32 * tn + 8 * g) =
            v4f{s[tm][tn][4 * g], s[tm][tn][4 * g + 1], s[tm][tn][4 * g + 2], s[tm][tn][4 * g + 3]};
  }
}

}  // namespace pipe

// Workgroup = head pair x token chunk, as in indexer_q.hip.
__global__ __launch_bounds__(pipe::NTHREADS, 1)
void IQP_PIPE_KERNEL(IndexerQArgs p) {
  using namespace pipe;
  __shared__ __attribute__((aligned(16))) uint8_t lds[LDS_BYTES];

  const int bid = blockIdx.x;
  uint64_t stamp0 = 0, rstamp0 = 0;   // the clock-stamp build's start stamps
  if constexpr (STAMP) {
    stamp0 = __builtin_amdgcn_s_memtime();
    rstamp0 = __builtin_amdgcn_s_memrealtime();
  }
  auto write_stamps = [&](bool ran) __attribute__((always_inline)) {
    // all four by thread 0, after its own waits; zeros for a workgroup with no tiles
    if (threadIdx.x == 0) {
      uint64_t* st = reinterpret_cast<uint64_t*>(p.dbg) + 4 * (int64_t)bid;
      const uint64_t t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
      *reinterpret_cast<v4u*>(st) = ran ? v4u{(uint32_t)stamp0, (uint32_t)(stamp0 >> 32), (uint32_t)t1,
                                              (uint32_t)(t1 >> 32)}
                                        : v4u{0, 0, 0, 0};
      *reinterpret_cast<v4u*>(st + 2) = ran ? v4u{(uint32_t)rstamp0, (uint32_t)(rstamp0 >> 32), (uint32_t)r1,
                                                  (uint32_t)(r1 >> 32)}
                                            : v4u{0, 0, 0, 0};
    }
  };
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
  // the chunk's tiles [t_begin, t_end) of the ceil(M / 128) tiles
  const int64_t ntiles = (p.M + TOKS - 1) / TOKS;
  const int64_t t_begin = ntiles * chunk / cpp;
  const int64_t t_end = ntiles * (chunk + 1) / cpp;
  if (t_begin >= t_end) {   // uniform over the workgroup
    if constexpr (STAMP) write_stamps(false);
    return;
  }

  Ctx c(p, lds, pair);
  auto tbase_of = [&](int64_t tile) __attribute__((always_inline)) { return TOKS * tile; };

  // prologue: blocks 0 and 1 of the first tile whole, block 2's first part
  // (split build: by the first tile's MFMA group, the one whose epilogue role
  // would have copied them)
  c.buffers(tbase_of(t_begin), c.ra, c.rs);
  c.buffers(t_begin + 1 < t_end ? tbase_of(t_begin + 1) : p.M, c.ra_n, c.rs_n);
  // past the chunk's last tile the next-tile copies read nothing (an empty buffer returns zeros)
  const rsrc_t rw_none = make_rsrc(p.w, 0);
  c.rw_n = t_begin + 1 < t_end ? c.rw : rw_none;
  if (!SPLIT || ((int)threadIdx.x >> 8) == 0) {
    static_for<0, NCOPY>([&](auto w) __attribute__((always_inline)) { c.template copy<0, false, decltype(w)::value, 0>(); });
    static_for<0, NCOPY>([&](auto w) __attribute__((always_inline)) { c.template copy<1, false, decltype(w)::value, 1>(); });
    static_for<0, PART1>([&](auto w) __attribute__((always_inline)) { c.template copy<2, false, decltype(w)::value, 2>(); });
    // block 0 has landed once only blocks 1 and 2's copies may be outstanding
    __builtin_amdgcn_s_waitcnt((((NCOPY + PART1) & 15) | (7 << 4) | (15 << 8) | (((NCOPY + PART1) >> 4) << 14)));
  }
  block_barrier();

  Frags f0, f1;
  int as0[MAX_TM] = {}, as1[MAX_TM] = {};
  Epi es;
  v16f acc[MAX_TM][4], accp[MAX_TM][4];   // the split build uses acc only
  if constexpr (!SPLIT) {
#pragma unroll
    for (int tm = 0; tm < MAX_TM; ++tm) as0[tm] = c.read_scale<0>(tm);
#pragma unroll
    for (int tm = 0; tm < MAX_TM; ++tm)
      f0.a[tm] = make_v8i(c.read16<0>(true, 0, 0, TM_STRIDE * tm), c.read16<0>(true, 0, 1, TM_STRIDE * tm));
#pragma unroll
    for (int tn = 0; tn < 4; ++tn)
      f0.w[tn] = make_v8i(c.read16<0>(false, 0, 0, 32 * tn), c.read16<0>(false, 0, 1, 32 * tn));
  }

  // Every tile is computed whole (4 sub-tiles; past M the copies read zeros
  // and nothing is stored), so the steady loop is one code path.
  int64_t tile = t_begin;
  auto advance = [&]() __attribute__((always_inline)) {
    // the copy buffers move to the next tile; the one after it streams in
    // during the next tile's last blocks
    c.ra = c.ra_n;
    c.rs = c.rs_n;
    c.buffers(tile + 2 < t_end ? tbase_of(tile + 2) : p.M, c.ra_n, c.rs_n);
    c.rw_n = tile + 2 < t_end ? c.rw : rw_none;
    ++tile;
  };
  if constexpr (!SPLIT) {
    auto one_tile = [&](auto ntmp_c) __attribute__((always_inline)) {
      tile_positions(c, es, tbase_of(tile));
      k_loop<ROLE_ALL, MAX_TM, decltype(ntmp_c)::value>(c, acc, f0, f1, as0, as1, es, accp);
      if constexpr (DUMP) dump_sums(accp, c, tbase_of(tile));
      hand_over(c, es, tbase_of(tile));
      advance();
    };
    one_tile(std::integral_constant<int, 0>{});
    while (tile < t_end) one_tile(std::integral_constant<int, DUMP ? 0 : MAX_TM>{});
    if constexpr (!DUMP) epilogue_alone<MAX_TM>(es, accp, c);
  } else {
    // Tile i is computed by group i % 2 while the other group runs the
    // epilogue of its own previous tile (none before the first) and copies.
    // Each iteration below is one group's K loop followed by its epilogue
    // role on the next tile (or, after the chunk's last tile, its epilogue
    // alone), so no accumulator is carried from one iteration to the next.
    const int group = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6) >> 2;
    if (group == 1) {
      c.copy_offsets(fresh(c.lane));
      k_loop<ROLE_EPI, MAX_TM, 0>(c, acc, f0, f1, as0, as1, es, acc);
      advance();
    }
    while (tile < t_end) {
      c.read_bases(fresh(c.lane));
      {
        const int64_t tb = tbase_of(tile);
        c.rp = make_rsrc(p.positions + tb, 8 * (uint64_t)(p.M - tb));
        c.pos_lds = P_OFF + P_BYTES * (int)(tile & 1);
      }
      k_loop<ROLE_MFMA, MAX_TM, 0>(c, acc, f0, f1, as0, as1, es, acc);
      if constexpr (DUMP) dump_sums(acc, c, tbase_of(tile));
      hand_over(c, es, tbase_of(tile));
      advance();
      if (tile < t_end) {
        c.copy_offsets(fresh(c.lane));
        k_loop<ROLE_EPI, MAX_TM, DUMP ? 0 : MAX_TM>(c, acc, f0, f1, as0, as1, es, acc);
        advance();
      } else if constexpr (!DUMP) {
        epilogue_owner<MAX_TM>(es, acc, c);
      }
    }
    // the group that did not compute the chunk's last tile takes its second sub-tile
    if constexpr (!DUMP) {
      if (group != (int)((t_end - 1 - t_begin) & 1)) epilogue_helper<MAX_TM>(es, acc, c, t_end - 1);
    }
  }
  __builtin_amdgcn_s_waitcnt(WAITCNT_VM0);   // no LDS copy may outlive the workgroup
  if constexpr (STAMP) {
    block_barrier();   // the workgroup's last wave is done
    write_stamps(true);
  }
}

}  // namespace

#if IQP_PIPE_VARIANT == 0 && !IQP_PIPE_SPLIT && !IQP_PIPE_DUMP && !IQP_PIPE_STAMP
// token indices are held in 32-bit registers
bool indexer_q_pipe_supported(const IndexerQArgs& a) {
  return a.nkb == pipe::NKB && a.M <= 0x7FFFFFFF - 2 * pipe::TOKS;
}
#endif
#if IQP_PIPE_VARIANT == 0 && IQP_PIPE_SPLIT && !IQP_PIPE_DUMP && !IQP_PIPE_STAMP && !IQP_PIPE_LANES
// as the pipelined kernel, with table positions held in 32-bit registers
bool indexer_q_split_supported(const IndexerQArgs& a) {
  return a.nkb == pipe::NKB && a.M <= 0x7FFFFFFF - 2 * pipe::TOKS && a.max_pos <= 0x7FFFFFFF;
}
#endif

hipError_t IQP_PIPE_LAUNCH(const IndexerQArgs& a, hipStream_t stream) {
  const dim3 grid((unsigned)((int64_t)((a.H + 1) / 2) * a.chunks)), block(pipe::NTHREADS);
  hipLaunchKernelGGL(IQP_PIPE_KERNEL, grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace iqp
