/*
 * iqprep.h — C ABI of libiqprep.so: DeepSeek-V4 indexer-Q preparation on
 * AMD Instinct MI355X (gfx950).
 *
 * The library computes, on the GPU, the calls of indexer-Q preparation:
 *
 *   1. fp8_quant_1x128_ue8m0     packed-UE8M0 FP8 1x128 activation quantization
 *      (tokenspeed PR "perf(deepseek-v4): accelerate indexer Q and packed FP8
 *      quantization", Summary; input contract in Risk and fallback).
 *   2. indexer_q_gemm_rope_fp4   block-scaled FP8 Q projection whose epilogue
 *      applies RoPE, a 128-point Hadamard rotation and FP4 e2m1 quantization
 *      (TensorRT-LLM PR "Fuse DeepSeek-V4 Indexer Q projection with CuTe DSL",
 *      sequence diagram: FP8 input + UE8M0 scales in, packed FP4 Q and scales
 *      out; the same tokenspeed PR, Summary: RoPE, Hadamard and FP4 make up
 *      the Q preparation); indexer_q_gemm_rope_fp4_ex takes convention flags.
 *   3. indexer_q_rope_hadamard_fp4   the same RoPE / Hadamard / FP4 epilogue as
 *      a standalone launch over a bf16 Q (the unfused chain's second half).
 *   4. indexer_q_prep_bf16   calls 1 and 2 as one launch for decode-sized
 *      batches (up to 256 tokens); indexer_q_prep_bf16_ex takes the flags;
 *      indexer_q_prep_bf16_with_quant also runs call 1 on an independent
 *      matrix in the same launch; indexer_q_prep_bf16_with_quant_ws is that
 *      call with a caller-owned workspace, which lets it split each head's
 *      K range over several workgroups at 12 to 64 tokens, and
 *      indexer_q_prep_bf16_with_quant_noalloc the same with the library's own
 *      scratch, for callers that cannot allocate.
 *   5. fp8_quant_weight_128x128_ue8m0   the weights' E4M3 codes and per-tile
 *      scales that calls 2 and 4 take (weight preparation, off the
 *      per-token path).
 *   6. iqp_rope_table_lanes   a RoPE table rearranged for the prefill kernel's
 *      16-byte loads (built once per table); indexer_q_gemm_rope_fp4_lanes
 *      is call 2 reading it.
 *
 * Conventions shared by every entry point:
 *
 *   - Every data pointer is a caller-owned DEVICE pointer on the current HIP
 *     device. The library never allocates, frees, copies or synchronizes; it
 *     enqueues kernels on `stream` (a hipStream_t; NULL = the null stream) and
 *     returns. Calls are therefore safe to capture into a HIP graph.
 *   - Inputs are never modified.
 *   - Sizes and leading dimensions are in elements of the named type unless
 *     stated otherwise; all offsets are computed in 64-bit.
 *   - Return value: IQP_OK, or an IQP_ERR_* code. Argument checks happen on
 *     the host before anything is enqueued; on any error nothing is enqueued
 *     (IQP_ERR_HIP: the launch itself failed). IQP_ERR_UNSUPPORTED means the
 *     arguments are well formed but outside the fast path's contract, and the
 *     caller should use another implementation: the library never falls back
 *     silently.
 *   - M == 0 is a successful no-op.
 *   - Entry points are reentrant and thread-safe; the only global state is a
 *     per-device cache of the device architecture, filled on first use, and
 *     the per-device scratch of indexer_q_prep_bf16_with_quant_noalloc (whose
 *     calls must not overlap on one GPU).
 *
 * Number formats: E4M3 is the OCP OFP8 "fn" variant (bias 7, max 448, no
 * infinities); E2M1 is OCP MX FP4 (magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6);
 * a UE8M0 byte b means 2^(b-127).
 */
#ifndef IQPREP_H
#define IQPREP_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define IQP_OK              0
#define IQP_ERR_INVALID     1  /* null pointer, negative size, leading dimension smaller than a row, overlapping scale strides */
#define IQP_ERR_UNSUPPORTED 2  /* well formed but outside the contract (K % 128, alignment, head shape, device): use another path */
#define IQP_ERR_HIP         3  /* a HIP runtime call or kernel launch failed */

#define IQP_ABI_VERSION     3

/* Convention flags of indexer_q_gemm_rope_fp4_ex, indexer_q_prep_bf16_ex and
 * indexer_q_rope_hadamard_fp4 (0: the defaults of indexer_q_gemm_rope_fp4).
 * The pages leave these conventions open. */
#define IQP_ROPE_INTERLEAVED     0x1  /* RoPE pairs (2i, 2i+1), i < rope_dim/2, instead of (i, i + rope_dim/2) */
#define IQP_FP4_SCALE_OCP_FLOOR  0x2  /* FP4 scale e = floor(log2 max(amax, 1e-4)) - 2 (OCP MX rule), codes
                                         saturating at +-6, instead of e = ceil(log2(amax / 6)) */
#define IQP_W_SCALES_PER_ROW     0x4  /* the projection calls only (not the standalone epilogue): w_scales holds one UE8M0 byte per
                                         weight row and K block, [H*D, K/128] row-major, instead of one per
                                         128x128 tile */

/*
 * fp8_quant_1x128_ue8m0 — packed-UE8M0 FP8 activation quantization.
 *
 * tokenspeed PR "perf(deepseek-v4): accelerate indexer Q and packed FP8
 * quantization", Summary (an online FP8 quantizer for DeepGEMM activations
 * with UE8M0 scale exponents packed into int32 words) and Risk and fallback
 * (a contiguous, aligned BF16 matrix with K divisible by 128; the existing
 * tiny-scale floor is kept).
 *
 * For every row m and 128-element block j of x:
 *   amax = max(max_k |x[m, 128j+k]|, 1e-4)          (1e-4: the tiny-scale floor)
 *   e    = ceil(log2(amax / 448))                     exact; -22 <= e <= 120
 *   q[m, 128j+k] = E4M3 round-to-nearest-even of x * 2^-e   (never saturates)
 *   byte(m, j) = e + 127
 * Four consecutive block bytes form one int32 word, block 4w+t in byte t
 * (little-endian): word (m, w) = scales[m * s_stride_m + w * s_stride_w], for
 * 0 <= w < ceil(K/512). Bytes for blocks past K/128 are written as zero.
 *
 *   x        bf16 [M, K], row stride ldx (elements, >= K); 16-byte aligned and
 *            ldx a multiple of 8, else IQP_ERR_UNSUPPORTED.
 *   q        E4M3 bytes [M, K], row stride ldq (bytes, >= K); 8-byte aligned
 *            and ldq a multiple of 8, else IQP_ERR_UNSUPPORTED.
 *   scales   int32 words, 4-byte aligned. Strides in int32 units; the two
 *            supported layouts are K-major (s_stride_w == 1, s_stride_m >=
 *            ceil(K/512)) and MN-major (s_stride_m == 1, s_stride_w >= M);
 *            anything else is IQP_ERR_INVALID.
 *   K        multiple of 128, else IQP_ERR_UNSUPPORTED.
 *
 * Inputs must be finite (NaN / Inf are outside the contract).
 */
int fp8_quant_1x128_ue8m0(const void* x, int64_t M, int64_t K, int64_t ldx,
                          void* q, int64_t ldq,
                          int32_t* scales, int64_t s_stride_m, int64_t s_stride_w,
                          void* stream);

/*
 * indexer_q_gemm_rope_fp4 — fused block-scaled FP8 Q projection + RoPE +
 * Hadamard-128 + FP4 e2m1 quantization, one launch.
 *
 * TensorRT-LLM PR "Fuse DeepSeek-V4 Indexer Q projection with CuTe DSL",
 * sequence diagram (FP8 input and UE8M0 scales from the quantizer feed a GEMM
 * with a RoPE and FP4 epilogue that returns packed FP4 Q and scales) and
 * Description / Paths compared (the unfused chain: Q GEMM, RoPE kernel, FP4
 * quantization kernel, scale copies); tokenspeed PR "perf(deepseek-v4):
 * accelerate indexer Q and packed FP8 quantization", Summary (the Hadamard
 * transform belongs to the optimized Q preparation).
 *
 * For every token m and head h (n = 128h + d, 0 <= d < 128):
 *   Q[m, n]  = sum_j 2^(ea(m,j) + ew(h,j)) * sum_{k in block j} A[m,k] W[n,k]
 *              (float32 accumulation)
 *   RoPE     for i < 32, p = positions[m], c = cos_sin[p, i], s = cos_sin[p, 32+i]:
 *              y_i = Q_i c - Q_{i+32} s,  y_{i+32} = Q_{i+32} c + Q_i s;  y_d = Q_d for d >= 64
 *   Hadamard z = (H_128 / sqrt(128)) y,  H[r][c] = (-1)^popcount(r & c)
 *   FP4      per 32-element block b: amax = max(max |z|, 1e-4),
 *              e = ceil(log2(amax / 6)) (so e >= -15), q_scales[m, h, b] = e + 127,
 *              codes = E2M1 round-to-nearest-even of z * 2^-e; two codes per
 *              byte, element 2t in the low nibble.
 * Q is never written to memory in any precision.
 *
 *   a          E4M3 [M, K] from fp8_quant_1x128_ue8m0, row stride lda (bytes);
 *              16-byte aligned, lda a multiple of 16.
 *   a_scales   the packed scale words that call wrote, with its strides
 *              (as_stride_m, as_stride_w), same layout rules.
 *   w          E4M3 weights [H*D, K], K contiguous, row stride ldw (bytes);
 *              16-byte aligned, ldw a multiple of 16.
 *   w_scales   UE8M0 bytes [H*D/128, K/128], row-major (one per 128x128 tile).
 *   M          tokens (>= 0); K: multiple of 128, at most 32768; H >= 1; D must
 *              be 128 and rope_dim 64 (else IQP_ERR_UNSUPPORTED). Row strides
 *              below 2^23 bytes and scale-word strides with
 *              as_stride_m < 2^20, (K/512) * as_stride_w < 2^28 (else
 *              IQP_ERR_UNSUPPORTED).
 *   positions  int64 [M]. A position outside [0, max_pos) is a precondition
 *              violation: it is clamped into range (the row's output is then
 *              meaningless, but no memory outside the table is read).
 *   cos_sin    float32 [max_pos, rope_dim]: cos of the rotation angles in
 *              columns [0, rope_dim/2), sin in [rope_dim/2, rope_dim); any
 *              frequencies may be used (iqp_rope_cos_sin_table builds the
 *              standard ones). 16-byte aligned; max_pos >= 1.
 *   q_fp4      uint8 [M, H, D/2] packed E2M1 codes, 16-byte aligned.
 *   q_scales   uint8 [M, H, D/32] UE8M0 bytes, 4-byte aligned.
 *
 * Q must fit float32: the output is undefined if |Q| would overflow, which
 * needs an exponent sum ea + ew near 99 or above (|A W| <= 448^2 per term);
 * activations from fp8_quant_1x128_ue8m0 and weights of ordinary magnitude
 * are far inside that range.
 */
int indexer_q_gemm_rope_fp4(const void* a, int64_t lda,
                            const int32_t* a_scales, int64_t as_stride_m, int64_t as_stride_w,
                            const void* w, int64_t ldw,
                            const uint8_t* w_scales,
                            int64_t M, int64_t K, int32_t H, int32_t D, int32_t rope_dim,
                            const int64_t* positions,
                            const float* cos_sin, int64_t max_pos,
                            uint8_t* q_fp4, uint8_t* q_scales,
                            void* stream);

/*
 * indexer_q_gemm_rope_fp4_ex — indexer_q_gemm_rope_fp4 with convention flags.
 *
 * The same pages as indexer_q_gemm_rope_fp4: they name the MLA RoPE kernel
 * and MX-style FP4 block scales but fix neither the RoPE pair layout nor the
 * scale rule. flags 0 is exactly indexer_q_gemm_rope_fp4 (same kernels, same
 * output). Otherwise, with the arguments, layouts and errors of that call:
 *   IQP_ROPE_INTERLEAVED      pair i < 32 is (Q_2i, Q_2i+1), rotated by the
 *                             angle of table columns i and 32 + i as before;
 *   IQP_FP4_SCALE_OCP_FLOOR   e = floor(log2 max(amax, 1e-4)) - 2 (so e >= -16),
 *                             codes = E2M1 RNE of z * 2^-e saturated at +-6;
 *   IQP_W_SCALES_PER_ROW      w_scales is UE8M0 [H*D, K/128] row-major (one
 *                             byte per weight row n and K block j), and the
 *                             projection uses ew(n, j) in place of ew(h, j).
 * Other bits: IQP_ERR_INVALID. Where the base call would run one of the
 * K = 1536 production kernels (small-batch up to 256 tokens, pipelined
 * above) the flags run that kernel's variant build (per-row weight scales
 * in the pipelined one need w_scales 4-byte aligned; flags without
 * IQP_W_SCALES_PER_ROW run its split-role build, with it the one-role one);
 * otherwise the general tiled kernel runs (slower than the
 * K = 1536 production kernels).
 */
int indexer_q_gemm_rope_fp4_ex(const void* a, int64_t lda,
                               const int32_t* a_scales, int64_t as_stride_m, int64_t as_stride_w,
                               const void* w, int64_t ldw,
                               const uint8_t* w_scales,
                               int64_t M, int64_t K, int32_t H, int32_t D, int32_t rope_dim,
                               const int64_t* positions,
                               const float* cos_sin, int64_t max_pos,
                               uint8_t* q_fp4, uint8_t* q_scales,
                               int32_t flags, void* stream);

/*
 * indexer_q_gemm_rope_fp4_lanes — indexer_q_gemm_rope_fp4 (default
 * conventions) that takes, beside the table, its lane-ordered copy from
 * iqp_rope_table_lanes (built once per table, like the weights).
 *
 * The same pages and the same computation: RoPE on the indexer Q with a
 * cos/sin table (tokenspeed PR "perf(deepseek-v4): accelerate indexer Q and
 * packed FP8 quantization", Summary; TensorRT-LLM PR "Fuse DeepSeek-V4
 * Indexer Q projection with CuTe DSL", sequence diagram). The output is
 * byte for byte that of indexer_q_gemm_rope_fp4 with the same arguments:
 * where that call runs the split-role K = 1536 kernel (257 tokens and
 * more) the rows are read from cos_sin_lanes, elsewhere from cos_sin. The
 * copy pays where a 32-token sub-tile's positions run consecutively (prefill;
 * 16-byte loads then read whole 1 KiB segments instead of gathering 32 rows);
 * for scattered positions it is somewhat slower than the table itself.
 *
 *   cos_sin_lanes  float32, ceil(max_pos / 32) * 2048 elements, 16-byte
 *                  aligned, filled by iqp_rope_table_lanes from this cos_sin
 *                  and max_pos (any other content gives undefined output);
 *                  NULL: IQP_ERR_INVALID.
 * Every other argument, layout and error is that of indexer_q_gemm_rope_fp4.
 */
int indexer_q_gemm_rope_fp4_lanes(const void* a, int64_t lda,
                                  const int32_t* a_scales, int64_t as_stride_m, int64_t as_stride_w,
                                  const void* w, int64_t ldw,
                                  const uint8_t* w_scales,
                                  int64_t M, int64_t K, int32_t H, int32_t D, int32_t rope_dim,
                                  const int64_t* positions,
                                  const float* cos_sin, const float* cos_sin_lanes, int64_t max_pos,
                                  uint8_t* q_fp4, uint8_t* q_scales,
                                  void* stream);

/*
 * indexer_q_prep_bf16 — the whole indexer-Q preparation in one launch for
 * decode-sized batches: bf16 activations in, packed FP4 Q and scales out.
 *
 * tokenspeed PR "perf(deepseek-v4): accelerate indexer Q and packed FP8
 * quantization", Summary and Perf (small shapes are kept off the multi-launch
 * path); TensorRT-LLM PR "Fuse DeepSeek-V4 Indexer Q projection with CuTe
 * DSL", kernel routing (a dedicated small-M route) and sequence diagram (FP8
 * quantization of the input, then the GEMM with the RoPE / FP4 epilogue).
 *
 * Computes exactly fp8_quant_1x128_ue8m0 on x followed by
 * indexer_q_gemm_rope_fp4 on its result (the same codes, scales and
 * rounding), without writing the FP8 activations anywhere.
 *
 *   x          bf16 [M, K], row stride ldx (elements, >= K); 16-byte aligned
 *              and ldx a multiple of 8.
 *   w, ldw, w_scales, H, D, rope_dim, positions, cos_sin, max_pos, q_fp4,
 *   q_scales   as in indexer_q_gemm_rope_fp4 (w_scales 4-byte aligned here).
 *   M          0 (no-op) to 256 tokens; K must be 1536; ldw below 2^22 bytes;
 *              H <= 65535. Anything else is IQP_ERR_UNSUPPORTED: a caller
 *              with more tokens uses the two calls above.
 */
int indexer_q_prep_bf16(const void* x, int64_t ldx, const void* w, int64_t ldw,
                        const uint8_t* w_scales,
                        int64_t M, int64_t K, int32_t H, int32_t D, int32_t rope_dim,
                        const int64_t* positions, const float* cos_sin, int64_t max_pos,
                        uint8_t* q_fp4, uint8_t* q_scales, void* stream);

/*
 * indexer_q_prep_bf16_ex — indexer_q_prep_bf16 with the convention flags of
 * indexer_q_gemm_rope_fp4_ex (same pages, same meaning: IQP_ROPE_INTERLEAVED,
 * IQP_FP4_SCALE_OCP_FLOOR, IQP_W_SCALES_PER_ROW with w_scales [H*D, K/128]
 * row-major, 4-byte aligned). flags 0 is exactly indexer_q_prep_bf16; the
 * output equals fp8_quant_1x128_ue8m0 followed by indexer_q_gemm_rope_fp4_ex
 * with the same flags. Other bits: IQP_ERR_INVALID; the other arguments,
 * limits and errors are those of indexer_q_prep_bf16.
 */
int indexer_q_prep_bf16_ex(const void* x, int64_t ldx, const void* w, int64_t ldw,
                           const uint8_t* w_scales,
                           int64_t M, int64_t K, int32_t H, int32_t D, int32_t rope_dim,
                           const int64_t* positions, const float* cos_sin, int64_t max_pos,
                           uint8_t* q_fp4, uint8_t* q_scales, int32_t flags, void* stream);

/*
 * indexer_q_prep_bf16_with_quant — indexer_q_prep_bf16 (default conventions)
 * and fp8_quant_1x128_ue8m0 of an independent bf16 matrix x2 in ONE launch:
 * extra workgroups of the one-launch kernel quantize x2 (a decode step's
 * other activation, e.g. the [M, 7168] input of a wider projection) while
 * the others prepare Q, saving a launch per step (tokenspeed PR
 * "perf(deepseek-v4): accelerate indexer Q and packed FP8 quantization",
 * Performance: the packed quantizer and the Q preparation timed as a decode
 * CUDA Graph replay per step; Summary for both operations).
 *
 * The first 15 arguments, their layouts and errors are indexer_q_prep_bf16's;
 * x2, M2, K2, ldx2, q2, ldq2, scales2, s_stride_m2, s_stride_w2 are
 * fp8_quant_1x128_ue8m0's (x, M, K, ldx, q, ldq, scales, s_stride_m,
 * s_stride_w), with the same checks and M2 at most 256 (else
 * IQP_ERR_UNSUPPORTED). Both outputs are byte for byte those of the two
 * separate calls. M2 == 0 or K2 == 0: the first call alone; M == 0: the
 * quantization alone (its own launch). The x2 / q2 / scales2 regions must
 * not overlap the other call's buffers.
 */
int indexer_q_prep_bf16_with_quant(const void* x, int64_t ldx, const void* w, int64_t ldw,
                                   const uint8_t* w_scales,
                                   int64_t M, int64_t K, int32_t H, int32_t D, int32_t rope_dim,
                                   const int64_t* positions, const float* cos_sin, int64_t max_pos,
                                   uint8_t* q_fp4, uint8_t* q_scales,
                                   const void* x2, int64_t M2, int64_t K2, int64_t ldx2,
                                   void* q2, int64_t ldq2, int32_t* scales2,
                                   int64_t s_stride_m2, int64_t s_stride_w2,
                                   void* stream);

/*
 * indexer_q_workspace_bytes — bytes of the workspace that
 * indexer_q_prep_bf16_with_quant_ws needs for H heads: 256 bytes of counters
 * per 32 heads (rounded up), then 64 KiB per head of float32 partial sums.
 * 4,194,816 bytes at H = 64. H <= 0: 0. (A workspace of B bytes keeps its
 * counters for the most heads it can hold, B / 65544, so one workspace
 * serves calls with any head count it is large enough for.)
 */
int64_t indexer_q_workspace_bytes(int32_t H);

/*
 * indexer_q_prep_bf16_with_quant_ws — indexer_q_prep_bf16_with_quant with a
 * workspace (the same arguments, then workspace, workspace_bytes). From 12
 * to 64 tokens the one-launch kernel then splits each head's K range (12
 * blocks of 128) over 3 workgroups (12 to 32 tokens) or 2 (33 to 64): each
 * quantizes only its blocks of X and streams only its blocks of W, stores
 * its float32 partial sums in the workspace and takes a ticket from the head
 * and tile's counter there; the workgroup that draws the last ticket adds the
 * partial sums in split order, resets the counter and runs the RoPE /
 * Hadamard / FP4 epilogue. Outside that range the workspace is not touched.
 * The GEMM is the same block-scaled FP8 contraction as in the unsplit kernel
 * (TensorRT-LLM PR "Fuse DeepSeek-V4 Indexer Q projection with CuTe DSL",
 * sequence diagram); only the order in which the float32 partial sums are
 * added differs, and it is fixed, so results are deterministic. Measured on
 * MI355X with an [M, 7168] quantization beside it, weights in the Infinity
 * Cache: 7.9 us against 8.6 at 24 tokens, 8.2 against 9.5 at 32, 8.7
 * against 9.6 at 48; weights in HBM: 8.7 against 9.9 at 16 tokens, 9.1
 * against 11.6 at 32.
 *
 * workspace: device memory of at least indexer_q_workspace_bytes(H) bytes,
 * 256-byte aligned, owned by the caller, filled with zeros before its first
 * use (each call leaves its counters at zero again; the partial sums need no
 * clearing). Calls that share a workspace must not run concurrently (one
 * workspace per stream, or order the calls): their counters would mix.
 *
 * Errors: null workspace or workspace_bytes too small: IQP_ERR_INVALID;
 * workspace not 256-byte aligned: IQP_ERR_UNSUPPORTED; everything else as in
 * indexer_q_prep_bf16_with_quant.
 */
int indexer_q_prep_bf16_with_quant_ws(const void* x, int64_t ldx, const void* w, int64_t ldw,
                                      const uint8_t* w_scales,
                                      int64_t M, int64_t K, int32_t H, int32_t D, int32_t rope_dim,
                                      const int64_t* positions, const float* cos_sin, int64_t max_pos,
                                      uint8_t* q_fp4, uint8_t* q_scales,
                                      const void* x2, int64_t M2, int64_t K2, int64_t ldx2,
                                      void* q2, int64_t ldq2, int32_t* scales2,
                                      int64_t s_stride_m2, int64_t s_stride_w2,
                                      void* workspace, int64_t workspace_bytes, void* stream);

/*
 * indexer_q_prep_bf16_with_quant_noalloc — indexer_q_prep_bf16_with_quant_ws
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same
 * arguments without the workspace, which is instead the library's own
 * scratch, a static device array of indexer_q_workspace_bytes(
 * IQP_NOALLOC_MAX_HEADS) = 4,194,816 bytes that each GPU the library runs on
 * holds until the process ends (it is zero when the library is loaded, and
 * every call leaves its counters at zero). The call allocates nothing.
 *
 * Every call on one GPU shares that GPU's scratch: calls that overlap on one
 * GPU (on different streams, or from several threads) race and must not be
 * made; order them on one stream. Results are byte for byte those of
 * indexer_q_prep_bf16_with_quant_ws.
 *
 * Errors: H > IQP_NOALLOC_MAX_HEADS: IQP_ERR_UNSUPPORTED (the scratch is too
 * small; use indexer_q_prep_bf16_with_quant_ws); otherwise as in
 * indexer_q_prep_bf16_with_quant (the scratch's address is looked up once per
 * device, at the first call that gets past the checks; IQP_ERR_HIP if that
 * fails).
 */
#define IQP_NOALLOC_MAX_HEADS 64
int indexer_q_prep_bf16_with_quant_noalloc(const void* x, int64_t ldx, const void* w, int64_t ldw,
                                           const uint8_t* w_scales,
                                           int64_t M, int64_t K, int32_t H, int32_t D, int32_t rope_dim,
                                           const int64_t* positions, const float* cos_sin, int64_t max_pos,
                                           uint8_t* q_fp4, uint8_t* q_scales,
                                           const void* x2, int64_t M2, int64_t K2, int64_t ldx2,
                                           void* q2, int64_t ldq2, int32_t* scales2,
                                           int64_t s_stride_m2, int64_t s_stride_w2, void* stream);

/*
 * indexer_q_rope_hadamard_fp4 — the epilogue of indexer_q_gemm_rope_fp4 as a
 * standalone launch over a bf16 Q: RoPE + Hadamard-128 + FP4 e2m1.
 *
 * TensorRT-LLM PR "Fuse DeepSeek-V4 Indexer Q projection with CuTe DSL",
 * Description / Paths compared (the unfused chain: the Q GEMM writes a bf16
 * Q, then an in-place RoPE kernel and an FP4 quantization kernel with scale
 * copies run on it); tokenspeed PR "perf(deepseek-v4): accelerate indexer Q
 * and packed FP8 quantization", Summary (the RoPE kernel, the Hadamard
 * transform and the fused FP4 cat kernel of the Q preparation).
 *
 * For every token m and head h, with Q_d = q[m * ldq + 128 h + d] widened to
 * float32, the RoPE, Hadamard and FP4 steps are those of
 * indexer_q_gemm_rope_fp4 (same table, same output layout and rounding)
 * when flags is 0. flags may select convention variants:
 *   IQP_ROPE_INTERLEAVED      pair i (angle row entries i and rope_dim/2 + i of
 *                             the table, as before) is dims (2i, 2i + 1);
 *   IQP_FP4_SCALE_OCP_FLOOR   e = floor(log2 max(amax, 1e-4)) - 2 (so e >= -16),
 *                             codes = E2M1 RNE of z * 2^-e saturated at +-6.
 * Other bits: IQP_ERR_INVALID.
 *
 *   q          bf16 [M, H*D], row stride ldq (elements, >= H*D); 16-byte
 *              aligned and ldq a multiple of 8, else IQP_ERR_UNSUPPORTED.
 *              Read only (no in-place RoPE).
 *   M          tokens (>= 0); H >= 1; D must be 128 and rope_dim 64 (else
 *              IQP_ERR_UNSUPPORTED); M < 2^31 and H <= 64 * 65535.
 *   positions  int64 [M]; outside [0, max_pos) is a precondition violation,
 *              clamped into range as in indexer_q_gemm_rope_fp4.
 *   cos_sin    float32 [max_pos, rope_dim] as in indexer_q_gemm_rope_fp4,
 *              16-byte aligned; max_pos >= 1.
 *   q_fp4      uint8 [M, H, D/2] packed E2M1 codes, 16-byte aligned.
 *   q_scales   uint8 [M, H, D/32] UE8M0 bytes, 4-byte aligned.
 *
 * Q must be finite.
 */
int indexer_q_rope_hadamard_fp4(const void* q, int64_t ldq, int64_t M, int32_t H, int32_t D,
                                int32_t rope_dim, const int64_t* positions,
                                const float* cos_sin, int64_t max_pos,
                                uint8_t* q_fp4, uint8_t* q_scales, int32_t flags, void* stream);

/*
 * fp8_quant_weight_128x128_ue8m0 — weight preparation: bf16 weights to the
 * E4M3 codes and per-tile UE8M0 scales that indexer_q_gemm_rope_fp4 and
 * indexer_q_prep_bf16 take as w / w_scales. Not on the per-token path: it
 * runs when weights are loaded or updated.
 *
 * The pages only say the Q projection is a block-scaled FP8 GEMM (tokenspeed
 * PR "perf(deepseek-v4): accelerate indexer Q and packed FP8 quantization",
 * Summary; TensorRT-LLM PR "Fuse DeepSeek-V4 Indexer Q projection with CuTe
 * DSL", sequence diagram); the weight format is a reading: one scale per
 * 128x128 tile, chosen like the activations' scales. For every tile (a, b):
 *   amax = max(max |w| over rows 128a.., columns 128b.., 1e-4)
 *   e    = ceil(log2(amax / 448)) exact;  scales[a * ld_scales + b] = e + 127
 *   q    = E4M3 round-to-nearest-even of w * 2^-e (never saturates)
 *
 *   w          bf16 [N, K], row stride ldw (elements, >= K); 16-byte aligned,
 *              ldw a multiple of 8.
 *   q          E4M3 bytes [N, K], row stride ldq (bytes, >= K); 8-byte
 *              aligned, ldq a multiple of 8.
 *   scales     uint8 [N/128, K/128], row stride ld_scales (bytes, >= K/128).
 *   N, K       multiples of 128 (else IQP_ERR_UNSUPPORTED); N/128 <= 65535.
 * Inputs must be finite.
 */
int fp8_quant_weight_128x128_ue8m0(const void* w, int64_t N, int64_t K, int64_t ldw,
                                   void* q, int64_t ldq, uint8_t* scales, int64_t ld_scales,
                                   void* stream);

/*
 * iqp_rope_cos_sin_table — builds the standard RoPE table that
 * indexer_q_gemm_rope_fp4 reads: for 0 <= p < max_pos and i < rope_dim/2,
 *   cos_sin[p, i] = cos(p * theta^(-2i/rope_dim)),
 *   cos_sin[p, rope_dim/2 + i] = sin(p * theta^(-2i/rope_dim)),
 * evaluated in float64 on the device and rounded to float32 once.
 * (tokenspeed PR "perf(deepseek-v4): accelerate indexer Q and packed FP8
 * quantization", Summary: RoPE on the indexer Q; the base and layout are not
 * on the page, theta = 10000 is the usual base.)
 *
 *   cos_sin   float32 [max_pos, rope_dim], 4-byte aligned. rope_dim even, > 0;
 *             theta > 0; max_pos >= 0 (0: no-op).
 */
int iqp_rope_cos_sin_table(double theta, int64_t max_pos, int32_t rope_dim,
                           float* cos_sin, void* stream);

/*
 * iqp_rope_table_lanes — the lane-ordered copy of a RoPE table that
 * indexer_q_gemm_rope_fp4_lanes reads (the same values, rearranged; built
 * once per table). Element k = 2048 b + 256 L + 4 (2 r + h) + e holds
 *   cos_sin[32 b + r, 32 (L % 2) + 8 (L / 2) + 4 h + e]
 * for 0 <= L < 8, 0 <= r < 32, h < 2, e < 4 where 32 b + r < max_pos, and 0.0
 * past max_pos: block b holds positions 32 b .. 32 b + 31, each 16-byte
 * piece the load one kernel lane makes. (tokenspeed PR "perf(deepseek-v4):
 * accelerate indexer Q and packed FP8 quantization", Summary: RoPE on the
 * indexer Q; the layout is this library's.)
 *
 *   cos_sin  float32 [max_pos, rope_dim], 16-byte aligned; rope_dim must be
 *            64 (else IQP_ERR_UNSUPPORTED).
 *   out      float32, ceil(max_pos / 32) * 2048 elements, 16-byte aligned;
 *            must not overlap cos_sin.
 *   max_pos >= 0 (0: no-op).
 */
int iqp_rope_table_lanes(const float* cos_sin, int64_t max_pos, int32_t rope_dim,
                         float* out, void* stream);

/*
 * iqp_debug_indexer_q_f32 — diagnostic twin of indexer_q_gemm_rope_fp4 for
 * parity testing of its stages (TensorRT-LLM PR "Fuse DeepSeek-V4 Indexer Q
 * projection with CuTe DSL", sequence diagram: the GEMM result feeds the
 * RoPE / FP4 epilogue): same inputs, but instead of FP4 codes it writes
 * float32 out[M, H*D] holding
 *   stage 0: Q (the GEMM output),
 *   stage 1: Q after RoPE,
 *   stage 2: z (after RoPE and the normalized Hadamard rotation),
 * all three from the general fused kernel (every supported shape), or
 *   stage 3: Q from the K loop of the kernel indexer_q_gemm_rope_fp4 runs
 *            for these arguments (the small-batch, pipelined or split-role
 *            kernel, built with its epilogue replaced by a float32 store; the
 *            general kernel's stage 0 where that is the kernel it runs).
 * out is 16-byte aligned; any other stage is IQP_ERR_INVALID.
 */
int iqp_debug_indexer_q_f32(const void* a, int64_t lda,
                            const int32_t* a_scales, int64_t as_stride_m, int64_t as_stride_w,
                            const void* w, int64_t ldw,
                            const uint8_t* w_scales,
                            int64_t M, int64_t K, int32_t H, int32_t D, int32_t rope_dim,
                            const int64_t* positions,
                            const float* cos_sin, int64_t max_pos,
                            float* out, int32_t stage,
                            void* stream);

/*
 * iqp_debug_indexer_q_prep_bf16_f32 — diagnostic twin of indexer_q_prep_bf16
 * (same pages, same arguments and limits): the one-launch kernel, quantizing
 * x itself, with its epilogue replaced by a float32 store of Q (the GEMM
 * output) to out[M, H*D], 16-byte aligned.
 */
int iqp_debug_indexer_q_prep_bf16_f32(const void* x, int64_t ldx, const void* w, int64_t ldw,
                                      const uint8_t* w_scales,
                                      int64_t M, int64_t K, int32_t H, int32_t D, int32_t rope_dim,
                                      const int64_t* positions, const float* cos_sin, int64_t max_pos,
                                      float* out, void* stream);

/*
 * iqp_debug_indexer_q_clock — indexer_q_gemm_rope_fp4 (same arguments, same
 * q_fp4 / q_scales bytes) from a build of its kernel that also records the
 * shader clock, for reading measured throughput against the clock the chip
 * ran at (tokenspeed PR "perf(deepseek-v4): accelerate indexer Q and packed
 * FP8 quantization", Performance: the pages quote kernel times with no
 * clock). Supported where the call runs the split-role kernel (K = 1536,
 * 257 tokens or more); elsewhere IQP_ERR_UNSUPPORTED with nothing enqueued.
 *
 *   cos_sin_lanes   NULL (the build that reads cos_sin), or the table's
 *                   lane-ordered copy as indexer_q_gemm_rope_fp4_lanes takes
 *                   it (the build that reads that; 16-byte aligned).
 *
 *   stamps          uint64 [4 * workgroups], 16-byte aligned: for workgroup
 *                   g, stamps[4g], [4g+1] = the shader clock counter
 *                   (s_memtime) at its start and end, [4g+2], [4g+3] = the
 *                   constant-rate counter (s_memrealtime, ticking at the
 *                   wall clock rate of iqp_device_clock_rates) at the same
 *                   points; all four 0 for a workgroup given no tokens.
 *   stamp_capacity  elements of stamps; below 4 * workgroups: IQP_ERR_INVALID,
 *                   nothing enqueued.
 *   n_workgroups    host pointer, set to the launch's workgroup count before
 *                   any other check of the stamps (0 when unsupported or
 *                   invalid otherwise).
 * Mean shader clock of a workgroup = (end - start of s_memtime) / (end -
 * start of s_memrealtime) * wall clock rate.
 */
int iqp_debug_indexer_q_clock(const void* a, int64_t lda,
                              const int32_t* a_scales, int64_t as_stride_m, int64_t as_stride_w,
                              const void* w, int64_t ldw,
                              const uint8_t* w_scales,
                              int64_t M, int64_t K, int32_t H, int32_t D, int32_t rope_dim,
                              const int64_t* positions,
                              const float* cos_sin, const float* cos_sin_lanes, int64_t max_pos,
                              uint8_t* q_fp4, uint8_t* q_scales,
                              uint64_t* stamps, int64_t stamp_capacity, int64_t* n_workgroups,
                              void* stream);

/*
 * iqp_device_clock_rates — the current device's constant-rate counter
 * frequency (the rate of iqp_debug_indexer_q_clock's realtime stamps) and its
 * peak shader clock, in Hz, into two host int64 values. IQP_ERR_HIP if the
 * runtime cannot report them.
 */
int iqp_device_clock_rates(int64_t* wall_clock_hz, int64_t* peak_shader_clock_hz);

/* Human-readable name of a status code (static storage; never NULL). */
const char* iqp_status_string(int status);

/* IQP_ABI_VERSION of the built library. */
int iqp_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* IQPREP_H */
