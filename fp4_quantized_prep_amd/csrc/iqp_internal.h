// Internal declarations shared by the library's translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace iqp {

// Arguments of the fused indexer-Q kernel (validated on the host).
struct IndexerQArgs {
  const uint8_t* a;              // E4M3 activations [M, K], row stride lda bytes
  int64_t lda;
  const uint8_t* a_scale_bytes;  // packed UE8M0 words viewed as bytes
  int64_t as_sm, as_sw;          // word strides (int32 units)
  const uint8_t* w;              // E4M3 weights [H*128, K], row stride ldw bytes
  int64_t ldw;
  const uint8_t* w_scales;       // UE8M0 [H, K/128]
  int64_t M;
  int32_t nkb;                   // K / 128
  int32_t H;
  const int64_t* positions;      // [M]
  const float* cos_sin;          // [max_pos, 64]
  int64_t max_pos;
  const float* cos_sin_lanes;    // null, or the table's lane-ordered copy (launch_rope_table_lanes),
                                 // which the split-role kernel then reads instead of cos_sin
  uint8_t* q_fp4;                // [M, H, 64]
  uint8_t* q_scales;             // [M, H, 4]
  float* dbg;                    // [M, H*128] for the diagnostic stages
  const uint16_t* x;             // bf16 activations [M, K], row stride ldx elements (one-launch small path)
  int64_t ldx;
  int32_t chunks;                // token chunks per head pair (set by the launcher)
  // one-launch kernel: the packed FP8 quantization of an independent bf16
  // matrix [side_words / side_nw rows, K] run by extra workgroups of the
  // same launch (none when side_words == 0); layout and strides as in
  // launch_fp8_quant
  const uint16_t* side_x;
  int64_t side_ldx;
  uint8_t* side_q;
  int64_t side_ldq;
  int32_t* side_scales;
  int64_t side_sm, side_sw;
  int32_t side_nw, side_nkb;
  int64_t side_words;
  // small-batch kernel, split over K (null: not split): the workspace, of
  // splitk_ws_bytes >= splitk_workspace_bytes(H) bytes, zero before its first
  // use and left zero by every call (the counters); calls sharing one must
  // not overlap
  uint8_t* splitk_ws;
  int64_t splitk_ws_bytes;
};

// the one-launch kernel's split-K workspace: the counters (one per head and
// 32-token tile), then each split's float32 partial sums of every head and
// tile (at most 4 sets of 16 KiB a head: 3 splits x 1 tile, 2 x 2). The
// counter region is sized by the workspace, for the most heads it can hold
// (8 bytes a head, in 256-byte units), so that calls with different head
// counts find their counters in one region and may share a workspace.
constexpr int64_t SPLITK_MIN_TOKENS = 12;
constexpr int64_t SPLITK_MAX_TOKENS = 64;
__host__ __device__ constexpr int64_t splitk_counter_bytes(int64_t H) { return (8 * H + 255) / 256 * 256; }
__host__ __device__ constexpr int64_t splitk_workspace_bytes(int64_t H) { return splitk_counter_bytes(H) + 65536 * H; }
__host__ __device__ constexpr int64_t splitk_counter_region(int64_t ws_bytes) {
  return splitk_counter_bytes(ws_bytes / (65536 + 8));
}

hipError_t launch_fp8_quant(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                            uint8_t* q, int64_t ldq, int32_t* scales,
                            int64_t s_stride_m, int64_t s_stride_w, hipStream_t stream);

// stage -1: FP4 output; 0, 1, 2: float32 diagnostics (see iqprep.h)
hipError_t launch_indexer_q(const IndexerQArgs& args, int stage, hipStream_t stream);
// the float32 GEMM sums of the kernel that launch_indexer_q(args, -1) runs
// (its diagnostic build; the general kernel's stage 0 where that one runs)
hipError_t launch_indexer_q_gemm_dump(const IndexerQArgs& args, hipStream_t stream);
// launch_indexer_q(args, -1) with shader-clock stamps (args.dbg, uint64
// [4 * workgroups]) where it runs the split-role kernel; *workgroups is set
// first; hipErrorNotSupported where another kernel would run, and
// hipErrorInvalidValue when stamp_capacity < 4 * workgroups (nothing launched)
hipError_t launch_indexer_q_clock(const IndexerQArgs& args, int64_t stamp_capacity, int64_t* workgroups,
                                  hipStream_t stream);
// FP4 output with convention variant v (bit 0: interleaved RoPE pairs, bit 1:
// OCP floor-rule FP4 scales, bit 2: per-row weight scales); v = 0 is
// launch_indexer_q(args, -1, stream); otherwise the variant build of the
// small-batch or pipelined kernel where the default call would run that
// kernel (per-row weight scales in the pipelined one: 4-byte aligned), and
// the general kernel everywhere else
hipError_t launch_indexer_q_variant(const IndexerQArgs& args, int variant, hipStream_t stream);

// the pipelined FP4-output kernel (indexer_q_pipe.hip) for the shapes it takes
// (K = 1536, token counts that fit in 31 bits); args.chunks set
bool indexer_q_pipe_supported(const IndexerQArgs& args);
hipError_t launch_indexer_q_pipe(const IndexerQArgs& args, hipStream_t stream);
// the same kernel with convention variant v = 1..7 compiled in
// (indexer_q_pipe_v<v>.hip; bits as in launch_indexer_q_variant; v >= 4 needs
// 4-byte aligned weight scales)
hipError_t launch_indexer_q_pipe_v1(const IndexerQArgs& args, hipStream_t stream);
hipError_t launch_indexer_q_pipe_v2(const IndexerQArgs& args, hipStream_t stream);
hipError_t launch_indexer_q_pipe_v3(const IndexerQArgs& args, hipStream_t stream);
hipError_t launch_indexer_q_pipe_v4(const IndexerQArgs& args, hipStream_t stream);
hipError_t launch_indexer_q_pipe_v5(const IndexerQArgs& args, hipStream_t stream);
hipError_t launch_indexer_q_pipe_v6(const IndexerQArgs& args, hipStream_t stream);
hipError_t launch_indexer_q_pipe_v7(const IndexerQArgs& args, hipStream_t stream);

// the split-role build of the pipelined kernel (indexer_q_split.hip): the
// pipelined kernel's shapes and arguments, table positions below 2^31
bool indexer_q_split_supported(const IndexerQArgs& args);
hipError_t launch_indexer_q_split(const IndexerQArgs& args, hipStream_t stream);
// the same kernel reading the RoPE rows from args.cos_sin_lanes (indexer_q_split_lanes.hip)
hipError_t launch_indexer_q_split_lanes(const IndexerQArgs& args, hipStream_t stream);
// the split-role kernel with convention variant v = 1..3 compiled in
// (indexer_q_split_v<v>.hip; per-row weight scales do not fit its registers);
// where indexer_q_split_supported holds
hipError_t launch_indexer_q_split_v1(const IndexerQArgs& args, hipStream_t stream);
hipError_t launch_indexer_q_split_v2(const IndexerQArgs& args, hipStream_t stream);
hipError_t launch_indexer_q_split_v3(const IndexerQArgs& args, hipStream_t stream);

// diagnostic builds: the float32 GEMM sums (Q before RoPE) of the pipelined,
// split-role and small-batch kernels' K loops in args.dbg [M, H*128]; the
// pipelined and split ones take the arguments of their FP4 launchers
// (args.chunks set); the small-batch one quantizes bf16 args.x itself when
// that is set (the one-launch kernel), else reads args.a
hipError_t launch_indexer_q_pipe_dump(const IndexerQArgs& args, hipStream_t stream);
hipError_t launch_indexer_q_split_dump(const IndexerQArgs& args, hipStream_t stream);
hipError_t launch_indexer_q_small_dump(const IndexerQArgs& args, hipStream_t stream);
// the split-role FP4 kernel with four uint64 stamps per workgroup in args.dbg
// (s_memtime start, end; s_memrealtime start, end; zeros for a workgroup with
// no tiles); args.chunks set
hipError_t launch_indexer_q_split_clock(const IndexerQArgs& args, hipStream_t stream);
// the same stamps from the build reading args.cos_sin_lanes (indexer_q_split_lanes_clock.hip)
hipError_t launch_indexer_q_split_lanes_clock(const IndexerQArgs& args, hipStream_t stream);

// the small-batch FP4-output kernel (indexer_q_small.hip): K = 1536, 1 to 256
// tokens, weight scales 4-byte aligned
bool indexer_q_small_supported(const IndexerQArgs& args);
hipError_t launch_indexer_q_small(const IndexerQArgs& args, hipStream_t stream);
// the same kernel with convention variant v = 1..7 compiled in
// (indexer_q_small_v<v>.hip; bits as in launch_indexer_q_variant)
hipError_t launch_indexer_q_small_v1(const IndexerQArgs& args, hipStream_t stream);
hipError_t launch_indexer_q_small_v2(const IndexerQArgs& args, hipStream_t stream);
hipError_t launch_indexer_q_small_v3(const IndexerQArgs& args, hipStream_t stream);
hipError_t launch_indexer_q_small_v4(const IndexerQArgs& args, hipStream_t stream);
hipError_t launch_indexer_q_small_v5(const IndexerQArgs& args, hipStream_t stream);
hipError_t launch_indexer_q_small_v6(const IndexerQArgs& args, hipStream_t stream);
hipError_t launch_indexer_q_small_v7(const IndexerQArgs& args, hipStream_t stream);
// the same kernel quantizing bf16 activations (args.x, args.ldx) itself: one
// launch from X to FP4 Q; K = 1536, 1 to 256 tokens
// (with args.splitk_ws set and SPLITK_MIN_TOKENS to SPLITK_MAX_TOKENS
// tokens, its split-K build)
bool indexer_q_small_bf16_supported(const IndexerQArgs& args);
hipError_t launch_indexer_q_small_bf16(const IndexerQArgs& args, hipStream_t stream);
// the same with convention variant v = 1..7 compiled in (indexer_q_small_v<v>.hip),
// and a dispatcher over v = 0..7 (0: launch_indexer_q_small_bf16)
hipError_t launch_indexer_q_small_bf16_v1(const IndexerQArgs& args, hipStream_t stream);
hipError_t launch_indexer_q_small_bf16_v2(const IndexerQArgs& args, hipStream_t stream);
hipError_t launch_indexer_q_small_bf16_v3(const IndexerQArgs& args, hipStream_t stream);
hipError_t launch_indexer_q_small_bf16_v4(const IndexerQArgs& args, hipStream_t stream);
hipError_t launch_indexer_q_small_bf16_v5(const IndexerQArgs& args, hipStream_t stream);
hipError_t launch_indexer_q_small_bf16_v6(const IndexerQArgs& args, hipStream_t stream);
hipError_t launch_indexer_q_small_bf16_v7(const IndexerQArgs& args, hipStream_t stream);
hipError_t launch_indexer_q_small_bf16_variant(const IndexerQArgs& args, int variant, hipStream_t stream);

// standalone epilogue: bf16 Q [M, H*128] (row stride ldq elements) -> RoPE,
// Hadamard-128, FP4 codes [M, H, 64] and scale bytes [M, H, 4]
// (interleaved: RoPE pairs (2i, 2i+1); floor_rule: OCP MX FP4 scales)
hipError_t launch_indexer_q_epilogue(const uint16_t* q, int64_t ldq, int64_t M, int32_t H,
                                     const int64_t* positions, const float* cos_sin, int64_t max_pos,
                                     uint8_t* q_fp4, uint8_t* q_scales, bool interleaved, bool floor_rule,
                                     hipStream_t stream);

// weight preparation: bf16 [N, K] -> E4M3 [N, K] + UE8M0 [N/128, K/128]
hipError_t launch_fp8_quant_weight(const uint16_t* w, int64_t N, int64_t K, int64_t ldw, uint8_t* q, int64_t ldq,
                                   uint8_t* scales, int64_t ld_scales, hipStream_t stream);

// compute units of the current device (cached per device)
int cu_count();

hipError_t launch_rope_table(double theta, int64_t max_pos, int32_t rope_dim,
                             float* cos_sin, hipStream_t stream);
// the lane-ordered copy of a [max_pos, 64] table: ceil(max_pos / 32) * 2048 floats
// (layout in rope_table.hip)
hipError_t launch_rope_table_lanes(const float* cos_sin, int64_t max_pos, float* out, hipStream_t stream);

}  // namespace iqp
