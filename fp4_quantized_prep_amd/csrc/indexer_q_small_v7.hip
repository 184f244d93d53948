// The small-batch fused indexer-Q kernel of indexer_q_small.hip (FP8 and
// bf16 inputs) compiled with a convention variant: interleaved RoPE pairs, OCP floor-rule FP4 scales and per-row weight scales.
#define IQP_SMALL_VARIANT 7
#define IQP_SMALL_LAUNCH launch_indexer_q_small_v7
#define IQP_SMALL_LAUNCH_BF16 launch_indexer_q_small_bf16_v7
#define IQP_SMALL_KERNEL indexer_q_small_kernel_v7
#include "indexer_q_small.hip"
