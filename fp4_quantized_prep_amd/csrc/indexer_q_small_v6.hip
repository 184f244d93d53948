// The small-batch fused indexer-Q kernel of indexer_q_small.hip (FP8 and
// bf16 inputs) compiled with a convention variant: OCP floor-rule FP4 scales and per-row weight scales.
#define IQP_SMALL_VARIANT 6
#define IQP_SMALL_LAUNCH launch_indexer_q_small_v6
#define IQP_SMALL_LAUNCH_BF16 launch_indexer_q_small_bf16_v6
#define IQP_SMALL_KERNEL indexer_q_small_kernel_v6
#include "indexer_q_small.hip"
