// The small-batch fused indexer-Q kernel of indexer_q_small.hip (FP8 and
// bf16 inputs) compiled with a convention variant: interleaved RoPE pairs (2i, 2i + 1).
#define IQP_SMALL_VARIANT 1
#define IQP_SMALL_LAUNCH launch_indexer_q_small_v1
#define IQP_SMALL_LAUNCH_BF16 launch_indexer_q_small_bf16_v1
#define IQP_SMALL_KERNEL indexer_q_small_kernel_v1
#include "indexer_q_small.hip"
