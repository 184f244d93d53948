// Split-role build of the pipelined fused kernel (indexer_q_split.hip) with a
// convention variant: interleaved RoPE pairs (2i, 2i + 1).
#define IQP_PIPE_VARIANT 1
#define IQP_PIPE_SPLIT 1
#define IQP_PIPE_LAUNCH launch_indexer_q_split_v1
#define IQP_PIPE_KERNEL indexer_q_split_kernel_v1
#include "indexer_q_pipe.hip"
