// Split-role build of the pipelined fused kernel (indexer_q_split.hip) with
// convention variants 1 and 2: interleaved RoPE pairs and OCP MX FP4 scales.
#define IQP_PIPE_VARIANT 3
#define IQP_PIPE_SPLIT 1
#define IQP_PIPE_LAUNCH launch_indexer_q_split_v3
#define IQP_PIPE_KERNEL indexer_q_split_kernel_v3
#include "indexer_q_pipe.hip"
