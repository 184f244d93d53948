// The pipelined fused indexer-Q kernel of indexer_q_pipe.hip compiled with a
// convention variant: interleaved RoPE pairs (2i, 2i + 1).
#define IQP_PIPE_VARIANT 1
#define IQP_PIPE_LAUNCH launch_indexer_q_pipe_v1
#define IQP_PIPE_KERNEL indexer_q_pipe_kernel_v1
#include "indexer_q_pipe.hip"
