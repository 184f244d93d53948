// The pipelined fused indexer-Q kernel of indexer_q_pipe.hip compiled with a
// convention variant: interleaved RoPE pairs and per-row weight scales.
#define IQP_PIPE_VARIANT 5
#define IQP_PIPE_LAUNCH launch_indexer_q_pipe_v5
#define IQP_PIPE_KERNEL indexer_q_pipe_kernel_v5
#include "indexer_q_pipe.hip"
