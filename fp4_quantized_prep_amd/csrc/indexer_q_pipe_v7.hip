// The pipelined fused indexer-Q kernel of indexer_q_pipe.hip compiled with a
// convention variant: interleaved RoPE pairs, OCP floor-rule FP4 scales and per-row weight scales.
#define IQP_PIPE_VARIANT 7
#define IQP_PIPE_LAUNCH launch_indexer_q_pipe_v7
#define IQP_PIPE_KERNEL indexer_q_pipe_kernel_v7
#include "indexer_q_pipe.hip"
