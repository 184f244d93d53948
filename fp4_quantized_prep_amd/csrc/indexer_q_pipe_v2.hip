// The pipelined fused indexer-Q kernel of indexer_q_pipe.hip compiled with a
// convention variant: OCP floor-rule FP4 scales.
#define IQP_PIPE_VARIANT 2
#define IQP_PIPE_LAUNCH launch_indexer_q_pipe_v2
#define IQP_PIPE_KERNEL indexer_q_pipe_kernel_v2
#include "indexer_q_pipe.hip"
