// The pipelined fused indexer-Q kernel of indexer_q_pipe.hip compiled with a
// convention variant: one weight scale per row and K block.
#define IQP_PIPE_VARIANT 4
#define IQP_PIPE_LAUNCH launch_indexer_q_pipe_v4
#define IQP_PIPE_KERNEL indexer_q_pipe_kernel_v4
#include "indexer_q_pipe.hip"
