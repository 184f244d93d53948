// Split-role build of the pipelined fused kernel (indexer_q_split.hip) with a
// convention variant: FP4 block scales by the OCP MX rule (codes saturate at
// 6).
#define IQP_PIPE_VARIANT 2
#define IQP_PIPE_SPLIT 1
#define IQP_PIPE_LAUNCH launch_indexer_q_split_v2
#define IQP_PIPE_KERNEL indexer_q_split_kernel_v2
#include "indexer_q_pipe.hip"
