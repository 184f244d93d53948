// Clock-stamp build of the split-role fused kernel (indexer_q_pipe.hip with
// the split roles): the FP4 kernel as the default build runs it, plus shader
// clock and constant-rate counter stamps at each workgroup's start and end.
#define IQP_PIPE_VARIANT 0
#define IQP_PIPE_SPLIT 1
#define IQP_PIPE_STAMP 1
#define IQP_PIPE_LAUNCH launch_indexer_q_split_clock
#define IQP_PIPE_KERNEL indexer_q_split_clock_kernel
#include "indexer_q_pipe.hip"
