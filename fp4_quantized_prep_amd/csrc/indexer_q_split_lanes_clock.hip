// Clock-stamp build of the split-role fused kernel that reads the RoPE table's
// lane-ordered copy (indexer_q_split_lanes.hip): that kernel, plus the shader
// clock and constant-rate counter stamps of indexer_q_split_clock.hip.
#define IQP_PIPE_VARIANT 0
#define IQP_PIPE_SPLIT 1
#define IQP_PIPE_STAMP 1
#define IQP_PIPE_LANES 1
#define IQP_PIPE_LAUNCH launch_indexer_q_split_lanes_clock
#define IQP_PIPE_KERNEL indexer_q_split_lanes_clock_kernel
#include "indexer_q_pipe.hip"
