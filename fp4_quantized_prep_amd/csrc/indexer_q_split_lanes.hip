// Split-role build of the pipelined fused kernel (indexer_q_split.hip) that
// reads the RoPE rows from the table's lane-ordered copy (args.cos_sin_lanes,
// built by rope_table.hip): with consecutive positions each of a sub-tile's
// eight row loads reads one 1 KiB segment instead of gathering 32 rows.
#define IQP_PIPE_VARIANT 0
#define IQP_PIPE_SPLIT 1
#define IQP_PIPE_LANES 1
#define IQP_PIPE_LAUNCH launch_indexer_q_split_lanes
#define IQP_PIPE_KERNEL indexer_q_split_lanes_kernel
#include "indexer_q_pipe.hip"
