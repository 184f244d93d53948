// Split-role build of the pipelined fused kernel (indexer_q_pipe.hip): eight
// waves, the K loop of a tile and the epilogue of the previous one in
// different waves of each SIMD, the roles alternating tile by tile.
#define IQP_PIPE_VARIANT 0
#define IQP_PIPE_SPLIT 1
#define IQP_PIPE_LAUNCH launch_indexer_q_split
#define IQP_PIPE_KERNEL indexer_q_split_kernel
#include "indexer_q_pipe.hip"
