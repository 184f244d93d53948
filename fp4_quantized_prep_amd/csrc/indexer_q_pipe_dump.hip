// Diagnostic build of the pipelined fused kernel (indexer_q_pipe.hip): the
// same K loop, with each tile's float32 GEMM sums written out in place of the
// RoPE / Hadamard / FP4 epilogue.
#define IQP_PIPE_VARIANT 0
#define IQP_PIPE_DUMP 1
#define IQP_PIPE_LAUNCH launch_indexer_q_pipe_dump
#define IQP_PIPE_KERNEL indexer_q_pipe_dump_kernel
#include "indexer_q_pipe.hip"
