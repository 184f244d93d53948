"""Kernel topology of the fused path: captured into a HIP graph, one indexer-Q
preparation is exactly two kernel nodes above the one-launch size (the FP8
quantizer and the fused projection / RoPE / Hadamard / FP4 kernel) and one
node up to it, with no separate RoPE, FP4 or scale-copy kernel and no memset
or copy node; the standalone epilogue is one kernel. This mirrors the
TensorRT-LLM page's check that a forced-fused graph holds no standalone RoPE
or FP4-concat kernel (TensorRT-LLM PR "Fuse DeepSeek-V4 Indexer Q projection
with CuTe DSL", Test Coverage, the Nsight Systems topology validation).

Graph nodes are read with hipGraphGetNodes / hipGraphNodeGetType from the
HIP runtime the process already has loaded (the one torch uses)."""
import ctypes

import pytest
import torch

import synthetic as S

pytestmark = pytest.mark.gpu

HIP_GRAPH_NODE_KERNEL = 0


def loaded_hip():
    with open("/proc/self/maps") as f:
        paths = {line.split()[-1] for line in f if "libamdhip64.so" in line and line.split()[-1].startswith("/")}
    assert len(paths) == 1, paths
    hip = ctypes.CDLL(paths.pop())
    hip.hipGraphGetNodes.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.POINTER(ctypes.c_size_t)]
    hip.hipGraphGetNodes.restype = ctypes.c_int
    hip.hipGraphNodeGetType.argtypes = [ctypes.c_void_p, ctypes.POINTER(ctypes.c_int)]
    hip.hipGraphNodeGetType.restype = ctypes.c_int
    return hip


def node_types(fn) -> list:
    """Run fn once eagerly, capture it into a graph and return its node types."""
    fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph(keep_graph=True)
    with torch.cuda.graph(g):
        fn()
    hip = loaded_hip()
    graph = ctypes.c_void_p(g.raw_cuda_graph())
    n = ctypes.c_size_t(0)
    assert hip.hipGraphGetNodes(graph, None, ctypes.byref(n)) == 0
    nodes = (ctypes.c_void_p * n.value)()
    assert hip.hipGraphGetNodes(graph, nodes, ctypes.byref(n)) == 0
    types = []
    for node in nodes[: n.value]:
        t = ctypes.c_int(-1)
        assert hip.hipGraphNodeGetType(ctypes.c_void_p(node), ctypes.byref(t)) == 0
        types.append(t.value)
    g.reset()
    return types


@pytest.fixture(scope="module")
def setup(gpu_lib):
    codes, sb = S.weights()
    cs = gpu_lib.rope_cos_sin_table(S.ROPE_THETA, 4632, 64)
    return codes.cuda(), sb.cuda(), cs


@pytest.mark.parametrize("M,expected", [(4632, 2), (300, 2), (64, 2), (8, 1), (1, 1)])
def test_preparation_kernel_nodes(gpu_lib, setup, M, expected):
    w, wsb, cs = setup
    inp = S.indexer_q_inputs("indexer_q_m4632", M=M)
    x, pos = inp["x"].cuda(), inp["positions"].cuda()
    print(f"[topology] indexer_q_prep M={M}", flush=True)
    types = node_types(lambda: gpu_lib.indexer_q_prep(x, w, wsb, pos, cs))
    assert types == [HIP_GRAPH_NODE_KERNEL] * expected, types


def test_standalone_epilogue_is_one_kernel(gpu_lib, setup):
    _, _, cs = setup
    inp = S.q_bf16_inputs("indexer_q_m4632", M=257)
    q, pos = inp["q"].cuda(), inp["positions"].cuda()
    types = node_types(lambda: gpu_lib.indexer_q_rope_hadamard_fp4(q, pos, cs))
    assert types == [HIP_GRAPH_NODE_KERNEL], types


def test_quantizer_is_one_kernel(gpu_lib):
    x = S.quant_input("quant_4632x7168", M=64).cuda()
    types = node_types(lambda: gpu_lib.fp8_quant_1x128_ue8m0(x))
    assert types == [HIP_GRAPH_NODE_KERNEL], types
