"""GPU: the allocation-free decode call (indexer_q_prep_bf16_with_quant_noalloc,
the library's per-GPU scratch in place of a workspace) against the call with
a caller workspace (indexer_q_prep_bf16_with_quant_ws), byte for byte, on
calls in a row with fewer tokens each time (two splits of two tiles, three
splits of one tile, then no split), and against the oracle's rule; and the
head-count limit of the scratch."""
import numpy as np
import pytest
import torch

import synthetic as S
from oracle import checker as C

from gpu_util import oracle_chain_from_x

pytestmark = pytest.mark.gpu

MAX_POS = 131072


def test_no_alloc_matches_the_workspace_call(gpu_lib):
    codes, sb = S.weights()
    wd, wsd = codes.cuda(), sb.cuda()
    cs = gpu_lib.rope_cos_sin_table(S.ROPE_THETA, MAX_POS, 64)
    ws = gpu_lib.indexer_q_workspace(64, device="cuda")
    for M in (64, 24, 8):
        print(f"[no_alloc] M={M}", flush=True)
        g = S.rng("indexer_q_m128", 7500 + M)
        x = S.activations_outlier(g, M, 1536)
        pos = torch.from_numpy(g.integers(0, MAX_POS, M).astype(np.int64))
        x2 = torch.from_numpy(g.standard_normal((M, 7168)).astype(np.float32)).to(torch.bfloat16).cuda()
        xd, pd = x.cuda(), pos.cuda()
        r1 = gpu_lib.indexer_q_prep_bf16(xd, wd, wsd, pd, cs, quant_beside=x2, no_alloc=True)
        r0 = gpu_lib.indexer_q_prep_bf16(xd, wd, wsd, pd, cs, quant_beside=x2, workspace=ws)
        torch.cuda.synchronize()
        assert all(torch.equal(a, b) for a, b in zip(r1, r0)), M
        ref = oracle_chain_from_x(x, codes, sb, pos, 64)
        rep = C.check_fp4(r1[0].cpu().numpy(), r1[1].cpu().numpy(), ref["z"], ref["q_fp4"], ref["q_scales"])
        assert rep["ok"], (M, rep)


def test_no_alloc_head_limit(gpu_lib):
    H = gpu_lib.IQP_NOALLOC_MAX_HEADS + 1
    codes = torch.zeros((H * 128, 1536), dtype=torch.uint8, device="cuda")
    sb = torch.full((H, 12), 127, dtype=torch.uint8, device="cuda")
    cs = gpu_lib.rope_cos_sin_table(S.ROPE_THETA, 4096, 64)
    x = torch.zeros((20, 1536), dtype=torch.bfloat16, device="cuda")
    pos = torch.zeros(20, dtype=torch.int64, device="cuda")
    with pytest.raises(gpu_lib.IqpError) as e:
        gpu_lib.indexer_q_prep_bf16(x, codes, sb, pos, cs, n_heads=H, no_alloc=True)
    assert e.value.status == gpu_lib.IQP_ERR_UNSUPPORTED
