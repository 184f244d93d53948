"""GPU parity: the one-launch decode call with a workspace
(indexer_q_prep_bf16_with_quant_ws), whose kernel splits each head's K range
over 3 workgroups at 12 to 32 tokens and 2 at 33 to 64, and adds their float32
partial sums in the workspace.

The split changes only the order in which float32 partial sums are added, so
its FP4 output is checked against the oracle's acceptance rule at every token
count, and against the unsplit call's bytes (a rounding difference may move a
value across an FP4 boundary, so a handful of differing bytes is allowed;
the oracle check decides whether they are legal). The second matrix's
quantization must be byte for byte the standalone quantizer's. The counters
must be back at zero after every call, repeated and graph-replayed calls must
give the same bytes, other workgroup counts must leave the workspace alone,
and other head counts must work."""
import numpy as np
import pytest
import torch

import synthetic as S
from oracle import checker as C

from gpu_util import oracle_chain_from_x, weights_for_heads

pytestmark = pytest.mark.gpu

MAX_POS = 131072


@pytest.fixture(scope="module")
def setup(gpu_lib):
    codes, sb = S.weights()
    cs = gpu_lib.rope_cos_sin_table(S.ROPE_THETA, MAX_POS, 64)
    ws = gpu_lib.indexer_q_workspace(64, device="cuda")
    return codes, sb, codes.cuda(), sb.cuda(), cs, ws


def inputs(M, seed, K2=7168):
    g = S.rng("indexer_q_m128", 7300 + seed)
    x = S.activations_outlier(g, M, 1536)
    pos = torch.from_numpy(g.integers(0, MAX_POS, M).astype(np.int64))
    x2 = torch.from_numpy(g.standard_normal((M, K2)).astype(np.float32)).to(torch.bfloat16)
    return x, pos, x2


def counters_zero(ws, H=64):
    return int(ws[: 8 * H].view(torch.int32).abs().sum()) == 0


@pytest.mark.parametrize("M", [12, 16, 17, 24, 31, 32, 33, 40, 48, 63, 64])
def test_split_matches_oracle_and_unsplit_call(gpu_lib, setup, M):
    codes, sb, wd, wsd, cs, ws = setup
    x, pos, x2 = inputs(M, M)
    print(f"[splitk] M={M}", flush=True)
    xd, pd, x2d = x.cuda(), pos.cuda(), x2.cuda()
    q1, s1, a1, w1 = gpu_lib.indexer_q_prep_bf16(xd, wd, wsd, pd, cs, quant_beside=x2d, workspace=ws)
    q0, s0, a0, w0 = gpu_lib.indexer_q_prep_bf16(xd, wd, wsd, pd, cs, quant_beside=x2d)
    a2, w2 = gpu_lib.fp8_quant_1x128_ue8m0(x2d)
    torch.cuda.synchronize()
    assert counters_zero(ws)
    assert torch.equal(a1, a2) and torch.equal(w1, w2), "the second matrix's quantization differs"
    ref = oracle_chain_from_x(x, codes, sb, pos, 64)
    rep = C.check_fp4(q1.cpu().numpy(), s1.cpu().numpy(), ref["z"], ref["q_fp4"], ref["q_scales"])
    print(rep)
    assert rep["ok"], rep
    nd = int((q1 != q0).sum()) + int((s1 != s0).sum())
    print(f"[splitk] M={M}: bytes differing from the unsplit call: {nd}")
    assert nd <= max(4, q1.numel() // 100000), nd


def test_split_without_second_matrix(gpu_lib, setup):
    codes, sb, wd, wsd, cs, ws = setup
    x, pos, _ = inputs(29, 1)
    q1, s1 = gpu_lib.indexer_q_prep_bf16(x.cuda(), wd, wsd, pos.cuda(), cs, workspace=ws)
    torch.cuda.synchronize()
    assert counters_zero(ws)
    ref = oracle_chain_from_x(x, codes, sb, pos, 64)
    rep = C.check_fp4(q1.cpu().numpy(), s1.cpu().numpy(), ref["z"], ref["q_fp4"], ref["q_scales"])
    assert rep["ok"], rep


def test_split_calls_in_a_row_and_in_a_graph(gpu_lib, setup):
    """Calls with different token counts reuse one workspace: each gives the
    bytes it gives alone, eagerly and replayed from a graph (three replays,
    with eager work between them)."""
    codes, sb, wd, wsd, cs, ws = setup
    cases = [inputs(M, 100 + M) for M in (32, 20, 64, 33, 17)]
    dev = [(x.cuda(), p.cuda(), x2.cuda()) for x, p, x2 in cases]
    alone = []
    for xd, pd, x2d in dev:
        alone.append([t.clone() for t in gpu_lib.indexer_q_prep_bf16(xd, wd, wsd, pd, cs, quant_beside=x2d,
                                                                    workspace=ws)])
        torch.cuda.synchronize()
        assert counters_zero(ws)
    outs = [[torch.empty_like(t) for t in ref] for ref in alone]

    def run():
        for (xd, pd, x2d), o in zip(dev, outs):
            gpu_lib.indexer_q_prep_bf16(xd, wd, wsd, pd, cs, q_fp4=o[0], q_scales=o[1], quant_beside=x2d,
                                        quant_beside_out=(o[2], o[3]), workspace=ws)
    run()
    torch.cuda.synchronize()
    for ref, o in zip(alone, outs):
        assert all(torch.equal(a, b) for a, b in zip(ref, o))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for rep in range(3):
        for o in outs:
            for t in o:
                t.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert counters_zero(ws)
        for ref, o in zip(alone, outs):
            assert all(torch.equal(a, b) for a, b in zip(ref, o)), rep
        gpu_lib.indexer_q_prep_bf16(dev[0][0], wd, wsd, dev[0][1], cs)   # eager work between replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("M", [1, 11, 65, 128])
def test_outside_the_split_range_the_workspace_is_untouched(gpu_lib, setup, M):
    codes, sb, wd, wsd, cs, _ = setup
    ws = gpu_lib.indexer_q_workspace(64, device="cuda")
    ws[8 * 64:].fill_(0xA5)   # partial sums: a marker; counters stay zero
    before = ws.clone()
    x, pos, x2 = inputs(M, 200 + M)
    xd, pd, x2d = x.cuda(), pos.cuda(), x2.cuda()
    r1 = gpu_lib.indexer_q_prep_bf16(xd, wd, wsd, pd, cs, quant_beside=x2d, workspace=ws)
    r0 = gpu_lib.indexer_q_prep_bf16(xd, wd, wsd, pd, cs, quant_beside=x2d)
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(r1, r0)), "the same kernel must give the same bytes"
    assert torch.equal(ws, before)


@pytest.mark.parametrize("H", [1, 3, 8])
def test_split_other_head_counts(gpu_lib, H):
    codes, sb = weights_for_heads(H)
    cs = gpu_lib.rope_cos_sin_table(S.ROPE_THETA, MAX_POS, 64)
    ws = gpu_lib.indexer_q_workspace(H, device="cuda")
    assert ws.numel() == gpu_lib.indexer_q_workspace_bytes(H)
    for M in (24, 50):
        x, pos, _ = inputs(M, 300 + 7 * H + M)
        q1, s1 = gpu_lib.indexer_q_prep_bf16(x.cuda(), codes.cuda(), sb.cuda(), pos.cuda(), cs, n_heads=H,
                                             workspace=ws)
        torch.cuda.synchronize()
        assert counters_zero(ws, H)
        ref = oracle_chain_from_x(x, codes, sb, pos, H)
        rep = C.check_fp4(q1.cpu().numpy(), s1.cpu().numpy(), ref["z"], ref["q_fp4"], ref["q_scales"])
        assert rep["ok"], (H, M, rep)


def test_one_workspace_serves_several_head_counts(gpu_lib, setup):
    """A workspace sized for 64 heads keeps its counters where a call with 3
    heads looks for them too, so calls with either head count can take turns
    on it (the counter region is sized by the workspace, not by the call)."""
    codes64, sb64, wd, wsd, cs, ws = setup
    c3, s3 = weights_for_heads(3)
    c3d, s3d = c3.cuda(), s3.cuda()
    for H, M in ((3, 24), (64, 40), (3, 50), (64, 20), (3, 30), (64, 64)):
        print(f"[splitk] shared workspace H={H} M={M}", flush=True)
        x, pos, _ = inputs(M, 500 + 10 * H + M)
        codes, sb, w_, s_ = (c3, s3, c3d, s3d) if H == 3 else (codes64, sb64, wd, wsd)
        q, qs = gpu_lib.indexer_q_prep_bf16(x.cuda(), w_, s_, pos.cuda(), cs, n_heads=H, workspace=ws)
        torch.cuda.synchronize()
        assert int(ws[:512].view(torch.int32).abs().sum()) == 0
        ref = oracle_chain_from_x(x, codes, sb, pos, H)
        rep = C.check_fp4(q.cpu().numpy(), qs.cpu().numpy(), ref["z"], ref["q_fp4"], ref["q_scales"])
        assert rep["ok"], (H, M, rep)


def test_split_strided_rows(gpu_lib, setup):
    """Rows of X 2048 elements apart (a view of a wider buffer), at both split
    counts: the same bytes as the contiguous call."""
    codes, sb, wd, wsd, cs, ws = setup
    for M in (12, 40):
        x, pos, _ = inputs(M, 700 + M)
        wide = torch.zeros((M, 2048), dtype=torch.bfloat16, device="cuda")
        wide[:, :1536] = x.cuda()
        xv = wide[:, :1536]
        assert xv.stride(0) == 2048
        q1, s1 = gpu_lib.indexer_q_prep_bf16(xv, wd, wsd, pos.cuda(), cs, workspace=ws)
        q2, s2 = gpu_lib.indexer_q_prep_bf16(x.cuda(), wd, wsd, pos.cuda(), cs, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(q1, q2) and torch.equal(s1, s2), M


@pytest.mark.parametrize("M", [40, 64, 65])
def test_routing_helper_with_a_workspace(gpu_lib, setup, M):
    """indexer_q_prep given a workspace: the split one-launch call up to 64
    tokens (its bytes), the two calls above; the oracle's rule either way."""
    codes, sb, wd, wsd, cs, ws = setup
    x, pos, _ = inputs(M, 600 + M)
    xd, pd = x.cuda(), pos.cuda()
    q1, s1 = gpu_lib.indexer_q_prep(xd, wd, wsd, pd, cs, workspace=ws)
    if M <= gpu_lib.ONE_LAUNCH_WITH_WORKSPACE_MAX_TOKENS:
        q2, s2 = gpu_lib.indexer_q_prep_bf16(xd, wd, wsd, pd, cs, workspace=ws)
    else:
        a, a_s = gpu_lib.fp8_quant_1x128_ue8m0(xd)
        q2, s2 = gpu_lib.indexer_q_gemm_rope_fp4(a, a_s, wd, wsd, pd, cs)
    torch.cuda.synchronize()
    assert torch.equal(q1, q2) and torch.equal(s1, s2)
    ref = oracle_chain_from_x(x, codes, sb, pos, 64)
    rep = C.check_fp4(q1.cpu().numpy(), s1.cpu().numpy(), ref["z"], ref["q_fp4"], ref["q_scales"])
    assert rep["ok"], rep


def test_workspace_binding_checks(gpu_lib, setup):
    codes, sb, wd, wsd, cs, ws = setup
    x, pos, _ = inputs(20, 400)
    with pytest.raises(ValueError):
        gpu_lib.indexer_q_prep_bf16(x.cuda(), wd, wsd, pos.cuda(), cs, workspace=ws[:1000])
    with pytest.raises(ValueError):
        gpu_lib.indexer_q_prep_bf16(x.cuda(), wd, wsd, pos.cuda(), cs, workspace=ws, scale_rule="ocp_floor")
    with pytest.raises(gpu_lib.IqpError):   # not 256-byte aligned
        gpu_lib.indexer_q_prep_bf16(x.cuda(), wd, wsd, pos.cuda(), cs,
                                    workspace=torch.zeros(ws.numel() + 512, dtype=torch.uint8, device="cuda")[16:])
