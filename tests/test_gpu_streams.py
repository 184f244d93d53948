"""The binding on an explicit stream that is not the current one: outputs
and the preparation's FP8 intermediates must come from that stream's pool,
so memory the current stream allocates right after the call can never be
the memory the call's kernels are still reading or writing."""
import pytest
import torch

import synthetic as S

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("M", [8, 300, 4632])
def test_prep_on_an_explicit_stream_matches_the_current_stream(gpu_lib, M):
    codes, sb = S.weights()
    wd, wsd = codes.cuda(), sb.cuda()
    inp = S.indexer_q_inputs("indexer_q_m4632" if M > 4096 else "indexer_q_m128", M=M)
    x, pos = inp["x"].cuda(), inp["positions"].cuda()
    cs = gpu_lib.rope_cos_sin_table(S.ROPE_THETA, 4632, 64)
    ref_q, ref_s = gpu_lib.indexer_q_prep(x, wd, wsd, pos, cs)
    torch.cuda.synchronize()
    print(f"M={M}", flush=True)
    for _ in range(3):
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        q, s = gpu_lib.indexer_q_prep(x, wd, wsd, pos, cs, stream=side)
        # the current stream allocates and overwrites at once, while the side
        # stream may still be running the call
        junk = [torch.full((M, 1536), 0x7F, dtype=torch.uint8, device="cuda") for _ in range(4)]
        junk += [torch.full((M, 64, 64), 0x55, dtype=torch.uint8, device="cuda") for _ in range(2)]
        side.synchronize()
        torch.cuda.synchronize()
        assert torch.equal(q, ref_q) and torch.equal(s, ref_s)
        del junk


def test_quant_and_fused_on_an_explicit_stream(gpu_lib):
    codes, sb = S.weights()
    wd, wsd = codes.cuda(), sb.cuda()
    inp = S.indexer_q_inputs("indexer_q_m128", M=128)
    x, pos = inp["x"].cuda(), inp["positions"].cuda()
    cs = gpu_lib.rope_cos_sin_table(S.ROPE_THETA, 4096, 64)
    a_ref, s_ref = gpu_lib.fp8_quant_1x128_ue8m0(x)
    q_ref, qs_ref = gpu_lib.indexer_q_gemm_rope_fp4(a_ref, s_ref, wd, wsd, pos, cs)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    a, s = gpu_lib.fp8_quant_1x128_ue8m0(x, stream=side)
    q, qs = gpu_lib.indexer_q_gemm_rope_fp4(a, s, wd, wsd, pos, cs, stream=side)
    junk = torch.full((128, 1536), 0x7F, dtype=torch.uint8, device="cuda")
    side.synchronize()
    torch.cuda.synchronize()
    assert torch.equal(a, a_ref) and torch.equal(s, s_ref)
    assert torch.equal(q, q_ref) and torch.equal(qs, qs_ref)
    del junk
