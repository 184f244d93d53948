"""GPU: the clock-stamp builds of the split-role fused kernel (bench.py reads
its shader clock from the one reading the RoPE table's lane-ordered copy)
compute the same bytes as the production call, and their stamps describe a
plausible clock."""
import pytest
import torch

import synthetic as S

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def setup(gpu_lib):
    w, wsb = S.weights()
    inp = S.indexer_q_inputs("indexer_q_m4632")
    cs = gpu_lib.rope_cos_sin_table(S.ROPE_THETA, inp["max_pos"], 64)
    return w.cuda(), wsb.cuda(), inp["x"].cuda(), inp["positions"].cuda(), cs


@pytest.mark.parametrize("lanes", [False, True], ids=["table", "lane_copy"])
@pytest.mark.parametrize("M", [1024, 1157, 4632])
def test_clock_build_gives_the_production_bytes(gpu_lib, setup, M, lanes):
    """Both clock-stamp builds: the one reading the table, and the one reading
    its lane-ordered copy (the kernel bench.py times)."""
    w, wsb, x, pos, cs = setup
    kw = dict(cos_sin_lanes=gpu_lib.rope_table_lanes(cs)) if lanes else {}
    a, a_s = gpu_lib.fp8_quant_1x128_ue8m0(x[:M])
    q, qs = gpu_lib.indexer_q_gemm_rope_fp4(a, a_s, w, wsb, pos[:M], cs, **kw)
    q2, qs2, st = gpu_lib.debug_indexer_q_clock(a, a_s, w, wsb, pos[:M], cs, **kw)
    torch.cuda.synchronize()
    assert torch.equal(q, q2) and torch.equal(qs, qs2)
    st = st.cpu()
    live = st[:, 3] != 0
    assert live.sum() >= 1
    d_clk = (st[live, 1] - st[live, 0]).double()
    d_rt = (st[live, 3] - st[live, 2]).double()
    assert (d_clk > 0).all() and (d_rt > 0).all()
    wall_hz, peak_hz = gpu_lib.device_clock_rates()
    sclk = d_clk.sum() / d_rt.sum() * wall_hz
    print(f"M={M}: {int(live.sum())} workgroups, mean shader clock {sclk / 1e9:.3f} GHz "
          f"(peak {peak_hz / 1e9:.3f} GHz, counter {wall_hz / 1e6:.1f} MHz)")
    assert 0.2e9 < sclk < 1.05 * peak_hz


def test_clock_build_limits(gpu_lib, setup):
    w, wsb, x, pos, cs = setup
    a, a_s = gpu_lib.fp8_quant_1x128_ue8m0(x[:200])
    with pytest.raises(gpu_lib.IqpError) as e:   # 200 tokens: the small-batch kernel runs
        gpu_lib.debug_indexer_q_clock(a, a_s, w, wsb, pos[:200], cs)
    assert e.value.status == gpu_lib.IQP_ERR_UNSUPPORTED
    a, a_s = gpu_lib.fp8_quant_1x128_ue8m0(x[:2048])
    with pytest.raises(gpu_lib.IqpError) as e:   # too few stamp slots: nothing launched
        gpu_lib.debug_indexer_q_clock(a, a_s, w, wsb, pos[:2048], cs,
                                      stamps=torch.zeros(8, dtype=torch.int64, device="cuda"))
    assert e.value.status == gpu_lib.IQP_ERR_INVALID
