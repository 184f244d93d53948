"""The C-ABI library on the host: it loads without a GPU, exports every entry
point include/iqprep.h declares, and rejects malformed arguments before it
would touch a device (no compute call is made here)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "iqprep.h")


@pytest.fixture(scope="module")
def iqp():
    import fp4_quantized_prep_amd as m
    return m


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", text, flags=re.M)


def test_header_declares_the_boundary():
    names = declared_functions()
    assert {"fp8_quant_1x128_ue8m0", "indexer_q_gemm_rope_fp4", "indexer_q_rope_hadamard_fp4",
            "indexer_q_prep_bf16", "fp8_quant_weight_128x128_ue8m0", "iqp_status_string",
            "iqp_abi_version", "iqp_rope_table_lanes", "indexer_q_gemm_rope_fp4_lanes",
            "indexer_q_workspace_bytes", "indexer_q_prep_bf16_with_quant_ws",
            "indexer_q_prep_bf16_with_quant_noalloc"} <= set(names)


def test_library_exports_every_declared_symbol(iqp):
    lib = ctypes.CDLL(iqp.library_path())
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_version_and_status_strings(iqp):
    assert iqp.abi_version() == 3
    for st in range(4):
        assert iqp._lib.iqp_status_string(st)
    assert b"unknown" in iqp._lib.iqp_status_string(99)


P = ctypes.c_void_p


def quant(iqp, x=16, M=4, K=128, ldx=128, q=16, ldq=128, s=16, sm=1, sw=1):
    return iqp._lib.fp8_quant_1x128_ue8m0(P(x), M, K, ldx, P(q), ldq, P(s), sm, sw, None)


def test_quant_argument_checks(iqp):
    # fake, never-dereferenced addresses: every case fails before any device call
    assert quant(iqp, M=-1) == iqp.IQP_ERR_INVALID
    assert quant(iqp, x=0) == iqp.IQP_ERR_INVALID
    assert quant(iqp, q=0) == iqp.IQP_ERR_INVALID
    assert quant(iqp, s=0) == iqp.IQP_ERR_INVALID
    assert quant(iqp, ldx=64) == iqp.IQP_ERR_INVALID
    assert quant(iqp, K=100, ldx=128, ldq=128) == iqp.IQP_ERR_UNSUPPORTED
    assert quant(iqp, x=24) == iqp.IQP_ERR_UNSUPPORTED        # not 16-byte aligned
    assert quant(iqp, ldx=132) == iqp.IQP_ERR_UNSUPPORTED     # row pitch not a multiple of 16 B
    assert quant(iqp, q=20) == iqp.IQP_ERR_UNSUPPORTED
    assert quant(iqp, sm=1, sw=2) == iqp.IQP_ERR_INVALID      # MN-major with stride < M
    assert quant(iqp, sm=2, sw=2) == iqp.IQP_ERR_INVALID      # neither layout
    assert quant(iqp, M=0) == iqp.IQP_OK                      # empty: no-op
    assert quant(iqp, x=0, q=0, s=0, M=0) == iqp.IQP_OK


def fused(iqp, M=4, K=256, H=2, D=128, rd=64, a=16, lda=256, s=16, sm=1, sw=1, w=16, ldw=256,
          ws=16, pos=16, cs=16, mp=10, q=16, qs=16):
    return iqp._lib.indexer_q_gemm_rope_fp4(P(a), lda, P(s), sm, sw, P(w), ldw, P(ws), M, K, H, D, rd,
                                            P(pos), P(cs), mp, P(q), P(qs), None)


def test_fused_argument_checks(iqp):
    assert fused(iqp, M=-3) == iqp.IQP_ERR_INVALID
    assert fused(iqp, a=0) == iqp.IQP_ERR_INVALID
    assert fused(iqp, pos=0) == iqp.IQP_ERR_INVALID
    assert fused(iqp, q=0) == iqp.IQP_ERR_INVALID
    assert fused(iqp, mp=0) == iqp.IQP_ERR_INVALID
    assert fused(iqp, lda=128) == iqp.IQP_ERR_INVALID
    assert fused(iqp, K=200, lda=256, ldw=256) == iqp.IQP_ERR_UNSUPPORTED
    assert fused(iqp, D=64) == iqp.IQP_ERR_UNSUPPORTED
    assert fused(iqp, rd=32) == iqp.IQP_ERR_UNSUPPORTED
    assert fused(iqp, a=8) == iqp.IQP_ERR_UNSUPPORTED
    assert fused(iqp, ldw=264) == iqp.IQP_ERR_UNSUPPORTED
    assert fused(iqp, q=20) == iqp.IQP_ERR_UNSUPPORTED
    assert fused(iqp, sm=3, sw=3) == iqp.IQP_ERR_INVALID
    assert fused(iqp, K=257 * 128, lda=257 * 128, ldw=257 * 128, sm=65) == iqp.IQP_ERR_UNSUPPORTED  # > 256 K blocks
    assert fused(iqp, M=0) == iqp.IQP_OK


def fused_ex(iqp, flags, M=4, K=256, H=2, D=128, rd=64, lda=256, ldw=256):
    return iqp._lib.indexer_q_gemm_rope_fp4_ex(P(16), lda, P(16), 1, 1, P(16), ldw, P(16), M, K, H, D, rd,
                                               P(16), P(16), 10, P(16), P(16), flags, None)


def test_fused_ex_argument_checks(iqp):
    inv, uns = iqp.IQP_ERR_INVALID, iqp.IQP_ERR_UNSUPPORTED
    assert fused_ex(iqp, 8) == inv                              # unknown convention bit
    assert fused_ex(iqp, -1) == inv
    assert fused_ex(iqp, iqp.IQP_W_SCALES_PER_ROW | 3, M=0) == iqp.IQP_OK
    assert epilogue(iqp, flags=iqp.IQP_W_SCALES_PER_ROW) == inv  # no weights in the standalone epilogue
    assert fused_ex(iqp, iqp.IQP_ROPE_INTERLEAVED, M=-3) == inv  # the base call's checks still apply
    assert fused_ex(iqp, iqp.IQP_FP4_SCALE_OCP_FLOOR, D=64) == uns
    assert fused_ex(iqp, 3, lda=128) == inv
    assert fused_ex(iqp, 3, M=0) == iqp.IQP_OK


def test_one_launch_ex_argument_checks(iqp):
    lib = iqp._lib
    args = [P(16), 1536, P(16), 1536, P(16), 4, 1536, 2, 128, 64, P(16), P(16), 10, P(16), P(16)]
    assert lib.indexer_q_prep_bf16_ex(*args, 8, None) == iqp.IQP_ERR_INVALID      # unknown convention bit
    assert lib.indexer_q_prep_bf16_ex(*args, -1, None) == iqp.IQP_ERR_INVALID
    zero = list(args)
    zero[5] = 0
    assert lib.indexer_q_prep_bf16_ex(*zero, 7, None) == iqp.IQP_OK               # M = 0: no-op
    wide = list(args)
    wide[6], wide[1], wide[3] = 1024, 1024, 1024
    assert lib.indexer_q_prep_bf16_ex(*wide, 1, None) == iqp.IQP_ERR_UNSUPPORTED  # K must be 1536


def test_one_launch_with_quant_argument_checks(iqp):
    lib, inv, uns = iqp._lib, iqp.IQP_ERR_INVALID, iqp.IQP_ERR_UNSUPPORTED
    base = [P(16), 1536, P(16), 1536, P(16), 4, 1536, 2, 128, 64, P(16), P(16), 10, P(16), P(16)]

    def call(M=4, x2=16, M2=3, K2=7168, ldx2=7168, q2=16, ldq2=7168, s2=16, sm=14, sw=1):
        args = list(base)
        args[5] = M
        return lib.indexer_q_prep_bf16_with_quant(*args, P(x2), M2, K2, ldx2, P(q2), ldq2, P(s2), sm, sw, None)
    assert call(M2=-1) == inv
    assert call(x2=0) == inv
    assert call(q2=0) == inv
    assert call(s2=0) == inv
    assert call(ldx2=4096) == inv
    assert call(K2=100, ldx2=128, ldq2=128) == uns          # K not a multiple of 128
    assert call(sm=2, sw=2) == inv                          # neither scale-word layout
    assert call(x2=8) == uns                                # not 16-byte aligned
    assert call(M2=257, sm=14) == uns                       # beyond decode sizes
    assert call(M=257) == uns                               # the one-launch call's own limit
    assert call(M=0, M2=0) == iqp.IQP_OK                    # nothing to do
    assert call(M2=0, x2=0, q2=0, s2=0, M=0) == iqp.IQP_OK


def test_workspace_size_and_argument_checks(iqp):
    lib, inv, uns = iqp._lib, iqp.IQP_ERR_INVALID, iqp.IQP_ERR_UNSUPPORTED
    # 8 bytes of counters a head rounded up to 256, then 64 KiB of partial sums a head
    assert iqp.indexer_q_workspace_bytes(64) == 512 + 64 * 65536 == 4194816
    assert iqp.indexer_q_workspace_bytes(1) == 256 + 65536
    assert iqp.indexer_q_workspace_bytes(33) == 512 + 33 * 65536
    assert lib.indexer_q_workspace_bytes(0) == 0 and lib.indexer_q_workspace_bytes(-3) == 0
    base = [P(16), 1536, P(16), 1536, P(16), 20, 1536, 2, 128, 64, P(16), P(16), 10, P(16), P(16)]
    need = iqp.indexer_q_workspace_bytes(2)

    def call(M=20, M2=3, ws=4096, nbytes=need):
        args = list(base)
        args[5] = M
        return lib.indexer_q_prep_bf16_with_quant_ws(*args, P(16), M2, 7168, 7168, P(16), 7168, P(16), 14, 1,
                                                     P(ws), nbytes, None)
    assert call(ws=0) == inv                                # no workspace
    assert call(nbytes=need - 1) == inv                     # too small for H = 2
    assert call(ws=4096 + 16) == uns                        # not 256-byte aligned
    assert call(M=257) == uns                               # the one-launch call's own limit
    assert call(M2=-1) == inv                               # the second matrix's checks
    assert call(M=0, M2=0) == iqp.IQP_OK                    # nothing to do


def test_no_alloc_argument_checks(iqp):
    lib, inv, uns = iqp._lib, iqp.IQP_ERR_INVALID, iqp.IQP_ERR_UNSUPPORTED
    base = [P(16), 1536, P(16), 1536, P(16), 20, 1536, 2, 128, 64, P(16), P(16), 10, P(16), P(16)]

    def call(M=20, H=2, x2=16, M2=3):
        args = list(base)
        args[5], args[7] = M, H
        return lib.indexer_q_prep_bf16_with_quant_noalloc(*args, P(x2), M2, 7168, 7168, P(16), 7168, P(16), 14, 1,
                                                          None)
    assert iqp.IQP_NOALLOC_MAX_HEADS == 64
    assert call(H=65) == uns                                # beyond what the scratch holds
    assert call(x2=0) == inv                                # the second matrix's checks
    assert call(M=257) == uns                               # the one-launch call's own limit
    assert call(M=-1) == inv
    assert call(M=0, M2=0) == iqp.IQP_OK                    # nothing to do, no device touched


def test_debug_and_table_argument_checks(iqp):
    lib = iqp._lib
    args = [P(16), 256, P(16), 1, 1, P(16), 256, P(16), 4, 256, 2, 128, 64, P(16), P(16), 10]
    assert lib.iqp_debug_indexer_q_f32(*args, P(16), 4, None) == iqp.IQP_ERR_INVALID
    assert lib.iqp_debug_indexer_q_f32(*args, P(16), -1, None) == iqp.IQP_ERR_INVALID
    assert lib.iqp_rope_cos_sin_table(10000.0, 10, 63, P(16), None) == iqp.IQP_ERR_INVALID
    assert lib.iqp_rope_cos_sin_table(-1.0, 10, 64, P(16), None) == iqp.IQP_ERR_INVALID
    assert lib.iqp_rope_cos_sin_table(10000.0, 10, 64, P(0), None) == iqp.IQP_ERR_INVALID
    assert lib.iqp_rope_cos_sin_table(10000.0, 0, 64, P(0), None) == iqp.IQP_OK


def fused_lanes(iqp, M=4, K=256, H=2, D=128, rd=64, lda=256, cs=16, lanes=16, q=16):
    return iqp._lib.indexer_q_gemm_rope_fp4_lanes(P(16), lda, P(16), 1, 1, P(16), 256, P(16), M, K, H, D, rd,
                                                  P(16), P(cs), P(lanes), 10, P(q), P(16), None)


def test_lane_table_argument_checks(iqp):
    lib, inv, uns = iqp._lib, iqp.IQP_ERR_INVALID, iqp.IQP_ERR_UNSUPPORTED
    assert lib.iqp_rope_table_lanes(P(16), -1, 64, P(16), None) == inv
    assert lib.iqp_rope_table_lanes(P(16), 10, -1, P(16), None) == inv
    assert lib.iqp_rope_table_lanes(P(0), 10, 64, P(16), None) == inv
    assert lib.iqp_rope_table_lanes(P(16), 10, 64, P(0), None) == inv
    assert lib.iqp_rope_table_lanes(P(16), 10, 32, P(16), None) == uns   # the copy is laid out for 64 columns
    assert lib.iqp_rope_table_lanes(P(8), 10, 64, P(16), None) == uns
    assert lib.iqp_rope_table_lanes(P(16), 10, 64, P(24), None) == uns
    assert lib.iqp_rope_table_lanes(P(0), 0, 64, P(0), None) == iqp.IQP_OK   # empty table: no-op
    assert fused_lanes(iqp, lanes=0) == inv
    assert fused_lanes(iqp, lanes=8) == uns
    assert fused_lanes(iqp, M=-3) == inv                       # the base call's checks still apply
    assert fused_lanes(iqp, cs=0) == inv
    assert fused_lanes(iqp, lda=128) == inv
    assert fused_lanes(iqp, D=64) == uns
    assert fused_lanes(iqp, q=20) == uns
    assert fused_lanes(iqp, M=0, lanes=0) == iqp.IQP_OK        # M = 0: no-op


def epilogue(iqp, q=16, ldq=256, M=4, H=2, D=128, rd=64, pos=16, cs=16, mp=10, out=16, sc=16, flags=0):
    return iqp._lib.indexer_q_rope_hadamard_fp4(P(q), ldq, M, H, D, rd, P(pos), P(cs), mp, P(out), P(sc), flags,
                                                None)


def test_epilogue_argument_checks(iqp):
    inv, uns = iqp.IQP_ERR_INVALID, iqp.IQP_ERR_UNSUPPORTED
    assert epilogue(iqp, M=0, q=0) == iqp.IQP_OK                  # M == 0: no-op before pointer checks
    assert epilogue(iqp, M=-1) == inv
    assert epilogue(iqp, q=0) == inv
    assert epilogue(iqp, pos=0) == inv
    assert epilogue(iqp, out=0) == inv
    assert epilogue(iqp, H=0) == inv
    assert epilogue(iqp, mp=0) == inv
    assert epilogue(iqp, ldq=255) == inv                          # row stride below H * 128
    assert epilogue(iqp, D=64, ldq=128) == uns
    assert epilogue(iqp, rd=32) == uns
    assert epilogue(iqp, q=8) == uns                              # bf16 input must be 16-byte aligned
    assert epilogue(iqp, ldq=260) == uns                          # row stride not a multiple of 8
    assert epilogue(iqp, cs=8) == uns
    assert epilogue(iqp, out=2) == uns
    assert epilogue(iqp, out=8) == uns                            # codes are stored 16 bytes at a time
    assert epilogue(iqp, flags=4) == inv                          # unknown convention bit
    assert epilogue(iqp, flags=-1) == inv


def prep(iqp, x=16, ldx=1536, w=16, ldw=1536, ws=16, M=4, K=1536, H=2, D=128, rd=64, pos=16, cs=16, mp=10,
         out=16, sc=16):
    return iqp._lib.indexer_q_prep_bf16(P(x), ldx, P(w), ldw, P(ws), M, K, H, D, rd, P(pos), P(cs), mp,
                                        P(out), P(sc), None)


def test_one_launch_argument_checks(iqp):
    inv, uns = iqp.IQP_ERR_INVALID, iqp.IQP_ERR_UNSUPPORTED
    assert prep(iqp, M=0, x=0) == iqp.IQP_OK
    assert prep(iqp, M=-1) == inv
    assert prep(iqp, x=0) == inv
    assert prep(iqp, w=0) == inv
    assert prep(iqp, out=0) == inv
    assert prep(iqp, ldx=1535) == inv
    assert prep(iqp, ldw=1024) == inv
    assert prep(iqp, M=257) == uns                 # more tokens: the two-call path
    assert prep(iqp, K=1024, ldx=1024, ldw=1024) == uns
    assert prep(iqp, D=64) == uns
    assert prep(iqp, x=8) == uns                   # bf16 rows must be 16-byte aligned
    assert prep(iqp, ldx=1540) == uns
    assert prep(iqp, ws=2) == uns                  # weight scales are read four at a time
    assert prep(iqp, out=4) == uns


def wq(iqp, w=16, N=256, K=384, ldw=384, q=16, ldq=384, s=16, lds=3):
    return iqp._lib.fp8_quant_weight_128x128_ue8m0(P(w), N, K, ldw, P(q), ldq, P(s), lds, None)


def test_weight_quant_argument_checks(iqp):
    inv, uns = iqp.IQP_ERR_INVALID, iqp.IQP_ERR_UNSUPPORTED
    assert wq(iqp, N=0, w=0) == iqp.IQP_OK
    assert wq(iqp, N=-128) == inv
    assert wq(iqp, w=0) == inv
    assert wq(iqp, s=0) == inv
    assert wq(iqp, ldw=256) == inv
    assert wq(iqp, ldq=256) == inv
    assert wq(iqp, lds=2) == inv
    assert wq(iqp, N=200) == uns
    assert wq(iqp, K=200, ldw=384, ldq=384, lds=2) == uns
    assert wq(iqp, w=8) == uns
    assert wq(iqp, ldw=388) == uns
    assert wq(iqp, q=4) == uns


def test_python_wrapper_rejects_wrong_dtypes(iqp):
    import torch
    with pytest.raises(TypeError):
        iqp.fp8_quant_1x128_ue8m0(torch.zeros(2, 128, dtype=torch.float32))


# ---------------------------------------------------------------- binding shape checks
#
# The C ABI takes row strides, not buffer sizes, so an output or scale buffer
# with too few rows or words could only be caught by the binding: it must
# raise before any launch. CPU tensors are used; every case fails in Python.


def test_binding_rejects_undersized_quant_outputs(iqp):
    import torch
    x = torch.zeros((4, 1536), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="q must be"):
        iqp.fp8_quant_1x128_ue8m0(x, q=torch.empty((3, 1536), dtype=torch.uint8))
    with pytest.raises(ValueError, match="q must be"):
        iqp.fp8_quant_1x128_ue8m0(x, q=torch.empty((4, 1024), dtype=torch.uint8))
    with pytest.raises(ValueError, match="scales must be"):
        iqp.fp8_quant_1x128_ue8m0(x, q=torch.empty((4, 1536), dtype=torch.uint8),
                                  scales=torch.empty((3, 3), dtype=torch.int32))
    with pytest.raises(ValueError, match="scales must be"):
        iqp.fp8_quant_1x128_ue8m0(x, q=torch.empty((4, 1536), dtype=torch.uint8),
                                  scales=torch.empty((4, 2), dtype=torch.int32))


def test_binding_rejects_short_activation_scale_rows(iqp):
    import torch
    M, K, H = 1, 1536, 2
    a = torch.zeros((M, K), dtype=torch.uint8)
    w = torch.zeros((H * 128, K), dtype=torch.uint8)
    ws = torch.zeros((H, K // 128), dtype=torch.uint8)
    pos = torch.zeros((M,), dtype=torch.int64)
    cs = torch.zeros((16, 64), dtype=torch.float32)
    # [M, 1] words for K = 1536 (12 blocks need 3 words): the kernel would read past them
    with pytest.raises(ValueError, match="a_scales must be"):
        iqp.indexer_q_gemm_rope_fp4(a, torch.zeros((M, 1), dtype=torch.int32), w, ws, pos, cs, n_heads=H)
    with pytest.raises(ValueError, match="a_scales must be"):
        iqp.debug_indexer_q_f32(a, torch.zeros((M, 2), dtype=torch.int32), w, ws, pos, cs, stage=0, n_heads=H)


def clock(iqp, M=2048, K=1536, H=64, stamps=16, cap=1024, nwg=True, q=16, qs=16, lanes=0):
    n = ctypes.c_int64(-1)
    st = iqp._lib.iqp_debug_indexer_q_clock(P(16), K, P(16), 3, 1, P(16), K, P(16), M, K, H, 128, 64,
                                            P(16), P(16), P(lanes), 10, P(q), P(qs), P(stamps), cap,
                                            ctypes.byref(n) if nwg else None, None)
    return st, n.value


def test_clock_and_debug_argument_checks(iqp):
    assert clock(iqp, nwg=False)[0] == iqp.IQP_ERR_INVALID
    assert clock(iqp, cap=-1) == (iqp.IQP_ERR_INVALID, 0)
    assert clock(iqp, M=-1) == (iqp.IQP_ERR_INVALID, 0)
    assert clock(iqp, q=0) == (iqp.IQP_ERR_INVALID, 0)
    assert clock(iqp, stamps=0) == (iqp.IQP_ERR_INVALID, 0)
    assert clock(iqp, stamps=24) == (iqp.IQP_ERR_UNSUPPORTED, 0)   # stamps not 16-byte aligned
    assert clock(iqp, M=0) == (iqp.IQP_ERR_UNSUPPORTED, 0)
    assert clock(iqp, lanes=8) == (iqp.IQP_ERR_UNSUPPORTED, 0)     # the lane-ordered copy not 16-byte aligned
    lib = iqp._lib
    assert lib.iqp_device_clock_rates(None, None) == iqp.IQP_ERR_INVALID
    # the debug GEMM stage 3 and the one-launch twin reject before any device call
    assert lib.iqp_debug_indexer_q_f32(P(16), 256, P(16), 1, 1, P(16), 256, P(16), 4, 256, 2, 128, 64,
                                       P(16), P(16), 10, P(16), 4, None) == iqp.IQP_ERR_INVALID
    assert lib.iqp_debug_indexer_q_f32(P(16), 256, P(16), 1, 1, P(16), 256, P(16), 4, 256, 2, 128, 64,
                                       P(16), P(16), 10, P(0), 3, None) == iqp.IQP_ERR_INVALID
    bf16 = lambda M=4, K=1536, x=16, out=16: lib.iqp_debug_indexer_q_prep_bf16_f32(
        P(x), K, P(16), K, P(16), M, K, 64, 128, 64, P(16), P(16), 10, P(out), None)
    assert bf16(M=-1) == iqp.IQP_ERR_INVALID
    assert bf16(x=0) == iqp.IQP_ERR_INVALID
    assert bf16(out=0) == iqp.IQP_ERR_INVALID
    assert bf16(M=257) == iqp.IQP_ERR_UNSUPPORTED
    assert bf16(K=1024) == iqp.IQP_ERR_UNSUPPORTED
    assert bf16(out=24) == iqp.IQP_ERR_UNSUPPORTED
    assert bf16(M=0) == iqp.IQP_OK
