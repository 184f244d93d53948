"""DeepSeek-V4 indexer-Q preparation on AMD Instinct MI355X (gfx950).

Thin Python binding over ``libiqprep.so`` (C ABI in ``include/iqprep.h``).
This module only checks and marshals arguments: every step of the path runs
in the library's HIP kernels, on torch's current stream. Torch provides device
memory and streams, nothing else.

If the library has not been built, importing this package raises ImportError
(build it with ``python fp4_quantized_prep_amd/build.py``); there is no
fallback implementation.
"""
import contextlib
import ctypes
import functools
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libiqprep.so")

__all__ = [
    "IqpError", "fp8_quant_1x128_ue8m0", "indexer_q_gemm_rope_fp4", "rope_cos_sin_table",
    "debug_indexer_q_f32", "debug_indexer_q_prep_bf16_f32", "debug_indexer_q_clock", "device_clock_rates",
    "indexer_q_rope_hadamard_fp4", "indexer_q_prep_bf16", "indexer_q_prep", "fp8_quant_weight_128x128_ue8m0", "abi_version", "library_path",
    "rope_table_lanes", "rope_table_lanes_size", "indexer_q_workspace_bytes", "indexer_q_workspace",
    "IQP_OK", "IQP_ERR_INVALID", "IQP_ERR_UNSUPPORTED", "IQP_ERR_HIP", "ONE_LAUNCH_MAX_TOKENS",
    "ONE_LAUNCH_WITH_QUANT_MAX_TOKENS", "ONE_LAUNCH_WITH_WORKSPACE_MAX_TOKENS",
    "IQP_ROPE_INTERLEAVED", "IQP_FP4_SCALE_OCP_FLOOR", "IQP_W_SCALES_PER_ROW", "IQP_NOALLOC_MAX_HEADS",
]

#: Up to this many tokens indexer_q_prep takes the one-launch path (measured on
#: MI355X: faster there; from 32 tokens the two calls are as fast or faster).
ONE_LAUNCH_MAX_TOKENS = 16

#: Up to this many tokens a decode step that also quantizes an independent
#: [M, 7168] activation is faster as one launch (indexer_q_prep_bf16 with
#: quant_beside) than as three (quantize, fused call, quantize): measured on
#: MI355X, 9.6 vs 11.2 us at 32 tokens, 11.8 vs 12.4 at 128, 17.9 vs 17.2 at 192.
ONE_LAUNCH_WITH_QUANT_MAX_TOKENS = 128

#: With a split-K workspace indexer_q_prep takes the one-launch path up to this
#: many tokens (measured on MI355X, Q preparation alone, weights hot / cold in
#: HBM: 32 tokens 8.3 / 9.1 us against 8.9 / 11.7 for the two calls, 64 tokens
#: 9.2 / 10.4 against 9.0 / 11.5).
ONE_LAUNCH_WITH_WORKSPACE_MAX_TOKENS = 64

#: Heads the allocation-free call's scratch holds (IQP_NOALLOC_MAX_HEADS).
IQP_NOALLOC_MAX_HEADS = 64

IQP_ROPE_INTERLEAVED = 0x1
IQP_FP4_SCALE_OCP_FLOOR = 0x2
IQP_W_SCALES_PER_ROW = 0x4

IQP_OK = 0
IQP_ERR_INVALID = 1
IQP_ERR_UNSUPPORTED = 2
IQP_ERR_HIP = 3


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python fp4_quantized_prep_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    c_i64, c_i32, c_p, c_dbl = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_double
    lib.fp8_quant_1x128_ue8m0.argtypes = [c_p, c_i64, c_i64, c_i64, c_p, c_i64, c_p, c_i64, c_i64, c_p]
    lib.fp8_quant_1x128_ue8m0.restype = ctypes.c_int
    iq_args = [c_p, c_i64, c_p, c_i64, c_i64, c_p, c_i64, c_p, c_i64, c_i64, c_i32, c_i32, c_i32,
               c_p, c_p, c_i64]
    lib.indexer_q_gemm_rope_fp4.argtypes = iq_args + [c_p, c_p, c_p]
    lib.indexer_q_gemm_rope_fp4.restype = ctypes.c_int
    lib.indexer_q_gemm_rope_fp4_ex.argtypes = iq_args + [c_p, c_p, c_i32, c_p]
    lib.indexer_q_gemm_rope_fp4_ex.restype = ctypes.c_int
    lib.indexer_q_gemm_rope_fp4_lanes.argtypes = iq_args[:-1] + [c_p, c_i64, c_p, c_p, c_p]
    lib.indexer_q_gemm_rope_fp4_lanes.restype = ctypes.c_int
    lib.iqp_rope_table_lanes.argtypes = [c_p, c_i64, c_i32, c_p, c_p]
    lib.iqp_rope_table_lanes.restype = ctypes.c_int
    lib.iqp_debug_indexer_q_f32.argtypes = iq_args + [c_p, c_i32, c_p]
    lib.iqp_debug_indexer_q_f32.restype = ctypes.c_int
    lib.indexer_q_prep_bf16.argtypes = [c_p, c_i64, c_p, c_i64, c_p, c_i64, c_i64, c_i32, c_i32, c_i32,
                                         c_p, c_p, c_i64, c_p, c_p, c_p]
    lib.indexer_q_prep_bf16.restype = ctypes.c_int
    lib.indexer_q_prep_bf16_ex.argtypes = lib.indexer_q_prep_bf16.argtypes[:-1] + [c_i32, c_p]
    lib.indexer_q_prep_bf16_ex.restype = ctypes.c_int
    lib.indexer_q_prep_bf16_with_quant.argtypes = lib.indexer_q_prep_bf16.argtypes[:-1] + \
        [c_p, c_i64, c_i64, c_i64, c_p, c_i64, c_p, c_i64, c_i64, c_p]
    lib.indexer_q_prep_bf16_with_quant.restype = ctypes.c_int
    lib.indexer_q_prep_bf16_with_quant_ws.argtypes = lib.indexer_q_prep_bf16_with_quant.argtypes[:-1] + \
        [c_p, c_i64, c_p]
    lib.indexer_q_prep_bf16_with_quant_ws.restype = ctypes.c_int
    lib.indexer_q_prep_bf16_with_quant_noalloc.argtypes = lib.indexer_q_prep_bf16_with_quant.argtypes
    lib.indexer_q_prep_bf16_with_quant_noalloc.restype = ctypes.c_int
    lib.indexer_q_workspace_bytes.argtypes = [c_i32]
    lib.indexer_q_workspace_bytes.restype = c_i64
    lib.fp8_quant_weight_128x128_ue8m0.argtypes = [c_p, c_i64, c_i64, c_i64, c_p, c_i64, c_p, c_i64, c_p]
    lib.fp8_quant_weight_128x128_ue8m0.restype = ctypes.c_int
    lib.indexer_q_rope_hadamard_fp4.argtypes = [c_p, c_i64, c_i64, c_i32, c_i32, c_i32, c_p, c_p, c_i64,
                                                 c_p, c_p, c_i32, c_p]
    lib.indexer_q_rope_hadamard_fp4.restype = ctypes.c_int
    lib.iqp_rope_cos_sin_table.argtypes = [c_dbl, c_i64, c_i32, c_p, c_p]
    lib.iqp_rope_cos_sin_table.restype = ctypes.c_int
    lib.iqp_status_string.argtypes = [ctypes.c_int]
    lib.iqp_status_string.restype = ctypes.c_char_p
    lib.iqp_abi_version.argtypes = []
    lib.iqp_abi_version.restype = ctypes.c_int
    lib.iqp_debug_indexer_q_prep_bf16_f32.argtypes = lib.indexer_q_prep_bf16.argtypes[:-3] + [c_p, c_p]
    lib.iqp_debug_indexer_q_prep_bf16_f32.restype = ctypes.c_int
    lib.iqp_debug_indexer_q_clock.argtypes = iq_args[:-1] + [c_p, c_i64] + [c_p, c_p, c_p, c_i64, c_p, c_p]
    lib.iqp_debug_indexer_q_clock.restype = ctypes.c_int
    lib.iqp_device_clock_rates.argtypes = [c_p, c_p]
    lib.iqp_device_clock_rates.restype = ctypes.c_int
    return lib


_lib = _load()


class IqpError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {_lib.iqp_status_string(status).decode()} (status {status})")


def _check(status: int, where: str):
    if status != IQP_OK:
        raise IqpError(status, where)


def library_path() -> str:
    return LIB_PATH


def abi_version() -> int:
    return _lib.iqp_abi_version()


def _stream(t: torch.Tensor, stream=None):
    if stream is None:
        stream = torch.cuda.current_stream(t.device)
    return ctypes.c_void_p(stream.cuda_stream)


def _on_stream(fn):
    """Run a wrapper with its explicit ``stream`` (if any) current, so that
    every tensor it allocates (outputs, the preparation's FP8 intermediates)
    comes from that stream's pool: the caching allocator then never hands
    that memory to another stream while the call's kernels may still use it."""
    @functools.wraps(fn)
    def wrapper(*args, stream=None, **kwargs):
        ctx = torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext()
        with ctx:
            return fn(*args, stream=stream, **kwargs)
    return wrapper


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _require(t: torch.Tensor, name: str, dtype, device: torch.device, ndim: int):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must have dtype {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must be {ndim}-D, got shape {tuple(t.shape)}")


def _bytes_u8(t: torch.Tensor) -> torch.Tensor:
    return t.view(torch.uint8) if t.dtype == torch.float8_e4m3fn else t


@_on_stream
def fp8_quant_1x128_ue8m0(x: torch.Tensor, scale_layout: str = "k", q: torch.Tensor = None,
                          scales: torch.Tensor = None, stream=None):
    """Packed-UE8M0 FP8 1x128 quantization of a bf16 [M, K] matrix.

    Returns ``(q, scales)``: q is uint8 [M, K] holding E4M3 codes and scales is
    an int32 [M, ceil(K/512)] view of the packed UE8M0 words. With
    ``scale_layout="k"`` the words are row-major (K-major); with ``"mn"`` the
    storage is [ceil(K/512), M rounded up to 4] and the returned view has
    strides (1, M_pad). Pre-allocated ``q`` / ``scales`` may be passed in.
    """
    q, scales = _quant_outputs(x, scale_layout, q, scales)
    M, K = x.shape
    st = _lib.fp8_quant_1x128_ue8m0(_ptr(x), M, K, x.stride(0), _ptr(q), q.stride(0), _ptr(scales),
                                    scales.stride(0), scales.stride(1), _stream(x, stream))
    _check(st, "fp8_quant_1x128_ue8m0")
    return q, scales


def _quant_outputs(x, scale_layout, q, scales):
    """Checks of a quantization's input and outputs (allocated when None)."""
    if not isinstance(x, torch.Tensor) or x.dim() != 2:
        raise ValueError("x must be a 2-D tensor")
    dev = x.device
    _require(x, "x", torch.bfloat16, dev, 2)
    if x.stride(1) != 1:
        raise ValueError("x rows must be contiguous")
    M, K = x.shape
    nw = (K // 128 + 3) // 4
    if q is None:
        q = torch.empty((M, K), dtype=torch.uint8, device=dev)
    q = _bytes_u8(q)
    _require(q, "q", torch.uint8, dev, 2)
    if tuple(q.shape) != (M, K) or q.stride(1) != 1:
        raise ValueError(f"q must be [{M}, {K}] with contiguous rows, got shape {tuple(q.shape)}")
    if scales is None:
        if scale_layout == "k":
            scales = torch.empty((M, nw), dtype=torch.int32, device=dev)
        elif scale_layout == "mn":
            m_pad = max(4, (M + 3) // 4 * 4)
            scales = torch.empty((nw, m_pad), dtype=torch.int32, device=dev).t()[:M]
        else:
            raise ValueError("scale_layout must be 'k' or 'mn'")
    _require(scales, "scales", torch.int32, dev, 2)
    if tuple(scales.shape) != (M, nw):
        raise ValueError(f"scales must be [{M}, {nw}] (one packed word per 512 columns), got {tuple(scales.shape)}")
    return q, scales


@_on_stream
def fp8_quant_weight_128x128_ue8m0(w: torch.Tensor, q: torch.Tensor = None, scales: torch.Tensor = None,
                                   stream=None):
    """Weight preparation: bf16 w [N, K] (rows contiguous, N and K multiples
    of 128) -> ``(q, scales)``: uint8 E4M3 codes [N, K] and uint8 UE8M0 bytes
    [N/128, K/128], one per 128x128 tile (any row strides)."""
    dev = w.device
    _require(w, "w", torch.bfloat16, dev, 2)
    if w.stride(1) != 1:
        raise ValueError("w rows must be contiguous")
    N, K = w.shape
    if q is None:
        q = torch.empty((N, K), dtype=torch.uint8, device=dev)
    q = _bytes_u8(q)
    if scales is None:
        scales = torch.empty((N // 128, K // 128), dtype=torch.uint8, device=dev)
    _require(q, "q", torch.uint8, dev, 2)
    _require(scales, "scales", torch.uint8, dev, 2)
    if q.stride(1) != 1 or scales.stride(1) != 1 or tuple(q.shape) != (N, K) or \
            tuple(scales.shape) != (N // 128, K // 128):
        raise ValueError("q must be [N, K] and scales [N/128, K/128], rows contiguous")
    st = _lib.fp8_quant_weight_128x128_ue8m0(_ptr(w), N, K, w.stride(0), _ptr(q), q.stride(0), _ptr(scales),
                                             scales.stride(0), _stream(w, stream))
    _check(st, "fp8_quant_weight_128x128_ue8m0")
    return q, scales


def _indexer_q_common(a, a_scales, w, w_scales, positions, cos_sin, n_heads, head_dim, rope_dim,
                      w_scale_rows: bool = False):
    a = _bytes_u8(a)
    w = _bytes_u8(w)
    dev = a.device
    _require(a, "a", torch.uint8, dev, 2)
    _require(a_scales, "a_scales", torch.int32, dev, 2)
    _require(w, "w", torch.uint8, dev, 2)
    _require(w_scales, "w_scales", torch.uint8, dev, 2)
    _require(positions, "positions", torch.int64, dev, 1)
    _require(cos_sin, "cos_sin", torch.float32, dev, 2)
    if a.stride(1) != 1 or w.stride(1) != 1 or not w_scales.is_contiguous() or not positions.is_contiguous() \
            or not cos_sin.is_contiguous():
        raise ValueError("a, w need contiguous rows; w_scales, positions, cos_sin must be contiguous")
    M, K = a.shape
    if w.shape[1] != K or w.shape[0] != n_heads * head_dim:
        raise ValueError(f"w must be [{n_heads * head_dim}, {K}], got {tuple(w.shape)}")
    ws_rows = n_heads * head_dim if w_scale_rows else n_heads * head_dim // 128
    if tuple(w_scales.shape) != (ws_rows, K // 128):
        raise ValueError(f"w_scales must be [{ws_rows}, {K // 128}]")
    if positions.shape[0] != M or a_scales.shape[0] != M:
        raise ValueError("positions and a_scales need one row per token")
    nw = (K // 128 + 3) // 4
    if a_scales.shape[1] != nw:
        raise ValueError(f"a_scales must be [M, {nw}] (one packed word per 512 columns), got {tuple(a_scales.shape)}")
    if cos_sin.shape[1] != rope_dim:
        raise ValueError(f"cos_sin must have {rope_dim} columns")
    args = [_ptr(a), a.stride(0), _ptr(a_scales), a_scales.stride(0), a_scales.stride(1),
            _ptr(w), w.stride(0), _ptr(w_scales), M, K, n_heads, head_dim, rope_dim,
            _ptr(positions), _ptr(cos_sin), cos_sin.shape[0]]
    return a, args


def _convention_flags(rope_layout: str, scale_rule: str) -> int:
    if rope_layout not in ("half_split", "interleaved") or scale_rule not in ("ceil", "ocp_floor"):
        raise ValueError("rope_layout must be 'half_split' or 'interleaved', scale_rule 'ceil' or 'ocp_floor'")
    return (IQP_ROPE_INTERLEAVED if rope_layout == "interleaved" else 0) | \
        (IQP_FP4_SCALE_OCP_FLOOR if scale_rule == "ocp_floor" else 0)


@_on_stream
def indexer_q_gemm_rope_fp4(a, a_scales, w, w_scales, positions, cos_sin, n_heads: int = 64,
                            head_dim: int = 128, rope_dim: int = 64, q_fp4=None, q_scales=None,
                            rope_layout: str = "half_split", scale_rule: str = "ceil",
                            w_scale_layout: str = "tile_128x128", cos_sin_lanes=None, stream=None):
    """Fused block-scaled FP8 Q projection + RoPE + Hadamard-128 + FP4 e2m1.

    a: E4M3 [M, K] (uint8 or float8_e4m3fn) and a_scales: the packed words from
    :func:`fp8_quant_1x128_ue8m0`; w: E4M3 [H*128, K]; w_scales: uint8
    [H, K/128]; positions: int64 [M]; cos_sin: float32 [max_pos, 64].
    Returns ``(q_fp4, q_scales)``: uint8 [M, H, 64] packed codes and uint8
    [M, H, 4] UE8M0 scale bytes. rope_layout "interleaved" / scale_rule
    "ocp_floor" / w_scale_layout "row_1x128" (w_scales uint8 [H*128, K/128])
    select the convention variants (indexer_q_gemm_rope_fp4_ex).
    cos_sin_lanes: the table's lane-ordered copy from :func:`rope_table_lanes`
    (default conventions only; indexer_q_gemm_rope_fp4_lanes): the same
    output, faster for prefill batches whose positions run consecutively.
    """
    if w_scale_layout not in ("tile_128x128", "row_1x128"):
        raise ValueError("w_scale_layout must be 'tile_128x128' or 'row_1x128'")
    rows = w_scale_layout == "row_1x128"
    flags = _convention_flags(rope_layout, scale_rule) | (IQP_W_SCALES_PER_ROW if rows else 0)
    a, args = _indexer_q_common(a, a_scales, w, w_scales, positions, cos_sin, n_heads, head_dim, rope_dim, rows)
    M = a.shape[0]
    dev = a.device
    if q_fp4 is None:
        q_fp4 = torch.empty((M, n_heads, head_dim // 2), dtype=torch.uint8, device=dev)
    if q_scales is None:
        q_scales = torch.empty((M, n_heads, head_dim // 32), dtype=torch.uint8, device=dev)
    _require(q_fp4, "q_fp4", torch.uint8, dev, 3)
    _require(q_scales, "q_scales", torch.uint8, dev, 3)
    if not (q_fp4.is_contiguous() and q_scales.is_contiguous()):
        raise ValueError("q_fp4 and q_scales must be contiguous")
    if tuple(q_fp4.shape) != (M, n_heads, head_dim // 2) or tuple(q_scales.shape) != (M, n_heads, head_dim // 32):
        raise ValueError("q_fp4 / q_scales have the wrong shape")
    if cos_sin_lanes is not None:
        if flags != 0:
            raise ValueError("cos_sin_lanes serves the default conventions only")
        _require(cos_sin_lanes, "cos_sin_lanes", torch.float32, dev, 1)
        if not cos_sin_lanes.is_contiguous() or cos_sin_lanes.numel() < rope_table_lanes_size(cos_sin.shape[0]):
            raise ValueError("cos_sin_lanes must be the contiguous copy rope_table_lanes builds from cos_sin")
        st = _lib.indexer_q_gemm_rope_fp4_lanes(*args[:-1], _ptr(cos_sin_lanes), args[-1], _ptr(q_fp4),
                                                _ptr(q_scales), _stream(a, stream))
        _check(st, "indexer_q_gemm_rope_fp4_lanes")
    elif flags == 0:
        st = _lib.indexer_q_gemm_rope_fp4(*args, _ptr(q_fp4), _ptr(q_scales), _stream(a, stream))
        _check(st, "indexer_q_gemm_rope_fp4")
    else:
        st = _lib.indexer_q_gemm_rope_fp4_ex(*args, _ptr(q_fp4), _ptr(q_scales), flags, _stream(a, stream))
        _check(st, "indexer_q_gemm_rope_fp4_ex")
    return q_fp4, q_scales


@_on_stream
def debug_indexer_q_f32(a, a_scales, w, w_scales, positions, cos_sin, stage: int, n_heads: int = 64,
                        head_dim: int = 128, rope_dim: int = 64, out=None, stream=None):
    """float32 [M, H*128] after stage 0 (GEMM), 1 (RoPE) or 2 (Hadamard) of the
    general fused kernel, or the GEMM output (stage 3) of the kernel that
    :func:`indexer_q_gemm_rope_fp4` runs for these arguments, for stage-wise
    parity checks."""
    a, args = _indexer_q_common(a, a_scales, w, w_scales, positions, cos_sin, n_heads, head_dim, rope_dim)
    M = a.shape[0]
    if out is None:
        out = torch.empty((M, n_heads * head_dim), dtype=torch.float32, device=a.device)
    _require(out, "out", torch.float32, a.device, 2)
    if not out.is_contiguous() or tuple(out.shape) != (M, n_heads * head_dim):
        raise ValueError("out must be a contiguous [M, H*128] float32 tensor")
    st = _lib.iqp_debug_indexer_q_f32(*args, _ptr(out), stage, _stream(a, stream))
    _check(st, "iqp_debug_indexer_q_f32")
    return out


@_on_stream
def indexer_q_rope_hadamard_fp4(q, positions, cos_sin, n_heads: int = 64, head_dim: int = 128,
                                rope_dim: int = 64, q_fp4=None, q_scales=None, rope_layout: str = "half_split",
                                scale_rule: str = "ceil", stream=None):
    """Standalone epilogue over a bf16 Q [M, H*128] (rows contiguous, any row
    stride): RoPE on each head's first 64 dims, Hadamard-128, FP4 e2m1.
    Returns ``(q_fp4, q_scales)`` laid out as :func:`indexer_q_gemm_rope_fp4`'s.
    rope_layout "interleaved" pairs dims (2i, 2i+1); scale_rule "ocp_floor"
    takes the OCP MX scale rule (codes saturate at 6)."""
    flags = _convention_flags(rope_layout, scale_rule)
    dev = q.device
    _require(q, "q", torch.bfloat16, dev, 2)
    _require(positions, "positions", torch.int64, dev, 1)
    _require(cos_sin, "cos_sin", torch.float32, dev, 2)
    if q.stride(1) != 1 or not positions.is_contiguous() or not cos_sin.is_contiguous():
        raise ValueError("q needs contiguous rows; positions and cos_sin must be contiguous")
    M = q.shape[0]
    if q.shape[1] != n_heads * head_dim:
        raise ValueError(f"q must be [M, {n_heads * head_dim}], got {tuple(q.shape)}")
    if positions.shape[0] != M:
        raise ValueError("positions needs one entry per token")
    if cos_sin.shape[1] != rope_dim:
        raise ValueError(f"cos_sin must have {rope_dim} columns")
    if q_fp4 is None:
        q_fp4 = torch.empty((M, n_heads, head_dim // 2), dtype=torch.uint8, device=dev)
    if q_scales is None:
        q_scales = torch.empty((M, n_heads, head_dim // 32), dtype=torch.uint8, device=dev)
    _require(q_fp4, "q_fp4", torch.uint8, dev, 3)
    _require(q_scales, "q_scales", torch.uint8, dev, 3)
    if not (q_fp4.is_contiguous() and q_scales.is_contiguous()):
        raise ValueError("q_fp4 and q_scales must be contiguous")
    if tuple(q_fp4.shape) != (M, n_heads, head_dim // 2) or tuple(q_scales.shape) != (M, n_heads, head_dim // 32):
        raise ValueError("q_fp4 / q_scales have the wrong shape")
    st = _lib.indexer_q_rope_hadamard_fp4(_ptr(q), q.stride(0), M, n_heads, head_dim, rope_dim, _ptr(positions),
                                          _ptr(cos_sin), cos_sin.shape[0], _ptr(q_fp4), _ptr(q_scales), flags,
                                          _stream(q, stream))
    _check(st, "indexer_q_rope_hadamard_fp4")
    return q_fp4, q_scales


@_on_stream
def rope_cos_sin_table(theta: float, max_pos: int, rope_dim: int = 64, device=None, out=None, stream=None):
    """float32 [max_pos, rope_dim] table of cos (first half) and sin (second
    half) of pos * theta^(-2i/rope_dim), computed on the device in float64."""
    if out is None:
        out = torch.empty((max_pos, rope_dim), dtype=torch.float32,
                          device=device if device is not None else "cuda")
    _require(out, "out", torch.float32, out.device, 2)
    if not out.is_contiguous() or tuple(out.shape) != (max_pos, rope_dim):
        raise ValueError("out must be a contiguous [max_pos, rope_dim] float32 tensor")
    st = _lib.iqp_rope_cos_sin_table(float(theta), max_pos, rope_dim, _ptr(out), _stream(out, stream))
    _check(st, "iqp_rope_cos_sin_table")
    return out


def rope_table_lanes_size(max_pos: int) -> int:
    """float32 elements of the lane-ordered copy of a [max_pos, 64] table."""
    return (max_pos + 31) // 32 * 2048


@_on_stream
def rope_table_lanes(cos_sin, out=None, stream=None):
    """The lane-ordered copy of a float32 [max_pos, 64] RoPE table that
    :func:`indexer_q_gemm_rope_fp4` takes as ``cos_sin_lanes`` (the same
    values rearranged, iqp_rope_table_lanes): a 1-D float32 tensor of
    :func:`rope_table_lanes_size` elements. Build it once per table."""
    dev = cos_sin.device
    _require(cos_sin, "cos_sin", torch.float32, dev, 2)
    if not cos_sin.is_contiguous():
        raise ValueError("cos_sin must be contiguous")
    max_pos, rope_dim = cos_sin.shape
    n = rope_table_lanes_size(max_pos)
    if out is None:
        out = torch.empty((n,), dtype=torch.float32, device=dev)
    _require(out, "out", torch.float32, dev, 1)
    if not out.is_contiguous() or out.numel() != n:
        raise ValueError(f"out must be a contiguous float32 tensor of {n} elements")
    st = _lib.iqp_rope_table_lanes(_ptr(cos_sin), max_pos, rope_dim, _ptr(out), _stream(cos_sin, stream))
    _check(st, "iqp_rope_table_lanes")
    return out


@_on_stream
def indexer_q_prep_bf16(x, w, w_scales, positions, cos_sin, n_heads: int = 64, head_dim: int = 128,
                        rope_dim: int = 64, q_fp4=None, q_scales=None, rope_layout: str = "half_split",
                        scale_rule: str = "ceil", w_scale_layout: str = "tile_128x128", quant_beside=None,
                        quant_beside_out=None, quant_beside_layout: str = "k", workspace=None,
                        no_alloc: bool = False, stream=None):
    """The whole preparation in one launch for up to 256 tokens (K = 1536):
    bf16 x [M, K] -> FP8 quantization (in the kernel, never stored) -> fused
    projection / RoPE / Hadamard / FP4. Returns ``(q_fp4, q_scales)``. The
    convention arguments are those of :func:`indexer_q_gemm_rope_fp4`
    (indexer_q_prep_bf16_ex).

    quant_beside: an independent bf16 [M2, K2] matrix (M2 <= 256) quantized
    as :func:`fp8_quant_1x128_ue8m0` would, in the same launch
    (indexer_q_prep_bf16_with_quant; default conventions only); the call then
    returns ``(q_fp4, q_scales, q2, scales2)``. quant_beside_out: preallocated
    ``(q2, scales2)``; quant_beside_layout: their words' layout ("k" or "mn")
    when allocated here.

    workspace: a uint8 device tensor from :func:`indexer_q_workspace` (zero
    before its first use; every call leaves it so): up to 64 tokens the
    kernel then splits each head's K range over 2 or 4 workgroups
    (indexer_q_prep_bf16_with_quant_ws; default conventions only). Calls
    sharing a workspace must not run concurrently.

    no_alloc: the same split with the library's own per-GPU scratch instead
    of a workspace (indexer_q_prep_bf16_with_quant_noalloc: the C call
    allocates nothing; up to IQP_NOALLOC_MAX_HEADS heads). Such calls must not
    overlap on one GPU. (Outputs not given are still allocated here.)"""
    if w_scale_layout not in ("tile_128x128", "row_1x128"):
        raise ValueError("w_scale_layout must be 'tile_128x128' or 'row_1x128'")
    rows = w_scale_layout == "row_1x128"
    flags = _convention_flags(rope_layout, scale_rule) | (IQP_W_SCALES_PER_ROW if rows else 0)
    args = _prep_bf16_common(x, w, w_scales, positions, cos_sin, n_heads, head_dim, rope_dim, rows)
    M, dev = x.shape[0], x.device
    if q_fp4 is None:
        q_fp4 = torch.empty((M, n_heads, head_dim // 2), dtype=torch.uint8, device=dev)
    if q_scales is None:
        q_scales = torch.empty((M, n_heads, head_dim // 32), dtype=torch.uint8, device=dev)
    _require(q_fp4, "q_fp4", torch.uint8, dev, 3)
    _require(q_scales, "q_scales", torch.uint8, dev, 3)
    if not (q_fp4.is_contiguous() and q_scales.is_contiguous()):
        raise ValueError("q_fp4 and q_scales must be contiguous")
    if tuple(q_fp4.shape) != (M, n_heads, head_dim // 2) or tuple(q_scales.shape) != (M, n_heads, head_dim // 32):
        raise ValueError("q_fp4 / q_scales have the wrong shape")
    args += [_ptr(q_fp4), _ptr(q_scales)]
    if no_alloc and workspace is not None:
        raise ValueError("no_alloc uses the library's scratch: pass no workspace")
    if workspace is not None or no_alloc:
        if flags != 0:
            raise ValueError("workspace / no_alloc serve the default conventions only")
    if workspace is not None:
        _require(workspace, "workspace", torch.uint8, dev, 1)
        if not workspace.is_contiguous() or workspace.numel() < indexer_q_workspace_bytes(n_heads):
            raise ValueError(f"workspace must be a contiguous uint8 tensor of at least "
                             f"{indexer_q_workspace_bytes(n_heads)} bytes (indexer_q_workspace)")
    if quant_beside is not None or workspace is not None or no_alloc:
        if flags != 0:
            raise ValueError("quant_beside serves the default conventions only")
        if quant_beside is not None:
            q2, s2 = quant_beside_out if quant_beside_out is not None else (None, None)
            q2, s2 = _quant_outputs(quant_beside, quant_beside_layout, q2, s2)
            if quant_beside.device != dev:
                raise ValueError("quant_beside must be on the device of x")
            M2, K2 = quant_beside.shape
            side = [_ptr(quant_beside), M2, K2, quant_beside.stride(0), _ptr(q2), q2.stride(0), _ptr(s2),
                    s2.stride(0), s2.stride(1)]
        else:
            side = [None, 0, 0, 0, None, 0, None, 0, 0]
        if workspace is not None:
            st = _lib.indexer_q_prep_bf16_with_quant_ws(*args, *side, _ptr(workspace), workspace.numel(),
                                                        _stream(x, stream))
            _check(st, "indexer_q_prep_bf16_with_quant_ws")
        elif no_alloc:
            st = _lib.indexer_q_prep_bf16_with_quant_noalloc(*args, *side, _stream(x, stream))
            _check(st, "indexer_q_prep_bf16_with_quant_noalloc")
        else:
            st = _lib.indexer_q_prep_bf16_with_quant(*args, *side, _stream(x, stream))
            _check(st, "indexer_q_prep_bf16_with_quant")
        return (q_fp4, q_scales, q2, s2) if quant_beside is not None else (q_fp4, q_scales)
    if flags == 0:
        st = _lib.indexer_q_prep_bf16(*args, _stream(x, stream))
        _check(st, "indexer_q_prep_bf16")
    else:
        st = _lib.indexer_q_prep_bf16_ex(*args, flags, _stream(x, stream))
        _check(st, "indexer_q_prep_bf16_ex")
    return q_fp4, q_scales


def indexer_q_workspace_bytes(n_heads: int = 64) -> int:
    """Bytes of the split-K workspace for n_heads heads (indexer_q_workspace_bytes)."""
    return int(_lib.indexer_q_workspace_bytes(n_heads))


def indexer_q_workspace(n_heads: int = 64, device=None):
    """A zeroed workspace for :func:`indexer_q_prep_bf16` (``workspace=``)."""
    return torch.zeros(indexer_q_workspace_bytes(n_heads), dtype=torch.uint8, device=device)


def _prep_bf16_common(x, w, w_scales, positions, cos_sin, n_heads, head_dim, rope_dim, w_scale_rows):
    """Checks of the one-launch call's inputs; its C arguments up to max_pos."""
    w = _bytes_u8(w)
    dev = x.device
    _require(x, "x", torch.bfloat16, dev, 2)
    _require(w, "w", torch.uint8, dev, 2)
    _require(w_scales, "w_scales", torch.uint8, dev, 2)
    _require(positions, "positions", torch.int64, dev, 1)
    _require(cos_sin, "cos_sin", torch.float32, dev, 2)
    if x.stride(1) != 1 or w.stride(1) != 1 or not w_scales.is_contiguous() or not positions.is_contiguous() \
            or not cos_sin.is_contiguous():
        raise ValueError("x, w need contiguous rows; w_scales, positions, cos_sin must be contiguous")
    M, K = x.shape
    if w.shape[1] != K or w.shape[0] != n_heads * head_dim:
        raise ValueError(f"w must be [{n_heads * head_dim}, {K}], got {tuple(w.shape)}")
    ws_rows = n_heads * head_dim if w_scale_rows else n_heads * head_dim // 128
    if tuple(w_scales.shape) != (ws_rows, K // 128):
        raise ValueError(f"w_scales must be [{ws_rows}, {K // 128}]")
    if positions.shape[0] != M:
        raise ValueError("positions needs one entry per token")
    if cos_sin.shape[1] != rope_dim:
        raise ValueError(f"cos_sin must have {rope_dim} columns")
    return [_ptr(x), x.stride(0), _ptr(w), w.stride(0), _ptr(w_scales), M, K, n_heads, head_dim, rope_dim,
            _ptr(positions), _ptr(cos_sin), cos_sin.shape[0]]


@_on_stream
def debug_indexer_q_prep_bf16_f32(x, w, w_scales, positions, cos_sin, n_heads: int = 64, head_dim: int = 128,
                                  rope_dim: int = 64, out=None, stream=None):
    """float32 [M, H*128]: the GEMM output of the one-launch kernel of
    :func:`indexer_q_prep_bf16` (its own FP8 quantization of x included)."""
    args = _prep_bf16_common(x, w, w_scales, positions, cos_sin, n_heads, head_dim, rope_dim, False)
    M = x.shape[0]
    if out is None:
        out = torch.empty((M, n_heads * head_dim), dtype=torch.float32, device=x.device)
    _require(out, "out", torch.float32, x.device, 2)
    if not out.is_contiguous() or tuple(out.shape) != (M, n_heads * head_dim):
        raise ValueError("out must be a contiguous [M, H*128] float32 tensor")
    st = _lib.iqp_debug_indexer_q_prep_bf16_f32(*args, _ptr(out), _stream(x, stream))
    _check(st, "iqp_debug_indexer_q_prep_bf16_f32")
    return out


@_on_stream
def debug_indexer_q_clock(a, a_scales, w, w_scales, positions, cos_sin, n_heads: int = 64, head_dim: int = 128,
                          rope_dim: int = 64, q_fp4=None, q_scales=None, stamps=None, cos_sin_lanes=None,
                          stream=None):
    """:func:`indexer_q_gemm_rope_fp4` from the clock-stamp build of its
    split-role kernel (the build reading ``cos_sin_lanes`` when that is given). Returns ``(q_fp4, q_scales, stamps)`` with stamps an
    int64 [workgroups, 4] device tensor (shader clock counter at start, end;
    constant-rate counter at start, end; all 0 for a workgroup with no
    tokens). Raises IqpError (IQP_ERR_UNSUPPORTED) where the call would not
    run the split-role kernel."""
    a, args = _indexer_q_common(a, a_scales, w, w_scales, positions, cos_sin, n_heads, head_dim, rope_dim)
    M, dev = a.shape[0], a.device
    if q_fp4 is None:
        q_fp4 = torch.empty((M, n_heads, head_dim // 2), dtype=torch.uint8, device=dev)
    if q_scales is None:
        q_scales = torch.empty((M, n_heads, head_dim // 32), dtype=torch.uint8, device=dev)
    _require(q_fp4, "q_fp4", torch.uint8, dev, 3)
    _require(q_scales, "q_scales", torch.uint8, dev, 3)
    if not (q_fp4.is_contiguous() and q_scales.is_contiguous()) or \
            tuple(q_fp4.shape) != (M, n_heads, head_dim // 2) or tuple(q_scales.shape) != (M, n_heads, head_dim // 32):
        raise ValueError("q_fp4 / q_scales must be contiguous [M, H, 64] / [M, H, 4]")
    if stamps is None:
        stamps = torch.empty((4 * 4096,), dtype=torch.int64, device=dev)
    _require(stamps, "stamps", torch.int64, dev, 1)
    if not stamps.is_contiguous():
        raise ValueError("stamps must be contiguous")
    nwg = ctypes.c_int64(0)
    if cos_sin_lanes is not None:
        _require(cos_sin_lanes, "cos_sin_lanes", torch.float32, dev, 1)
        if not cos_sin_lanes.is_contiguous() or cos_sin_lanes.numel() < rope_table_lanes_size(cos_sin.shape[0]):
            raise ValueError("cos_sin_lanes must be the contiguous copy rope_table_lanes builds from cos_sin")
    st = _lib.iqp_debug_indexer_q_clock(*args[:-1], _ptr(cos_sin_lanes), args[-1], _ptr(q_fp4), _ptr(q_scales),
                                        _ptr(stamps), stamps.numel(), ctypes.byref(nwg), _stream(a, stream))
    _check(st, "iqp_debug_indexer_q_clock")
    return q_fp4, q_scales, stamps[: 4 * nwg.value].view(nwg.value, 4)


def device_clock_rates():
    """(constant-rate counter Hz, peak shader clock Hz) of the current device."""
    wall, sclk = ctypes.c_int64(0), ctypes.c_int64(0)
    _check(_lib.iqp_device_clock_rates(ctypes.byref(wall), ctypes.byref(sclk)), "iqp_device_clock_rates")
    return wall.value, sclk.value


@_on_stream
def indexer_q_prep(x, w, w_scales, positions, cos_sin, n_heads: int = 64, rope_layout: str = "half_split",
                   scale_rule: str = "ceil", w_scale_layout: str = "tile_128x128", cos_sin_lanes=None,
                   workspace=None, stream=None):
    """The whole indexer-Q preparation for a bf16 [M, K] activation batch:
    up to ONE_LAUNCH_MAX_TOKENS tokens at K = 1536 the one-launch call (up to
    ONE_LAUNCH_WITH_WORKSPACE_MAX_TOKENS given a ``workspace`` from
    :func:`indexer_q_workspace` and the default conventions: the call then
    splits each head's K range from 12 tokens), else FP8 quantization then the
    fused projection / RoPE / Hadamard / FP4 call, both on one stream. Returns
    ``(q_fp4, q_scales)``; the paths pass the same acceptance rule (without a
    workspace they give the same bytes). The convention arguments and
    ``cos_sin_lanes`` are those of :func:`indexer_q_gemm_rope_fp4` (the
    one-launch call reads the table)."""
    conv = dict(rope_layout=rope_layout, scale_rule=scale_rule, w_scale_layout=w_scale_layout)
    default = rope_layout == "half_split" and scale_rule == "ceil" and w_scale_layout == "tile_128x128"
    limit = ONE_LAUNCH_WITH_WORKSPACE_MAX_TOKENS if (workspace is not None and default) else ONE_LAUNCH_MAX_TOKENS
    if (1 <= x.shape[0] <= limit and x.dim() == 2 and x.shape[1] == 1536
            and x.data_ptr() % 16 == 0 and x.stride(0) % 8 == 0 and w_scales.data_ptr() % 4 == 0):
        if workspace is not None and default:
            return indexer_q_prep_bf16(x, w, w_scales, positions, cos_sin, n_heads=n_heads, workspace=workspace,
                                       stream=stream)
        return indexer_q_prep_bf16(x, w, w_scales, positions, cos_sin, n_heads=n_heads, stream=stream, **conv)
    a, a_scales = fp8_quant_1x128_ue8m0(x, stream=stream)
    return indexer_q_gemm_rope_fp4(a, a_scales, w, w_scales, positions, cos_sin, n_heads=n_heads,
                                   cos_sin_lanes=cos_sin_lanes, stream=stream, **conv)
