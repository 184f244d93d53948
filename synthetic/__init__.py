"""Seeded synthetic inputs shaped like the indexer-Q workloads.

Shared by the tests, the benchmark and the oracle's callers. This module holds
no step of the method: it draws random numbers and rounds them to the storage
types (bf16 activations, E4M3 weights) with torch's CPU casts.

Every tensor comes from ``numpy.random.default_rng([workload_id, tensor_id])``
(the weights from ``default_rng([100])``), so a given workload is the same on
every machine.

Workloads (token counts and widths from the pages' microbenchmarks: 128 and
4,632 tokens, K divisible by 128):

* ``indexer_q_m128``   X[128,1536] ~ N(0,1) with 4 outlier channels x30;
  positions uniform in [0,4096)
* ``quant_4632x7168``  X[4632,7168] ~ N(0,1); 1 % of the 128-blocks x1e3 and a
  disjoint 1 % x1e-6
* ``indexer_q_m4632``  X[4632,1536] as the M=128 case; positions 0..4631
* ``decode_mix``       M drawn from {1,2,4,8,16,32,64}; positions uniform in
  [0,131072); plus a standalone X'[M,7168] ~ N(0,1)
* ``prefill_m32768``   X[32768,1536] ~ Student-t (nu=3); positions 0..32767;
  plus a standalone X'[32768,7168] ~ t3

The standalone epilogue takes a bf16 Q [M, 64*128] instead of X: each token
row is N(0,1) times a per-token factor 2^u, u uniform in [-4, 4] (the spread
of magnitudes a projection output has across tokens), with the positions of
the workload it stands beside (``q_bf16_inputs``).

Weights: W[8192,1536] ~ N(0, 0.02^2), stored as E4M3 codes with one UE8M0
exponent per 128x128 tile. The tile exponents are drawn from {-12, -11}
(about the natural exponent for N(0, 0.02^2) data), and the codes are the
normal sample divided by the tile's power of two, cast to E4M3 (saturating at
448). The weights are thus synthesized directly in their stored form.
"""
import numpy as np
import torch

WORKLOAD_IDS = {
    "indexer_q_m128": 0,
    "quant_4632x7168": 1,
    "indexer_q_m4632": 2,
    "decode_mix": 3,
    "prefill_m32768": 4,
}

N_HEADS = 64
HEAD_DIM = 128
ROPE_DIM = 64
ROPE_THETA = 10000.0
K_PROJ = 1536
K_WIDE = 7168
DECODE_M_CHOICES = (1, 2, 4, 8, 16, 32, 64)


def rng(workload: str, tensor_id: int) -> np.random.Generator:
    return np.random.default_rng([WORKLOAD_IDS[workload], tensor_id])


def to_bf16(x: np.ndarray) -> torch.Tensor:
    """float array -> bf16 CPU tensor (torch's round-to-nearest-even cast)."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)


def activations_outlier(g: np.random.Generator, M: int, K: int, n_outliers: int = 4,
                        factor: float = 30.0) -> torch.Tensor:
    """N(0,1) with ``n_outliers`` channels scaled by ``factor``."""
    x = g.standard_normal((M, K), dtype=np.float32)
    ch = g.choice(K, size=min(n_outliers, K), replace=False)
    x[:, ch] *= factor
    return to_bf16(x)


def activations_block_extremes(g: np.random.Generator, M: int, K: int,
                               frac: float = 0.01) -> torch.Tensor:
    """N(0,1) with ``frac`` of the 128-blocks x1e3 and a disjoint ``frac`` x1e-6."""
    x = g.standard_normal((M, K), dtype=np.float32)
    nb = M * (K // 128)
    n_sel = int(round(frac * nb))
    sel = g.choice(nb, size=2 * n_sel, replace=False)
    blocks = x.reshape(nb, 128)
    blocks[sel[:n_sel]] *= 1e3
    blocks[sel[n_sel:]] *= 1e-6
    return to_bf16(x)


def activations_student_t(g: np.random.Generator, M: int, K: int, nu: float = 3.0) -> torch.Tensor:
    return to_bf16(g.standard_t(nu, size=(M, K)).astype(np.float32))


def weights(N: int = N_HEADS * HEAD_DIM, K: int = K_PROJ, std: float = 0.02,
            seed: int = 100) -> tuple:
    """E4M3 weight codes [N, K] (uint8 tensor) and tile exponent bytes
    [N/128, K/128] (uint8 tensor)."""
    g = np.random.default_rng([seed])
    w = g.standard_normal((N, K), dtype=np.float32) * np.float32(std)
    tile_exp = g.integers(-12, -10, size=(N // 128, K // 128))          # {-12, -11}
    inv = np.ldexp(np.float32(1.0), -np.repeat(np.repeat(tile_exp, 128, 0), 128, 1)).astype(np.float32)
    scaled = np.clip(w * inv, -448.0, 448.0)
    codes = torch.from_numpy(scaled).to(torch.float8_e4m3fn).view(torch.uint8)
    scale_bytes = torch.from_numpy((tile_exp + 127).astype(np.uint8))
    return codes.contiguous(), scale_bytes.contiguous()


def positions_uniform(g: np.random.Generator, M: int, max_pos: int) -> torch.Tensor:
    return torch.from_numpy(g.integers(0, max_pos, size=M).astype(np.int64))


def positions_arange(M: int) -> torch.Tensor:
    return torch.arange(M, dtype=torch.int64)


def indexer_q_inputs(workload: str, M: int = None) -> dict:
    """Activations, positions and table size for one indexer-Q workload."""
    if workload == "indexer_q_m128":
        M = 128 if M is None else M
        x = activations_outlier(rng(workload, 0), M, K_PROJ)
        pos = positions_uniform(rng(workload, 1), M, 4096)
        max_pos = 4096
    elif workload == "indexer_q_m4632":
        M = 4632 if M is None else M
        x = activations_outlier(rng(workload, 0), M, K_PROJ)
        pos = positions_arange(M)
        max_pos = max(M, 1)
    elif workload == "prefill_m32768":
        M = 32768 if M is None else M
        x = activations_student_t(rng(workload, 0), M, K_PROJ)
        pos = positions_arange(M)
        max_pos = max(M, 1)
    else:
        raise ValueError(workload)
    return {"x": x, "positions": pos, "max_pos": max_pos, "M": M}


def q_bf16_inputs(workload: str, M: int = None, n_heads: int = N_HEADS) -> dict:
    """bf16 Q [M, n_heads*128] and positions for the standalone epilogue, at the
    token counts and positions of an indexer-Q workload."""
    base = indexer_q_inputs(workload, M=M)
    M = base["M"]
    g = rng(workload, 5)
    q = g.standard_normal((M, n_heads * HEAD_DIM), dtype=np.float32)
    q *= np.exp2(g.uniform(-4.0, 4.0, size=(M, 1))).astype(np.float32)
    return {"q": to_bf16(q), "positions": base["positions"], "max_pos": base["max_pos"], "M": M}


def decode_calls(n_calls: int = 256) -> list:
    """Per-call inputs of the decode-shaped mix: list of dicts with x [M,1536],
    x_wide [M,7168], positions [M]."""
    g = rng("decode_mix", 0)
    ms = g.choice(np.array(DECODE_M_CHOICES), size=n_calls)
    calls = []
    for i, m in enumerate(ms):
        gi = np.random.default_rng([WORKLOAD_IDS["decode_mix"], 1000 + i])
        calls.append({
            "x": activations_outlier(gi, int(m), K_PROJ),
            "x_wide": to_bf16(gi.standard_normal((int(m), K_WIDE), dtype=np.float32)),
            "positions": positions_uniform(gi, int(m), 131072),
        })
    return calls


def quant_input(workload: str = "quant_4632x7168", M: int = None, K: int = None) -> torch.Tensor:
    """Standalone quantizer input."""
    if workload == "quant_4632x7168":
        return activations_block_extremes(rng(workload, 0), M or 4632, K or K_WIDE)
    if workload == "prefill_m32768":
        return activations_student_t(rng(workload, 2), M or 32768, K or K_WIDE)
    raise ValueError(workload)
