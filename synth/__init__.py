"""Seeded synthetic inputs for the Prox sparse SwiGLU FFN.

This module only draws random numbers and stores them in the dtypes the
layer uses.  It holds none of the method's arithmetic, and both the CPU
oracle and the HIP path are fed from it, so it imports neither.

Recipe (stands in for the trained weights and decode activations of the
ten LLMs the Prox pages evaluate, which are not available):

* one NumPy ``Generator(PCG64(SeedSequence([seed, layer, role])))`` per
  tensor, role 0 = gate, 1 = up, 2 = down, 3 = x;
* weights: float32 standard normals times ``std`` (float32 multiply),
  stored as float32 (fp32 layers) or rounded to bfloat16 with
  round-to-nearest-even (bf16 layers), drawn in row-major nn.Linear order:
  ``w_gate[F][d]``, ``w_up[F][d]``, ``w_down[d][F]``;
* x: float32 standard normals per token; per token ``round(0.01 * d)``
  positions drawn uniformly without replacement are multiplied by 20
  (activation outliers), then stored like the weights.

bf16 tensors are returned as ``uint16`` bit patterns; float32 tensors as
``float32``.
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

ROLE_GATE, ROLE_UP, ROLE_DOWN, ROLE_X = 0, 1, 2, 3

# Rows generated per chunk; bounds host memory for the 8192 x 28672 layer.
_CHUNK_ELEMS = 1 << 25


def _rng(seed: int, layer: int, role: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, layer, role])))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); uint16 bits."""
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    return ((b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal_matrix(rows: int, cols: int, std: float, dtype: str, rng: np.random.Generator) -> np.ndarray:
    out = np.empty((rows, cols), dtype=np.float32 if dtype == "f32" else np.uint16)
    step = max(1, _CHUNK_ELEMS // cols)
    s32 = np.float32(std)
    for r0 in range(0, rows, step):
        r1 = min(rows, r0 + step)
        v = rng.standard_normal((r1 - r0) * cols, dtype=np.float32) * s32
        v = v.reshape(r1 - r0, cols)
        out[r0:r1] = v if dtype == "f32" else f32_to_bf16_bits(v)
    return out


def make_weights(d: int, F: int, std: float, dtype: str, seed: int = 0, layer: int = 0):
    """(w_gate[F][d], w_up[F][d], w_down[d][F]) in nn.Linear orientation.

    The three matrices come from independent streams, so they are drawn in
    three threads (NumPy fills and converts large arrays without the GIL);
    the values do not depend on it."""
    assert dtype in ("f32", "bf16")
    jobs = ((F, d, ROLE_GATE), (F, d, ROLE_UP), (d, F, ROLE_DOWN))
    with ThreadPoolExecutor(max_workers=3) as ex:
        futs = [ex.submit(_normal_matrix, r, c, std, dtype, _rng(seed, layer, role)) for r, c, role in jobs]
        wg, wu, wd = [f.result() for f in futs]
    return wg, wu, wd


def make_x(B: int, d: int, dtype: str, seed: int = 0, layer: int = 0,
           outlier_frac: float = 0.01, outlier_scale: float = 20.0) -> np.ndarray:
    """Decode activations x[B][d]: N(0,1) with a few large-magnitude outliers per token."""
    rng = _rng(seed, layer, ROLE_X)
    x = rng.standard_normal((B, d), dtype=np.float32)
    n_out = int(round(outlier_frac * d))
    for b in range(B):
        pos = rng.choice(d, size=n_out, replace=False)
        x[b, pos] *= np.float32(outlier_scale)
    return x if dtype == "f32" else f32_to_bf16_bits(x)


def to_f32(a: np.ndarray) -> np.ndarray:
    """float32 view of a generated tensor (bf16 bits widened exactly)."""
    return a if a.dtype == np.float32 else bf16_bits_to_f32(a)


@dataclass(frozen=True)
class Workload:
    """One of the layer shapes the Prox pages evaluate on (LLM FFN shapes)."""
    name: str
    d: int
    F: int
    dtype: str
    std: float
    mode: str                      # proxy format: "int8_row" or "int4_g128"
    input_keep: float
    sparsities: tuple
    batches: tuple
    layers: int = 1
    extra_modes: tuple = field(default_factory=tuple)


WORKLOADS = {
    # toy fp32 layer, 512 x 1376
    "toy_fp32": Workload("toy_fp32", 512, 1376, "f32", 0.02, "int8_row", 0.5, (0.5,), (1,)),
    # 7B-like 4096 x 11008
    "llama7b": Workload("llama7b", 4096, 11008, "bf16", 0.02, "int8_row", 0.5, (0.0, 0.5, 0.7, 0.9), (1,)),
    # 8B-like 4096 x 14336
    "llama8b": Workload("llama8b", 4096, 14336, "bf16", 0.02, "int8_row", 0.5, (0.7,), (1, 4, 16)),
    # 70B-like 8192 x 28672, int4 group-128 proxy and int8 proxy
    "llama70b": Workload("llama70b", 8192, 28672, "bf16", 0.015, "int4_g128", 0.4, (0.5, 0.7, 0.9), (1,),
                         extra_modes=("int8_row",)),
    # 32 layers of the 8B-like FFN with RMSNorm and residual adds
    "llama8b_chain32": Workload("llama8b_chain32", 4096, 14336, "bf16", 0.02, "int8_row", 0.5, (0.7,), (1, 8),
                                layers=32),
}
