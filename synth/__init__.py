"""Seeded synthetic inputs shared by the HIP path's tests/bench and the oracle.

This module holds no arithmetic of the BitLinear method itself: it only draws
latent fp32 weights, bf16 activation tokens (as raw bit patterns) and describes
the layer shapes of the five workloads.  Both sides receive the identical bytes.

Workload shapes follow the model families the source pages discuss:
  * a single 2048x2048 layer;
  * a BitNet-2B-shaped stack (hidden 2560, FFN 6912, 30 layers), the model
    of "BitNet-2B-4T: Inside the 2B-Parameter, 4T-Token 1-Bit LLM";
  * a LLaMA-3-8B-shaped stack (hidden 4096, FFN 14336, 32 layers), the model
    of "BitNet b1.58 in Production" (introduction) and of the architecture
    breakdown page's headline figure;
  * a 70B-shaped layer (d_model 8192, FFN 28672), the model size of
    "BitNet 1-bit LLM Inference Framework", section "Why 1-bit".
Latent weights are N(0, 0.02); activations are N(0, 1) rounded to bf16, with a
fixed fraction of positions per token multiplied by 10 (outliers).
"""
from __future__ import annotations

import concurrent.futures as _cf
from dataclasses import dataclass, field
from typing import Iterator, List, Sequence, Tuple

import numpy as np

WEIGHT_STD = np.float32(0.02)
OUTLIER_SCALE = np.float32(10.0)


@dataclass(frozen=True)
class Matrix:
    """One BitLinear: K inputs -> N outputs; latent weight is [N][K] row-major."""
    name: str
    k: int
    n: int


@dataclass(frozen=True)
class Workload:
    key: str                      # short name used by tests and bench
    title: str
    layers: int
    matrices: Tuple[Matrix, ...]
    ms: Tuple[int, ...]           # token counts M exercised
    outlier_frac: float           # fraction of positions per token scaled x10
    weight_seed: int = -1         # >= 0: single-matrix workload with a fixed seed
    act_seed: int = -1
    index: int = 0                # position in the workload list (seed namespace)
    weight_index: int = -1        # >= 0: draw the weights of that workload instead (same layers)


_L2B = (Matrix("qkv", 2560, 3840), Matrix("o", 2560, 2560),
        Matrix("gate_up", 2560, 13824), Matrix("down", 6912, 2560))
_L8B = (Matrix("qkv", 4096, 6144), Matrix("o", 4096, 4096),
        Matrix("gate_up", 4096, 28672), Matrix("down", 14336, 4096))

WORKLOADS: Tuple[Workload, ...] = (
    Workload("single2048", "single BitLinear 2048->2048, M=1", 1,
             (Matrix("w", 2048, 2048),), (1,), 0.01, weight_seed=0, act_seed=1, index=0),
    Workload("b2b_decode", "BitNet-2B-shaped stack, 30 layers, decode M=1", 30,
             _L2B, (1,), 0.0, index=1),
    Workload("l8b_decode", "LLaMA-3-8B-shaped stack, 32 layers, decode M=1/4/8", 32,
             _L8B, (1, 4, 8), 0.005, index=2),
    # prefill: the decode stack's weights (same seeds), 512 tokens per matrix
    Workload("l8b_prefill", "LLaMA-3-8B-shaped stack, 32 layers, prefill M=512", 32,
             _L8B, (512,), 0.005, index=3, weight_index=2),
    Workload("l70b_layer", "70B-shaped layer, d_model 8192, M=1/64", 1,
             (Matrix("gate_up", 8192, 57344), Matrix("down", 28672, 8192)), (1, 64), 0.0,
             index=4),
)
BY_KEY = {w.key: w for w in WORKLOADS}

ROLE_WEIGHT = 0
ROLE_ACT = 1
ROLE_GAIN = 2


def seed_for(wl: Workload, layer: int, mat: int, role: int, extra: int = 0):
    """Seed of one tensor of a workload.

    The single-layer 2048 workload uses the fixed seeds 0 (weights) and 1
    (activations); every other tensor uses SeedSequence([workload, layer,
    matrix, role, extra]), where a workload that shares another's weights
    (weight_index) names that workload for its weight tensors."""
    if role == ROLE_WEIGHT and wl.weight_seed >= 0:
        return wl.weight_seed
    if role == ROLE_ACT and wl.act_seed >= 0 and extra == 0:
        return wl.act_seed
    index = wl.weight_index if role == ROLE_WEIGHT and wl.weight_index >= 0 else wl.index
    return np.random.SeedSequence([index, layer, mat, role, extra])


def _rng(seed) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def latent_weights(seed, n: int, k: int, std: np.float32 = WEIGHT_STD) -> np.ndarray:
    """fp32 [n][k] ~ N(0, std): standard normals scaled by std in fp32."""
    w = _rng(seed).standard_normal((n, k), dtype=np.float32)
    w *= np.float32(std)
    return w


def fp32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round finite fp32 values to bf16 (nearest, ties to even); returns uint16 bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    bias = ((u >> np.uint64(16)) & np.uint64(1)) + np.uint64(0x7FFF)
    return ((u + bias) >> np.uint64(16)).astype(np.uint16)


def bf16_bits_to_fp32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32 (for building test inputs)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def activations_bf16(seed, m: int, k: int, outlier_frac: float = 0.0,
                     outlier_scale: np.float32 = OUTLIER_SCALE) -> np.ndarray:
    """bf16 bits [m][k]: N(0,1) in fp32, a fixed count round(frac*k) of positions
    per token (drawn without replacement) multiplied by outlier_scale in fp32,
    then rounded to bf16."""
    rng = _rng(seed)
    x = rng.standard_normal((m, k), dtype=np.float32)
    n_out = int(round(outlier_frac * k))
    if n_out > 0:
        keys = rng.random((m, k))
        idx = np.argpartition(keys, n_out - 1, axis=1)[:, :n_out]
        rows = np.arange(m)[:, None]
        x[rows, idx] *= np.float32(outlier_scale)
    return fp32_to_bf16_bits(x)


def activations_f32(seed, m: int, k: int, scale: float = 1.0) -> np.ndarray:
    """fp32 [m][k]: scale * N(0,1), for inputs produced in fp32 on the device."""
    rng = _rng(seed)
    return (np.float32(scale) * rng.standard_normal((m, k), dtype=np.float32)).astype(np.float32)


def norm_gain(seed, k: int) -> np.ndarray:
    """fp32 [k] per-channel RMSNorm gains: 1 + 0.1 * N(0,1), a synthetic
    stand-in for trained gains (initialised to one)."""
    rng = _rng(seed)
    return (np.float32(1.0) + np.float32(0.1) * rng.standard_normal(k, dtype=np.float32)).astype(np.float32)


def iter_layer_matrices(wl: Workload) -> Iterator[Tuple[int, int, Matrix]]:
    """(layer, matrix index, Matrix) in layer order."""
    for layer in range(wl.layers):
        for j, mat in enumerate(wl.matrices):
            yield layer, j, mat


def generate_many(jobs: Sequence[Tuple[object, int, int]], threads: int = 8) -> List[np.ndarray]:
    """Draw several latent weight matrices concurrently: jobs = [(seed, n, k)].
    Each matrix has its own generator, so the result does not depend on threads."""
    with _cf.ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
        return list(ex.map(lambda j: latent_weights(j[0], j[1], j[2]), jobs))


def packed_weight_bytes_2bit(wl: Workload) -> int:
    """Dense 2-bit weight bytes of the whole workload (N*K/4 per matrix)."""
    return wl.layers * sum((m.n * m.k + 3) // 4 for m in wl.matrices)
