"""Seeded synthetic inputs for the residual-binarized linear layer.

This module only draws random numbers and names shapes.  It holds none of
the method's arithmetic (no signs, means, packing or products), so both the
CPU oracle side (tests) and the HIP side (tests, bench) can take their
inputs from it without sharing any computation.

Workloads (weights are out x in, row-major fp32; activations fp16):

* ``small``      256x512, K=2, per-row scales.  W ~ N(0, 0.02^2) seed 0,
                 x ~ N(0, 1) seed 1, one token.
* ``llama2_7b``  the seven decoder linears of Llama-2-7B (q, k, v, o
                 4096x4096; gate, up 11008x4096; down 4096x11008), K=2,
                 per-row scales, W ~ N(0, 0.02^2) with 0.1 % of positions
                 (drawn without replacement) multiplied by 20.  Seeds:
                 W 1000 + 7*layer + i, outlier positions W seed + 500000,
                 x seed 2 (one token) and seed 3 (skinny batches 4 and 16:
                 the first rows of one 16-row draw).
* ``llama2_13b_g128``  5120x5120 (q, k, v, o), 13824x5120 (gate, up),
                 5120x13824 (down); K=4 with one scale per row per group of
                 128 input columns; W ~ N(0, 0.02^2) seeds 2000 + 7*layer + i;
                 x seed 4.
* ``llama3_8b_prefill``  14336x4096 and 4096x14336, K=2 per-row, 2048
                 tokens; W seeds 3000 and 3001, X seed 5.

The pages evaluate trained Llama checkpoints; none is available here, so
these Gaussian matrices of the same shapes stand in for them.
"""
from __future__ import annotations

import dataclasses

import numpy as np

W_STD = np.float32(0.02)
OUTLIER_FRACTION = 0.001
OUTLIER_FACTOR = np.float32(20.0)


@dataclasses.dataclass(frozen=True)
class Linear:
    name: str
    out_features: int
    in_features: int


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    linears: tuple
    num_planes: int
    group_size: int          # 0 = one scale per row, else columns per group
    outliers: bool
    w_seed_base: int
    x_seed: int
    tokens: tuple            # token counts this workload is run at


LLAMA2_7B_LINEARS = (
    Linear("q_proj", 4096, 4096),
    Linear("k_proj", 4096, 4096),
    Linear("v_proj", 4096, 4096),
    Linear("o_proj", 4096, 4096),
    Linear("gate_proj", 11008, 4096),
    Linear("up_proj", 11008, 4096),
    Linear("down_proj", 4096, 11008),
)

LLAMA2_13B_LINEARS = (
    Linear("q_proj", 5120, 5120),
    Linear("k_proj", 5120, 5120),
    Linear("v_proj", 5120, 5120),
    Linear("o_proj", 5120, 5120),
    Linear("gate_proj", 13824, 5120),
    Linear("up_proj", 13824, 5120),
    Linear("down_proj", 5120, 13824),
)

WORKLOADS = {
    "small": Workload("small", (Linear("linear", 256, 512),), 2, 0, False, 0, 1, (1,)),
    "llama2_7b": Workload("llama2_7b", LLAMA2_7B_LINEARS, 2, 0, True, 1000, 2, (1,)),
    "llama2_7b_skinny": Workload("llama2_7b_skinny", LLAMA2_7B_LINEARS, 2, 0, True, 1000, 3, (4, 16)),
    "llama2_13b_g128": Workload("llama2_13b_g128", LLAMA2_13B_LINEARS, 4, 128, False, 2000, 4, (1,)),
    "llama3_8b_prefill": Workload(
        "llama3_8b_prefill",
        (Linear("gate_proj", 14336, 4096), Linear("down_proj", 4096, 14336)),
        2, 0, False, 3000, 5, (2048,)),
}


def weight_seed(wl: Workload, index: int, layer: int = 0) -> int:
    """Seed of linear ``index`` of layer ``layer`` (7 linears per layer)."""
    if wl.name == "llama3_8b_prefill":
        return wl.w_seed_base + index
    return wl.w_seed_base + 7 * layer + index


def gaussian_weight(out_features: int, in_features: int, seed: int,
                    outliers: bool = False) -> np.ndarray:
    """W ~ N(0, 0.02^2) fp32, optionally with 0.1 % of entries times 20.

    Exactly round(0.001 * out * in) positions are drawn without replacement
    from a second generator seeded ``seed + 500000``.
    """
    rng = np.random.default_rng(seed)
    w = rng.standard_normal((out_features, in_features), dtype=np.float32)
    w *= W_STD
    if outliers:
        count = int(round(OUTLIER_FRACTION * out_features * in_features))
        orng = np.random.default_rng(seed + 500000)
        pos = orng.choice(out_features * in_features, size=count, replace=False)
        w.reshape(-1)[pos] *= OUTLIER_FACTOR
    return w


def gaussian_activations(tokens: int, in_features: int, seed: int) -> np.ndarray:
    """x ~ N(0, 1), drawn in fp32 and rounded to fp16 (round to nearest even).

    Returned as a uint16 array of fp16 bit patterns, shape [tokens][in].
    """
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((tokens, in_features), dtype=np.float32)
    return x.astype(np.float16).view(np.uint16)


def workload_weight(wl: Workload, index: int, layer: int = 0) -> np.ndarray:
    lin = wl.linears[index]
    return gaussian_weight(lin.out_features, lin.in_features,
                           weight_seed(wl, index, layer), wl.outliers)


def workload_activations(wl: Workload, in_features: int, tokens: int) -> np.ndarray:
    """Activations for ``tokens`` tokens: the first rows of one draw of the
    workload's largest token count, so smaller batches are prefixes."""
    full = max(max(wl.tokens), tokens)
    return gaussian_activations(full, in_features, wl.x_seed)[:tokens]


def layer_activations(wl: Workload, in_features: int, layers: int, slot: int) -> np.ndarray:
    """One fp16 token per layer for one input of a decoder layer (slot 0:
    attention input, read by q, k, v; 1: o_proj input; 2: MLP input, read
    by gate and up; 3: down_proj input), so that no two launches of a step
    read the same activations unless a decoder's would.  x ~ N(0, 1), seed
    100 * x_seed + 10 + slot; uint16 [layers][in]."""
    return gaussian_activations(layers, in_features, 100 * wl.x_seed + 10 + slot)


def random_scales(num_planes: int, out_features: int, groups: int, seed: int,
                  signed: bool = True) -> np.ndarray:
    """Arbitrary finite fp16 scales (as learned scales would be), uint16 bits."""
    rng = np.random.default_rng(seed)
    s = rng.uniform(0.001, 0.05, size=(num_planes, out_features, groups)).astype(np.float32)
    if signed:
        s *= rng.choice(np.array([-1.0, 1.0], dtype=np.float32), size=s.shape)
    return s.astype(np.float16).view(np.uint16)


def random_planes(num_planes: int, out_features: int, in_features: int, seed: int) -> np.ndarray:
    """Uniformly random sign-plane words, uint32 [K][out][in/32]."""
    rng = np.random.default_rng(seed)
    return rng.integers(0, 2**32, size=(num_planes, out_features, in_features // 32),
                        dtype=np.uint64).astype(np.uint32)
