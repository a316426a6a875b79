"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module only draws random numbers and rounds them to bfloat16; it holds none of the
quantization, routing or linear arithmetic, and imports neither the HIP library nor the
oracle.  The workloads stand in for the LLaMA-2/3 and Qwen2.5 layers that the MoBiQuant
explainer evaluates (section 4 of the English gist.science page), which are not available
here: weights ~ N(0, 0.02^2) with a few input columns scaled up as outliers, activations
~ N(0, 1), router weights ~ N(0, 0.1^2).

Draw order for one linear (numpy ``default_rng(seed)``):
  1. W = standard_normal((N, K), float32) * 0.02
  2. outlier columns = rng.choice(K, n_out, replace=False), multiplied by the outlier scale
  3. W rounded to bfloat16 (round to nearest even) unless the workload is float32
  4. X = standard_normal((T, K), float32), rounded to bfloat16 unless float32
  5. Wr = standard_normal((K, S), float32) * 0.1
  6. forced budget mixes: rng.permutation(T) over a block-sorted budget vector

The low-rank side path's factors come from ``make_lowrank``: A ~ N(0, 1/K), B ~ N(0, s^2)
(s = 0.005 unless stated), both rounded to bfloat16.

The MLP router's weights have a generator of their own (``make_mlp_router``): hidden width
256 unless stated, W1 ~ N(0, 1/K) rounded to bfloat16 (pre-activations ~ N(0, 1) on the
activations above), b1 ~ N(0, 0.1^2), W2 ~ N(0, 2/H), b2 ~ N(0, 0.1^2), all float32.
"""
from __future__ import annotations

import numpy as np


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def bf16_values(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> their exact float32 values."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


def round_bf16(a: np.ndarray) -> np.ndarray:
    return bf16_values(bf16_bits(a))


def make_linear(seed: int, N: int, K: int, T: int, *, group: int = 128, slices: int = 3,
                dtype: str = "bf16", n_outliers: int = 0, outlier_scale: float = 1.0,
                forced_counts=None, rng=None) -> dict:
    """One linear layer's synthetic inputs.

    Returns float32 arrays holding exactly the values the device sees (bfloat16-rounded
    when ``dtype == "bf16"``): W [N, K], X [T, K], Wr [K, S]; plus ``budget`` (int32 [T])
    when ``forced_counts`` (tokens with budget 1, 2, ...) is given, else None.
    """
    rng = np.random.default_rng(seed) if rng is None else rng
    W = rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02)
    if n_outliers:
        cols = rng.choice(K, n_outliers, replace=False)
        W[:, cols] *= np.float32(outlier_scale)
    if dtype == "bf16":
        W = round_bf16(W)
    X = rng.standard_normal((T, K), dtype=np.float32)
    if dtype == "bf16":
        X = round_bf16(X)
    Wr = rng.standard_normal((K, slices), dtype=np.float32) * np.float32(0.1)
    budget = None
    if forced_counts is not None:
        counts = list(forced_counts)
        assert sum(counts) == T and len(counts) <= slices
        base = np.repeat(np.arange(1, len(counts) + 1, dtype=np.int32), counts)
        budget = base[rng.permutation(T)].astype(np.int32)
    return {"W": W, "X": X, "Wr": Wr, "budget": budget, "N": N, "K": K, "T": T,
            "group": group, "slices": slices, "dtype": dtype}


def make_mlp_router(seed: int, K: int, slices: int = 3, hidden: int = 256) -> dict:
    """Synthetic weights of the 2-layer MLP router: one score per residual slice.

    Draw order (``default_rng(seed)``): W1 [hidden, K], b1 [hidden], W2 [hidden, slices-1],
    b2 [slices-1].  W1 holds bfloat16-representable float32 values.
    """
    rng = np.random.default_rng(seed)
    W1 = rng.standard_normal((hidden, K), dtype=np.float32) * np.float32(1.0 / np.sqrt(K))
    W1 = round_bf16(W1)
    b1 = rng.standard_normal(hidden, dtype=np.float32) * np.float32(0.1)
    W2 = rng.standard_normal((hidden, slices - 1), dtype=np.float32) * np.float32(np.sqrt(2.0 / hidden))
    b2 = rng.standard_normal(slices - 1, dtype=np.float32) * np.float32(0.1)
    return {"W1": W1, "b1": b1, "W2": W2, "b2": b2, "hidden": hidden, "K": K,
            "slices": slices}


def make_lowrank(seed: int, N: int, K: int, rank: int = 16, b_scale: float = 0.005) -> dict:
    """Synthetic low-rank side-path factors, bfloat16-representable float32.

    Draw order (``default_rng(seed)``): A [rank, K] ~ N(0, 1/K), then B [N, rank] ~
    N(0, b_scale^2).  With activations ~ N(0, 1), x . A^T is ~ N(0, 1) per rank, so the
    side path is ~ sqrt(rank) * b_scale per output.
    """
    rng = np.random.default_rng(seed)
    A = round_bf16(rng.standard_normal((rank, K), dtype=np.float32) * np.float32(1.0 / np.sqrt(K)))
    B = round_bf16(rng.standard_normal((N, rank), dtype=np.float32) * np.float32(b_scale))
    return {"A": A, "B": B, "rank": rank}


def forced_mix(T: int, fractions) -> list:
    """Token counts for a budget mix: each fraction rounded, the remainder to the last."""
    counts = [int(round(f * T)) for f in fractions[:-1]]
    counts.append(T - sum(counts))
    return counts


# The five workloads, by number.  Sizes follow the Qwen2.5-7B up-projection, the
# Llama-7B MLP, a 14B-class decoder layer and a 14336x4096 projection.
CONFIG_NAMES = {
    1: "tiny single linear 512x256, G64, S3, fp32, T16",
    2: "decode GEMV 18944x3584 (Qwen2.5-7B-like up-proj), G128, S3, bf16, T 1/4/16",
    3: "prefill GEMM 11008x4096 (Llama-7B-like), G128, S3, bf16, T2048, budget mix 30/50/20",
    4: "14B-like decoder-layer linears (hidden 5120, ffn 13824), G128, S3, bf16, T64",
    5: "elasticity sweep 14336x4096, G128, S3, bf16, T 32/1024",
}

LAYER14B = [("q", 5120, 5120), ("k", 5120, 5120), ("v", 5120, 5120), ("o", 5120, 5120),
            ("gate", 13824, 5120), ("up", 13824, 5120), ("down", 5120, 13824)]


WORKLOADS = ("tiny_512x256", "decode_18944x3584", "prefill_11008x4096", "layer14b_t64", "sweep_14336x4096")


def make_workload(name: str) -> dict:
    """One of the full-size synthetic workloads, by name:
    tiny_512x256 (G 64, float32, 16 tokens, outlier columns), decode_18944x3584 (16 tokens,
    router), prefill_11008x4096 (2048 tokens at forced budgets 30/50/20 %), layer14b_t64
    (the seven linears of a 14B-like decoder layer at 64 tokens) and sweep_14336x4096 (1024
    tokens, forced budgets or the router)."""
    if name == "tiny_512x256":
        return make_linear(1, 512, 256, 16, group=64, dtype="f32", n_outliers=4,
                           outlier_scale=20.0)
    if name == "decode_18944x3584":
        return make_linear(2, 18944, 3584, 16, n_outliers=round(0.005 * 3584),
                           outlier_scale=10.0)
    if name == "prefill_11008x4096":
        return make_linear(3, 11008, 4096, 2048, forced_counts=forced_mix(2048, [0.3, 0.5, 0.2]))
    if name == "sweep_14336x4096":
        return make_linear(5, 14336, 4096, 1024)
    if name == "layer14b_t64":
        return make_layer14b()
    raise ValueError(name)


def make_layer14b(T: int = 64, seed: int = 4, scale_down: int = 1) -> dict:
    """Seven linears of one 14B-like decoder layer; one router on the layer input.

    ``scale_down`` divides every dimension (for small tests with the same structure).
    """
    rng = np.random.default_rng(seed)
    lin = []
    for name, N, K in LAYER14B:
        W = rng.standard_normal((N // scale_down, K // scale_down), dtype=np.float32) * np.float32(0.02)
        lin.append({"name": name, "W": round_bf16(W)})
    for d in lin:
        K = d["W"].shape[1]
        d["X"] = round_bf16(rng.standard_normal((T, K), dtype=np.float32))
    hidden = LAYER14B[0][2] // scale_down
    Wr = rng.standard_normal((hidden, 3), dtype=np.float32) * np.float32(0.1)
    return {"linears": lin, "Wr": Wr, "X_layer": lin[0]["X"], "T": T, "group": 128,
            "slices": 3, "dtype": "bf16"}
