"""Seeded synthetic inputs for the nested-weight speculative round.

Both the HIP path (tests, benchmark) and the CPU oracle take their inputs from
here. This module holds none of the method's arithmetic. It only draws
random numbers, converts dtypes and lists workload shapes. Every tensor comes
from its own numpy stream, ``SeedSequence(0, spawn_key=key)``, so a tensor is
reproducible on its own, whatever else was drawn before it.

Workloads (names give what they are):
  * ``linear_4096``: one nested 4096x4096 linear layer. Draft GEMV with 1
    row, verify with 5 rows (k=4).
  * ``qwen2.5-7b_layer``: the linears of one Qwen2.5-7B-shaped decoder
    layer. hidden 3584, QKV 3584->4608 (28 q / 4 kv heads, d=128), O
    3584->3584, gate and up 3584->18944, down 18944->3584.
  * ``qwen2.5-7b_lm_head``: the nested 3584x152064 LM head with k=8 verify
    rows and planted acceptance 0.58 / 0.66 / 0.95. These are the acceptance
    rates that SpecQuant's Table II and BitNest's abstract report.
  * ``llama3-8b_batched_verify``: 16 sequences x 9 rows = 144-row verify over
    the LLaMA-3-8B-shaped linears (hidden 4096, QKV 4096->6144, O
    4096->4096, gate and up 4096->14336 each, stored as one 28672 x 4096
    matrix since both read the same rows, down 14336->4096), 32 layers.
  * ``kv_32k``: nested KV cache with 32 q heads / 8 kv heads, d=128 and a
    32768-token context. bf16 queries; 1 draft query; 9 verify queries.

Distributions: weights ~ N(0, 0.02) (read as standard deviation 0.02).
Activations, K, V and queries ~ N(0, 1). Queries are rounded to bf16
(nearest, ties to even).
"""
from __future__ import annotations

import os

import numpy as np

SEED = 0

WORKLOADS = {
    "linear_4096": {"K": 4096, "N": 4096, "group": 128, "draft_rows": 1,
                    "verify_rows": 5, "k": 4},
    "qwen2.5-7b_layer": {
        "hidden": 3584, "group": 128, "k": 4,
        # name -> (N out, K in)
        "linears": {"qkv": (4608, 3584), "o": (3584, 3584), "gate_up": (2 * 18944, 3584),
                    "down": (3584, 18944)},
        "q_heads": 28, "kv_heads": 4, "head_dim": 128,
    },
    "qwen2.5-7b_lm_head": {"K": 3584, "V": 152064, "group": 128, "k": 8,
                           "alphas": (0.58, 0.66, 0.95), "rounds": 10000, "pool": 16},
    "llama3-8b_batched_verify": {
        "hidden": 4096, "group": 128, "layers": 32, "sequences": 16, "rows_per_seq": 9,
        "linears": {"qkv": (6144, 4096), "o": (4096, 4096), "gate_up": (28672, 4096),
                    "down": (4096, 14336)},
    },
    "kv_32k": {"q_heads": 32, "kv_heads": 8, "head_dim": 128, "context": 32768,
               "block": 128, "draft_queries": 1, "verify_queries": 9},
}

# Stable small integers for the spawn keys of each workload.
WORKLOAD_KEY = {name: i + 1 for i, name in enumerate(WORKLOADS)}


def rng(*key: int) -> np.random.Generator:
    """Generator for one tensor: seed 0 and spawn key ``key``."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(SEED, spawn_key=key)))


CHUNK = 1 << 22  # elements per independently seeded chunk of a large tensor
MAX_THREADS = 16  # a one-GPU host share


def _fill(out: np.ndarray, key, std: float) -> None:
    rng(*key).standard_normal(out=out, dtype=np.float32)
    if std != 1.0:
        out *= np.float32(std)


def normal(shape, key, std: float = 1.0) -> np.ndarray:
    """float32 normal draws, scaled by ``std`` in float32.

    A tensor of at most CHUNK elements is one stream with spawn key ``key``.
    A larger one is cut along its first axis into slabs of about CHUNK
    elements. Slab c draws from spawn key ``key + (c,)``, so the values do
    not depend on how many threads fill them.
    """
    shape = tuple(int(s) for s in np.atleast_1d(shape))
    a = np.empty(shape, dtype=np.float32)
    key = tuple(key)
    if a.size <= CHUNK or len(shape) == 1:
        _fill(a, key, std)
        return a
    row = int(np.prod(shape[1:])) if len(shape) > 1 else 1
    rows_per = max(1, CHUNK // max(row, 1))
    slabs = [(c, a[r:r + rows_per]) for c, r in enumerate(range(0, shape[0], rows_per))]
    import concurrent.futures as cf

    workers = min(len(slabs), MAX_THREADS, len(os.sched_getaffinity(0)))
    with cf.ThreadPoolExecutor(workers) as ex:
        list(ex.map(lambda cs: _fill(cs[1], key + (cs[0],), std), slabs))
    return a


def weights(n: int, k: int, key, std: float = 0.02) -> np.ndarray:
    """fp32 [n][k] weights ~ N(0, std)."""
    return normal((n, k), key, std)


def activations(m: int, k: int, key) -> np.ndarray:
    """fp32 [m][k] activations ~ N(0, 1)."""
    return normal((m, k), key)


def kv(n_kv_heads: int, capacity: int, head_dim: int, key, k_std: float = 1.0, v_std: float = 1.0):
    """fp32 K and V, each [Hkv][capacity][d], ~ N(0, k_std) and N(0, v_std)."""
    return (normal((n_kv_heads, capacity, head_dim), tuple(key) + (0,), k_std),
            normal((n_kv_heads, capacity, head_dim), tuple(key) + (1,), v_std))


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even) and return the bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_float(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def queries_bf16(nq: int, n_q_heads: int, head_dim: int, key, std: float = 1.0) -> np.ndarray:
    """bf16 bit patterns [nq][Hq][d] of N(0, std) draws."""
    return to_bf16_bits(normal((nq, n_q_heads, head_dim), key, std))


def plant_drafts(target: np.ndarray, alpha: float, vocab: int, key) -> np.ndarray:
    """Draft tokens planted to match the target's choices at rate ``alpha``.

    ``target`` is int [R][k+1]: the target's choices t_0..t_k of R rounds.
    Slot i (1..k) holds d_i = t_{i-1} with probability alpha. Otherwise it
    holds an id drawn uniformly from the other vocab-1 ids. Slots are
    independent, which is the assumption behind the blog's Eq. (1). The
    result is int32 [R][k].
    """
    target = np.asarray(target, dtype=np.int64)
    R, k1 = target.shape
    k = k1 - 1
    g = rng(*key)
    u = g.random((R, k))
    other = g.integers(0, vocab - 1, size=(R, k))
    prev = target[:, :k]
    other = np.where(other >= prev, other + 1, other)
    return np.where(u < alpha, prev, other).astype(np.int32)


def logits(rows: int, vocab: int, key, spread: float = 2.0, peaks: int = 3, lift: float = 9.0) -> np.ndarray:
    """float32 [rows][vocab] language-model-like logits.

    N(0, spread) for every id, plus ``lift`` * U(0.6, 1) on ``peaks`` random ids
    of each row, so that a few ids hold most of the probability and a long
    tail holds the rest, as in a trained model's next-token scores.
    """
    g = rng(*key)
    y = g.standard_normal((rows, vocab), dtype=np.float32) * np.float32(spread)
    for r in range(rows):
        ids = g.choice(vocab, size=min(peaks, vocab), replace=False)
        y[r, ids] += (lift * g.uniform(0.6, 1.0, size=ids.size)).astype(np.float32)
    return y


def logits_near(y: np.ndarray, key, noise: float = 0.3) -> np.ndarray:
    """``y`` plus N(0, noise) per element: a second model's logits that
    mostly agree with ``y`` (a draft close to its target)."""
    g = rng(*key)
    return (y + g.standard_normal(y.shape, dtype=np.float32) * np.float32(noise)).astype(np.float32)


def uniforms(shape, key) -> np.ndarray:
    """float32 uniforms in [0, 1): the random numbers a sampling step consumes."""
    return rng(*key).random(shape, dtype=np.float32)


# A small synthetic pre-norm decoder (Llama / Qwen style) for running rounds
# end to end: 2 layers, hidden 512 (4 q heads / 2 kv heads of 128), SwiGLU
# width 1024, vocabulary 4096, nested KV cache of 1024 tokens.
TINY_DECODER = {"vocab": 4096, "hidden": 512, "layers": 2, "q_heads": 4, "kv_heads": 2, "head_dim": 128,
                "inter": 1024, "theta": 10000.0, "eps": 1e-6, "capacity": 1024}


def decoder_weights(cfg: dict, key) -> dict:
    """fp32 weights of the decoder in ``cfg``: linears ~ N(0, 1/fan_in)
    (std 1/sqrt(fan_in)), the LM head at twice that, embeddings N(0, 1), norm
    gains 1 + N(0, 0.1). Linears are [out][in]; gate and up are stored
    concatenated as gate_up [2 * inter][hidden]."""
    H, I, V = cfg["hidden"], cfg["inter"], cfg["vocab"]
    qd = cfg["q_heads"] * cfg["head_dim"]
    kvd = cfg["kv_heads"] * cfg["head_dim"]
    key = tuple(key)
    w = {"embed": normal((V, H), key + (0,)),
         "lm_head": normal((V, H), key + (1,), std=2.0 / np.sqrt(H)),
         "norm_final": (1.0 + normal(H, key + (2,), std=0.1)).astype(np.float32),
         "layers": []}
    for li in range(cfg["layers"]):
        k2 = key + (10 + li,)
        w["layers"].append({
            "norm_attn": (1.0 + normal(H, k2 + (0,), std=0.1)).astype(np.float32),
            "norm_mlp": (1.0 + normal(H, k2 + (1,), std=0.1)).astype(np.float32),
            "qkv": normal((qd + 2 * kvd, H), k2 + (2,), std=1.0 / np.sqrt(H)),
            "o": normal((H, qd), k2 + (3,), std=1.0 / np.sqrt(qd)),
            "gate_up": normal((2 * I, H), k2 + (4,), std=1.0 / np.sqrt(H)),
            "down": normal((H, I), k2 + (5,), std=1.0 / np.sqrt(I)),
        })
    return w


def tokens(n: int, vocab: int, key) -> np.ndarray:
    """int32 token ids, uniform over the vocabulary (a synthetic prompt)."""
    return rng(*key).integers(0, vocab, size=n).astype(np.int32)
