"""Test-side helpers: bit-pattern conversions and independent dense references.

Nothing here is shared with the oracle or the GPU path; these are the yardsticks
the oracle is pinned against and the converters a test uses to read results.
"""

from __future__ import annotations

import math
import os

import numpy as np

REPO = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN = os.path.join(REPO, "tests", "golden")


def bits_to_f64(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Storage bit patterns -> float64 (numpy's own format conversions)."""
    bits = np.asarray(bits)
    if dtype == "f32":
        return bits.astype(np.uint32).view(np.float32).astype(np.float64)
    if dtype == "bf16":
        return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if dtype == "f16":
        return bits.astype(np.uint16).view(np.float16).astype(np.float64)
    raise ValueError(dtype)


def f64_to_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    """float64 -> storage bits, round-to-nearest-even through float32 (tests only)."""
    x32 = np.asarray(x, dtype=np.float32)
    if dtype == "f32":
        return x32.view(np.uint32).copy()
    if dtype == "f16":
        return np.asarray(x, dtype=np.float64).astype(np.float16).view(np.uint16)
    u = x32.view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def dense_numpy(wl, q_bits=None) -> np.ndarray:
    """softmax(scale * q K^T) V per (s, h) on the generator's logical (contiguous)
    history, in float64 with numpy.  Query head h reads KV head h // (Hq / Hkv)."""
    q = bits_to_f64(wl.q if q_bits is None else q_bits, wl.dtype)
    S, Hq, D = q.shape
    G = Hq // wl.num_kv_heads
    out = np.zeros((S, Hq, D))
    scale = float(np.float32(wl.scale))
    for s in range(S):
        L = int(wl.seq_lens[s])
        if L == 0:
            continue
        K = bits_to_f64(wl.logical_k(s), wl.dtype)  # [L, Hkv, D]
        V = bits_to_f64(wl.logical_v(s), wl.dtype)
        for h in range(Hq):
            kv = h // G
            x = scale * (K[:, kv, :] @ q[s, h])
            p = np.exp(x - x.max())
            out[s, h] = (p @ V[:, kv, :]) / p.sum()
    return out


def online_tiles_numpy(wl, tile: int = 16) -> np.ndarray:
    """The same attention by a tile-wise online softmax (running max, sum and
    accumulator rescaled by exp(m_old - m_new)), float64."""
    q = bits_to_f64(wl.q, wl.dtype)
    S, Hq, D = q.shape
    G = Hq // wl.num_kv_heads
    out = np.zeros((S, Hq, D))
    scale = float(np.float32(wl.scale))
    for s in range(S):
        L = int(wl.seq_lens[s])
        if L == 0:
            continue
        K = bits_to_f64(wl.logical_k(s), wl.dtype)
        V = bits_to_f64(wl.logical_v(s), wl.dtype)
        for h in range(Hq):
            kv = h // G
            m, l, acc = -math.inf, 0.0, np.zeros(D)
            for t0 in range(0, L, tile):
                x = scale * (K[t0:t0 + tile, kv, :] @ q[s, h])
                m_new = max(m, float(x.max()))
                alpha = math.exp(m - m_new) if m != -math.inf else 0.0
                p = np.exp(x - m_new)
                l = alpha * l + p.sum()
                acc = alpha * acc + p @ V[t0:t0 + tile, kv, :]
                m = m_new
            out[s, h] = acc / l
    return out


def pool_view(wl, pool_arr: np.ndarray, which: str = "k") -> np.ndarray:
    """Index a pool image as [block, token, head, dim] through the workload's strides."""
    from numpy.lib.stride_tricks import as_strided
    es = pool_arr.itemsize
    base = pool_arr if which == "k" or wl.layout != "combined" else pool_arr[wl.v_offset:]
    return as_strided(base, shape=(wl.num_blocks, wl.block_size, wl.num_kv_heads, wl.head_size),
                      strides=(wl.block_stride * es, wl.token_stride * es, wl.head_stride * es, es),
                      writeable=False)


def with_abs_values(wl):
    """The same workload with every V element replaced by its magnitude (sign bit of
    the value rows cleared, history and step rows alike).  Dense attention over it
    gives sum_t p_t |v_t| / sum_t p_t per output element -- the scale of the error
    that rounding the probabilities p_t before P.V can cause."""
    import dataclasses
    sign = np.uint32(0x80000000) if wl.dtype == "f32" else np.uint16(0x8000)
    return dataclasses.replace(wl, pre_value=wl.pre_value & ~sign, value=wl.value & ~sign)


# relative error of a probability as P.V sees it: fp16 rounds it once (unit roundoff
# 2^-11, an 11-bit significand); bf16 (8-bit significand, unit roundoff 2^-8) carries it
# as the rounded value plus the rounded residual, 2^-8 of a residual of at most 2^-8
PROB_ROUNDOFF = {"bf16": 2.0 ** -16, "f16": 2.0 ** -11, "f32": 0.0}
