"""Pure-Python brute force for tiny paged decode problems (a pin for the oracle).

It walks each sequence's block table token by token and folds every score into a
running (max, sum, accumulator) online softmax -- the per-token form described in
"Splitting the KV cache into 16-token blocks" (section "Online softmax: scanning
blocks into a weighted mean") and in "PagedAttention kernel: paged KV cache & block
tables" (section "Code"), written here from that description.  Element values are
decoded from their bit patterns with ``struct``, independently of numpy and the
oracle.  Only for inputs of a few thousand elements.
"""

from __future__ import annotations

import math
import struct


def _elem(bits: int, dtype: str) -> float:
    if dtype == "f32":
        return struct.unpack("<f", struct.pack("<I", bits))[0]
    if dtype == "bf16":
        return struct.unpack("<f", struct.pack("<I", bits << 16))[0]
    return struct.unpack("<e", struct.pack("<H", bits))[0]


def paged_decode(wl, k_flat, v_flat, v_base: int = 0):
    """[S][Hq][D] nested lists.  ``k_flat``/``v_flat`` are flat pool images (bit
    patterns); V elements start ``v_base`` elements into ``v_flat``."""
    S, Hq, Hkv, D, B = wl.num_seqs, wl.num_q_heads, wl.num_kv_heads, wl.head_size, wl.block_size
    group = Hq // Hkv
    scale = float(wl.scale)
    out = []
    for s in range(S):
        L = int(wl.seq_lens[s])
        row_out = []
        for h in range(Hq):
            kv = h // group
            q = [_elem(int(wl.q[s, h, d]), wl.dtype) for d in range(D)]
            m, l, acc = -math.inf, 0.0, [0.0] * D
            pos = 0
            for j in range(wl.block_tables.shape[1]):
                if pos >= L:
                    break
                phys = int(wl.block_tables[s, j])
                for r in range(B):
                    if pos >= L:
                        break
                    base = phys * wl.block_stride + r * wl.token_stride + kv * wl.head_stride
                    k = [_elem(int(k_flat[base + d]), wl.dtype) for d in range(D)]
                    v = [_elem(int(v_flat[v_base + base + d]), wl.dtype) for d in range(D)]
                    x = scale * sum(qi * ki for qi, ki in zip(q, k))
                    m_new = max(m, x)
                    corr = math.exp(m - m_new) if m != -math.inf else 0.0
                    p = math.exp(x - m_new)
                    l = l * corr + p
                    acc = [a * corr + p * vi for a, vi in zip(acc, v)]
                    m = m_new
                    pos += 1
            row_out.append([a / l for a in acc] if L > 0 else [0.0] * D)
        out.append(row_out)
    return out
