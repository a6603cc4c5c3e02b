"""Pure-Python brute force for tiny paged decode problems (a pin for the oracle).

Built from the mathematics of the operation, not from any printed listing:

* element values come from their bit patterns by the IEEE-754 field rules (sign,
  biased exponent, fraction; subnormals, infinities and NaN included), written out
  here with ``math.ldexp`` -- no ``struct``, numpy or C cast takes part;
* the logical history of a sequence is resolved position by position through its
  block table: position t lives in physical block ``table[t // block_size]`` at row
  ``t % block_size``, and the element address follows from the pool's strides;
* every dot product is summed exactly and rounded once (``math.fsum`` over products
  that are themselves exact in double, since each factor carries at most 24
  significant bits);
* the softmax is taken in log-sum-exp form: lse = M + log(sum_t exp(x_t - M)), each
  weight exp(x_t - lse) is already normalised, and each output element is the
  exactly rounded sum of weight times value.

The oracle instead keeps an unnormalised sum and divides at the end, in C; the two
agree to a few ulps of double.  Only for inputs of a few thousand elements.
"""

from __future__ import annotations

import math

# (exponent bits, fraction bits) of the storage formats
_FORMATS = {"f32": (8, 23), "f16": (5, 10), "bf16": (8, 7)}


def decode_bits(bits: int, dtype: str) -> float:
    """The real number (or inf / NaN) a storage bit pattern stands for."""
    ebits, fbits = _FORMATS[dtype]
    bias = (1 << (ebits - 1)) - 1
    frac = bits & ((1 << fbits) - 1)
    exp = (bits >> fbits) & ((1 << ebits) - 1)
    neg = (bits >> (fbits + ebits)) & 1
    if exp == (1 << ebits) - 1:
        mag = math.nan if frac else math.inf
    elif exp == 0:  # subnormal (or zero): no implicit leading one
        mag = math.ldexp(frac, 1 - bias - fbits)
    else:
        mag = math.ldexp(frac + (1 << fbits), exp - bias - fbits)
    return -mag if neg else mag


def _row(flat, base: int, n: int, dtype: str) -> list:
    return [decode_bits(int(flat[base + d]), dtype) for d in range(n)]


def paged_decode(wl, k_flat, v_flat, v_base: int = 0):
    """[S][Hq][D] nested lists of floats.  ``k_flat``/``v_flat`` are flat pool images
    (bit patterns); V elements start ``v_base`` elements into ``v_flat``."""
    D, Bs = wl.head_size, wl.block_size
    heads_per_kv = wl.num_q_heads // wl.num_kv_heads
    scale = float(wl.scale)
    result = []
    for s in range(wl.num_seqs):
        L = int(wl.seq_lens[s])
        table = [int(x) for x in wl.block_tables[s]]
        per_head = []
        for h in range(wl.num_q_heads):
            if L == 0:
                per_head.append([0.0] * D)
                continue
            kvh = h // heads_per_kv
            q = [decode_bits(int(x), wl.dtype) for x in wl.q[s, h]]
            # element address of (position t, dim 0) of this kv head
            addr = [table[t // Bs] * wl.block_stride + (t % Bs) * wl.token_stride + kvh * wl.head_stride
                    for t in range(L)]
            scores = [scale * math.fsum(a * b for a, b in zip(q, _row(k_flat, base, D, wl.dtype))) for base in addr]
            top = max(scores)
            lse = top + math.log(math.fsum(math.exp(x - top) for x in scores))
            weights = [math.exp(x - lse) for x in scores]
            values = [_row(v_flat, v_base + base, D, wl.dtype) for base in addr]
            per_head.append([math.fsum(w * v[d] for w, v in zip(weights, values)) for d in range(D)])
        result.append(per_head)
    return result
