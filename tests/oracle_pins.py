"""Pins for the CPU oracle: checks against what the pages and mathematics fix.

Each ``pin_*`` function raises ``AssertionError`` (or ``oracle.OracleError``) when
the oracle disagrees with something it does not compute itself:

* worked values printed on the pages (``tests/golden/*.json``, each cites its page);
* closed forms (one visible token, q = 0, identical keys, two tokens, huge logits);
* invariants (any physical placement of the blocks, unread memory, padding rows);
* independent references (numpy and torch float64 dense attention on the contiguous
  history, a tile-wise online softmax, a pure-Python per-token brute force);
* the split identity (per-partition partials merged = the whole sequence);
* for the 8-bit cache: the OCP E4M3 landmarks and torch's float8_e4m3fn converter,
  and dense attention on dequantised rows;
* for ALiBi: zero slopes change nothing, torch's attention with the bias as an
  additive mask, the geometric weights of q = 0, and the partials' maxima;
* for multi-token (varlen) queries: single tokens reproduce the decode, numpy and
  torch references with the causal limit written out, prefix means of q = 0, a
  first token that sees exactly one row, and the non-causal form.

``tests/test_oracle_pins.py`` runs them; ``tests/test_oracle_mutants.py`` plants
mistakes in copies of the oracle and requires some pin to fail for each.
"""

from __future__ import annotations

import functools
import json
import math
import os
from types import SimpleNamespace

import numpy as np

import brute
import oracle
from helpers import GOLDEN, bits_to_f64, dense_numpy, f64_to_bits, online_tiles_numpy
from workloads import alibi_variant, custom, fp8_variant, make_config, nan_bits, varlen_variant

B = 16


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


@functools.lru_cache(maxsize=None)
def _cfg(idx, contents=True):
    return make_config(idx, contents=contents)


def hand_wl(dtype, Hq, Hkv, D, num_blocks, block_tables, seq_lens, q_f64):
    """A hand-built HND workload ([num_blocks, Hkv, B, D] per buffer)."""
    wl = SimpleNamespace(dtype=dtype, num_seqs=len(seq_lens), num_q_heads=Hq, num_kv_heads=Hkv, head_size=D,
                         block_size=B, layout="hnd", num_blocks=num_blocks, block_stride=Hkv * B * D,
                         token_stride=D, head_stride=B * D, v_offset=0, pool_elems=num_blocks * Hkv * B * D,
                         seq_lens=np.asarray(seq_lens, np.int32),
                         block_tables=np.asarray(block_tables, np.int32).reshape(len(seq_lens), -1),
                         scale=np.float32(1.0 / math.sqrt(D)), q=f64_to_bits(np.asarray(q_f64), dtype))
    bits = np.uint32 if dtype == "f32" else np.uint16
    wl.nan_pool = lambda: np.full(wl.pool_elems, nan_bits(dtype), dtype=bits)
    return wl


def hand_pool(wl, K, V):
    """Pool image from per-physical-slot rows K, V shaped [num_blocks, B, Hkv, D] (float64);
    the HND buffer is [num_blocks, Hkv, B, D]."""
    k = f64_to_bits(np.ascontiguousarray(np.transpose(K, (0, 2, 1, 3))), wl.dtype).reshape(-1)
    v = f64_to_bits(np.ascontiguousarray(np.transpose(V, (0, 2, 1, 3))), wl.dtype).reshape(-1)
    return oracle.Pool(k, v, 0, wl.pool_elems)


def _rounded(x, dtype):
    return bits_to_f64(f64_to_bits(x, dtype), dtype)


# ---------------------------------------------------------------------------------
# worked examples printed on the pages
# ---------------------------------------------------------------------------------

def pin_slot_write():
    """Slot 36 of the worked example lands at physical block 2, offset 4, and nowhere else."""
    g = _golden("slot_example.json")
    Hkv, D = 2, 8
    wl = hand_wl("f32", Hkv, Hkv, D, 10, [g["block_table"]], [g["position"] + 1], np.zeros((1, Hkv, D)))
    pool = oracle.empty_pool(wl)
    key = f64_to_bits(np.arange(1, Hkv * D + 1, dtype=float).reshape(1, Hkv, D), "f32")
    value = f64_to_bits(-np.arange(1, Hkv * D + 1, dtype=float).reshape(1, Hkv, D), "f32")
    oracle.write(wl, pool, key, value, np.array([g["slot"]], np.int64))
    for arr, row in ((pool.k, key[0]), (pool.v, value[0])):
        img = arr.reshape(10, Hkv, B, D)
        assert np.array_equal(img[g["physical_block"], :, g["offset"], :], row)
        rest = np.ones(img.shape, bool)
        rest[g["physical_block"], :, g["offset"], :] = False
        assert (img[rest] == nan_bits("f32")).all()


def _saturating_read(g, position_key, length_key, target_block, target_offset, table):
    """All keys zero except one physical slot whose key scores 50 against q: the output
    is that slot's value row iff the read resolves the position to that slot."""
    D = 8
    rng = np.random.default_rng(1)
    wl = hand_wl("f32", 1, 1, D, 10, [table], [g[length_key]], rng.standard_normal((1, 1, D)))
    qv = bits_to_f64(wl.q, "f32")[0, 0]
    scale = float(wl.scale)
    K = np.zeros((10, B, 1, D))
    V = _rounded(rng.standard_normal((10, B, 1, D)), "f32")
    K[target_block, target_offset, 0] = qv * (50.0 / (scale * float(qv @ qv)))
    pool = hand_pool(wl, K, V)
    out = oracle.decode(wl, pool)[0, 0]
    assert np.abs(out - V[target_block, target_offset, 0]).max() < 1e-12
    # one token shorter: the target position is not visible, every score is 0, and the
    # output is the plain mean of the rows the table maps positions 0..L-2 to
    L = g[length_key] - 1
    out2 = oracle.decode(wl, pool, seq_lens=np.array([L], np.int32))[0, 0]
    rows = [V[table[t // B], t % B, 0] for t in range(L)]
    assert np.abs(out2 - np.mean(rows, axis=0)).max() < 1e-13
    assert np.abs(out2 - V[target_block, target_offset, 0]).max() > 1e-3


def pin_slot_read():
    """Position 20 under block_table [7, 2, 9] is read from physical block 2, offset 4."""
    g = _golden("slot_example.json")
    g = dict(g, seq_len=g["position"] + 1)
    _saturating_read(g, "position", "seq_len", g["physical_block"], g["offset"], g["block_table"])


def pin_invariant_line():
    """seq_len 17 with block_table [7, 2]: logical token 16 is physical block 2, offset 0."""
    g = _golden("invariant_example.json")
    _saturating_read(g, "logical_token", "seq_len", g["physical_block"], g["offset"], g["block_table"])


def pin_gqa_mapping():
    """Query head h reads KV head h / (Hq / Hkv) (printed examples)."""
    g = _golden("gqa_examples.json")
    for case in g["cases"]:
        Hq, Hkv, D = case["num_q_heads"], case["num_kv_heads"], 8
        rng = np.random.default_rng(2)
        wl = hand_wl("f32", Hq, Hkv, D, 2, [[1]], [5], rng.standard_normal((1, Hq, D)))
        K = _rounded(rng.standard_normal((2, B, Hkv, D)), "f32")
        V = np.zeros((2, B, Hkv, D))
        for kv in range(Hkv):
            V[:, :, kv, :] = kv + 1.0  # every value row of KV head kv is (kv + 1)
        out = oracle.decode(wl, hand_pool(wl, K, V))[0]
        for h, kv in case["pairs"]:
            assert np.abs(out[h] - (kv + 1.0)).max() < 1e-14, (h, kv, out[h][:2])


def pin_worked_decode():
    """8 query heads / 2 KV heads, seq_len 35 over [7, 2, 9]: query head 5 reads KV head 1
    and position 34 sits in physical block 9, offset 2."""
    g = _golden("worked_decode.json")
    Hq, Hkv, D = g["num_q_heads"], g["num_kv_heads"], g["head_size"]
    rng = np.random.default_rng(3)
    wl = hand_wl("bf16", Hq, Hkv, D, 10, [g["block_table"]], [g["seq_len"]], rng.standard_normal((1, Hq, D)))
    q = bits_to_f64(wl.q, "bf16")[0]
    K = np.zeros((10, B, Hkv, D))
    V = _rounded(rng.standard_normal((10, B, Hkv, D)), "bf16")
    pb = g["last_block_tokens"]["physical_block"]
    off = g["last_block_tokens"]["offsets"][-1]
    qh = q[g["query_head"]]
    K[pb, off, g["kv_head"]] = _rounded(qh * (60.0 / (float(wl.scale) * float(qh @ qh))), "bf16")
    out = oracle.decode(wl, hand_pool(wl, K, V))[0]
    assert np.abs(out[g["query_head"]] - V[pb, off, g["kv_head"]]).max() < 1e-9
    # heads of KV head 0 saw only zero keys: the plain mean of the 35 rows of KV head 0
    rows = [V[g["block_table"][t // B], t % B, 0] for t in range(g["seq_len"])]
    for h in range(Hq // Hkv):
        assert np.abs(out[h] - np.mean(rows, axis=0)).max() < 1e-13


def pin_combined_block_layout():
    """tiny-vllm's combined block: V_OFFSET 16384 B, 32768 B blocks, 65536 blocks in 2 GiB,
    128 blocks per 2048-token sequence; bytes land where its address rule says."""
    g = _golden("combined_block_constants.json")
    w = _cfg(2, contents=False)
    assert w.v_offset * w.esize == g["v_offset_bytes"]
    assert w.block_stride * w.esize == g["block_bytes"]
    assert w.num_blocks == g["num_blocks"] == g["cache_bytes"] // g["block_bytes"]
    assert w.block_tables.shape[1] == g["max_blocks_per_seq"] == g["max_seq_len"] // g["block_size"]
    assert w.num_kv_heads * w.head_size == g["kv_dim"]
    assert 2 * 16 * g["max_blocks_per_seq"] == g["block_table_entries_2_seqs_16_layers"]
    small = custom(0, "bf16", 32, 8, 64, [5], layout="combined", pool_factor=3.0)
    pool = oracle.empty_pool(small)
    rng = np.random.default_rng(4)
    key = f64_to_bits(rng.standard_normal((1, 8, 64)), "bf16")
    value = f64_to_bits(rng.standard_normal((1, 8, 64)), "bf16")
    blk, tok = 2, 3
    oracle.write(small, pool, key, value, np.array([blk * B + tok], np.int64))
    raw = pool.k.view(np.uint8)
    for h in range(8):
        for d in range(64):
            a = blk * g["block_bytes"] + tok * g["kv_dim"] * 2 + h * g["head_dim"] * 2 + d * 2
            assert raw[a:a + 2].view(np.uint16)[0] == key[0, h, d]
            a += g["v_offset_bytes"]
            assert raw[a:a + 2].view(np.uint16)[0] == value[0, h, d]


# ---------------------------------------------------------------------------------
# closed forms
# ---------------------------------------------------------------------------------

def pin_one_token_exact():
    """One visible token: the output is that token's value row, exactly."""
    for dt in ("f32", "bf16", "f16"):
        w = custom(3, dt, 4, 2, 64, [1, 1, 1])
        out = oracle.decode(w, oracle.filled_pool(w))
        for s in range(3):
            for h in range(4):
                assert np.array_equal(out[s, h], bits_to_f64(w.logical_v(s)[0, h // 2], dt)), (dt, s, h)


def pin_special_values_exact():
    """Format decoding: subnormals, zeros, the largest finite values and ordinary
    normals come back exactly through a one-token read (a zero's sign is not kept:
    the weighted sum starts from +0)."""
    specials = {
        "f16": [0x0001, 0x03FF, 0x0400, 0x8001, 0x8000, 0x7BFF, 0xFBFF, 0x3C00, 0x3555, 0xC800],
        "bf16": [0x0001, 0x007F, 0x0080, 0x8001, 0x8000, 0x7F7F, 0xFF7F, 0x3F80, 0x3EAB, 0xC120],
        "f32": [0x00000001, 0x007FFFFF, 0x00800000, 0x80000001, 0x80000000, 0x7F7FFFFF, 0xFF7FFFFF,
                0x3F800000, 0x3EAAAAAB, 0xC1200000],
    }
    for dt, pats in specials.items():
        D = 64
        w = custom(20, dt, 1, 1, D, [1])
        row = np.resize(np.array(pats, dtype=w.bits_dtype), D)
        w.key[0, 0, :] = row
        w.bank_v[w.logical_src[0][0], 0, :] = row
        w.value[0, 0, :] = row
        out = oracle.decode(w, oracle.filled_pool(w))[0, 0]
        expect = bits_to_f64(row, dt)
        assert np.array_equal(out, expect), dt


def pin_zero_query_mean():
    """q = 0: every score is 0 and the output is the mean of the visible value rows."""
    w = custom(4, "bf16", 8, 2, 64, [1, 7, 33, 100])
    out = oracle.decode(w, oracle.filled_pool(w), q=np.zeros_like(w.q))
    for s in range(w.num_seqs):
        V = bits_to_f64(w.logical_v(s), "bf16")
        for h in range(8):
            assert np.abs(out[s, h] - V[:, h // 4].mean(axis=0)).max() < 1e-13


def pin_equal_keys_mean():
    """All keys identical: uniform softmax, the output is the mean of the value rows."""
    w = custom(5, "f16", 4, 4, 128, [3, 40, 64])
    w.pre_key[:] = w.key[0]
    w.key[:] = w.key[0]
    out = oracle.decode(w, oracle.filled_pool(w))
    for s in range(w.num_seqs):
        V = bits_to_f64(w.logical_v(s), "f16")
        for h in range(4):
            assert np.abs(out[s, h] - V[:, h].mean(axis=0)).max() < 1e-13


def _sig(z):
    return 1.0 / (1.0 + math.exp(-z))


def pin_two_tokens_sigmoid():
    """Two tokens: out = sigma(x0 - x1) v0 + sigma(x1 - x0) v1, x_t = scale q.k_t."""
    w = custom(6, "f32", 4, 2, 64, [2, 2])
    out = oracle.decode(w, oracle.filled_pool(w))
    sc = float(w.scale)
    q = bits_to_f64(w.q, "f32")
    for s in range(2):
        K = bits_to_f64(w.logical_k(s), "f32")
        V = bits_to_f64(w.logical_v(s), "f32")
        for h in range(4):
            kv = h // 2
            x0 = sc * math.fsum(q[s, h] * K[0, kv])
            x1 = sc * math.fsum(q[s, h] * K[1, kv])
            exp = _sig(x0 - x1) * V[0, kv] + _sig(x1 - x0) * V[1, kv]
            assert np.abs(out[s, h] - exp).max() < 1e-14


def pin_huge_logits():
    """Scores near 800 overflow exp() unless the running maximum is subtracted first."""
    D = 8
    q = np.zeros((1, 1, D))
    q[0, 0, 0] = 1.0
    wl = hand_wl("f32", 1, 1, D, 1, [[0]], [2], q)
    K = np.zeros((1, B, 1, D))
    K[0, 0, 0, 0] = 2262.75
    K[0, 1, 0, 0] = 2234.5
    rng = np.random.default_rng(5)
    V = _rounded(rng.standard_normal((1, B, 1, D)), "f32")
    out = oracle.decode(wl, hand_pool(wl, K, V))[0, 0]
    sc = float(wl.scale)
    x0, x1 = sc * 2262.75, sc * 2234.5
    assert x0 > 790 and x1 > 780
    exp = _sig(x0 - x1) * V[0, 0, 0] + _sig(x1 - x0) * V[0, 1, 0]
    assert np.isfinite(out).all() and np.abs(out - exp).max() < 1e-12


# ---------------------------------------------------------------------------------
# invariants
# ---------------------------------------------------------------------------------

def pin_placement_invariance():
    """Any physical arrangement of the blocks gives exactly the same output."""
    args = (11, "bf16", 8, 2, 64, [1, 17, 40, 64, 100])
    outs, tables = [], []
    for pl in (None, "identity", 123, 456):
        w = custom(*args, placement=pl)
        tables.append(w.block_tables)
        outs.append(oracle.decode(w, oracle.filled_pool(w)))
    assert not np.array_equal(tables[0], tables[1]) and not np.array_equal(tables[2], tables[3])
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


def pin_negative_slot_skipped():
    """A negative slot has no destination: the pool is left byte-identical, and the
    filled pool holds exactly the valid tokens (the padding row landed nowhere)."""
    w = _cfg(0)
    pool = oracle.filled_pool(w, step_write=False)
    before = [a.copy() for a in pool.arrays()]
    oracle.write(w, pool, w.key, w.value, np.full(len(w.slot_mapping), -1, np.int64))
    assert all(np.array_equal(b, a) for b, a in zip(before, pool.arrays()))
    pool = oracle.filled_pool(w)
    written = sum(int((a != nan_bits(w.dtype)).sum()) for a in pool.arrays())
    assert written == 2 * int(w.seq_lens.sum()) * w.num_kv_heads * w.head_size


def pin_unread_memory():
    """Memory outside the visible tokens (block tails, unused blocks) is never read:
    overwriting it with other values leaves the output bit-identical and finite."""
    for w in (_cfg(0), custom(18, "bf16", 8, 2, 64, [1, 17, 31]), custom(21, "f16", 4, 4, 64, [2, 47], layout="nhd")):
        pool = oracle.filled_pool(w)
        out = oracle.decode(w, pool)
        assert np.isfinite(out).all()
        garbage = f64_to_bits(np.array([1.0e4]), w.dtype)[0]
        for a in pool.arrays():
            a[a == nan_bits(w.dtype)] = garbage
        assert np.array_equal(oracle.decode(w, pool), out)


def pin_table_padding():
    """Entries past ceil(L/B) are padding (-1) and never dereferenced; a length that
    would need them is refused."""
    w = custom(19, "f32", 4, 4, 64, [3, 40], table_width=8)
    assert (w.block_tables == -1).sum() >= 8
    pool = oracle.filled_pool(w)
    oracle.decode(w, pool)
    for bad in (17, 8 * B + 1):
        sl = w.seq_lens.copy()
        sl[0] = bad
        try:
            oracle.decode(w, pool, seq_lens=sl)
        except oracle.OracleError:
            continue
        raise AssertionError(f"seq_len {bad} over a padded row was accepted")


def pin_write_out_of_range():
    """A slot past the pool is refused rather than written."""
    w = _cfg(0)
    pool = oracle.empty_pool(w)
    try:
        oracle.write(w, pool, w.key[:1], w.value[:1], np.array([w.num_blocks * B], np.int64))
    except oracle.OracleError:
        return
    raise AssertionError("out-of-range slot accepted")


# ---------------------------------------------------------------------------------
# independent references
# ---------------------------------------------------------------------------------

def _ref_cases():
    return [
        _cfg(0),
        custom(7, "bf16", 32, 8, 128, [1, 15, 16, 17, 100, 511, 513]),
        custom(8, "f16", 8, 8, 128, [3, 200]),
        custom(9, "bf16", 32, 8, 64, [1, 2, 1000], layout="combined"),
        custom(10, "f32", 8, 2, 64, [5, 64], layout="nhd"),
        custom(22, "f16", 16, 4, 128, [40, 70], prefix_blocks=2, pad_count=1),
    ]


def pin_numpy_dense():
    """numpy softmax(scale q K^T) V on the contiguous history agrees to 1e-12."""
    for w in _ref_cases():
        out = oracle.decode(w, oracle.filled_pool(w))
        assert np.abs(out - dense_numpy(w)).max() < 1e-12, w.name


def pin_block_sizes():
    """Blocks of 8 and 32 tokens, every layout: numpy dense attention agrees to 1e-12."""
    for B in (8, 32):
        for layout in ("hnd", "nhd", "combined"):
            w = custom(23 + B, "bf16", 8, 2, 64, [1, 7, 8, 9, 31, 33, 300], layout=layout, block_size=B)
            out = oracle.decode(w, oracle.filled_pool(w))
            assert np.abs(out - dense_numpy(w)).max() < 1e-12, (B, layout)


def pin_torch_sdpa():
    """torch scaled_dot_product_attention in float64 on the CPU agrees to 1e-12."""
    import torch
    w = custom(12, "bf16", 16, 4, 64, [1, 9, 130])
    out = oracle.decode(w, oracle.filled_pool(w))
    G = w.num_q_heads // w.num_kv_heads
    q = torch.from_numpy(bits_to_f64(w.q, w.dtype))
    for s in range(w.num_seqs):
        K = torch.from_numpy(bits_to_f64(w.logical_k(s), w.dtype)).permute(1, 0, 2).repeat_interleave(G, 0)
        V = torch.from_numpy(bits_to_f64(w.logical_v(s), w.dtype)).permute(1, 0, 2).repeat_interleave(G, 0)
        ref = torch.nn.functional.scaled_dot_product_attention(q[s].unsqueeze(1).unsqueeze(0), K.unsqueeze(0),
                                                               V.unsqueeze(0), scale=float(w.scale))
        assert (ref[0, :, 0, :].numpy() - out[s]).__abs__().max() < 1e-12


def pin_online_tiles():
    """A tile-wise online softmax (running max/sum/accumulator) agrees to 1e-12."""
    w = custom(16, "bf16", 32, 8, 128, [1, 16, 17, 300])
    out = oracle.decode(w, oracle.filled_pool(w))
    assert np.abs(out - online_tiles_numpy(w)).max() < 1e-12


def pin_brute_force():
    """A pure-Python per-token walk of the block table agrees to 1e-12."""
    cases = [_cfg(0), custom(13, "bf16", 4, 2, 64, [1, 16, 17, 33]), custom(14, "f16", 2, 1, 64, [20]),
             custom(15, "bf16", 4, 2, 64, [5, 30], layout="combined")]
    for w in cases:
        pool = oracle.filled_pool(w)
        out = oracle.decode(w, pool)
        ref = np.array(brute.paged_decode(w, pool.k, pool.v, pool.v_offset))
        assert np.abs(out - ref).max() < 1e-12, w.name


# ---------------------------------------------------------------------------------
# the split identity
# ---------------------------------------------------------------------------------

def pin_split_identity():
    """Partials of P-token partitions, merged by log-sum-exp, equal the whole-sequence
    result; partitions past seq_len are left untouched; each partial is dense
    attention over its own token range."""
    w = custom(17, "f32", 4, 2, 64, [1, 15, 16, 17, 511, 512, 513, 1100])
    pool = oracle.filled_pool(w)
    dense = oracle.decode(w, pool)
    q = bits_to_f64(w.q, w.dtype)
    sc = float(w.scale)
    for P in (16, 32, 48, 512):
        tmp, ml, es = oracle.partials(w, pool, P)
        for s in range(w.num_seqs):
            L = int(w.seq_lens[s])
            n = -(-L // P)
            assert np.isnan(ml[s, :, n:]).all() and np.isnan(tmp[s, :, n:]).all()
            assert np.isfinite(ml[s, :, :n]).all() and np.isfinite(tmp[s, :, :n]).all()
            if s == w.num_seqs - 1:  # spot-check each partial of the longest sequence
                K = bits_to_f64(w.logical_k(s), w.dtype)
                V = bits_to_f64(w.logical_v(s), w.dtype)
                for p in range(n):
                    for h in (0, 3):
                        x = sc * (K[p * P:(p + 1) * P, h // 2] @ q[s, h])
                        e = np.exp(x - x.max())
                        assert abs(ml[s, h, p] - x.max()) < 1e-13
                        assert abs(es[s, h, p] - e.sum()) < 1e-12 * e.sum()
                        assert np.abs(tmp[s, h, p] - e @ V[p * P:(p + 1) * P, h // 2] / e.sum()).max() < 1e-13
        merged = oracle.merge(tmp, ml, es, w.seq_lens, P)
        assert np.abs(merged - dense).max() < 1e-13, P


# ---------------------------------------------------------------------------------
# 8-bit (OCP E4M3) cache
# ---------------------------------------------------------------------------------

def _torch_e4m3_value(codes: np.ndarray) -> np.ndarray:
    import torch
    return torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn).double().numpy()


def _torch_e4m3_code(x32: np.ndarray) -> np.ndarray:
    """torch's nearest-even float8_e4m3fn conversion, after clamping to +-448 (torch
    maps larger magnitudes to NaN)."""
    import torch
    y = np.where(np.isnan(x32), x32, np.clip(x32, -448.0, 448.0)).astype(np.float32)
    codes = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()
    codes[np.isnan(x32)] = 0xFF
    return codes


def pin_e4m3_values():
    """Every code's value: the OCP definition's landmarks and torch's float8_e4m3fn."""
    codes = np.arange(256, dtype=np.uint8)
    v = oracle.e4m3_decode(codes)
    t = _torch_e4m3_value(codes)
    assert np.array_equal(np.isnan(v), np.isnan(t)) and np.array_equal(v[~np.isnan(v)], t[~np.isnan(t)])
    assert np.isnan(v[[0x7F, 0xFF]]).all() and np.isnan(v).sum() == 2  # no infinities, one NaN per sign
    assert v[0x38] == 1.0 and v[0x7E] == 448.0 and v[0xFE] == -448.0  # 1.75 * 2^8 is the largest
    assert v[0x01] == 2.0 ** -9 and v[0x07] == 7 * 2.0 ** -9 and v[0x08] == 2.0 ** -6  # subnormals, min normal
    assert v[0x00] == 0.0 and np.signbit(v[0x80])
    assert (np.diff(v[:0x7F]) > 0).all()  # codes 0..0x7E increase


def pin_e4m3_rounding():
    """Nearest code, ties to the even mantissa, saturation at 448, NaN -> 0xFF."""
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = oracle.e4m3_decode(finite).astype(np.float32)
    back = oracle.e4m3_encode(vals)
    assert np.array_equal(back[vals != 0], finite[vals != 0])  # every finite value maps to its own code
    pos = oracle.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mid = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)  # exact in binary32
    tie = oracle.e4m3_encode(mid)
    lo = np.arange(0x7E)
    assert np.array_equal(tie, np.where(lo % 2 == 0, lo, lo + 1).astype(np.uint8))
    up = oracle.e4m3_encode(np.nextafter(mid, np.float32(1e9)))
    down = oracle.e4m3_encode(np.nextafter(mid, np.float32(-1e9)))
    assert np.array_equal(up, lo + 1) and np.array_equal(down, lo)
    big = np.array([448, 449, 463.9, 464, 480, 1e4, 3e38, np.inf], dtype=np.float32)
    assert (oracle.e4m3_encode(big) == 0x7E).all() and (oracle.e4m3_encode(-big) == 0xFE).all()
    assert oracle.e4m3_encode(np.array([np.nan], dtype=np.float32))[0] == 0xFF
    x = (np.random.default_rng(3).standard_normal(50000) * 60).astype(np.float32)
    assert np.array_equal(oracle.e4m3_encode(x), _torch_e4m3_code(x))


@functools.lru_cache(maxsize=None)
def _fp8_wl(per_head=True):
    # small scales: values beyond ~2.2 sigma saturate, so that branch is exercised
    return fp8_variant(custom(21, "bf16", 8, 2, 64, [1, 16, 17, 40, 530], extra_pad_rows=1), per_head=per_head,
                       lo=0.005, hi=0.02)


def _quantised_history(w):
    """Per sequence [L, Hkv, D]: codes of the logical history, by torch's converter."""
    ks, vs = w.k_scale.astype(np.float32), w.v_scale.astype(np.float32)
    kh = np.repeat(ks, w.num_kv_heads) if w.scale_stride == 0 else ks
    vh = np.repeat(vs, w.num_kv_heads) if w.scale_stride == 0 else vs
    out = []
    for s in range(w.num_seqs):
        K = bits_to_f64(w.logical_k(s), w.dtype).astype(np.float32)
        V = bits_to_f64(w.logical_v(s), w.dtype).astype(np.float32)
        out.append((_torch_e4m3_code(K / kh[None, :, None]), _torch_e4m3_code(V / vh[None, :, None]), kh, vh))
    return out


def pin_kv8_write():
    """The 8-bit write stores the code of x / scale of its head (torch's converter), in
    the slot the flattening names; nothing else changes."""
    sat = 0
    for per_head in (True, False):
        w = _fp8_wl(per_head)
        pool = oracle.filled_pool(w)
        hist = _quantised_history(w)
        written = np.zeros(w.pool_elems, bool)
        for s in range(w.num_seqs):
            kc, vc, _, _ = hist[s]
            for t in range(int(w.seq_lens[s])):
                phys = int(w.block_tables[s, t // B])
                for h in range(w.num_kv_heads):
                    base = phys * w.block_stride + (t % B) * w.token_stride + h * w.head_stride
                    assert np.array_equal(pool.k[base:base + w.head_size], kc[t, h]), (per_head, s, t, h)
                    assert np.array_equal(pool.v[base:base + w.head_size], vc[t, h]), (per_head, s, t, h)
                    written[base:base + w.head_size] = True
        assert (pool.k[~written] == 0x7F).all() and (pool.v[~written] == 0x7F).all()
        sat += sum(int((np.abs(oracle.e4m3_decode(c)) == 448).sum()) for kc, vc, _, _ in hist for c in (kc, vc))
    assert sat > 0  # the scales make some values saturate: that branch is exercised


def pin_kv8_decode():
    """Decode over the 8-bit pool = dense attention on code value * scale (numpy),
    q = 0 gives the mean of the dequantised V, and the partials merge to it."""
    w = _fp8_wl(True)
    pool = oracle.filled_pool(w)
    out = oracle.decode(w, pool)
    hist = _quantised_history(w)
    q = bits_to_f64(w.q, w.dtype)
    G = w.num_q_heads // w.num_kv_heads
    zero = oracle.decode(w, pool, q=np.zeros_like(w.q))
    for s in range(w.num_seqs):
        kc, vc, kh, vh = hist[s]
        K = _torch_e4m3_value(kc) * kh[None, :, None].astype(np.float64)
        V = _torch_e4m3_value(vc) * vh[None, :, None].astype(np.float64)
        for h in range(w.num_q_heads):
            x = float(w.scale) * (K[:, h // G] @ q[s, h])
            e = np.exp(x - x.max())
            assert np.abs(out[s, h] - e @ V[:, h // G] / e.sum()).max() < 1e-12, (s, h)
            assert np.abs(zero[s, h] - V[:, h // G].mean(axis=0)).max() < 1e-12, (s, h)
    for P in (16, 512):
        tmp, ml, es = oracle.partials(w, pool, P)
        assert np.abs(oracle.merge(tmp, ml, es, w.seq_lens, P) - out).max() < 1e-13


# ---------------------------------------------------------------------------------
# ALiBi ("vLLM 源码完全拆解（七）", 第一步: score of token t gains a_h * (t - (L - 1)))
# ---------------------------------------------------------------------------------

def _alibi_wl(dtype="bf16", lengths=(1, 2, 17, 300, 700), Hq=8, Hkv=2, D=64, seed=30):
    w = custom(seed, dtype, Hq, Hkv, D, list(lengths))
    # slopes of both signs and sizes, one per query head (distinct within a kv group)
    slopes = np.linspace(-0.05, 0.4, Hq).astype(np.float32)[::-1].copy()
    return alibi_variant(w, slopes)


def pin_alibi_zero_slopes():
    """All slopes 0: bit-identical to the decode without ALiBi (and the partials)."""
    w = custom(31, "f16", 8, 4, 128, [1, 33, 520])
    z = alibi_variant(w, np.zeros(8, np.float32))
    pool = oracle.filled_pool(w)
    assert np.array_equal(oracle.decode(z, pool), oracle.decode(w, pool))
    a, b = oracle.partials(z, pool, 512), oracle.partials(w, pool, 512)
    for x, y in zip(a, b):
        assert np.array_equal(x, y, equal_nan=True)


def pin_alibi_torch_sdpa():
    """torch scaled_dot_product_attention in float64 with the bias a_h * (t - (L - 1))
    as an additive float mask agrees to 1e-12 (query head h uses slope a_h)."""
    import torch
    w = _alibi_wl()
    out = oracle.decode(w, oracle.filled_pool(w))
    G = w.num_q_heads // w.num_kv_heads
    q = torch.from_numpy(bits_to_f64(w.q, w.dtype))
    a = torch.from_numpy(w.alibi_slopes.astype(np.float64))
    for s in range(w.num_seqs):
        L = int(w.seq_lens[s])
        K = torch.from_numpy(bits_to_f64(w.logical_k(s), w.dtype)).permute(1, 0, 2).repeat_interleave(G, 0)
        V = torch.from_numpy(bits_to_f64(w.logical_v(s), w.dtype)).permute(1, 0, 2).repeat_interleave(G, 0)
        dist = torch.arange(L, dtype=torch.float64) - (L - 1)  # <= 0, 0 at the newest token
        mask = (a[:, None] * dist[None, :]).unsqueeze(1)         # [Hq, 1, L]
        ref = torch.nn.functional.scaled_dot_product_attention(q[s].unsqueeze(1), K, V, attn_mask=mask,
                                                               scale=float(w.scale))
        assert (ref[:, 0, :].numpy() - out[s]).__abs__().max() < 1e-12, s


def pin_alibi_geometric_weights():
    """q = 0 leaves only the bias: token t weighs r^(L-1-t) with r = e^(-a_h), so the
    output is that geometric average of V (numpy, written from the powers)."""
    w = _alibi_wl(dtype="f32", lengths=(1, 5, 64, 129))
    pool = oracle.filled_pool(w)
    out = oracle.decode(w, pool, q=np.zeros_like(w.q))
    G = w.num_q_heads // w.num_kv_heads
    for s in range(w.num_seqs):
        L = int(w.seq_lens[s])
        V = bits_to_f64(w.logical_v(s), w.dtype)
        for h in range(w.num_q_heads):
            r = math.exp(-float(w.alibi_slopes[h]))
            wts = np.array([r ** (L - 1 - t) for t in range(L)])
            ref = wts @ V[:, h // G] / wts.sum()
            assert np.abs(out[s, h] - ref).max() < 1e-12, (s, h)


def pin_alibi_partials():
    """With q = 0 the max score of partition p is a_h * (last position of p - (L - 1))
    (a_h >= 0) or a_h * (first position of p - (L - 1)) (a_h < 0), exactly; the partials
    merge to the whole-sequence result."""
    w = _alibi_wl(dtype="bf16", lengths=(1, 511, 512, 513, 1500))
    pool = oracle.filled_pool(w)
    zq = np.zeros_like(w.q)
    dense = oracle.decode(w, pool, q=zq)
    for P in (16, 512):
        tmp, ml, es = oracle.partials(w, pool, P, q=zq)
        for s in range(w.num_seqs):
            L = int(w.seq_lens[s])
            for p in range(-(-L // P)):
                first, last = p * P, min(L, (p + 1) * P) - 1
                for h in range(w.num_q_heads):
                    a = float(w.alibi_slopes[h])
                    want = a * ((last if a >= 0 else first) - (L - 1))
                    assert abs(ml[s, h, p] - want) < 1e-12, (P, s, p, h)
        assert np.abs(oracle.merge(tmp, ml, es, w.seq_lens, P) - dense).max() < 1e-13, P


# ---------------------------------------------------------------------------------
# multi-token queries ("Inside vLLM CUDA Kernels", Part 3, "How Metadata Connects a Q
# Tile to Paged K/V"): request r's rows [qs[r], qs[r+1]) are its newest n_r tokens;
# token i sits at p = L_r - n_r + i and, causally, sees positions t <= p
# ---------------------------------------------------------------------------------

def _varlen_case(causal=True, alibi=False, dtype="bf16"):
    w = custom(60, dtype, 8, 2, 64, [1, 5, 16, 17, 40, 300])
    if alibi:
        w = alibi_variant(w, np.linspace(0.3, -0.02, 8).astype(np.float32))
    return w, varlen_variant(w, [1, 5, 3, 17, 1, 33], causal=causal)


def _varlen_numpy(w, vq):
    """Dense attention per packed row from the generator's contiguous history."""
    q = bits_to_f64(vq.q, w.dtype)
    G = w.num_q_heads // w.num_kv_heads
    out = np.zeros(q.shape)
    qs = vq.query_start_loc
    for r in range(w.num_seqs):
        L, n = int(w.seq_lens[r]), int(qs[r + 1] - qs[r])
        K = bits_to_f64(w.logical_k(r), w.dtype)
        V = bits_to_f64(w.logical_v(r), w.dtype)
        for i in range(n):
            p = L - n + i
            vis = p + 1 if vq.causal else L
            for h in range(w.num_q_heads):
                x = float(w.scale) * (K[:vis, h // G] @ q[qs[r] + i, h])
                if getattr(w, "alibi_slopes", None) is not None:
                    x = x + float(w.alibi_slopes[h]) * (np.arange(vis) - p)
                e = np.exp(x - x.max())
                out[qs[r] + i, h] = e @ V[:vis, h // G] / e.sum()
    return out


def pin_varlen_single_tokens_are_decode():
    """One query token per request with the decode's q: bit-identical to the decode."""
    w = custom(61, "f16", 8, 4, 128, [1, 33, 520])
    pool = oracle.filled_pool(w)
    v1 = varlen_variant(w, [1, 1, 1])
    assert np.array_equal(oracle.varlen(w, pool, v1, q=w.q), oracle.decode(w, pool))


def pin_varlen_numpy():
    """numpy dense attention with the causal limit t <= L - n + i (and without it, and
    with an ALiBi bias measured from the token's own position) agrees to 1e-12."""
    for causal, alibi in ((True, False), (False, False), (True, True)):
        w, vq = _varlen_case(causal, alibi)
        out = oracle.varlen(w, oracle.filled_pool(w), vq)
        assert np.abs(out - _varlen_numpy(w, vq)).max() < 1e-12, (causal, alibi)


def pin_varlen_torch_sdpa():
    """torch SDPA in float64 with a boolean mask built from the causal limit."""
    import torch
    w, vq = _varlen_case(True, dtype="f32")
    out = oracle.varlen(w, oracle.filled_pool(w), vq)
    G = w.num_q_heads // w.num_kv_heads
    q = torch.from_numpy(bits_to_f64(vq.q, w.dtype))
    qs = vq.query_start_loc
    for r in range(w.num_seqs):
        L, n = int(w.seq_lens[r]), int(qs[r + 1] - qs[r])
        if n == 0:
            continue
        K = torch.from_numpy(bits_to_f64(w.logical_k(r), w.dtype)).permute(1, 0, 2).repeat_interleave(G, 0)
        V = torch.from_numpy(bits_to_f64(w.logical_v(r), w.dtype)).permute(1, 0, 2).repeat_interleave(G, 0)
        allowed = torch.arange(L)[None, :] <= (L - n + torch.arange(n))[:, None]  # [n, L]
        ref = torch.nn.functional.scaled_dot_product_attention(q[qs[r]:qs[r + 1]].permute(1, 0, 2), K, V,
                                                               attn_mask=allowed, scale=float(w.scale))
        assert (ref.permute(1, 0, 2).numpy() - out[qs[r]:qs[r + 1]]).__abs__().max() < 1e-12, r


def pin_varlen_prefix_means():
    """q = 0, causal: token i's output is the plain mean of V over positions 0 .. p."""
    w, vq = _varlen_case(True, dtype="f32")
    zq = np.zeros_like(vq.q)
    out = oracle.varlen(w, oracle.filled_pool(w), vq, q=zq)
    G = w.num_q_heads // w.num_kv_heads
    qs = vq.query_start_loc
    for r in range(w.num_seqs):
        L, n = int(w.seq_lens[r]), int(qs[r + 1] - qs[r])
        V = bits_to_f64(w.logical_v(r), w.dtype)
        for i in range(n):
            p = L - n + i
            for h in range(w.num_q_heads):
                assert np.abs(out[qs[r] + i, h] - V[:p + 1, h // G].mean(axis=0)).max() < 1e-12, (r, i, h)


def pin_varlen_first_token_sees_one_row():
    """A request whose query covers its whole history (n = L): its first token sees only
    position 0, so its output is that V row exactly, in every format."""
    for dtype in ("f32", "f16", "bf16"):
        w = custom(62, dtype, 4, 2, 64, [9, 20])
        vq = varlen_variant(w, [9, 20])
        out = oracle.varlen(w, oracle.filled_pool(w), vq)
        for r, row in ((0, 0), (1, 9)):
            V0 = bits_to_f64(w.logical_v(r)[0], dtype)  # [Hkv, D]
            assert np.array_equal(out[row], np.repeat(V0, 2, axis=0)), (dtype, r)


PINS = [
    pin_slot_write, pin_slot_read, pin_invariant_line, pin_gqa_mapping, pin_worked_decode,
    pin_combined_block_layout, pin_one_token_exact, pin_special_values_exact, pin_zero_query_mean,
    pin_equal_keys_mean, pin_two_tokens_sigmoid, pin_huge_logits, pin_placement_invariance,
    pin_negative_slot_skipped, pin_unread_memory, pin_table_padding, pin_write_out_of_range,
    pin_numpy_dense, pin_block_sizes, pin_torch_sdpa, pin_online_tiles, pin_brute_force, pin_split_identity,
    pin_e4m3_values, pin_e4m3_rounding, pin_kv8_write, pin_kv8_decode, pin_alibi_zero_slopes,
    pin_alibi_torch_sdpa, pin_alibi_geometric_weights, pin_alibi_partials, pin_varlen_single_tokens_are_decode,
    pin_varlen_numpy, pin_varlen_torch_sdpa, pin_varlen_prefix_means, pin_varlen_first_token_sees_one_row,
]
