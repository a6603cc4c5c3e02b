"""The seeded generator: determinism, shapes and the structure each workload promises."""

import numpy as np
import pytest
import torch

from workloads import BLOCK_SIZE, custom, make_config
from workloads.gen import _to_bits

B = BLOCK_SIZE


def _valid_ids(w):
    ids = []
    for s in range(w.num_seqs):
        n = -(-int(w.seq_lens[s]) // B)
        row = w.block_tables[s]
        assert (row[:n] >= 0).all() and (row[:n] < w.num_blocks).all()
        assert (row[n:] == -1).all()
        ids.append(row[:n])
    return ids


def test_deterministic():
    a, b = make_config(0), make_config(0)
    for f in ("seq_lens", "block_tables", "q", "pre_key", "pre_value", "pre_slots", "key", "value", "slot_mapping"):
        assert np.array_equal(getattr(a, f), getattr(b, f)), f
    c = make_config(0, seed=7)
    assert not np.array_equal(a.q, c.q)


def test_bf16_rounding_matches_torch():
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32)
    x[:4] = [1.00390625, 1.01171875, -1.00390625, 3.0e-39]  # ties and a subnormal
    ours = _to_bits(x, "bf16")
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(_to_bits(x, "f16"), torch.from_numpy(x).half().view(torch.int16).numpy().view(np.uint16))


def test_config0():
    w = make_config(0)
    assert w.dtype == "f32" and w.num_blocks == 16 and list(w.seq_lens) == [20, 37]
    assert (w.num_q_heads, w.num_kv_heads, w.head_size) == (4, 4, 64)
    ids = np.concatenate(_valid_ids(w))
    assert len(ids) == 5 and len(set(ids.tolist())) == 5
    assert w.key.shape == (3, 4, 64) and w.slot_mapping[2] == -1 and (w.slot_mapping[:2] >= 0).all()
    assert len(w.pre_slots) == 19 + 36


def test_config1_structure():
    w = make_config(1, contents=False)
    assert w.num_seqs == 64 and w.dtype == "bf16" and (w.num_q_heads, w.num_kv_heads, w.head_size) == (32, 8, 128)
    assert w.seq_lens.min() >= 512 and w.seq_lens.max() <= 2048
    ids = np.concatenate(_valid_ids(w))
    assert len(set(ids.tolist())) == len(ids) and w.num_blocks == 2 * len(ids)
    assert w.block_tables.shape[1] == 128 and (w.slot_mapping >= 0).all()


def test_config2_structure():
    w = make_config(2, contents=False)
    assert w.layout == "combined" and w.num_blocks == 65536 and w.pool_elems * 2 == 2 ** 31
    assert w.seq_lens.min() >= 1 and w.seq_lens.max() <= 2048 and w.num_seqs == 128
    ids = np.concatenate(_valid_ids(w))
    assert len(set(ids.tolist())) == len(ids)


def test_config3_structure():
    w = make_config(3, contents=False)
    assert (w.seq_lens == 32768).all() and w.num_blocks == 8192 and w.block_tables.shape == (4, 2048)
    ids = np.concatenate(_valid_ids(w))
    assert sorted(ids.tolist()) == list(range(8192))


def test_config4_structure():
    w = make_config(4, contents=False)
    assert w.num_seqs == 256 and w.dtype == "f16" and w.num_q_heads == w.num_kv_heads == 32
    assert w.seq_lens.min() >= 16 and w.seq_lens.max() <= 8192
    assert (w.slot_mapping == -1).sum() == 26
    ids = _valid_ids(w)
    prefix = None
    for s, row in enumerate(ids):
        if len(row) >= 65:
            prefix = row[:64]
            break
    assert prefix is not None
    private = []
    for row in ids:
        sh = min(64, len(row) - 1)
        assert np.array_equal(row[:sh], prefix[:sh])
        private.extend(row[sh:].tolist())
    assert len(set(private)) == len(private) and not set(private) & set(prefix.tolist())
    assert w.num_blocks == 64 + len(private)
    # the log-uniform draw covers both ends
    assert (w.seq_lens < 64).any() and (w.seq_lens > 4096).any()


@pytest.mark.parametrize("layout", ["hnd", "nhd", "combined"])
def test_custom_write_lists(layout):
    w = custom(3, "bf16", 8, 2, 64, [1, 16, 17, 40], layout=layout, extra_pad_rows=2, pad_count=1)
    # every visible position is written exactly once: history rows, then the step
    valid = w.slot_mapping[w.slot_mapping >= 0]
    assert len(set(w.pre_slots.tolist()) | set(valid.tolist())) == len(w.pre_slots) + len(valid) == int(
        w.seq_lens.sum())
    assert (w.slot_mapping == -1).sum() == 3
