"""The one-pass decode's one-workgroup-per-unit kernel: the library runs it (16-bit
pools) when the longest sequence fits one 512-token partition, or for at least 32 units
per compute unit with sequences up to 2048 tokens.  Every case is checked against the
fp64 oracle; the lengths are chosen so that the decode takes this kernel."""

import numpy as np
import pytest
import torch

import gpu_harness as gh
import oracle
from test_gpu_parity import check_attention
from workloads import alibi_variant, custom

pytestmark = pytest.mark.gpu

SHORT = [1, 2, 15, 16, 17, 31, 100, 255, 256, 257, 511, 512]
CASES = [(dt, D, G, layout, B) for dt in ("bf16", "f16") for D in (64, 128) for G in (1, 2, 4, 8)
         for layout, B in (("hnd", 16),)] + [
    ("bf16", 64, 4, "combined", 16), ("f16", 128, 2, "nhd", 16), ("bf16", 128, 4, "hnd", 8),
    ("f16", 64, 1, "hnd", 32), ("bf16", 64, 4, "nhd", 8), ("bf16", 128, 8, "hnd", 32)]


@pytest.mark.parametrize("dt,D,G,layout,B", CASES, ids=[f"{a}-d{b}-g{c}-{d}-b{e}" for a, b, c, d, e in CASES])
def test_grid_kernel_matches_oracle(dt, D, G, layout, B):
    Hkv = 2
    wl = custom(500 + D + G + B, dt, Hkv * G, Hkv, D, SHORT, layout=layout, extra_pad_rows=1, block_size=B)
    assert int(wl.seq_lens.max()) <= 512
    hpool = oracle.filled_pool(wl)
    out, used = gh.decode(gh.filled_pool(wl), gh.DecodeInputs(wl), "single")
    torch.cuda.synchronize()
    check_attention(gh.out_f64(out), oracle.decode(wl, hpool), dt, f"grid kernel {dt} D{D} G{G} {layout} B{B}")


def test_grid_kernel_alibi_and_empty_sequences():
    rng = np.random.default_rng(5)
    wl = custom(531, "bf16", 16, 4, 128, [0, 5, 0, 300, 512, 77], layout="hnd")
    wl = alibi_variant(wl, slopes=rng.uniform(-0.2, 0.2, 16).astype(np.float32))
    out, _ = gh.decode(gh.filled_pool(wl), gh.DecodeInputs(wl), "single")
    got = gh.out_f64(out)
    assert (got[0] == 0).all() and (got[2] == 0).all()
    check_attention(got, oracle.decode(wl, oracle.filled_pool(wl)), "bf16", "grid kernel, ALiBi, empty sequences")


def test_grid_kernel_invalid_block_id_poisons_only_its_sequence():
    wl = custom(532, "bf16", 8, 2, 128, [40, 400, 33])
    hpool = oracle.filled_pool(wl)
    bt = wl.block_tables.copy()
    bt[1, 3] = wl.num_blocks + 9
    out, _ = gh.decode(gh.filled_pool(wl), gh.DecodeInputs(wl, block_tables=bt), "single")
    got = gh.out_f64(out)
    assert np.isnan(got[1]).all()
    check_attention(got[[0, 2]], oracle.decode(wl, hpool)[[0, 2]], "bf16", "grid kernel, neighbours of a bad row")


def test_grid_kernel_length_past_table_row():
    wl = custom(533, "f16", 4, 4, 64, [40, 20], table_width=3)
    sl = wl.seq_lens.copy()
    sl[1] = 3 * 16 + 5  # needs a 4th block the row does not have; max_seq_len understated below
    out, _ = gh.decode(gh.filled_pool(wl), gh.DecodeInputs(wl, seq_lens=sl), "single", max_seq_len=48)
    got = gh.out_f64(out)
    assert np.isnan(got[1]).all() and np.isfinite(got[0]).all()


def test_grid_kernel_many_units():
    """At least 32 units per compute unit with sequences up to 2048 tokens (the second
    condition of the rule): 256 sequences x 32 kv heads = 8192 units.  Outputs of a
    sample of sequences are compared with the oracle's decode of those sequences over
    the same pool."""
    rng = np.random.default_rng(21)
    lengths = rng.integers(1, 2049, size=256)
    lengths[0] = 2048
    wl = custom(534, "bf16", 32, 32, 64, lengths, pool_factor=1.05)
    out, _ = gh.decode(gh.filled_pool(wl), gh.DecodeInputs(wl), "single")
    got = gh.out_f64(out)
    pick = np.sort(rng.choice(256, 10, replace=False))
    ref = oracle.decode(wl, oracle.filled_pool(wl), q=wl.q[pick], seq_lens=wl.seq_lens[pick],
                        block_tables=wl.block_tables[pick])
    check_attention(got[pick], ref, "bf16", "grid kernel, 8192 units")
