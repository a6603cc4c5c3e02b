"""Head size 64 with a token's kv heads side by side (NHD, or K then V per block): the
decode reads kv heads 2p and 2p+1 together and computes them as one head of 128 with
twice the query heads.  Every case is checked against the fp64 oracle, which knows
nothing of the pairing; odd kv head counts and groups of 8 take the unpaired kernels.
"""

import numpy as np
import pytest
import torch

import gpu_harness as gh
import oracle
from test_gpu_parity import check_attention
from workloads import alibi_variant, custom

pytestmark = pytest.mark.gpu

LENGTHS = [1, 15, 16, 17, 100, 511, 512, 513, 1100]
CASES = [(dt, layout, G, Hkv) for dt in ("bf16", "f16") for layout in ("nhd", "combined") for G in (1, 2, 4)
         for Hkv in (2, 6)] + [("bf16", "nhd", 4, 3), ("f16", "combined", 2, 5), ("bf16", "nhd", 8, 2)]


@pytest.mark.parametrize("dt,layout,G,Hkv", CASES, ids=[f"{a}-{b}-g{c}-kv{d}" for a, b, c, d in CASES])
@pytest.mark.parametrize("path", ["single", "split"])
def test_pairs_match_oracle(dt, layout, G, Hkv, path):
    wl = custom(400 + 10 * G + Hkv, dt, Hkv * G, Hkv, 64, LENGTHS, layout=layout, extra_pad_rows=1)
    hpool = oracle.filled_pool(wl)
    out, _ = gh.decode(gh.filled_pool(wl), gh.DecodeInputs(wl), path)
    torch.cuda.synchronize()
    check_attention(gh.out_f64(out), oracle.decode(wl, hpool), dt, f"pairs {dt} {layout} G{G} Hkv{Hkv} {path}")


def test_pair_partials_match_oracle():
    """The split path's partials of paired heads, element by element (head size 64 rows)."""
    wl = custom(431, "bf16", 16, 4, 64, [1, 511, 512, 513, 1500], layout="nhd")
    hpool = oracle.filled_pool(wl)
    es, ml, tmp = gh.partials_call(gh.filled_pool(wl), gh.DecodeInputs(wl), int(wl.seq_lens.max()))
    torch.cuda.synchronize()
    P = es.shape[2]
    rt, rm, re = oracle.partials(wl, hpool, 512, P)
    written = ~np.isnan(rm)
    assert np.array_equal(written, ~np.isnan(ml.double().cpu().numpy()))
    assert np.abs(ml.double().cpu().numpy()[written] - rm[written]).max() < 1e-5
    assert (np.abs(es.double().cpu().numpy()[written] - re[written]) / re[written]).max() < 1e-5
    assert np.abs(tmp.double().cpu().numpy()[written] - rt[written]).max() <= 1e-2


@pytest.mark.parametrize("path", ["single", "split"])
def test_pairs_with_alibi(path):
    rng = np.random.default_rng(7)
    wl = custom(432, "bf16", 16, 4, 64, LENGTHS, layout="combined")
    wl = alibi_variant(wl, slopes=rng.uniform(-0.2, 0.2, 16).astype(np.float32))
    out, _ = gh.decode(gh.filled_pool(wl), gh.DecodeInputs(wl), path)
    check_attention(gh.out_f64(out), oracle.decode(wl, oracle.filled_pool(wl)), "bf16", f"pairs ALiBi {path}")


@pytest.mark.parametrize("B", [8, 32])
@pytest.mark.parametrize("path", ["single", "split"])
def test_pairs_other_block_sizes(B, path):
    wl = custom(433 + B, "f16", 8, 4, 64, LENGTHS, layout="nhd", block_size=B)
    out, _ = gh.decode(gh.filled_pool(wl), gh.DecodeInputs(wl), path)
    check_attention(gh.out_f64(out), oracle.decode(wl, oracle.filled_pool(wl)), "f16", f"pairs B{B} {path}")


def test_pairs_many_units():
    """More paired units than persistent workgroups (ranked later turns)."""
    rng = np.random.default_rng(11)
    lengths = rng.integers(1, 700, size=160)
    wl = custom(434, "bf16", 32, 8, 64, lengths, layout="combined")
    out, _ = gh.decode(gh.filled_pool(wl), gh.DecodeInputs(wl), "single")
    check_attention(gh.out_f64(out), oracle.decode(wl, oracle.filled_pool(wl)), "bf16", "pairs, 640 units")
