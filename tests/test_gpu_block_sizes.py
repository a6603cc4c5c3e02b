"""GPU parity of the decode over pools of 8- and 32-token blocks ("vLLM 源码完全拆解
（七）", section GQA、向量化加载与 Block Size 的联动: the block size is a storage
choice; attention over it is unchanged).  The kernels keep 16-token score tiles: a
32-token block holds two tiles, an 8-token block half of one.  Bars as for 16-token
blocks: bit-exact writes, max-abs 1e-2 of the fp64 oracle.
"""

import dataclasses

import numpy as np
import pytest
import torch

import gpu_harness as gh
import oracle
from helpers import bits_to_f64
from workloads import alibi_variant, custom, fp8_variant

pytestmark = pytest.mark.gpu

TOL = 1e-2
LENGTHS = [1, 7, 8, 9, 15, 16, 17, 31, 32, 33, 100, 511, 512, 513, 1100]


def say(msg):
    print(msg, flush=True)


def check(got, ref, what):
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got - ref)
    say(f"{what}: max|err| {err.max():.3e}, max|o| {np.abs(ref).max():.3f}")
    assert err.max() <= TOL, what


def pools_equal(dev, host):
    return all(np.array_equal(d, h) for d, h in zip(dev.bits(), host.arrays()))


CASES = [(B, dt, D, G) for B in (8, 32) for dt in ("bf16", "f16") for D in (64, 128) for G in (1, 4, 8)]


@pytest.mark.parametrize("B,dt,D,G", CASES, ids=[f"b{a}-{b}-d{c}-g{d}" for a, b, c, d in CASES])
@pytest.mark.parametrize("path", ["single", "split"])
def test_block_size_parity(B, dt, D, G, path):
    wl = custom(600 + B + D + G, dt, 2 * G, 2, D, LENGTHS, extra_pad_rows=1, block_size=B)
    hpool = oracle.filled_pool(wl)
    dpool = gh.filled_pool(wl)
    assert pools_equal(dpool, hpool)
    out, _ = gh.decode(dpool, gh.DecodeInputs(wl), path)
    check(gh.out_f64(out), oracle.decode(wl, hpool), f"B{B} {dt} D{D} G{G} {path}")


@pytest.mark.parametrize("B", [8, 32])
@pytest.mark.parametrize("variant", ["fp8", "nhd", "combined", "alibi"])
def test_block_size_variants(B, variant):
    layout = variant if variant in ("nhd", "combined") else "hnd"
    wl = custom(650 + B, "bf16", 16, 4, 128, [3, 8, 40, 600, 1300], layout=layout, block_size=B)
    if variant == "fp8":
        wl = fp8_variant(wl)
    if variant == "alibi":
        wl = alibi_variant(wl, np.linspace(0.2, -0.01, 16).astype(np.float32))
    hpool = oracle.filled_pool(wl)
    dpool = gh.filled_pool(wl)
    assert pools_equal(dpool, hpool)
    ref = oracle.decode(wl, hpool)
    for path in ("single", "split"):
        out, _ = gh.decode(dpool, gh.DecodeInputs(wl), path)
        check(gh.out_f64(out), ref, f"B{B} {variant} {path}")


@pytest.mark.parametrize("B", [8, 32])
@pytest.mark.parametrize("path", ["single", "split"])
def test_block_size_mean_of_v(B, path):
    """q = 0 over histories that span several staged id chunks: the exact mean of V
    (one block counted twice or skipped shows far above the bound)."""
    wl = custom(660 + B, "bf16", 8, 2, 128, [1, 9, 17, 511, 16416, 40000], pool_factor=1.2, block_size=B)
    zq = np.zeros_like(wl.q)
    ref = oracle.decode(dataclasses.replace(wl, q=zq), oracle.filled_pool(wl))
    for s in range(wl.num_seqs):
        mean = bits_to_f64(wl.logical_v(s), "bf16").mean(axis=0)
        assert np.allclose(ref[s], np.repeat(mean, 4, axis=0), rtol=0, atol=1e-12)
    dpool = gh.filled_pool(wl)
    out, _ = gh.decode(dpool, gh.DecodeInputs(wl, q_bits=zq), path)
    got = gh.out_f64(out)
    err = np.abs(got - ref)
    bound = 2.0 ** -8 * np.abs(ref) + 1e-6
    say(f"B{B} mean-of-V {path}: worst err/bound {(err / bound).max():.3f}")
    assert (err <= bound).all()


@pytest.mark.parametrize("B", [8, 32])
def test_block_size_bad_id(B):
    wl = custom(670 + B, "bf16", 8, 2, 128, [40, 700, 33], block_size=B)
    hpool = oracle.filled_pool(wl)
    dpool = gh.filled_pool(wl)
    bt = wl.block_tables.copy()
    bt[1, 3] = wl.num_blocks + 2
    ref = oracle.decode(wl, hpool)
    for path in ("single", "split"):
        out, _ = gh.decode(dpool, gh.DecodeInputs(wl, block_tables=bt), path)
        got = gh.out_f64(out)
        assert np.isnan(got[1]).all()
        check(got[[0, 2]], ref[[0, 2]], f"B{B} neighbours of a bad id ({path})")


@pytest.mark.parametrize("B", [8, 32])
def test_block_size_gqa_full(B):
    """64 sequences of 512..2048 tokens, GQA 32/8, D = 128 (the headline shape)."""
    rng = np.random.default_rng(B)
    wl = custom(680 + B, "bf16", 32, 8, 128, rng.integers(512, 2049, size=64), block_size=B)
    hpool = oracle.filled_pool(wl)
    dpool = gh.filled_pool(wl)
    assert pools_equal(dpool, hpool)
    ref = oracle.decode(wl, hpool)
    for path in ("single", "split"):
        out, _ = gh.decode(dpool, gh.DecodeInputs(wl), path)
        check(gh.out_f64(out), ref, f"B{B} GQA 64 x 512..2048 {path}")
