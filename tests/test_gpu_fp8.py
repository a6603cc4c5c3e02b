"""GPU parity of the 8-bit (OCP E4M3) cache: the quantising write and the decode over
codes, against the oracle's kv8 functions on the same seeded inputs.

Bars: the write is bit-exact over the whole pool (every code, the untouched NaN
fill included).  Every E4M3 value is exact in bf16 and fp16, so the decode sees
the same dequantised K and V as the oracle and keeps the 16-bit path's bar: max-abs
1e-2 of the fp64 output.
"""

import dataclasses
import functools

import numpy as np
import pytest
import torch

import gpu_harness as gh
import oracle
import paged_kv_cache_reshape_amd as pc
from helpers import PROB_ROUNDOFF, with_abs_values
from workloads import custom, fp8_variant, make_config

pytestmark = pytest.mark.gpu

TOL = 1e-2


def say(msg):
    print(msg, flush=True)


def pools_equal(dev: gh.DevicePool, host: oracle.Pool) -> bool:
    for d, h in zip(dev.bits(), host.arrays()):
        if not np.array_equal(d, h):
            n = int((d != h).sum())
            i = int(np.argmax(d != h))
            say(f"pool differs in {n} bytes, first at {i}: gpu {d[i]:#04x} oracle {h[i]:#04x}")
            return False
    return True


def check_attention(got, ref, what, tol=TOL):
    assert got.shape == ref.shape
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got - ref)
    i = np.unravel_index(int(err.argmax()), err.shape)
    say(f"{what}: max|err| {err.max():.3e} at {tuple(int(x) for x in i)} (ref {ref[i]:.5f} got {got[i]:.5f}), "
        f"max|o| {np.abs(ref).max():.3f}, tol {tol}")
    assert err.max() <= tol, what


# ---------------------------------------------------------------------------------
# the quantising write
# ---------------------------------------------------------------------------------

WRITE_CASES = [("bf16", "hnd", True), ("f16", "nhd", True), ("f32", "hnd", False), ("bf16", "combined", False),
               ("f32", "nhd", True)]


@pytest.mark.parametrize("dt,layout,per_head", WRITE_CASES,
                         ids=[f"{a}-{b}-{'head' if c else 'shared'}" for a, b, c in WRITE_CASES])
def test_write_bit_exact(dt, layout, per_head):
    # scales small enough that a few standard-normal values pass 448 * scale and saturate
    wl = fp8_variant(custom(200, dt, 8, 4, 128, [1, 16, 33, 700], layout=layout, extra_pad_rows=2),
                     per_head=per_head, lo=0.003, hi=0.01)
    hpool = oracle.filled_pool(wl)
    dpool = gh.filled_pool(wl)
    assert pools_equal(dpool, hpool)
    codes = np.concatenate([a.ravel() for a in hpool.arrays()])
    assert ((codes & 0x7F) == 0x7E).any(), "no saturated code: the case lost its point"


def _special_rows(shape, dt):
    """Rows (fp32 values) that hit the conversion's edge cases at scale 2^-6: ties
    between neighbouring codes (to even), the subnormal range and its ties, the
    largest finite value and past it, infinities, NaN and signed zeros."""
    vals = np.array([
        1.0625, 1.1875, 1.0, -1.0625, -1.1875,        # ties in [1, 2): to the even mantissa
        2.0 ** -10, 3 * 2.0 ** -10, 2.0 ** -9, 5 * 2.0 ** -10, 2.0 ** -11,  # subnormal steps and ties
        2.0 ** -6 * 1.0625, 240.0, 448.0, 464.0, 470.0, 1e6, -1e6,  # top of the range and saturation
        np.inf, -np.inf, np.nan, 0.0, -0.0, 0.3, -7.7,
    ], dtype=np.float64) / 64.0  # divided again by the scale 2^-6 in the write
    flat = np.resize(vals, int(np.prod(shape)))
    out = flat.reshape(shape).astype(np.float32)
    if dt == "f32":
        return out.view(np.uint32)
    if dt == "f16":
        return out.astype(np.float16).view(np.uint16)
    return (out.view(np.uint32) >> 16).astype(np.uint16)  # exact: every value above fits bf16


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
def test_write_special_values(dt):
    base = custom(201, dt, 4, 2, 64, [40, 9])
    wl = fp8_variant(base, per_head=True)
    two = np.full(2, 2.0 ** -6, np.float32)
    wl = dataclasses.replace(wl, k_scale=two, v_scale=two.copy(), pre_key=_special_rows(wl.pre_key.shape, dt),
                             pre_value=_special_rows(wl.pre_value.shape, dt)[::-1].copy())
    hpool = oracle.filled_pool(wl)
    dpool = gh.filled_pool(wl)
    assert pools_equal(dpool, hpool)
    codes = hpool.k
    assert (codes == 0x7E).any() and (codes == 0xFE).any() and (codes == 0xFF).any()


def test_write_skips_negative_and_out_of_range_slots():
    wl = fp8_variant(custom(202, "bf16", 8, 2, 128, [5, 9]))
    dpool = gh.filled_pool(wl)
    before = dpool.bits()
    slots = np.array([-1, -9, wl.num_blocks * 16, wl.num_blocks * 16 + 5], np.int64)
    rows = np.repeat(wl.key[:1], 4, axis=0)
    gh.write(dpool, rows, rows, slots)
    for b, a in zip(before, dpool.bits()):
        assert np.array_equal(b, a)


# ---------------------------------------------------------------------------------
# decode over codes
# ---------------------------------------------------------------------------------

LENGTHS = [1, 15, 16, 17, 100, 511, 512, 513, 1100]
VARIANTS = [(dt, D, G) for dt in ("bf16", "f16") for D in (64, 128) for G in (1, 2, 4, 8)]


@pytest.mark.parametrize("dt,D,G", VARIANTS, ids=[f"{a}-d{b}-g{c}" for a, b, c in VARIANTS])
@pytest.mark.parametrize("path", ["single", "split"])
def test_decode_parity(dt, D, G, path):
    Hkv = 2
    wl = fp8_variant(custom(300 + D + G, dt, Hkv * G, Hkv, D, LENGTHS, extra_pad_rows=1))
    hpool = oracle.filled_pool(wl)
    dpool = gh.filled_pool(wl)
    assert pools_equal(dpool, hpool)
    out, _ = gh.decode(dpool, gh.DecodeInputs(wl), path)
    check_attention(gh.out_f64(out), oracle.decode(wl, hpool), f"fp8 {dt} D{D} G{G} {path}")


@pytest.mark.parametrize("layout,per_head", [("nhd", False), ("combined", True)])
def test_decode_other_layouts_and_shared_scale(layout, per_head):
    wl = fp8_variant(custom(310, "bf16", 16, 4, 128, [3, 70, 600, 1300], layout=layout), per_head=per_head)
    hpool = oracle.filled_pool(wl)
    dpool = gh.filled_pool(wl)
    assert pools_equal(dpool, hpool)
    ref = oracle.decode(wl, hpool)
    for path in ("single", "split"):
        out, _ = gh.decode(dpool, gh.DecodeInputs(wl), path)
        check_attention(gh.out_f64(out), ref, f"fp8 {layout} {'per-head' if per_head else 'shared'} {path}")


@pytest.mark.parametrize("path", ["single", "split"])
def test_uniform_scores_give_mean_of_v(path):
    """q = 0: every probability is exactly 1, so the output is the mean of the
    dequantised V over the visible tokens times nothing else; the oracle's value is
    that mean (pinned on the CPU), and the bound is one storage ulp plus fp32 sums."""
    wl = fp8_variant(custom(311, "bf16", 8, 2, 128, [1, 17, 511, 16416, 40000], pool_factor=1.2))
    zq = np.zeros_like(wl.q)
    hpool = oracle.filled_pool(wl)
    ref = oracle.decode(dataclasses.replace(wl, q=zq), hpool)
    dpool = gh.filled_pool(wl)
    out, _ = gh.decode(dpool, gh.DecodeInputs(wl, q_bits=zq), path)
    got = gh.out_f64(out)
    err = np.abs(got - ref)
    bound = 2.0 ** -8 * np.abs(ref) + 1e-6
    say(f"fp8 mean-of-V {path}: worst err/bound {(err / bound).max():.3f}")
    assert (err <= bound).all()


def test_split_partials_against_oracle():
    wl = fp8_variant(custom(312, "f16", 8, 2, 128, [1, 511, 512, 513, 1500]))
    hpool = oracle.filled_pool(wl)
    dpool = gh.filled_pool(wl)
    inp = gh.DecodeInputs(wl)
    es, ml, tmp = gh.partials_call(dpool, inp, inp.max_seq_len)
    torch.cuda.synchronize()
    P = es.shape[2]
    rt, rm, re = oracle.partials(wl, hpool, 512, P)
    gt, gm, ge = tmp.double().cpu().numpy(), ml.double().cpu().numpy(), es.double().cpu().numpy()
    written = ~np.isnan(rm)
    assert np.array_equal(written, ~np.isnan(gm)), "partitions written differ"
    assert np.abs(gm[written] - rm[written]).max() < 1e-5
    assert (np.abs(ge[written] - re[written]) / re[written]).max() < 1e-5
    # probabilities enter P.V rounded to the query's 16-bit type (relative error <= u),
    # so element d moves by at most u * sum_t p_t |v_t[d]| / sum_t p_t (v dequantised):
    # the oracle's partials over |V| (E4M3 encoding is symmetric, so clearing the sign
    # of the rows before the write clears it in the codes)
    A, _, _ = oracle.partials(with_abs_values(wl), oracle.filled_pool(with_abs_values(wl)), 512, P)
    err = np.abs(gt[written] - rt[written])
    bound = (PROB_ROUNDOFF[wl.dtype] + 2.0 ** -14) * A[written] + 1e-6
    say(f"fp8 split partials: max err {err.max():.3e}, worst err/bound {(err / bound).max():.3f}")
    assert (err <= bound).all()
    assert err.max() <= 1e-2


@pytest.mark.parametrize("path", ["single", "split"])
def test_bad_scale_poisons_only_its_head(path):
    wl = fp8_variant(custom(313, "bf16", 8, 2, 128, [40, 700, 33]))
    hpool = oracle.filled_pool(wl)
    dpool = gh.filled_pool(wl)
    dpool.k_scale[1] = 0.0  # kv head 1 (query heads 4..7) can no longer be dequantised
    out, _ = gh.decode(dpool, gh.DecodeInputs(wl), path)
    got = gh.out_f64(out)
    assert np.isnan(got[:, 4:]).all()
    check_attention(got[:, :4], oracle.decode(wl, hpool)[:, :4], f"heads beside a bad scale ({path})")


# ---------------------------------------------------------------------------------
# full-size workloads over an 8-bit cache, in the launch configuration the benchmark times
# ---------------------------------------------------------------------------------

@functools.lru_cache(maxsize=1)
def _config_state(idx):
    say(f"[fp8 config {idx}] generating")
    wl = fp8_variant(make_config(idx))
    say(f"[fp8 config {idx}] oracle write + decode")
    hpool = oracle.filled_pool(wl)
    ref = oracle.decode(wl, hpool)
    say(f"[fp8 config {idx}] GPU write")
    dpool = gh.filled_pool(wl)
    return wl, hpool, ref, dpool


@pytest.mark.parametrize("idx,path", [(1, "single"), (3, "split")])
def test_config_fp8(idx, path):
    wl, hpool, ref, dpool = _config_state(idx)
    assert pools_equal(dpool, hpool)
    out, used = gh.decode(dpool, gh.DecodeInputs(wl), path)
    check_attention(gh.out_f64(out), ref, f"[fp8 config {idx}] {used} path")
