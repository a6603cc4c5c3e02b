"""GPU parity: the HIP library against the fp64 oracle on the same seeded inputs.

Bars: the cache write is bit-exact over the whole pool; attention is within
max-abs 1e-5 (fp32 storage) or 1e-2 (bf16/fp16 storage) of the oracle.  The five
named workloads run at full size in the path the benchmark times; smaller cases
cover ragged tails, every (dtype, head size, group, layout) kernel, both paths,
empty sequences and partitions, and invalid data.
"""

import dataclasses
import functools
import math

import numpy as np
import pytest
import torch

import gpu_harness as gh
import oracle
import paged_kv_cache_reshape_amd as pc
from helpers import PROB_ROUNDOFF, bits_to_f64, with_abs_values
from workloads import custom, make_config, nan_bits

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "f16": 1e-2, "bf16": 1e-2}
CONFIG_PATH = {0: "single", 1: "single", 2: "plan", 3: "split", 4: "plan"}


def say(msg):
    print(msg, flush=True)


def check_attention(got: np.ndarray, ref: np.ndarray, dtype: str, what: str):
    assert got.shape == ref.shape
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got - ref)
    i = np.unravel_index(int(err.argmax()), err.shape)
    say(f"{what}: max|err| {err.max():.3e} at {tuple(int(x) for x in i)} (ref {ref[i]:.5f} got {got[i]:.5f}), "
        f"max|o| {np.abs(ref).max():.3f}, tol {TOL[dtype]}")
    assert err.max() <= TOL[dtype], what


def pools_equal(dev: gh.DevicePool, host: oracle.Pool) -> bool:
    torch.cuda.synchronize()
    for d, h in zip(dev.arrays(), host.arrays()):
        if not np.array_equal(gh.to_bits(d, dev.wl.dtype), h):
            return False
    return True


# ---------------------------------------------------------------------------------
# the five named workloads, full size
# ---------------------------------------------------------------------------------

@functools.lru_cache(maxsize=1)
def _config_state(idx):
    say(f"[config {idx}] generating")
    wl = make_config(idx)
    say(f"[config {idx}] oracle write + decode")
    hpool = oracle.filled_pool(wl)
    ref = oracle.decode(wl, hpool)
    say(f"[config {idx}] GPU write")
    dpool = gh.filled_pool(wl)
    return wl, hpool, ref, dpool


@pytest.mark.parametrize("idx", [0, 1, 2, 3, 4])
def test_config_write_bit_exact(idx):
    wl, hpool, _, dpool = _config_state(idx)
    say(f"[config {idx}] comparing {sum(a.nbytes for a in hpool.arrays()) / 1e9:.2f} GB of pool")
    assert pools_equal(dpool, hpool)


@pytest.mark.parametrize("idx", [0, 1, 2, 3, 4])
def test_config_decode(idx):
    wl, _, ref, dpool = _config_state(idx)
    inp = gh.DecodeInputs(wl)
    out, used = gh.decode(dpool, inp, CONFIG_PATH[idx])
    torch.cuda.synchronize()
    check_attention(gh.out_f64(out), ref, wl.dtype, f"[config {idx}] {used} path")
    if idx == 1:
        assert used == "single"
    if idx == 3:
        assert used == "split"


@pytest.mark.parametrize("idx", [0, 1, 2, 3, 4])
def test_config_other_path(idx):
    """The path the planner did not pick must agree too."""
    wl, _, ref, dpool = _config_state(idx)
    inp = gh.DecodeInputs(wl)
    _, used = gh.decode(dpool, inp, "plan")
    other = "split" if used == "single" else "single"
    out, _ = gh.decode(dpool, inp, other)
    torch.cuda.synchronize()
    check_attention(gh.out_f64(out), ref, wl.dtype, f"[config {idx}] {other} path")


# ---------------------------------------------------------------------------------
# every kernel variant on ragged lengths
# ---------------------------------------------------------------------------------

LENGTHS = [1, 15, 16, 17, 100, 511, 512, 513, 1100]
VARIANTS = [(dt, D, G, layout) for dt in ("f32", "f16", "bf16") for D in (64, 128) for G in (1, 2, 4)
            for layout in ("hnd",)] + [("bf16", 64, 4, "combined"), ("f16", 128, 4, "nhd"), ("f32", 64, 2, "nhd"),
                                        ("bf16", 128, 1, "combined")]


@pytest.mark.parametrize("dt,D,G,layout", VARIANTS, ids=[f"{a}-d{b}-g{c}-{d}" for a, b, c, d in VARIANTS])
@pytest.mark.parametrize("path", ["single", "split"])
def test_variant_parity(dt, D, G, layout, path):
    Hkv = 2
    wl = custom(100 + D + G, dt, Hkv * G, Hkv, D, LENGTHS, layout=layout, extra_pad_rows=1)
    hpool = oracle.filled_pool(wl)
    dpool = gh.filled_pool(wl)
    assert pools_equal(dpool, hpool)
    out, _ = gh.decode(dpool, gh.DecodeInputs(wl), path)
    torch.cuda.synchronize()
    check_attention(gh.out_f64(out), oracle.decode(wl, hpool), dt, f"{dt} D{D} G{G} {layout} {path}")


MANY_UNITS = [
    ("ranked, partial second round", 40, 8, 8, 128),    # 320 units over 256 workgroups
    ("kv heads not dividing the grid", 200, 12, 3, 128),  # 600 units, rounds in index order
    ("more sequences than ranked", 600, 2, 1, 128),       # S > 512: rounds in index order
    ("ranked, several rounds, D=64", 300, 16, 4, 64),     # 1200 units
]


@pytest.mark.parametrize("what,S,Hq,Hkv,D", MANY_UNITS, ids=[m[0] for m in MANY_UNITS])
def test_onepass_unit_dealing(what, S, Hq, Hkv, D):
    """More (sequence, kv head) units than persistent workgroups: every unit must be
    computed exactly once, whichever way the later rounds are dealt."""
    rng = np.random.default_rng(S + Hq)
    lengths = rng.integers(1, 400, size=S)
    lengths[::7] = 0
    wl = custom(20 + S, "bf16", Hq, Hkv, D, lengths)
    out, _ = gh.decode(gh.filled_pool(wl), gh.DecodeInputs(wl), "single")
    got = gh.out_f64(out)
    check_attention(got, oracle.decode(wl, oracle.filled_pool(wl)), "bf16", f"one pass, {what}")


@pytest.mark.parametrize("path", ["single", "split"])
def test_zero_length_sequences(path):
    wl = custom(7, "bf16", 8, 2, 128, [0, 37, 0, 600])
    dpool = gh.filled_pool(wl)
    out, _ = gh.decode(dpool, gh.DecodeInputs(wl), path)
    got = gh.out_f64(out)
    assert (got[0] == 0).all() and (got[2] == 0).all()
    check_attention(got, oracle.decode(wl, oracle.filled_pool(wl)), "bf16", f"zero-length {path}")


def test_shared_prefix_and_padding_rows():
    wl = custom(8, "f16", 16, 16, 128, [20, 64, 65, 300, 1030], prefix_blocks=4, pad_count=2, table_width=80)
    hpool = oracle.filled_pool(wl)
    dpool = gh.filled_pool(wl)
    assert pools_equal(dpool, hpool)
    for path in ("single", "split"):
        out, _ = gh.decode(dpool, gh.DecodeInputs(wl), path)
        check_attention(gh.out_f64(out), oracle.decode(wl, hpool), "f16", f"prefix+padding {path}")


@pytest.mark.parametrize("dt,D", [("bf16", 128), ("f16", 64), ("bf16", 64), ("f32", 128)])
@pytest.mark.parametrize("path", ["single", "split"])
def test_uniform_scores_give_mean_of_v(dt, D, path):
    """q = 0 makes every score 0: each probability is exactly 1 in any precision and the
    output is the plain mean of V over the visible tokens ("Inside vLLM CUDA Kernels",
    Part 3, "How Each K/V Tile Contributes to the Output": softmax of equal scores).
    With no rounding in the weights, the only error left is the fp32 sum and the final
    rounding, so one block counted twice or skipped shows far above the bound.  The
    long rows span several staged id chunks of the one-pass kernel."""
    wl = custom(11 + D, dt, 8, 2, D, [1, 17, 511, 16416, 40000], pool_factor=1.2)
    zq = np.zeros_like(wl.q)
    ref = oracle.decode(dataclasses.replace(wl, q=zq), oracle.filled_pool(wl))
    for s in range(wl.num_seqs):  # the closed form itself, for the oracle too
        mean = bits_to_f64(wl.logical_v(s), dt).mean(axis=0)  # [Hkv, D]
        assert np.allclose(ref[s], np.repeat(mean, 4, axis=0), rtol=0, atol=1e-12)
    dpool = gh.filled_pool(wl)
    out, _ = gh.decode(dpool, gh.DecodeInputs(wl, q_bits=zq), path)
    got = gh.out_f64(out)
    err = np.abs(got - ref)
    bound = 2.0 ** -8 * np.abs(ref) + 1e-6  # one storage ulp + fp32 summation
    i = np.unravel_index(int((err - bound).argmax()), err.shape)
    say(f"mean-of-V {dt} D{D} {path}: worst err {err[i]:.3e} vs bound {bound[i]:.3e} at {tuple(int(x) for x in i)}")
    assert (err <= bound).all()


def test_split_partials_against_oracle():
    wl = custom(9, "bf16", 8, 2, 128, [1, 511, 512, 513, 1500])
    hpool = oracle.filled_pool(wl)
    dpool = gh.filled_pool(wl)
    inp = gh.DecodeInputs(wl)
    S, Hq, D = wl.q.shape
    P = -(-inp.max_seq_len // 512)
    es = torch.full((S, Hq, P), float("nan"), device="cuda")
    ml = torch.full((S, Hq, P), float("nan"), device="cuda")
    tmp = torch.full((S, Hq, P, D), float("nan"), device="cuda")
    pc.paged_attention_decode(None, inp.q, dpool.k, dpool.v, inp.block_tables, inp.seq_lens, inp.max_seq_len,
                              num_kv_heads=wl.num_kv_heads, scale=float(wl.scale), partition_size=512,
                              exp_sums=es, max_logits=ml, tmp_out=tmp, **dpool.layout_kwargs())
    torch.cuda.synchronize()
    rt, rm, re = oracle.partials(wl, hpool, 512, P)
    gt, gm, ge = tmp.double().cpu().numpy(), ml.double().cpu().numpy(), es.double().cpu().numpy()
    written = ~np.isnan(rm)
    assert np.array_equal(written, ~np.isnan(gm)), "partitions written differ"
    assert np.abs(gm[written] - rm[written]).max() < 1e-5
    assert (np.abs(ge[written] - re[written]) / re[written]).max() < 1e-5
    # The kernel rounds each probability to the storage type before P.V (relative error
    # <= u) and sums the normaliser from the unrounded values, so element d of a partial
    # moves by at most u * sum_t p_t |v_t[d]| / sum_t p_t: the oracle's partials of the
    # same workload with |V|.  Slack for the fp32 scores, exponentials and sums on top.
    A, _, _ = oracle.partials(with_abs_values(wl), oracle.filled_pool(with_abs_values(wl)), 512, P)
    err = np.abs(gt[written] - rt[written])
    bound = (PROB_ROUNDOFF[wl.dtype] + 2.0 ** -14) * A[written] + 1e-6
    say(f"split partials bf16: max err {err.max():.3e}, worst err/bound {(err / bound).max():.3f}")
    assert (err <= bound).all()
    assert err.max() <= 1e-2


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_reduce_alone(dt):
    """Oracle partials rounded to fp32 in, GPU merge out, against the oracle merge."""
    wl = custom(10, dt, 8, 4, 64, [3, 512, 513, 2000])
    hpool = oracle.filled_pool(wl)
    P = 4
    rt, rm, re = oracle.partials(wl, hpool, 512, P, fill=0.0)
    rt32, rm32, re32 = (np.asarray(x, np.float32) for x in (rt, rm, re))
    ref = oracle.merge(rt32.astype(np.float64), rm32.astype(np.float64), re32.astype(np.float64), wl.seq_lens, 512)
    out = torch.empty(wl.q.shape, dtype=gh.TORCH_DT[dt], device="cuda")
    pc.paged_attention_reduce(out, torch.from_numpy(re32).cuda(), torch.from_numpy(rm32).cuda(),
                              torch.from_numpy(rt32).cuda(), torch.from_numpy(wl.seq_lens).cuda())
    check_attention(gh.out_f64(out), ref, dt, f"reduce alone {dt}")


def synthetic_partials(rng, S, Hq, P, D):
    """Seeded fp32 partials: maxima spread over about +-12 (weights from e^-24 to 1), sums
    in [0.5, 200), outputs N(0, 1)."""
    ml = (rng.standard_normal((S, Hq, P)) * 4.0).astype(np.float32)
    es = rng.uniform(0.5, 200.0, (S, Hq, P)).astype(np.float32)
    tmp = rng.standard_normal((S, Hq, P, D)).astype(np.float32)
    return tmp, ml, es


def reduce_on_gpu(tmp, ml, es, lens, dt):
    S, Hq, _, D = tmp.shape
    out = torch.empty((S, Hq, D), dtype=gh.TORCH_DT[dt], device="cuda")
    pc.paged_attention_reduce(out, torch.from_numpy(es).cuda(), torch.from_numpy(ml).cuda(),
                              torch.from_numpy(tmp).cuda(), torch.from_numpy(np.asarray(lens, np.int32)).cuda())
    torch.cuda.synchronize()
    return gh.out_f64(out)


@pytest.mark.parametrize("dt,D,P", [("f32", 128, 40), ("bf16", 64, 300), ("f16", 96, 17)])
def test_reduce_many_partitions(dt, D, P):
    """More partitions per row than the one-wave rows kernel takes (and, at 300, more than
    one 256-partition batch): rows of 0, 1, 2, about P/2 and P partitions, against the
    oracle's merge of the same fp32 values."""
    lens = np.array([0, 1, 512, 513, 512 * (P // 2) + 7, 512 * P, 512 * (P - 1) + 1], np.int32)
    tmp, ml, es = synthetic_partials(np.random.default_rng(1000 + P), len(lens), 3, P, D)
    ref = oracle.merge(tmp.astype(np.float64), ml.astype(np.float64), es.astype(np.float64), lens, 512)
    check_attention(reduce_on_gpu(tmp, ml, es, lens, dt), ref, dt, f"reduce of {P} partitions, {dt}, D {D}")


def test_reduce_many_partitions_nan_and_empty_partitions():
    """A NaN element of one partial reaches only that output element; a NaN maximum, the
    whole row; a partition with maximum -inf and sum 0 weighs nothing.  As the oracle."""
    P, D = 40, 64
    lens = np.array([512 * 40, 512 * 40, 512 * 39 + 100], np.int32)
    tmp, ml, es = synthetic_partials(np.random.default_rng(77), 3, 2, P, D)
    tmp[1, 0, 33, 5] = np.nan
    ml[2, 1, 7] = np.nan
    ml[0, 1, 12], es[0, 1, 12] = -np.inf, 0.0
    ml[0, 0, 3], es[0, 0, 3] = -np.inf, 0.0
    ref = oracle.merge(tmp.astype(np.float64), ml.astype(np.float64), es.astype(np.float64), lens, 512)
    got = reduce_on_gpu(tmp, ml, es, lens, "f32")
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.isnan(got[1, 0, 5]) and np.isfinite(np.delete(got[1, 0], 5)).all() and np.isnan(got[2, 1]).all()
    fin = np.isfinite(ref)
    assert np.abs(got[fin] - ref[fin]).max() <= TOL["f32"]


# ---------------------------------------------------------------------------------
# invalid data: kernels turn it into NaN or a skipped write, never an out-of-range access
# ---------------------------------------------------------------------------------

@pytest.mark.parametrize("path", ["single", "split"])
def test_invalid_block_id_poisons_only_its_sequence(path):
    wl = custom(11, "bf16", 8, 2, 128, [40, 700, 33])
    hpool = oracle.filled_pool(wl)
    dpool = gh.filled_pool(wl)
    bt = wl.block_tables.copy()
    bt[1, 1] = wl.num_blocks + 3
    out, _ = gh.decode(dpool, gh.DecodeInputs(wl, block_tables=bt), path)
    got = gh.out_f64(out)
    assert np.isnan(got[1]).all()
    ref = oracle.decode(wl, hpool)
    check_attention(got[[0, 2]], ref[[0, 2]], "bf16", f"neighbours of a bad table row ({path})")


def test_length_past_table_row_is_flagged():
    wl = custom(12, "f16", 4, 4, 64, [40, 20], table_width=3)
    dpool = gh.filled_pool(wl)
    sl = wl.seq_lens.copy()
    sl[1] = 3 * 16 + 5  # needs a 4th block the row does not have
    inp = gh.DecodeInputs(wl, seq_lens=sl)
    with pytest.raises(pc.PagedCacheError):  # the host knows max_seq_len exceeds the row: refused
        gh.decode(dpool, inp, "single")
    out, _ = gh.decode(dpool, inp, "single", max_seq_len=48)  # a caller that understates it: kernel flags NaN
    got = gh.out_f64(out)
    assert np.isnan(got[1]).all() and np.isfinite(got[0]).all()


def test_write_skips_negative_and_out_of_range_slots():
    wl = custom(13, "bf16", 8, 2, 128, [5, 9])
    dpool = gh.filled_pool(wl)
    before = [gh.to_bits(a, wl.dtype).copy() for a in dpool.arrays()]
    slots = np.array([-1, -7, wl.num_blocks * 16, wl.num_blocks * 16 + 99], np.int64)
    rows = np.repeat(wl.key[:1], 4, axis=0)
    gh.write(dpool, rows, rows, slots)
    torch.cuda.synchronize()
    for b, a in zip(before, dpool.arrays()):
        assert np.array_equal(b, gh.to_bits(a, wl.dtype))


def test_write_unaligned_rows_fall_back_to_element_copies():
    wl = custom(14, "bf16", 8, 2, 128, [3, 30])
    hpool = oracle.filled_pool(wl)
    dpool = gh.DevicePool(wl)
    for key, value, slots in ((wl.pre_key, wl.pre_value, wl.pre_slots), (wl.key, wl.value, wl.slot_mapping)):
        T = len(slots)
        big_k = torch.zeros(T * 257 + 1, dtype=torch.bfloat16, device="cuda")
        big_v = torch.zeros(T * 257 + 1, dtype=torch.bfloat16, device="cuda")
        kk = big_k[1:].as_strided((T, 2, 128), (257, 128, 1))  # odd element offset and row stride
        vv = big_v[1:].as_strided((T, 2, 128), (257, 128, 1))
        kk.copy_(gh.to_dev(key, "bf16"))
        vv.copy_(gh.to_dev(value, "bf16"))
        pc.reshape_and_cache(kk, vv, dpool.k, dpool.v, torch.from_numpy(slots).cuda(), **dpool.layout_kwargs())
    assert pools_equal(dpool, hpool)


def test_side_stream_ordering():
    """Write then decode on a non-default stream: the decode sees the written tokens."""
    wl = custom(15, "bf16", 8, 2, 128, [77, 300])
    hpool = oracle.filled_pool(wl)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        dpool = gh.DevicePool(wl)
        gh.write(dpool, wl.pre_key, wl.pre_value, wl.pre_slots)
        gh.write(dpool, wl.key, wl.value, wl.slot_mapping)
        out, _ = gh.decode(dpool, gh.DecodeInputs(wl), "single")
    s.synchronize()
    check_attention(gh.out_f64(out), oracle.decode(wl, hpool), "bf16", "side stream")


# ---------------------------------------------------------------------------------
# sharp attention on large values: bf16 outputs of 2 to 4, whose own rounding costs up
# to 2^-7, where one bf16 rounding of the probabilities in P.V (relative 2^-8) could
# carry the result past 1e-2; P.V takes each probability as two bf16 operands instead
# ---------------------------------------------------------------------------------

def _scaled(bits, power, dtype):
    """16-bit storage bits times 2**power (exact for the normal values N(0,1) draws give)."""
    if dtype == "bf16":
        f = (bits.astype(np.uint32) << 16).view(np.float32) * np.float32(2.0 ** power)
        return (f.view(np.uint32) >> 16).astype(np.uint16)
    return (bits.view(np.float16).astype(np.float32) * np.float32(2.0 ** power)).astype(np.float16).view(np.uint16)


def sharp_workload(seed, dtype="bf16"):
    """q x 4 (scores 4x wider, so few tokens carry the weight) and V x 2, over short
    histories: outputs up to a few units."""
    wl = custom(seed, dtype, 8, 2, 128, [2, 3, 4, 5, 6, 8, 12, 16, 24, 40])
    sv = lambda b: _scaled(b, 1, dtype)
    return dataclasses.replace(wl, q=_scaled(wl.q, 2, dtype), pre_value=sv(wl.pre_value), value=sv(wl.value),
                               bank_v=sv(wl.bank_v))


@pytest.mark.parametrize("seed", [800, 801, 802, 803])
@pytest.mark.parametrize("path", ["single", "split"])
def test_sharp_attention_on_large_values(seed, path):
    """Seeds where one bf16 rounding of the probabilities misses the oracle by 1.06e-2 to
    1.24e-2 (a host emulation of that arithmetic): within 1e-2 where the output is below
    4; above, within bf16's own rounding of it (half a spacing, at most 2^-8 relative) plus
    2^-12 relative and 1e-4 for the arithmetic."""
    wl = sharp_workload(seed)
    ref = oracle.decode(wl, oracle.filled_pool(wl))
    out, used = gh.decode(gh.filled_pool(wl), gh.DecodeInputs(wl), path)
    got = gh.out_f64(out)
    assert np.isfinite(got).all()
    err = np.abs(got - ref)
    small = np.abs(ref) < 4
    say(f"sharp attention seed {seed} ({used}): max|o| {np.abs(ref).max():.3f}, max err below 4 "
        f"{err[small].max():.3e}, outputs of 4 or more {int((~small).sum())}")
    assert err[small].max() <= TOL["bf16"]
    assert (err[~small] <= np.abs(ref[~small]) * (2.0 ** -8 + 2.0 ** -12) + 1e-4).all()


@pytest.mark.parametrize("path", ["single", "split"])
def test_sharp_attention_on_large_values_fp16(path):
    """fp16 keeps one rounding of the probabilities (relative 2^-11): on the same kind of
    workload every output, up to 8 in size, stays within 1e-2 (a host emulation of that
    arithmetic puts the worst near 2.4e-3)."""
    wl = sharp_workload(800, "f16")
    ref = oracle.decode(wl, oracle.filled_pool(wl))
    out, used = gh.decode(gh.filled_pool(wl), gh.DecodeInputs(wl), path)
    check_attention(gh.out_f64(out), ref, "f16", f"sharp attention fp16 ({used})")
