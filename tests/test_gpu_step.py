"""GPU parity of the fused decode step (pc_reshape_and_cache_decode).

The step is the write of "How vLLM CUDA Kernels Write and Read the Paged KV Cache"
(each new token's K/V row to its slot) followed by the decode of "vLLM 源码完全拆解
（七）" on the same stream; the fused launch must give what those two give in that
order: the pool bit for bit equal to the oracle's write, the output within the
decode's bars (1e-2 max-abs of the fp64 oracle for 16-bit storage) and, since the
same decode arithmetic runs on the same row values, bit for bit equal to the two
separate launches.
"""

import numpy as np
import pytest
import torch

import gpu_harness as gh
import oracle
import paged_kv_cache_reshape_amd as pc
from workloads import alibi_variant, custom, make_config

pytestmark = pytest.mark.gpu

TOL = 1e-2


def say(msg):
    print(msg, flush=True)


def step_rows(wl):
    """The step's rows one per sequence: key/value bits [S, Hkv, D] and slots [S] -- the
    workload's step token written at position L_s - 1 of sequence s, or none (slot -1)."""
    sm = np.asarray(wl.slot_mapping)
    L = np.asarray(wl.seq_lens)
    bt = np.asarray(wl.block_tables)
    B = wl.block_size
    S = len(L)
    key = np.zeros((S,) + wl.key.shape[1:], wl.key.dtype)
    value = np.zeros_like(key)
    slots = np.full(S, -1, np.int64)
    for s in range(S):
        if L[s] < 1:
            continue
        e = int(bt[s, (L[s] - 1) // B]) * B + (int(L[s]) - 1) % B
        t = np.nonzero(sm == e)[0]
        if len(t):
            key[s], value[s], slots[s] = wl.key[t[0]], wl.value[t[0]], e
    return key, value, slots


def fused(wl, path, key, value, slots, inp=None):
    """The fused step on the history-only pool; returns (out, device pool)."""
    dpool = gh.filled_pool(wl, step_write=False)
    inp = inp or gh.DecodeInputs(wl)
    S, Hq, D = inp.q.shape
    kd, vd = gh.to_dev(key, wl.dtype), gh.to_dev(value, wl.dtype)
    sd = torch.from_numpy(slots).cuda()
    out = torch.full_like(inp.q, float("nan"))
    common = dict(num_kv_heads=wl.num_kv_heads, scale=float(wl.scale), alibi_slopes=inp.alibi,
                  **dpool.layout_kwargs())
    if path == "single":
        pc.reshape_and_cache_decode(out, inp.q, kd, vd, dpool.k, dpool.v, sd, inp.block_tables, inp.seq_lens,
                                    inp.max_seq_len, **common)
    else:
        P = max(1, -(-inp.max_seq_len // pc.PARTITION_SIZE))
        es = torch.full((S, Hq, P), float("nan"), device="cuda")
        ml = torch.full_like(es, float("nan"))
        tmp = torch.full((S, Hq, P, D), float("nan"), device="cuda")
        pc.reshape_and_cache_decode(None, inp.q, kd, vd, dpool.k, dpool.v, sd, inp.block_tables, inp.seq_lens,
                                    inp.max_seq_len, partition_size=pc.PARTITION_SIZE, exp_sums=es, max_logits=ml,
                                    tmp_out=tmp, **common)
        pc.paged_attention_reduce(out, es, ml, tmp, inp.seq_lens)
    torch.cuda.synchronize()
    return out, dpool


def separate(wl, path, key, value, slots, inp=None):
    """The same step as two launches: the write, then the decode."""
    dpool = gh.filled_pool(wl, step_write=False)
    gh.write(dpool, key, value, slots)
    inp = inp or gh.DecodeInputs(wl)
    out, _ = gh.decode(dpool, inp, path)
    torch.cuda.synchronize()
    return out, dpool


def pools_bits(dpool):
    torch.cuda.synchronize()
    return [gh.to_bits(a, dpool.wl.dtype) for a in dpool.arrays()]


CASES = [(dt, D, G, B) for dt in ("bf16", "f16") for D in (64, 128) for G in (1, 4, 8) for B in (16,)] + \
        [("bf16", 128, 4, 8), ("bf16", 128, 4, 32), ("f16", 64, 2, 32)]
LENS = [1, 15, 16, 17, 100, 511, 512, 513, 1100]


@pytest.mark.parametrize("dt,D,G,B", CASES, ids=[f"{a}-d{b}-g{c}-b{d}" for a, b, c, d in CASES])
@pytest.mark.parametrize("path", ["single", "split"])
def test_step_parity(dt, D, G, B, path):
    wl = custom(600 + D + G + B, dt, 2 * G, 2, D, LENS, block_size=B)
    key, value, slots = step_rows(wl)
    assert (slots >= 0).all()
    out, dpool = fused(wl, path, key, value, slots)
    ref = oracle.decode(wl, oracle.filled_pool(wl))
    got = gh.out_f64(out)
    err = np.abs(got - ref).max()
    say(f"step {dt} D{D} G{G} B{B} {path}: max|err| {err:.3e}")
    assert np.isfinite(got).all() and err <= TOL
    host = oracle.filled_pool(wl)
    for d, h in zip(pools_bits(dpool), host.arrays()):
        assert np.array_equal(d, h), "pool differs from the oracle's write"
    sep, spool = separate(wl, path, key, value, slots)
    assert torch.equal(out.view(torch.int16), sep.view(torch.int16)), "fused and separate launches differ"
    for a, b in zip(pools_bits(dpool), pools_bits(spool)):
        assert np.array_equal(a, b)


def test_step_padding_and_invalid_slots():
    """Slot -1 (padding) and a slot past the pool write nothing and leave the decode as
    after a write that skipped them; a slot inside the pool that is not position L - 1
    of its sequence turns that sequence's outputs (only) to NaN and writes nothing."""
    wl = custom(610, "bf16", 8, 2, 128, [40, 300, 60, 17, 520])
    key, value, slots = step_rows(wl)
    bad_slot = int(slots[0])          # sequence 0's own position L - 1: wrong for sequence 2
    slots[1] = -1
    slots[2] = bad_slot
    slots[3] = wl.num_blocks * wl.block_size + 5
    for path in ("single", "split"):
        out, dpool = fused(wl, path, key, value, slots)
        ok = [0, 4]
        s_slots = slots.copy()
        s_slots[2] = -1                # the separate reference: the invalid token writes nothing
        sep, spool = separate(wl, path, key, value, s_slots)
        got, ref = gh.out_f64(out), gh.out_f64(sep)
        assert np.isnan(got[2]).all(), "invalid slot: NaN expected"
        assert np.array_equal(got[ok], ref[ok])
        # sequences 1 and 3 read their pools' (unwritten, NaN-filled) row L - 1 in both
        assert np.array_equal(np.isnan(got[[1, 3]]), np.isnan(ref[[1, 3]]))
        for a, b in zip(pools_bits(dpool), pools_bits(spool)):
            assert np.array_equal(a, b), "the pools differ"


def test_step_alibi():
    wl = alibi_variant(custom(611, "bf16", 16, 4, 128, LENS), np.linspace(0.3, -0.01, 16).astype(np.float32))
    key, value, slots = step_rows(wl)
    for path in ("single", "split"):
        out, _ = fused(wl, path, key, value, slots)
        sep, _ = separate(wl, path, key, value, slots)
        assert torch.equal(out.view(torch.int16), sep.view(torch.int16)), path
    ref = oracle.decode(wl, oracle.filled_pool(wl))
    assert np.abs(gh.out_f64(out) - ref).max() <= TOL


@pytest.mark.parametrize("cfg,path", [(1, "single"), (3, "split")])
def test_step_headline_workloads(cfg, path):
    """The benchmark's decode workloads at full size in the path the benchmark times:
    fused and separate launches agree bit for bit, outputs and pools."""
    say(f"[step cfg{cfg}] generating")
    wl = make_config(cfg)
    key, value, slots = step_rows(wl)
    assert (slots >= 0).all() and np.array_equal(slots, np.asarray(wl.slot_mapping))
    out, dpool = fused(wl, path, key, value, slots)
    sep, spool = separate(wl, path, key, value, slots)
    assert torch.equal(out.view(torch.int16), sep.view(torch.int16))
    for a, b in zip(dpool.arrays(), spool.arrays()):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))  # bits: the pools hold NaN padding
