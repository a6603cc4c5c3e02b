"""pc_paged_attention_decode_prefix: the split path for sequences sharing a prefix, the
partitions a sequence's shared tokens cover completely computed for 16 / G sequences at
once.  Checked against the fp64 oracle (which knows nothing of the sharing): final
outputs after the reduce, and partials element by element; against the plain split path
without a prefix; and on tables that contradict the stated sharing (NaN for those
sequences only)."""

import numpy as np
import pytest
import torch

import gpu_harness as gh
import oracle
import paged_kv_cache_reshape_amd as pc
from helpers import PROB_ROUNDOFF, with_abs_values
from test_gpu_parity import check_attention
from workloads import alibi_variant, custom, make_config

pytestmark = pytest.mark.gpu

# lengths around the partition and prefix edges (a sequence's last block is private)
LENGTHS = [1, 15, 16, 17, 511, 512, 513, 527, 528, 529, 1023, 1024, 1025, 1040, 1041, 1500, 2100, 3000]


def prefix_table_of(wl):
    """The shared blocks, as the generator reports them."""
    assert wl.shared_lens().max() == wl.prefix_blocks * wl.block_size
    return wl.prefix_table()


def prefix_partials(pool, inp, wl, shared=None, table=None, block_tables=None):
    S, Hq, D = inp.q.shape
    P = max(1, -(-inp.max_seq_len // 512))
    es = torch.full((S, Hq, P), float("nan"), device="cuda")
    ml = torch.full((S, Hq, P), float("nan"), device="cuda")
    tmp = torch.full((S, Hq, P, D), float("nan"), device="cuda")
    pt = torch.from_numpy(prefix_table_of(wl) if table is None else table).cuda()
    sl = torch.from_numpy(np.ascontiguousarray(wl.shared_lens() if shared is None else shared, np.int32)).cuda()
    bt = inp.block_tables if block_tables is None else torch.from_numpy(np.ascontiguousarray(block_tables)).cuda()
    pc.paged_attention_decode_prefix(inp.q, pool.k, pool.v, bt, inp.seq_lens, inp.max_seq_len,
                                     num_kv_heads=wl.num_kv_heads, scale=float(wl.scale), exp_sums=es, max_logits=ml,
                                     tmp_out=tmp, prefix_table=pt, shared_lens=sl, alibi_slopes=inp.alibi,
                                     **pool.layout_kwargs())
    return es, ml, tmp


def prefix_decode(pool, inp, wl, **kw):
    es, ml, tmp = prefix_partials(pool, inp, wl, **kw)
    out = torch.empty_like(inp.q)
    pc.paged_attention_reduce(out, es, ml, tmp, inp.seq_lens)
    torch.cuda.synchronize()
    return gh.out_f64(out)


CASES = [(dt, D, G, P) for dt in ("bf16", "f16") for D in (64, 128) for G in (1, 2, 4, 8)
         for P in ((64,) if (D + G) % 2 == 0 else (40,))] + [("bf16", 128, 1, 32), ("f16", 128, 4, 96)]


@pytest.mark.parametrize("dt,D,G,P", CASES, ids=[f"{a}-d{b}-g{c}-p{d}" for a, b, c, d in CASES])
def test_prefix_matches_oracle(dt, D, G, P):
    Hkv = 2
    lengths = LENGTHS + [P * 16 + 600] + ([1700] if G == 1 else [])  # 19-20 sequences: a ragged last group
    wl = custom(600 + D + G + P, dt, Hkv * G, Hkv, D, lengths, prefix_blocks=P)
    assert wl.shared_lens().max() == P * 16
    got = prefix_decode(gh.filled_pool(wl), gh.DecodeInputs(wl), wl)
    check_attention(got, oracle.decode(wl, oracle.filled_pool(wl)), dt, f"prefix {dt} D{D} G{G} P{P}")


def test_prefix_partials_against_oracle():
    """Partials, element by element, of an MHA batch: the covered partitions come from the
    prefix kernel, the rest from the split kernel; the same bound as the split path's."""
    wl = custom(620, "bf16", 4, 4, 128, LENGTHS, prefix_blocks=64)
    hpool = oracle.filled_pool(wl)
    inp = gh.DecodeInputs(wl)
    es, ml, tmp = prefix_partials(gh.filled_pool(wl), inp, wl)
    torch.cuda.synchronize()
    P = es.shape[2]
    rt, rm, re = oracle.partials(wl, hpool, 512, P)
    gt, gm, ge = tmp.double().cpu().numpy(), ml.double().cpu().numpy(), es.double().cpu().numpy()
    written = ~np.isnan(rm)
    assert np.array_equal(written, ~np.isnan(gm)), "partitions written differ"
    assert np.abs(gm[written] - rm[written]).max() < 1e-5
    assert (np.abs(ge[written] - re[written]) / re[written]).max() < 1e-5
    A, _, _ = oracle.partials(with_abs_values(wl), oracle.filled_pool(with_abs_values(wl)), 512, P)
    err = np.abs(gt[written] - rt[written])
    bound = (PROB_ROUNDOFF[wl.dtype] + 2.0 ** -14) * A[written] + 1e-6
    assert (err <= bound).all()
    assert err.max() <= 1e-2


def test_prefix_with_alibi():
    rng = np.random.default_rng(9)
    wl = custom(621, "bf16", 16, 4, 128, LENGTHS, prefix_blocks=64)
    wl = alibi_variant(wl, slopes=rng.uniform(-0.2, 0.2, 16).astype(np.float32))
    got = prefix_decode(gh.filled_pool(wl), gh.DecodeInputs(wl), wl)
    check_attention(got, oracle.decode(wl, oracle.filled_pool(wl)), "bf16", "prefix, ALiBi")


def test_no_prefix_is_the_split_path():
    """prefix_blocks = 0: the split decode itself, bit for bit."""
    wl = custom(622, "f16", 8, 2, 128, LENGTHS, prefix_blocks=64)
    pool, inp = gh.filled_pool(wl), gh.DecodeInputs(wl)
    es, ml, tmp = prefix_partials(pool, inp, wl, table=np.zeros(0, np.int32), shared=np.zeros(wl.num_seqs))
    e2, m2, t2 = gh.partials_call(pool, inp, inp.max_seq_len)
    torch.cuda.synchronize()
    for a, b in ((es, e2), (ml, m2), (tmp, t2)):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))


def test_understated_sharing_is_still_exact():
    """A sequence that shares the prefix but states fewer (or no) shared tokens is read
    through its own table for the rest: still the same attention."""
    wl = custom(623, "bf16", 8, 8, 128, LENGTHS, prefix_blocks=64)
    shared = wl.shared_lens().copy()
    shared[12] = 0         # 1025 tokens, shares 64 blocks, states none
    shared[15] = 512       # 1500 tokens, states one partition of two
    got = prefix_decode(gh.filled_pool(wl), gh.DecodeInputs(wl), wl, shared=shared)
    check_attention(got, oracle.decode(wl, oracle.filled_pool(wl)), "bf16", "prefix, understated sharing")


def test_contradicted_sharing_gives_nan_for_that_sequence_only():
    wl = custom(624, "bf16", 8, 8, 128, LENGTHS, prefix_blocks=64)
    ref = oracle.decode(wl, oracle.filled_pool(wl))
    shared = wl.shared_lens().copy()
    bt = wl.block_tables.copy()
    i_tab = 16                      # 2100 tokens: partitions 0 and 1 covered
    bt[i_tab, 40] = bt[17, 70]      # a block of another sequence where the prefix block should be
    i_len = 4                       # 511 tokens: states a whole partition it does not have
    shared[i_len] = 512
    got = prefix_decode(gh.filled_pool(wl), gh.DecodeInputs(wl, block_tables=bt), wl, shared=shared, block_tables=bt)
    assert np.isnan(got[i_tab]).all() and np.isnan(got[i_len]).all()
    keep = [i for i in range(wl.num_seqs) if i not in (i_tab, i_len)]
    check_attention(got[keep], ref[keep], "bf16", "prefix, neighbours of contradicted sequences")


def test_prefix_refuses_fp32_and_other_block_sizes():
    wl = custom(625, "f32", 4, 4, 64, [600, 900], prefix_blocks=32)
    with pytest.raises(pc.PagedCacheError) as e:
        prefix_partials(gh.filled_pool(wl), gh.DecodeInputs(wl), wl)
    assert e.value.status == -2
    wl = custom(626, "bf16", 4, 4, 64, [600, 1500], prefix_blocks=32, block_size=32)
    with pytest.raises(pc.PagedCacheError) as e:
        prefix_partials(gh.filled_pool(wl), gh.DecodeInputs(wl), wl)
    assert e.value.status == -2


def test_prefix_on_the_mixed_serving_workload():
    """The full-size mixed-serving workload (256 sequences, 1024-token shared prefix): a
    sample of sequences against the oracle, and every output against the split path's."""
    wl = make_config(4)
    pool, inp = gh.filled_pool(wl), gh.DecodeInputs(wl)
    got = prefix_decode(pool, inp, wl)
    plain, path = gh.decode(pool, inp, "split")
    plain = gh.out_f64(plain)
    rows = np.isfinite(plain).all(axis=(1, 2))
    assert np.array_equal(rows, np.isfinite(got).all(axis=(1, 2)))
    assert np.abs(got[rows] - plain[rows]).max() <= 2e-2
    rng = np.random.default_rng(4)
    pick = np.sort(rng.choice(wl.num_seqs, 12, replace=False))
    pick = np.union1d(pick, [int(np.argmax(wl.seq_lens))])
    ref = oracle.decode(wl, oracle.filled_pool(wl), q=wl.q[pick], seq_lens=wl.seq_lens[pick],
                        block_tables=wl.block_tables[pick])
    check_attention(got[pick], ref, "f16", "prefix path, mixed serving, sampled sequences")
