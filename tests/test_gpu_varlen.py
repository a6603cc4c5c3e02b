"""GPU parity of multi-token (varlen) queries over the paged K/V against the oracle.

Request r owns rows [qs[r], qs[r+1]) of the packed query, its newest n_r tokens;
token i attends positions t <= L_r - n_r + i (causal) or all of [0, L_r).  Bars as
for the decode: max-abs 1e-2 of the fp64 oracle for 16-bit storage.
"""

import numpy as np
import pytest
import torch

import gpu_harness as gh
import oracle
from workloads import alibi_variant, custom, varlen_variant

pytestmark = pytest.mark.gpu

TOL = 1e-2


def say(msg):
    print(msg, flush=True)


def check(got, ref, what, rows=None):
    g = gh.out_f64(got)
    if rows is not None:
        g, ref = g[rows], ref[rows]
    assert np.isfinite(g).all(), f"{what}: non-finite output"
    err = np.abs(g - ref)
    say(f"{what}: max|err| {err.max():.3e}, max|o| {np.abs(ref).max():.3f}")
    assert err.max() <= TOL, what


LENS = [1, 16, 17, 40, 300, 700, 33]
QLENS = [1, 16, 3, 40, 0, 21, 33]   # includes a request with no query, one whose query is its whole history
CASES = [(dt, D, G) for dt in ("bf16", "f16") for D in (64, 128) for G in (1, 2, 4, 8)]


@pytest.mark.parametrize("dt,D,G", CASES, ids=[f"{a}-d{b}-g{c}" for a, b, c in CASES])
@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
def test_varlen_parity(dt, D, G, causal):
    Hkv = 2
    wl = custom(500 + D + G, dt, Hkv * G, Hkv, D, LENS)
    vq = varlen_variant(wl, QLENS, causal=causal)
    hpool = oracle.filled_pool(wl)
    dpool = gh.filled_pool(wl)
    out = gh.varlen(dpool, vq)
    check(out, oracle.varlen(wl, hpool, vq), f"varlen {dt} D{D} G{G} {'causal' if causal else 'full'}")


SHORT_QLENS = [1, 2, 4, 3, 0, 4, 1]  # G <= 4: the multi-token decode; G = 8 (32 columns): K/V split over waves
# at most 16 (token, head) columns per request and kv head: the one-pass decode's unit
MT_QLENS = {1: [1, 16, 9, 0, 16, 5, 1], 2: [1, 8, 3, 0, 8, 2, 1], 4: [1, 4, 4, 0, 2, 4, 3], 8: [1, 2, 1, 0, 2, 2, 1]}


@pytest.mark.parametrize("dt,D,G", CASES, ids=[f"{a}-d{b}-g{c}" for a, b, c in CASES])
def test_varlen_parity_short_queries(dt, D, G):
    wl = custom(520 + D + G, dt, 2 * G, 2, D, LENS)
    vq = varlen_variant(wl, SHORT_QLENS)
    dpool = gh.filled_pool(wl)
    check(gh.varlen(dpool, vq), oracle.varlen(wl, oracle.filled_pool(wl), vq), f"varlen short {dt} D{D} G{G}")


@pytest.mark.parametrize("G", [1, 2, 4, 8])
@pytest.mark.parametrize("causal", [True, False])
def test_varlen_multitoken_decode(G, causal):
    """Up to 16 (query token, head) columns per request and kv head run on the one-pass
    decode's unit with one 16-column score tile: column c is token c / G, head c % G."""
    wl = custom(540 + G, "bf16", 2 * G, 2, 128, LENS)
    vq = varlen_variant(wl, MT_QLENS[G])
    dpool = gh.filled_pool(wl)
    check(gh.varlen(dpool, vq, causal=causal), oracle.varlen(wl, oracle.filled_pool(wl), vq, causal=causal),
          f"varlen multi-token G{G} {'causal' if causal else 'full'}")


@pytest.mark.parametrize("R", [8, 128, 130])
def test_varlen_dispatch_order(R):
    """Workgroups take requests longest history first (ranked inside the kernel up to 128
    requests, in index order past that): with tied lengths and either side of that
    bound, every request's rows are still computed exactly once."""
    rng = np.random.default_rng(530 + R)
    if R == 8:
        lens = np.array([300, 40, 300, 300, 17, 40, 300, 5])
    else:
        lens = rng.choice([24, 64, 65, 150], size=R)  # many ties
    qlens = np.minimum(lens, rng.integers(1, 25, size=R))
    qlens[0] = min(lens[0], 24)                       # 24 tokens x 4 heads: the LDS-sharing kernel
    wl = custom(530 + R, "bf16", 16, 4, 128, lens.tolist())
    vq = varlen_variant(wl, qlens.astype(np.int32))
    dpool = gh.filled_pool(wl)
    check(gh.varlen(dpool, vq), oracle.varlen(wl, oracle.filled_pool(wl), vq), f"varlen order R{R}")


@pytest.mark.parametrize("causal", [True, False])
def test_varlen_alibi_multitoken(causal):
    """The bias on the multi-token decode (origin at each query token's own position,
    causal or not)."""
    wl = alibi_variant(custom(512, "bf16", 16, 4, 128, LENS), np.linspace(0.25, -0.01, 16).astype(np.float32))
    vq = varlen_variant(wl, MT_QLENS[4])
    dpool = gh.filled_pool(wl)
    check(gh.varlen(dpool, vq, causal=causal), oracle.varlen(wl, oracle.filled_pool(wl), vq, causal=causal),
          f"varlen + ALiBi, multi-token {'causal' if causal else 'full'}")


@pytest.mark.parametrize("qlens", ["long", "short"])
def test_varlen_alibi(qlens):
    """The bias on both kernels: long queries (K/V shared through LDS) and at most 32
    (token, head) columns per request (K/V split over the waves)."""
    wl = alibi_variant(custom(510, "bf16", 16, 4, 128, LENS), np.linspace(0.25, -0.01, 16).astype(np.float32))
    vq = varlen_variant(wl, QLENS if qlens == "long" else SHORT_QLENS)
    dpool = gh.filled_pool(wl)
    check(gh.varlen(dpool, vq), oracle.varlen(wl, oracle.filled_pool(wl), vq), f"varlen + ALiBi, {qlens} queries")


def test_varlen_single_tokens_match_decode():
    """One token per request: the varlen kernel and the decode kernel agree (and both the oracle)."""
    wl = custom(511, "bf16", 32, 8, 128, [5, 77, 513, 1500])
    dpool = gh.filled_pool(wl)
    vq = varlen_variant(wl, [1, 1, 1, 1])
    out = gh.varlen(dpool, vq, q_bits=wl.q)
    ref = oracle.decode(wl, oracle.filled_pool(wl))
    check(out, ref.reshape(out.shape), "varlen n=1 vs decode oracle")
    dec, _ = gh.decode(dpool, gh.DecodeInputs(wl), "single")
    assert np.abs(gh.out_f64(dec).reshape(out.shape) - gh.out_f64(out)).max() <= TOL


def test_varlen_chunked_prefill_step():
    """A chunked-prefill step: the chunk's K/V rows are written through slot_mapping
    (pc_reshape_and_cache), then the chunk attends causally to the whole history."""
    wl = custom(512, "bf16", 32, 8, 128, [600, 1300, 2048, 257])
    vq = varlen_variant(wl, [128, 64, 128, 100])
    hpool = oracle.empty_pool(wl)
    # history before the chunk, then the chunk itself (what the step writes)
    oracle.write(wl, hpool, wl.pre_key, wl.pre_value, wl.pre_slots)
    oracle.write(wl, hpool, wl.key, wl.value, wl.slot_mapping)
    dpool = gh.DevicePool(wl)
    gh.write(dpool, wl.pre_key, wl.pre_value, wl.pre_slots)
    gh.write(dpool, wl.key, wl.value, wl.slot_mapping)
    gh.write(dpool, vq.key, vq.value, vq.slot_mapping)  # rewrites the chunk's own rows, unchanged
    oracle.write(wl, hpool, vq.key, vq.value, vq.slot_mapping)
    torch.cuda.synchronize()
    for d, h in zip(dpool.arrays(), hpool.arrays()):
        assert np.array_equal(gh.to_bits(d, wl.dtype), h)
    check(gh.varlen(dpool, vq), oracle.varlen(wl, hpool, vq), "chunked prefill step")


@pytest.mark.parametrize("mql", [2, 8, 16])
def test_varlen_understated_max_query_len(mql):
    """A request longer than max_query_len is still computed in full (2 x 4 columns: the
    multi-token decode, in passes of 4 tokens; 8 x 4: the K/V-splitting kernel; 16 x 4:
    the LDS-sharing kernel, whose grid then holds one 32-token chunk per request)."""
    wl = custom(513, "f16", 8, 2, 64, [100, 300])
    vq = varlen_variant(wl, [90, 7])
    dpool = gh.filled_pool(wl)
    check(gh.varlen(dpool, vq, max_query_len=mql), oracle.varlen(wl, oracle.filled_pool(wl), vq), f"short grid {mql}")


@pytest.mark.parametrize("qlens", [[4, 30, 5], [2, 3, 4]], ids=["lds", "multitoken"])
def test_varlen_bad_request_is_nan_only_there(qlens):
    wl = custom(514, "bf16", 8, 2, 128, [40, 300, 60])
    vq = varlen_variant(wl, qlens)
    dpool = gh.filled_pool(wl)
    ref = oracle.varlen(wl, oracle.filled_pool(wl), vq)
    qs = vq.query_start_loc
    bt = wl.block_tables.copy()
    bt[1, 3] = wl.num_blocks + 7          # request 1 names a block outside the pool
    sl = wl.seq_lens.copy()
    sl[2] = 3                              # request 2 claims fewer tokens than its query
    out = gh.out_f64(gh.varlen(dpool, vq, seq_lens=sl, block_tables=bt))
    assert np.isnan(out[qs[1]:qs[2]]).all() and np.isnan(out[qs[2]:qs[3]]).all()
    err = np.abs(out[qs[0]:qs[1]] - ref[qs[0]:qs[1]]).max()
    assert err <= TOL


@pytest.mark.parametrize("kind,sample", [("spec", None), ("prefill", [0, 5])])
def test_varlen_bench_workloads(kind, sample):
    """The benchmark's multi-token workloads at full size, in the configuration it times;
    for the prefill workload the oracle covers the rows of a sample of requests."""
    from workloads import varlen_config
    say(f"[varlen {kind}] generating")
    wl, vq = varlen_config(kind)
    dpool = gh.filled_pool(wl)
    out = gh.out_f64(gh.varlen(dpool, vq))
    hpool = oracle.filled_pool(wl)
    qs = vq.query_start_loc
    if sample is None:
        check_rows = np.arange(vq.total_q)
        ref = oracle.varlen(wl, hpool, vq)
    else:
        # only the sampled requests keep their rows; the others get empty ranges
        n = np.zeros(wl.num_seqs, np.int64)
        for r in sample:
            n[r] = qs[r + 1] - qs[r]
        qs_s = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
        check_rows = np.concatenate([np.arange(qs[r], qs[r + 1]) for r in sample])
        ref = oracle.varlen(wl, hpool, vq, q=vq.q[check_rows], query_start_loc=qs_s)
    got = out[check_rows]
    assert np.isfinite(out).all()
    err = np.abs(got - ref)
    say(f"[varlen {kind}] {len(check_rows)} rows: max|err| {err.max():.3e}, max|o| {np.abs(ref).max():.3f}")
    assert err.max() <= TOL
