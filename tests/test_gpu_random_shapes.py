"""Seeded random draws over the decode's options at once -- storage type, 8-bit cache,
head size, query heads per kv head, kv heads, pool layout, block size, path, ALiBi and
length mix -- each against the oracle.  The parametrised tests pin each option on its
own; these draws reach combinations none of them names (odd kv-head counts, 8-token
blocks in a combined pool over the split path, ...).  Every draw is printed before it
runs."""

import numpy as np
import pytest

import gpu_harness as gh
import oracle
from test_gpu_parity import TOL, check_attention, say
from workloads import alibi_variant, custom, fp8_variant, varlen_variant

pytestmark = pytest.mark.gpu

N_DRAWS = 32
WORK_LIMIT = 4e8  # sum over sequences of q heads x length x head size, so the oracle takes seconds


def draw(k: int) -> dict:
    rng = np.random.default_rng(7000 + k)
    dt = str(rng.choice(["f32", "f16", "bf16"]))
    fp8 = dt != "f32" and rng.random() < 0.3
    D = int(rng.choice([64, 128]))
    G = int(rng.choice([1, 2, 4] if dt == "f32" else [1, 2, 4, 8]))
    Hkv = int(rng.choice([1, 2, 3, 4, 8]))
    layout = str(rng.choice(["hnd", "nhd", "combined"]))
    B = 16 if dt == "f32" else int(rng.choice([8, 16, 32]))
    path = str(rng.choice(["plan", "single", "split"]))
    hi = int(rng.choice([600, 3000, 9000]))
    S = int(rng.integers(1, 25))
    lens = rng.integers(0 if k % 4 == 0 else 1, hi + 1, S)
    while S > 1 and float(lens.sum()) * Hkv * G * D > WORK_LIMIT:
        S -= 1
        lens = lens[:S]
    alibi = bool(rng.random() < 0.4)
    # fp32: slopes of ALiBi's own sign.  A negative slope puts the weight on the oldest
    # tokens, whose biases of |slope| * L (hundreds here) fp32 holds only to their spacing
    # (about 6e-5 at 900), above the 1e-5 bar; the 16-bit bars hold for either sign.
    lo = 0.0 if dt == "f32" else -0.3
    return dict(k=k, dt=dt, fp8=fp8, D=D, G=G, Hkv=Hkv, layout=layout, B=B, path=path, lens=lens.astype(np.int32),
                alibi=alibi, slopes=rng.uniform(lo, 0.3, Hkv * G).astype(np.float32))


@pytest.mark.parametrize("k", range(N_DRAWS))
def test_random_draw(k):
    d = draw(k)
    say(f"[draw {k}] {d['dt']}{' fp8 cache' if d['fp8'] else ''} D{d['D']} G{d['G']} Hkv{d['Hkv']} {d['layout']} "
        f"B{d['B']} {d['path']} alibi={d['alibi']} S={len(d['lens'])} lens={d['lens'].tolist()}")
    wl = custom(7000 + k, d["dt"], d["Hkv"] * d["G"], d["Hkv"], d["D"], d["lens"], layout=d["layout"],
                block_size=d["B"])
    if d["alibi"]:
        wl = alibi_variant(wl, slopes=d["slopes"])
    if d["fp8"]:
        wl = fp8_variant(wl)
    out, used = gh.decode(gh.filled_pool(wl), gh.DecodeInputs(wl), d["path"])
    ref = oracle.decode(wl, oracle.filled_pool(wl))
    check_attention(gh.out_f64(out), ref, d["dt"], f"draw {k} ({used} path)")


# ---------------------------------------------------------------------------------
# several query tokens per request (pc_paged_attention_varlen)
# ---------------------------------------------------------------------------------

N_VARLEN = 24


def draw_varlen(k: int) -> dict:
    rng = np.random.default_rng(7100 + k)
    dt = str(rng.choice(["f16", "bf16"]))
    D = int(rng.choice([64, 128]))
    G = int(rng.choice([1, 2, 4, 8]))
    Hkv = int(rng.choice([1, 2, 3, 4]))
    layout = str(rng.choice(["hnd", "nhd", "combined"]))
    R = int(rng.integers(1, 13))
    lens = rng.integers(1, int(rng.choice([100, 1000, 3000])) + 1, R)
    # query lengths: a few tokens (the decode's unit), up to 40 (two score tiles or the
    # prefill kernel) or up to 600; zero for some requests
    qmax = int(rng.choice([4, 40, 600]))
    qlens = np.minimum(rng.integers(0, qmax + 1, R), lens)
    while R > 1 and float((qlens * lens).sum()) * Hkv * G * D > WORK_LIMIT:
        R -= 1
        lens, qlens = lens[:R], qlens[:R]
    return dict(k=k, dt=dt, D=D, G=G, Hkv=Hkv, layout=layout, lens=lens.astype(np.int32),
                qlens=qlens.astype(np.int32), causal=bool(rng.random() < 0.7), alibi=bool(rng.random() < 0.4),
                slopes=rng.uniform(-0.3, 0.3, Hkv * G).astype(np.float32))


@pytest.mark.parametrize("k", range(N_VARLEN))
def test_random_varlen_draw(k):
    d = draw_varlen(k)
    say(f"[varlen draw {k}] {d['dt']} D{d['D']} G{d['G']} Hkv{d['Hkv']} {d['layout']} causal={d['causal']} "
        f"alibi={d['alibi']} lens={d['lens'].tolist()} qlens={d['qlens'].tolist()}")
    wl = custom(7100 + k, d["dt"], d["Hkv"] * d["G"], d["Hkv"], d["D"], d["lens"], layout=d["layout"])
    if d["alibi"]:
        wl = alibi_variant(wl, slopes=d["slopes"])
    vq = varlen_variant(wl, d["qlens"], causal=d["causal"])
    if vq.total_q == 0:
        pytest.skip("no query rows drawn")
    out = gh.varlen(gh.filled_pool(wl), vq)
    check_attention(gh.out_f64(out), oracle.varlen(wl, oracle.filled_pool(wl), vq), d["dt"], f"varlen draw {k}")


# ---------------------------------------------------------------------------------
# the split path given a shared prefix (pc_paged_attention_decode_prefix)
# ---------------------------------------------------------------------------------

N_PREFIX = 16


def draw_prefix(k: int) -> dict:
    rng = np.random.default_rng(7200 + k)
    P = int(rng.choice([32, 40, 64, 96, 160]))  # prefix blocks: whole partitions, or one and a part
    S = int(rng.integers(1, 41))
    # most sequences run past the prefix, some end inside it
    lens = np.where(rng.random(S) < 0.8, P * 16 + rng.integers(1, 2000, S), rng.integers(1, P * 16 + 1, S))
    Hkv = int(rng.choice([1, 2, 4]))
    G = int(rng.choice([1, 2, 4, 8]))
    D = int(rng.choice([64, 128]))
    while S > 1 and float(lens[:S].sum()) * Hkv * G * D > WORK_LIMIT:
        S -= 1
    return dict(k=k, dt=str(rng.choice(["f16", "bf16"])), P=P, lens=lens[:S].astype(np.int32), Hkv=Hkv, G=G, D=D,
                alibi=bool(rng.random() < 0.3), slopes=rng.uniform(-0.3, 0.3, Hkv * G).astype(np.float32))


@pytest.mark.parametrize("k", range(N_PREFIX))
def test_random_prefix_draw(k):
    from test_gpu_prefix import prefix_decode
    d = draw_prefix(k)
    say(f"[prefix draw {k}] {d['dt']} D{d['D']} G{d['G']} Hkv{d['Hkv']} prefix {d['P']} blocks alibi={d['alibi']} "
        f"lens={d['lens'].tolist()}")
    wl = custom(7200 + k, d["dt"], d["Hkv"] * d["G"], d["Hkv"], d["D"], d["lens"], prefix_blocks=d["P"])
    if d["alibi"]:
        wl = alibi_variant(wl, slopes=d["slopes"])
    if wl.shared_lens().max() < 512:
        pytest.skip("no sequence's shared tokens cover a whole partition")
    got = prefix_decode(gh.filled_pool(wl), gh.DecodeInputs(wl), wl)
    check_attention(got, oracle.decode(wl, oracle.filled_pool(wl)), d["dt"], f"prefix draw {k}")
