"""GPU parity of the ALiBi score bias against the oracle on the same seeded inputs.

The bias of query head h at token t is slope_h * (t - (L - 1)) ("vLLM 源码完全拆解
（七）", section 第一步), added to the scaled score before the softmax.  Bars as for
the plain decode: max-abs 1e-5 (fp32 storage) or 1e-2 (16-bit and 8-bit caches) of
the fp64 oracle; the split partials' maxima, which carry the bias, within 1e-4.
"""

import numpy as np
import pytest
import torch

import gpu_harness as gh
import oracle
from workloads import alibi_variant, custom, fp8_variant, make_config

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "f16": 1e-2, "bf16": 1e-2}
LENGTHS = [1, 15, 16, 17, 100, 511, 512, 513, 1100]


def say(msg):
    print(msg, flush=True)


def check(got, ref, tol, what):
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got - ref)
    say(f"{what}: max|err| {err.max():.3e}, max|o| {np.abs(ref).max():.3f}, tol {tol}")
    assert err.max() <= tol, what


def slopes_for(Hq, seed):
    """Slopes of both signs and very different sizes, one per query head."""
    rng = np.random.default_rng(seed)
    s = rng.uniform(-0.02, 0.3, size=Hq).astype(np.float32)
    s[0] = 0.0
    return s


CASES = [(dt, D, G, kv) for dt, kv in (("f32", ""), ("f16", ""), ("bf16", ""), ("bf16", "fp8"), ("f16", "fp8"))
         for D in (64, 128) for G in (1, 4)] + [("bf16", 128, 8, ""), ("f16", 64, 2, "fp8")]


@pytest.mark.parametrize("dt,D,G,kv", CASES, ids=[f"{a}-d{b}-g{c}{'-' + d if d else ''}" for a, b, c, d in CASES])
@pytest.mark.parametrize("path", ["single", "split"])
def test_alibi_parity(dt, D, G, kv, path):
    Hkv = 2
    wl = custom(400 + D + G, dt, Hkv * G, Hkv, D, LENGTHS, extra_pad_rows=1)
    if kv == "fp8":
        wl = fp8_variant(wl)
    wl = alibi_variant(wl, slopes_for(Hkv * G, D + G))
    hpool = oracle.filled_pool(wl)
    dpool = gh.filled_pool(wl)
    out, _ = gh.decode(dpool, gh.DecodeInputs(wl), path)
    check(gh.out_f64(out), oracle.decode(wl, hpool), TOL[dt], f"alibi {dt} D{D} G{G} {kv or 'native'} {path}")


def test_alibi_partials():
    wl = alibi_variant(custom(410, "bf16", 8, 2, 128, [1, 511, 512, 513, 1500]), slopes_for(8, 3))
    hpool = oracle.filled_pool(wl)
    dpool = gh.filled_pool(wl)
    inp = gh.DecodeInputs(wl)
    es, ml, tmp = gh.partials_call(dpool, inp, inp.max_seq_len)
    torch.cuda.synchronize()
    rt, rm, re = oracle.partials(wl, hpool, 512, es.shape[2])
    gm, ge = ml.double().cpu().numpy(), es.double().cpu().numpy()
    written = ~np.isnan(rm)
    assert np.array_equal(written, ~np.isnan(gm))
    err_m = np.abs(gm[written] - rm[written]).max()
    say(f"alibi partials: max|dm| {err_m:.3e}")
    assert err_m < 1e-4
    assert (np.abs(ge[written] - re[written]) / re[written]).max() < 1e-4


def test_alibi_zero_slopes_match_plain():
    """Slopes of zero give the plain decode's bits (the bias adds exactly zero)."""
    wl = custom(411, "bf16", 16, 4, 128, [3, 70, 600])
    dpool = gh.filled_pool(wl)
    plain, _ = gh.decode(dpool, gh.DecodeInputs(wl), "single")
    z = alibi_variant(wl, np.zeros(16, np.float32))
    zero, _ = gh.decode(dpool, gh.DecodeInputs(z), "single")
    assert torch.equal(plain.view(torch.int16), zero.view(torch.int16))


def test_alibi_long_context_split():
    """The long-context workload (4 x 32768 tokens) with the usual geometric slopes."""
    wl = alibi_variant(make_config(3))
    hpool = oracle.filled_pool(wl)
    ref = oracle.decode(wl, hpool)
    dpool = gh.filled_pool(wl)
    for path in ("split", "single"):
        out, _ = gh.decode(dpool, gh.DecodeInputs(wl), path)
        check(gh.out_f64(out), ref, TOL["bf16"], f"alibi long context {path}")
