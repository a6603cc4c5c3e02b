"""The C ABI on the host: every declared symbol is exported, invalid arguments are
refused before anything is enqueued, and the planner's choices (CPU only).

Every call here either fails validation or is a documented no-op, so no kernel is
ever launched (the pointers passed are never dereferenced).
"""

import ctypes
import os
import re

import pytest
import torch

import paged_kv_cache_reshape_amd as pc
from paged_kv_cache_reshape_amd import _native

REPO = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = ctypes.c_void_p(0x10000)  # 16-byte aligned, never dereferenced: every call below fails validation


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(pc.LIB_PATH):
        from paged_kv_cache_reshape_amd import build
        build.build()
    return pc.library()


def declared_symbols():
    text = open(os.path.join(REPO, "include", "pc.h")).read()
    return sorted(set(re.findall(r"\b(pc_[a-z_0-9]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(lib):
    names = declared_symbols()
    assert {"pc_reshape_and_cache", "pc_paged_attention_decode", "pc_paged_attention_reduce",
            "pc_paged_attention_plan", "pc_reshape_and_cache_fp8", "pc_paged_attention_decode_fp8",
            "pc_paged_attention_varlen", "pc_reshape_and_cache_decode"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings(lib):
    assert pc.abi_version() == 10
    assert pc.status_string(0) == "ok"
    assert "invalid" in pc.status_string(-1)
    assert "unsupported" in pc.status_string(-2)
    assert "launch" in pc.status_string(-3)
    assert "buffer" in pc.status_string(-4)


def _decode(lib, **kw):
    a = dict(out=FAKE, q=FAKE, k=FAKE, v=FAKE, nb=100, bs=8 * 16 * 128, ts=128, hs=16 * 128, bt=FAKE, W=128,
             sl=FAKE, S=4, msl=2048, Hq=32, Hkv=8, D=128, B=16, scale=0.088, ps=0, es=None, ml=None, tmp=None,
             alibi=None, dt=2, stream=None)
    a.update(kw)
    return lib.pc_paged_attention_decode(a["out"], a["q"], a["k"], a["v"], a["nb"], a["bs"], a["ts"], a["hs"],
                                         a["bt"], a["W"], a["sl"], a["S"], a["msl"], a["Hq"], a["Hkv"], a["D"],
                                         a["B"], a["scale"], a["ps"], a["es"], a["ml"], a["tmp"], a["alibi"],
                                         a["dt"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(dt=7), -1),                      # unknown dtype
    (dict(Hq=30), -1),                     # Hq not a multiple of Hkv
    (dict(S=-1), -1),
    (dict(msl=2049), -1),                  # longer than a table row can hold
    (dict(out=None), -1),                  # one-pass path without out
    (dict(q=None), -1),
    (dict(nb=0), -1),
    (dict(ps=512), -1),                    # split path without partials
    (dict(es=FAKE), -1),                   # partials on the one-pass path
    (dict(ps=256), -2),                    # partition size not offered
    (dict(D=96, bs=8 * 16 * 96, hs=16 * 96, ts=96), -2),
    (dict(B=64, W=32), -2),                # block sizes 8, 16 and 32 only
    (dict(B=8, W=256, dt=0), -2),          # fp32 storage: 16-token blocks only
    (dict(Hq=128), -2),                    # group of 16 not built
    (dict(q=ctypes.c_void_p(0x10008)), -2),  # not 16-byte aligned
    (dict(ts=100), -2),                    # stride not a multiple of 16 bytes
    (dict(ts=1 << 26), -2),                # 16 token rows span 2 GiB: past 32-bit offsets
])
def test_decode_validation(lib, kw, status):
    assert _decode(lib, **kw) == status


def test_decode_empty_batch_is_a_noop(lib):
    assert _decode(lib, S=0) == 0
    assert _decode(lib, S=0, q=None, k=None, v=None, bt=None, sl=None, out=None) == 0


def test_write_validation(lib):
    f = lib.pc_reshape_and_cache
    ok = dict(key=FAKE, value=FAKE, krs=1024, vrs=1024, k=FAKE, v=FAKE, nb=10, bs=16384, ts=128, hs=2048,
              sm=FAKE, T=3, Hkv=8, D=128, B=16, dt=2)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["key"], a["value"], a["krs"], a["vrs"], a["k"], a["v"], a["nb"], a["bs"], a["ts"], a["hs"],
                 a["sm"], a["T"], a["Hkv"], a["D"], a["B"], a["dt"], None)

    assert call(T=0) == 0  # no tokens: nothing to do
    for bad in (dict(dt=3), dict(T=-1), dict(Hkv=0), dict(D=0), dict(B=0), dict(nb=0), dict(key=None),
                dict(sm=None), dict(krs=100), dict(ts=0)):
        assert call(**bad) == -1, bad


def _decode_fp8(lib, **kw):
    a = dict(out=FAKE, q=FAKE, k=FAKE, v=FAKE, nb=100, bs=8 * 16 * 128, ts=128, hs=16 * 128, bt=FAKE, W=128,
             sl=FAKE, S=4, msl=2048, Hq=32, Hkv=8, D=128, B=16, scale=0.088, ps=0, es=None, ml=None, tmp=None,
             alibi=None, ksc=FAKE, vsc=FAKE, sst=1, dt=2, stream=None)
    a.update(kw)
    return lib.pc_paged_attention_decode_fp8(a["out"], a["q"], a["k"], a["v"], a["nb"], a["bs"], a["ts"], a["hs"],
                                             a["bt"], a["W"], a["sl"], a["S"], a["msl"], a["Hq"], a["Hkv"], a["D"],
                                             a["B"], a["scale"], a["ps"], a["es"], a["ml"], a["tmp"], a["alibi"],
                                             a["ksc"], a["vsc"], a["sst"], a["dt"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(dt=7), -1),
    (dict(ksc=None), -1),                  # scales are required
    (dict(vsc=None), -1),
    (dict(sst=-1), -1),
    (dict(out=None), -1),
    (dict(ps=512), -1),
    (dict(dt=0), -2),                      # fp32 queries have no 8-bit kernel
    (dict(ts=72), -2),                     # byte stride not a multiple of 16
    (dict(D=96, bs=8 * 16 * 96, hs=16 * 96, ts=96), -2),
    (dict(B=12, W=171), -2),
    (dict(ts=1 << 27), -2),                # 16 token rows span 2 GiB
])
def test_decode_fp8_validation(lib, kw, status):
    assert _decode_fp8(lib, **kw) == status


def test_decode_fp8_empty_batch_is_a_noop(lib):
    assert _decode_fp8(lib, S=0) == 0


def test_write_fp8_validation(lib):
    f = lib.pc_reshape_and_cache_fp8
    ok = dict(key=FAKE, value=FAKE, krs=1024, vrs=1024, k=FAKE, v=FAKE, nb=10, bs=16384, ts=128, hs=2048,
              sm=FAKE, T=3, Hkv=8, D=128, B=16, ksc=FAKE, vsc=FAKE, sst=1, dt=2)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["key"], a["value"], a["krs"], a["vrs"], a["k"], a["v"], a["nb"], a["bs"], a["ts"], a["hs"],
                 a["sm"], a["T"], a["Hkv"], a["D"], a["B"], a["ksc"], a["vsc"], a["sst"], a["dt"], None)

    assert call(T=0) == 0
    assert call(T=0, ksc=None, vsc=None) == 0
    for bad in (dict(dt=3), dict(T=-1), dict(Hkv=0), dict(ksc=None), dict(vsc=None), dict(sst=-1), dict(key=None),
                dict(krs=100), dict(nb=0)):
        assert call(**bad) == -1, bad
    for unsup in (dict(D=126, krs=1008, vrs=1008, hs=2016), dict(ts=130), dict(k=ctypes.c_void_p(0x10002))):
        assert call(**unsup) == -2, unsup


def _varlen(lib, **kw):
    a = dict(out=FAKE, q=FAKE, k=FAKE, v=FAKE, nb=100, bs=8 * 16 * 128, ts=128, hs=16 * 128, bt=FAKE, W=128,
             qsl=FAKE, sl=FAKE, R=4, T=40, mq=16, Hq=32, Hkv=8, D=128, B=16, scale=0.088, causal=1, alibi=None, dt=2)
    a.update(kw)
    return lib.pc_paged_attention_varlen(a["out"], a["q"], a["k"], a["v"], a["nb"], a["bs"], a["ts"], a["hs"],
                                         a["bt"], a["W"], a["qsl"], a["sl"], a["R"], a["T"], a["mq"], a["Hq"],
                                         a["Hkv"], a["D"], a["B"], a["scale"], a["causal"], a["alibi"], a["dt"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(dt=7), -1), (dict(R=-1), -1), (dict(T=-1), -1), (dict(mq=-1), -1), (dict(causal=2), -1),
    (dict(qsl=None), -1), (dict(out=None), -1), (dict(Hq=30), -1), (dict(scale=0.0), -1), (dict(nb=0), -1),
    (dict(dt=0), -2),                                  # fp32: no varlen kernel
    (dict(B=32, W=64), -2), (dict(D=96, bs=8 * 16 * 96, hs=16 * 96, ts=96), -2), (dict(Hq=128), -2),
    (dict(out=ctypes.c_void_p(0x10008)), -2), (dict(ts=100), -2),
])
def test_varlen_validation(lib, kw, status):
    assert _varlen(lib, **kw) == status


def test_varlen_empty_is_a_noop(lib):
    assert _varlen(lib, R=0) == 0
    assert _varlen(lib, T=0, q=None, out=None) == 0


def _step(lib, **kw):
    a = dict(out=FAKE, q=FAKE, key=FAKE, value=FAKE, krs=1024, vrs=1024, sm=FAKE, k=FAKE, v=FAKE, nb=100,
             bs=8 * 16 * 128, ts=128, hs=16 * 128, bt=FAKE, W=128, sl=FAKE, S=4, msl=2048, Hq=32, Hkv=8, D=128, B=16,
             scale=0.088, ps=0, es=None, ml=None, tmp=None, alibi=None, dt=2)
    a.update(kw)
    return lib.pc_reshape_and_cache_decode(a["out"], a["q"], a["key"], a["value"], a["krs"], a["vrs"], a["sm"],
                                           a["k"], a["v"], a["nb"], a["bs"], a["ts"], a["hs"], a["bt"], a["W"],
                                           a["sl"], a["S"], a["msl"], a["Hq"], a["Hkv"], a["D"], a["B"], a["scale"],
                                           a["ps"], a["es"], a["ml"], a["tmp"], a["alibi"], a["dt"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(dt=7), -1), (dict(S=-1), -1), (dict(key=None), -1), (dict(sm=None), -1), (dict(krs=100), -1),
    (dict(out=None), -1), (dict(ps=512), -1), (dict(nb=0), -1),
    (dict(dt=0), -2),                                  # fp32: the fused write lives in the matrix-core decode
    (dict(key=ctypes.c_void_p(0x10008)), -2),          # rows moved in 16-byte pieces
    (dict(vrs=1028), -2),
    (dict(D=96, bs=8 * 16 * 96, hs=16 * 96, ts=96, krs=768, vrs=768), -2),
    (dict(B=8, Hq=64, bs=8 * 8 * 128, hs=8 * 128, W=256), -2),  # no fused kernel: 8-token blocks, G=8, D=128
])
def test_step_validation(lib, kw, status):
    assert _step(lib, **kw) == status


def test_step_empty_batch_is_a_noop(lib):
    assert _step(lib, S=0) == 0


def test_reduce_validation(lib):
    f = lib.pc_paged_attention_reduce
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 0, 32, 128, 4, 512, 2, None) == 0
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 32, 128, 4, 256, 2, None) == -2
    assert f(None, FAKE, FAKE, FAKE, FAKE, 4, 32, 128, 4, 512, 2, None) == -1
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 32, 128, 4, 512, 9, None) == -1


def test_stream_read_validation(lib):
    f = lib.pc_stream_read
    assert f(None, 1 << 20, FAKE, 64, 0, None) == -1  # no source
    assert f(FAKE, 0, FAKE, 64, 0, None) == -1  # nothing to read
    assert f(FAKE, 1 << 20, FAKE, 0, 0, None) == -1  # no workgroups
    assert f(FAKE, 1 << 20, FAKE, 64, 1, None) == -1  # cache policy is 0 or 2
    assert f(FAKE, (1 << 20) + 8, FAKE, 64, 0, None) == -2  # not whole 16-byte vectors
    assert f(FAKE, 1 << 40, FAKE, 1, 0, None) == -2  # a chunk past 32-bit offsets


def _gather(lib, **kw):
    a = dict(k=FAKE, v=FAKE, nb=64, bs=8 * 16 * 128, ts=128, hs=16 * 128, bt=FAKE, W=4, sl=FAKE, S=2, msl=64, Hkv=8,
             D=128, eb=2, sink=FAKE, pol=0)
    a.update(kw)
    return lib.pc_gather_read(a["k"], a["v"], a["nb"], a["bs"], a["ts"], a["hs"], a["bt"], a["W"], a["sl"], a["S"],
                              a["msl"], a["Hkv"], a["D"], a["eb"], a["sink"], a["pol"], None)


def test_gather_read_validation(lib):
    assert _gather(lib, S=0) == 0 and _gather(lib, msl=0) == 0  # nothing to read: no launch
    assert _gather(lib, eb=3) == -1  # element size 1, 2 or 4
    assert _gather(lib, pol=1) == -1  # cache policy 0 or 2
    assert _gather(lib, msl=65) == -1  # longer than a table row holds
    assert _gather(lib, sink=None) == -1
    assert _gather(lib, nb=0) == -1
    assert _gather(lib, D=96) == -2  # a row of 192 bytes
    assert _gather(lib, ts=127, hs=16 * 127) == -2  # strides not whole 16-byte vectors
    assert _gather(lib, ts=1 << 27) == -2  # a tile past 32-bit offsets


def test_plan_choices():
    bf16 = torch.bfloat16
    # 64 sequences x 8 kv heads = 512 units: enough work units for a single pass
    assert pc.paged_attention_plan(64, 32, 8, 128, 2048, bf16) == (0, 1, 0)
    # 4 sequences x 8 kv heads = 32 units over 32768 tokens: split into 64 partitions
    ps, P, ws = pc.paged_attention_plan(4, 32, 8, 128, 32768, bf16)
    assert (ps, P) == (512, 64) and ws == 4 * 32 * 64 * (128 + 2) * 4
    # a single partition never splits
    assert pc.paged_attention_plan(1, 32, 8, 128, 512, bf16)[0] == 0
    # many MHA units
    assert pc.paged_attention_plan(256, 32, 32, 128, 8192, torch.float16)[0] == 0
    with pytest.raises(pc.PagedCacheError):
        pc.paged_attention_plan(4, 30, 8, 128, 100, bf16)


def test_binding_refuses_host_tensors():
    x = torch.zeros(2, 8, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        pc.reshape_and_cache(x, x, x, x, torch.zeros(2, dtype=torch.int64), num_blocks=1, block_stride=1,
                             token_stride=1, head_stride=1)


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(_native, "_lib", None)
    monkeypatch.setattr(_native, "LIB_PATH", str(tmp_path / "absent.so"))
    with pytest.raises(RuntimeError, match="not built"):
        _native.abi_version()


def prototypes():
    """{name: number of parameters} of every function prototype in include/pc.h."""
    text = open(os.path.join(REPO, "include", "pc.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)  # comments
    out = {}
    for m in re.finditer(r"\b(?:int|const char\s*\*)\s*(pc_[a-z_0-9]+)\s*\(([^)]*)\)\s*;", text):
        params = [p.strip() for p in m.group(2).split(",") if p.strip() and p.strip() != "void"]
        out[m.group(1)] = len(params)
    return out


def test_binding_argtypes_match_the_header(lib):
    """Each prototype's parameter count equals the binding's ctypes argtypes: a signature
    change in the header cannot leave the binding passing the old argument list."""
    protos = prototypes()
    assert set(protos) == set(declared_symbols())
    for name, n in protos.items():
        fn = getattr(lib, name)
        assert fn.argtypes is not None, f"{name}: no argtypes in the binding"
        assert len(fn.argtypes) == n, f"{name}: header {n} parameters, binding {len(fn.argtypes)}"
