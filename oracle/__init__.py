"""CPU oracle for the paged KV-cache write and paged decode attention (fp64).

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` use it.  The product library never imports, links or
calls anything here, and nothing here touches the GPU library.

The arithmetic lives in ``pc_oracle.c`` (plain C loops, double precision); this
module compiles it with gcc when the shared object is missing or older than the
source, and marshals numpy arrays into it.  Storage types are handled as raw bit
patterns (uint32 for fp32, uint16 for fp16/bf16, uint8 for an OCP E4M3 cache).

Parity pins: every function here is pinned by tests that do not reuse its code
(worked examples printed on the pages, closed forms, invariants, numpy and torch
float64 dense attention, a pure-Python brute force); see ``tests/test_oracle_pins.py``.
"""

from __future__ import annotations

import contextlib
import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pc_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_FMT = {"f32": 0, "f16": 1, "bf16": 2}
_lock = threading.Lock()
_lib = None

OK, EINVAL, ERANGE = 0, -1, -2


class OracleError(RuntimeError):
    pass


def build(force: bool = False, src: str = _SRC, out: str = _LIB, defines=()) -> str:
    """Compile the oracle with gcc (strict IEEE double: no fast-math, no contraction)."""
    if force or not os.path.exists(out) or os.path.getmtime(out) < os.path.getmtime(src):
        tmp = out + f".tmp{os.getpid()}"
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-ffp-contract=off",
               *[f"-D{d}" for d in defines], "-o", tmp, src, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, out)
    return out


def _bind(lib):
    i64, i32, f32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_void_p
    lib.oracle_write.restype = i32
    lib.oracle_write.argtypes = [vp, vp, i64, i64, i64, i64, i64, vp, vp, i64, i64, vp, i64, i32, i32, i32, i32]
    lib.oracle_decode.restype = i32
    lib.oracle_decode.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i64, vp, i32, vp, i32, i32, i32, i32, i32,
                                  f32, vp, i32, i32]
    lib.oracle_partials.restype = i32
    lib.oracle_partials.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, vp, i32, vp, i32, i32, i32,
                                    i32, i32, f32, vp, i32, i32, i32, i32]
    lib.oracle_varlen.restype = i32
    lib.oracle_varlen.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i64, vp, i32, vp, vp, i32, i64, i32, i32, i32,
                                  i32, f32, i32, vp, i32, i32]
    lib.oracle_merge.restype = i32
    lib.oracle_merge.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32]
    lib.oracle_write_kv8.restype = i32
    lib.oracle_write_kv8.argtypes = [vp, vp, i64, i64, i64, i64, i64, vp, vp, i64, i64, vp, i64, i32, i32, i32, i32,
                                     vp, vp, i64]
    lib.oracle_decode_kv8.restype = i32
    lib.oracle_decode_kv8.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i64, vp, i32, vp, i32, i32, i32, i32, i32,
                                      f32, vp, i32, vp, vp, i64, i32]
    lib.oracle_partials_kv8.restype = i32
    lib.oracle_partials_kv8.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, vp, i32, vp, i32, i32, i32,
                                        i32, i32, f32, vp, i32, i32, i32, vp, vp, i64, i32]
    lib.oracle_e4m3_decode.restype = None
    lib.oracle_e4m3_decode.argtypes = [vp, vp, i64]
    lib.oracle_e4m3_encode.restype = None
    lib.oracle_e4m3_encode.argtypes = [vp, vp, i64]
    return lib


def load(path: str | None = None):
    """Load (building if needed) the oracle library; ``path`` loads another build."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    with _lock:
        if _lib is None:
            _lib = _bind(ctypes.CDLL(build()))
    return _lib


@contextlib.contextmanager
def using(path: str):
    """Route every call through another build of the oracle (used to check that the
    pins catch planted mistakes); restores the default build afterwards."""
    global _lib
    other = _bind(ctypes.CDLL(path))
    with _lock:
        saved = _lib
        _lib = other
    try:
        yield other
    finally:
        with _lock:
            _lib = saved


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(rc: int, what: str):
    if rc != OK:
        raise OracleError(f"{what} returned {rc} ({'invalid argument' if rc == EINVAL else 'out-of-range data'})")


def _nthreads(n):
    return n if n else (os.cpu_count() or 1)


# ---------------------------------------------------------------------------------
# pool images
# ---------------------------------------------------------------------------------

class Pool:
    """Host image of a paged K/V pool: K and V bases inside one or two bit arrays."""

    def __init__(self, k: np.ndarray, v: np.ndarray, v_offset: int, bound: int):
        self.k, self.v, self.v_offset, self.bound = k, v, v_offset, bound

    def k_ptr(self):
        return self.k.ctypes.data

    def v_ptr(self):
        return self.v.ctypes.data + self.v_offset * self.v.itemsize

    def copy(self) -> "Pool":
        if self.v is self.k:
            k = self.k.copy()
            return Pool(k, k, self.v_offset, self.bound)
        return Pool(self.k.copy(), self.v.copy(), self.v_offset, self.bound)

    def arrays(self):
        return (self.k,) if self.v is self.k else (self.k, self.v)


def empty_pool(wl) -> Pool:
    """The workload's pool filled with its quiet-NaN pattern."""
    k = wl.nan_pool()
    if wl.layout == "combined":
        return Pool(k, k, wl.v_offset, wl.pool_elems - wl.v_offset)
    return Pool(k, wl.nan_pool(), 0, wl.pool_elems)


# ---------------------------------------------------------------------------------
# operations
# ---------------------------------------------------------------------------------

def _scales(wl):
    return (np.ascontiguousarray(wl.k_scale, dtype=np.float32), np.ascontiguousarray(wl.v_scale, dtype=np.float32),
            int(wl.scale_stride))


def _slopes(wl, alibi_slopes):
    """ALiBi slopes (float32, one per query head) passed explicitly, else the workload's, else None."""
    a = alibi_slopes if alibi_slopes is not None else getattr(wl, "alibi_slopes", None)
    if a is None:
        return None
    a = np.ascontiguousarray(a, dtype=np.float32)
    if a.shape != (wl.num_q_heads,):
        raise ValueError("alibi_slopes must hold one float per query head")
    return a


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """Values (float64) of OCP E4M3 codes."""
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(c.shape, dtype=np.float64)
    load().oracle_e4m3_decode(_ptr(out), _ptr(c), c.size)
    return out


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """Nearest OCP E4M3 codes (ties to even, saturating at 448, NaN -> 0xFF) of float32 values."""
    v = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(v.shape, dtype=np.uint8)
    load().oracle_e4m3_encode(_ptr(out), _ptr(v), v.size)
    return out


def write(wl, pool: Pool, key: np.ndarray, value: np.ndarray, slot_mapping: np.ndarray):
    """Scatter ``key``/``value`` rows [T, Hkv, D] into ``pool`` through ``slot_mapping``
    (quantised with the workload's scales when its cache is 8-bit)."""
    lib = load()
    key = np.ascontiguousarray(key)
    value = np.ascontiguousarray(value)
    slots = np.ascontiguousarray(slot_mapping, dtype=np.int64)
    T = int(slots.shape[0])
    row = wl.num_kv_heads * wl.head_size
    if getattr(wl, "fp8", False):
        ks, vs, st = _scales(wl)
        rc = lib.oracle_write_kv8(pool.k_ptr(), pool.v_ptr(), pool.bound, wl.num_blocks, wl.block_stride,
                                  wl.token_stride, wl.head_stride, _ptr(key), _ptr(value), row, row, _ptr(slots), T,
                                  wl.num_kv_heads, wl.head_size, wl.block_size, _FMT[wl.dtype], _ptr(ks), _ptr(vs), st)
        _check(rc, "oracle_write_kv8")
        return pool
    rc = lib.oracle_write(pool.k_ptr(), pool.v_ptr(), pool.bound, wl.num_blocks, wl.block_stride,
                          wl.token_stride, wl.head_stride, _ptr(key), _ptr(value), row, row, _ptr(slots), T,
                          wl.num_kv_heads, wl.head_size, wl.block_size, _FMT[wl.dtype])
    _check(rc, "oracle_write")
    return pool


def filled_pool(wl, step_write: bool = True) -> Pool:
    """NaN pool -> history write (``pre_*``) -> the step's write (``key``/``value``)."""
    pool = empty_pool(wl)
    write(wl, pool, wl.pre_key, wl.pre_value, wl.pre_slots)
    if step_write:
        write(wl, pool, wl.key, wl.value, wl.slot_mapping)
    return pool


def decode(wl, pool: Pool, q: np.ndarray | None = None, seq_lens=None, block_tables=None, scale=None,
           nthreads: int | None = None, alibi_slopes=None) -> np.ndarray:
    """fp64 decode attention, [S, Hq, D] (with ALiBi when the workload or the call gives slopes)."""
    lib = load()
    al = _slopes(wl, alibi_slopes)
    q = np.ascontiguousarray(wl.q if q is None else q)
    sl = np.ascontiguousarray(wl.seq_lens if seq_lens is None else seq_lens, dtype=np.int32)
    bt = np.ascontiguousarray(wl.block_tables if block_tables is None else block_tables, dtype=np.int32)
    S = int(sl.shape[0])
    out = np.zeros((S, wl.num_q_heads, wl.head_size), dtype=np.float64)
    if getattr(wl, "fp8", False):
        ks, vs, st = _scales(wl)
        rc = lib.oracle_decode_kv8(_ptr(out), _ptr(q), pool.k_ptr(), pool.v_ptr(), pool.bound, wl.num_blocks,
                                   wl.block_stride, wl.token_stride, wl.head_stride, _ptr(bt), int(bt.shape[1]),
                                   _ptr(sl), S, wl.num_q_heads, wl.num_kv_heads, wl.head_size, wl.block_size,
                                   float(wl.scale if scale is None else scale), _ptr(al), _FMT[wl.dtype], _ptr(ks),
                                   _ptr(vs), st, _nthreads(nthreads))
        _check(rc, "oracle_decode_kv8")
        return out
    rc = lib.oracle_decode(_ptr(out), _ptr(q), pool.k_ptr(), pool.v_ptr(), pool.bound, wl.num_blocks,
                           wl.block_stride, wl.token_stride, wl.head_stride, _ptr(bt), int(bt.shape[1]), _ptr(sl), S,
                           wl.num_q_heads, wl.num_kv_heads, wl.head_size, wl.block_size,
                           float(wl.scale if scale is None else scale), _ptr(al), _FMT[wl.dtype],
                           _nthreads(nthreads))
    _check(rc, "oracle_decode")
    return out


def partials(wl, pool: Pool, partition_size: int, max_partitions: int | None = None, q=None, seq_lens=None,
             block_tables=None, nthreads: int | None = None, fill: float = np.nan, alibi_slopes=None):
    """Per-partition (tmp_out [S,Hq,P,D], max_logits [S,Hq,P], exp_sums [S,Hq,P]); slots of
    partitions that hold no token keep ``fill``."""
    lib = load()
    al = _slopes(wl, alibi_slopes)
    q = np.ascontiguousarray(wl.q if q is None else q)
    sl = np.ascontiguousarray(wl.seq_lens if seq_lens is None else seq_lens, dtype=np.int32)
    bt = np.ascontiguousarray(wl.block_tables if block_tables is None else block_tables, dtype=np.int32)
    S = int(sl.shape[0])
    if max_partitions is None:
        max_partitions = max(1, -(-int(sl.max()) // partition_size)) if S else 1
    H, D = wl.num_q_heads, wl.head_size
    tmp = np.full((S, H, max_partitions, D), fill, dtype=np.float64)
    ml = np.full((S, H, max_partitions), fill, dtype=np.float64)
    es = np.full((S, H, max_partitions), fill, dtype=np.float64)
    if getattr(wl, "fp8", False):
        ks, vs, st = _scales(wl)
        rc = lib.oracle_partials_kv8(_ptr(tmp), _ptr(ml), _ptr(es), _ptr(q), pool.k_ptr(), pool.v_ptr(), pool.bound,
                                     wl.num_blocks, wl.block_stride, wl.token_stride, wl.head_stride, _ptr(bt),
                                     int(bt.shape[1]), _ptr(sl), S, H, wl.num_kv_heads, D, wl.block_size,
                                     float(wl.scale), _ptr(al), partition_size, max_partitions, _FMT[wl.dtype],
                                     _ptr(ks), _ptr(vs), st, _nthreads(nthreads))
        _check(rc, "oracle_partials_kv8")
        return tmp, ml, es
    rc = lib.oracle_partials(_ptr(tmp), _ptr(ml), _ptr(es), _ptr(q), pool.k_ptr(), pool.v_ptr(), pool.bound,
                             wl.num_blocks, wl.block_stride, wl.token_stride, wl.head_stride, _ptr(bt),
                             int(bt.shape[1]), _ptr(sl), S, H, wl.num_kv_heads, D, wl.block_size, float(wl.scale),
                             _ptr(al), partition_size, max_partitions, _FMT[wl.dtype], _nthreads(nthreads))
    _check(rc, "oracle_partials")
    return tmp, ml, es


def varlen(wl, pool: Pool, vq, q=None, causal=None, alibi_slopes=None, seq_lens=None, query_start_loc=None,
           nthreads: int | None = None) -> np.ndarray:
    """fp64 attention of the packed multi-token queries of ``vq`` (a VarlenStep) over
    the pool, [total_q, Hq, D]."""
    lib = load()
    q = np.ascontiguousarray(vq.q if q is None else q)
    qs = np.ascontiguousarray(vq.query_start_loc if query_start_loc is None else query_start_loc, dtype=np.int32)
    sl = np.ascontiguousarray(wl.seq_lens if seq_lens is None else seq_lens, dtype=np.int32)
    bt = np.ascontiguousarray(wl.block_tables, dtype=np.int32)
    al = _slopes(wl, alibi_slopes)
    total = int(qs[-1])
    out = np.zeros((total, wl.num_q_heads, wl.head_size), dtype=np.float64)
    rc = lib.oracle_varlen(_ptr(out), _ptr(q), pool.k_ptr(), pool.v_ptr(), pool.bound, wl.num_blocks,
                           wl.block_stride, wl.token_stride, wl.head_stride, _ptr(bt), int(bt.shape[1]), _ptr(qs),
                           _ptr(sl), int(sl.shape[0]), total, wl.num_q_heads, wl.num_kv_heads, wl.head_size,
                           wl.block_size, float(wl.scale), int(vq.causal if causal is None else causal), _ptr(al),
                           _FMT[wl.dtype], _nthreads(nthreads))
    _check(rc, "oracle_varlen")
    return out


def merge(tmp_out: np.ndarray, max_logits: np.ndarray, exp_sums: np.ndarray, seq_lens,
          partition_size: int) -> np.ndarray:
    """Log-sum-exp merge of partials (fp64 in, fp64 out)."""
    lib = load()
    tmp = np.ascontiguousarray(tmp_out, dtype=np.float64)
    ml = np.ascontiguousarray(max_logits, dtype=np.float64)
    es = np.ascontiguousarray(exp_sums, dtype=np.float64)
    sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
    S, H, P, D = tmp.shape
    out = np.zeros((S, H, D), dtype=np.float64)
    rc = lib.oracle_merge(_ptr(out), _ptr(tmp), _ptr(ml), _ptr(es), _ptr(sl), S, H, D, P, partition_size)
    _check(rc, "oracle_merge")
    return out
