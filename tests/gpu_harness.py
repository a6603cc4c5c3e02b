"""Drive a workload through the HIP library (GPU) and read the results back.

Inputs are the generator's seeded arrays; device memory comes from torch.  Every
step of the path -- the history write, the step's write, the decode and the reduce
-- runs in ``libpcache.so`` through the package's binding.
"""

from __future__ import annotations

import numpy as np
import torch

import paged_kv_cache_reshape_amd as pc
from workloads import nan_bits

TORCH_DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
INT_VIEW = {"f32": (np.int32, torch.int32), "f16": (np.int16, torch.int16), "bf16": (np.int16, torch.int16)}


def to_dev(bits: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    """Storage bit patterns (numpy) -> a device tensor of the storage dtype."""
    npi, _ = INT_VIEW[dtype]
    t = torch.from_numpy(np.ascontiguousarray(bits).view(npi)).to(device)
    return t.view(TORCH_DT[dtype])


def to_bits(t: torch.Tensor, dtype: str) -> np.ndarray:
    npi, ti = INT_VIEW[dtype]
    u = np.uint32 if dtype == "f32" else np.uint16
    return t.contiguous().view(ti).cpu().numpy().view(u)


class DevicePool:
    """The workload's pool in device memory, filled with its quiet-NaN pattern (an
    8-bit cache: uint8 codes, NaN 0x7F, plus its per-head scales on the device)."""

    def __init__(self, wl, device="cuda"):
        self.wl = wl
        self.fp8 = bool(getattr(wl, "fp8", False))
        if self.fp8:
            def make():
                return torch.full((wl.pool_elems,), 0x7F, dtype=torch.uint8, device=device)

            self.k_scale = torch.from_numpy(np.ascontiguousarray(wl.k_scale, np.float32)).to(device)
            self.v_scale = torch.from_numpy(np.ascontiguousarray(wl.v_scale, np.float32)).to(device)
        else:
            _, ti = INT_VIEW[wl.dtype]
            fill = nan_bits(wl.dtype)  # 0x7FC00000 / 0x7E00 / 0x7FC0: positive in the signed view

            def make():
                return torch.full((wl.pool_elems,), fill, dtype=ti, device=device).view(TORCH_DT[wl.dtype])

        self.k = make()
        self.v = self.k if wl.layout == "combined" else make()
        self.v_offset = wl.v_offset if wl.layout == "combined" else 0

    def layout_kwargs(self):
        w = self.wl
        return dict(num_blocks=w.num_blocks, block_stride=w.block_stride, token_stride=w.token_stride,
                    head_stride=w.head_stride, block_size=w.block_size, v_offset=self.v_offset)

    def arrays(self):
        return (self.k,) if self.v is self.k else (self.k, self.v)

    def scale_kwargs(self):
        return dict(kv_scale_stride=int(self.wl.scale_stride)) if self.fp8 else {}

    def bits(self):
        """Host copies of the pool buffers as stored bits (uint8 codes for an 8-bit cache)."""
        torch.cuda.synchronize()
        if self.fp8:
            return [a.cpu().numpy() for a in self.arrays()]
        return [to_bits(a, self.wl.dtype) for a in self.arrays()]


def write(pool: DevicePool, key_bits, value_bits, slots, chunk: int = 1 << 16):
    """pc_reshape_and_cache of host rows, uploaded in chunks of ``chunk`` tokens."""
    wl = pool.wl
    T = len(slots)
    for t0 in range(0, T, chunk):
        t1 = min(T, t0 + chunk)
        key = to_dev(key_bits[t0:t1], wl.dtype)
        value = to_dev(value_bits[t0:t1], wl.dtype)
        sm = torch.from_numpy(np.ascontiguousarray(slots[t0:t1], dtype=np.int64)).cuda()
        if pool.fp8:
            pc.reshape_and_cache_fp8(key, value, pool.k, pool.v, sm, pool.k_scale, pool.v_scale,
                                     **pool.layout_kwargs(), **pool.scale_kwargs())
        else:
            pc.reshape_and_cache(key, value, pool.k, pool.v, sm, **pool.layout_kwargs())


def filled_pool(wl, step_write: bool = True) -> DevicePool:
    pool = DevicePool(wl)
    write(pool, wl.pre_key, wl.pre_value, wl.pre_slots)
    if step_write:
        write(pool, wl.key, wl.value, wl.slot_mapping)
    torch.cuda.synchronize()
    return pool


class DecodeInputs:
    def __init__(self, wl, q_bits=None, seq_lens=None, block_tables=None):
        self.wl = wl
        self.q = to_dev(wl.q if q_bits is None else q_bits, wl.dtype)
        sl = wl.seq_lens if seq_lens is None else seq_lens
        bt = wl.block_tables if block_tables is None else block_tables
        self.seq_lens_host = np.asarray(sl, np.int32)
        self.seq_lens = torch.from_numpy(np.ascontiguousarray(sl, dtype=np.int32)).cuda()
        self.block_tables = torch.from_numpy(np.ascontiguousarray(bt, dtype=np.int32)).cuda()
        self.max_seq_len = int(self.seq_lens_host.max()) if len(self.seq_lens_host) else 0
        al = getattr(wl, "alibi_slopes", None)
        self.alibi = None if al is None else torch.from_numpy(np.ascontiguousarray(al, np.float32)).cuda()


def decode(pool: DevicePool, inp: DecodeInputs, path: str = "plan", max_seq_len: int | None = None):
    """Run the decode; ``path`` is 'single', 'split' or 'plan'.  Returns (out tensor, path used)."""
    wl = pool.wl
    S, Hq, D = inp.q.shape
    msl = inp.max_seq_len if max_seq_len is None else max_seq_len
    if path == "plan":
        shared = wl.shared_lens() if max_seq_len is None and np.array_equal(inp.seq_lens_host, wl.seq_lens) else None
        ps, _, _ = pc.paged_attention_plan_lens(inp.seq_lens_host, Hq, wl.num_kv_heads, D, wl.head_stride,
                                                TORCH_DT[wl.dtype], kv_fp8=pool.fp8, shared_lens=shared)
        path = "split" if ps else "single"
    out = torch.empty_like(inp.q)
    if path == "single":
        decode_call(pool, inp, out, msl)
        return out, path
    es, ml, tmp = partials_call(pool, inp, msl)
    pc.paged_attention_reduce(out, es, ml, tmp, inp.seq_lens)
    return out, path


def decode_call(pool: DevicePool, inp: DecodeInputs, out, msl: int, **kw):
    """One pc_paged_attention_decode(_fp8) call on the pool (``kw``: split-path partials)."""
    wl = pool.wl
    common = dict(num_kv_heads=wl.num_kv_heads, scale=float(wl.scale), alibi_slopes=inp.alibi,
                  **pool.layout_kwargs(), **kw)
    if pool.fp8:
        pc.paged_attention_decode_fp8(out, inp.q, pool.k, pool.v, inp.block_tables, inp.seq_lens, msl, pool.k_scale,
                                      pool.v_scale, **pool.scale_kwargs(), **common)
    else:
        pc.paged_attention_decode(out, inp.q, pool.k, pool.v, inp.block_tables, inp.seq_lens, msl, **common)


def partials_call(pool: DevicePool, inp: DecodeInputs, msl: int):
    """The split path's decode: (exp_sums, max_logits, tmp_out), NaN where unwritten."""
    S, Hq, D = inp.q.shape
    P = max(1, -(-msl // pc.PARTITION_SIZE))
    es = torch.full((S, Hq, P), float("nan"), device="cuda")
    ml = torch.full((S, Hq, P), float("nan"), device="cuda")
    tmp = torch.full((S, Hq, P, D), float("nan"), device="cuda")
    decode_call(pool, inp, None, msl, partition_size=pc.PARTITION_SIZE, exp_sums=es, max_logits=ml, tmp_out=tmp)
    return es, ml, tmp


def out_f64(out: torch.Tensor) -> np.ndarray:
    return out.double().cpu().numpy()


def varlen(pool: DevicePool, vq, wl=None, q_bits=None, causal=None, max_query_len=None, seq_lens=None,
           block_tables=None):
    """pc_paged_attention_varlen of a VarlenStep's packed queries; returns out [total_q, Hq, D]."""
    wl = pool.wl if wl is None else wl
    q = to_dev(vq.q if q_bits is None else q_bits, wl.dtype)
    out = torch.full_like(q, float("nan"))
    qs = torch.from_numpy(np.ascontiguousarray(vq.query_start_loc, np.int32)).cuda()
    sl = torch.from_numpy(np.ascontiguousarray(wl.seq_lens if seq_lens is None else seq_lens, np.int32)).cuda()
    bt = torch.from_numpy(np.ascontiguousarray(wl.block_tables if block_tables is None else block_tables,
                                               np.int32)).cuda()
    al = getattr(wl, "alibi_slopes", None)
    al = None if al is None else torch.from_numpy(np.ascontiguousarray(al, np.float32)).cuda()
    pc.paged_attention_varlen(out, q, pool.k, pool.v, bt, qs, sl,
                              vq.max_query_len if max_query_len is None else max_query_len,
                              num_kv_heads=wl.num_kv_heads, scale=float(wl.scale),
                              causal=vq.causal if causal is None else causal, alibi_slopes=al,
                              **pool.layout_kwargs())
    torch.cuda.synchronize()
    return out
