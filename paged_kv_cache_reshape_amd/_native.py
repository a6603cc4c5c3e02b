"""ctypes binding of ``libpcache.so`` (the C ABI in ``include/pc.h``).

Argument marshalling only: torch tensors are reduced to device pointers, sizes and
the current HIP stream, and every step runs in the library's kernels.  There is
no CPU fallback -- a missing library raises at import of this module's functions.
"""

from __future__ import annotations

import ctypes
import os

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libpcache.so")

PC_OK, PC_ERR_INVALID_ARG, PC_ERR_UNSUPPORTED, PC_ERR_LAUNCH, PC_ERR_TOO_LARGE = 0, -1, -2, -3, -4
NOALLOC_SCRATCH_BYTES = 128 << 20  # PC_NOALLOC_SCRATCH_BYTES
PARTITION_SIZE = 512
_DTYPES = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}
_lib = None


class PagedCacheError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: status {status} ({status_string(status)})")


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"HIP library not built: {LIB_PATH} is missing (run __graft_entry__.build() or "
                               "python -m paged_kv_cache_reshape_amd.build)")
        lib = ctypes.CDLL(LIB_PATH)
        i64, i32, f32, vp, sz = ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t
        lib.pc_abi_version.restype = i32
        lib.pc_abi_version.argtypes = []
        lib.pc_status_string.restype = ctypes.c_char_p
        lib.pc_status_string.argtypes = [i32]
        lib.pc_reshape_and_cache.restype = i32
        lib.pc_reshape_and_cache.argtypes = [vp, vp, i64, i64, vp, vp, i64, i64, i64, i64, vp, i64, i32, i32, i32,
                                             i32, vp]
        lib.pc_paged_attention_decode.restype = i32
        lib.pc_paged_attention_decode.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, vp, i32, vp, i32, i32, i32,
                                                  i32, i32, i32, f32, i32, vp, vp, vp, vp, i32, vp]
        lib.pc_reshape_and_cache_fp8.restype = i32
        lib.pc_reshape_and_cache_fp8.argtypes = [vp, vp, i64, i64, vp, vp, i64, i64, i64, i64, vp, i64, i32, i32,
                                                 i32, vp, vp, i64, i32, vp]
        lib.pc_paged_attention_decode_fp8.restype = i32
        lib.pc_paged_attention_decode_fp8.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, vp, i32, vp, i32, i32,
                                                      i32, i32, i32, i32, f32, i32, vp, vp, vp, vp, vp, vp, i64,
                                                      i32, vp]
        lib.pc_paged_attention_varlen.restype = i32
        lib.pc_paged_attention_varlen.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, vp, i32, vp, vp, i32, i64, i32,
                                                  i32, i32, i32, i32, f32, i32, vp, i32, vp]
        lib.pc_reshape_and_cache_decode.restype = i32
        lib.pc_reshape_and_cache_decode.argtypes = [vp, vp, vp, vp, i64, i64, vp, vp, vp, i64, i64, i64, i64, vp,
                                                    i32, vp, i32, i32, i32, i32, i32, i32, f32, i32, vp, vp, vp,
                                                    vp, i32, vp]
        lib.pc_paged_attention_reduce.restype = i32
        lib.pc_paged_attention_reduce.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, vp]
        lib.pc_paged_attention_plan.restype = i32
        lib.pc_paged_attention_plan.argtypes = [i32, i32, i32, i32, i32, i32, ctypes.POINTER(i32),
                                                ctypes.POINTER(i32), ctypes.POINTER(sz)]
        lib.pc_paged_attention_plan_lens.restype = i32
        lib.pc_paged_attention_plan_lens.argtypes = [vp, vp, i32, i32, i32, i32, i64, i32, i32, ctypes.POINTER(i32),
                                                     ctypes.POINTER(i32), ctypes.POINTER(sz)]
        lib.pc_paged_attention_decode_prefix.restype = i32
        lib.pc_paged_attention_decode_prefix.argtypes = [vp, vp, vp, i64, i64, i64, i64, vp, i32, vp, i32, i32, i32,
                                                         i32, i32, i32, f32, vp, vp, vp, vp, vp, i32, vp, i32, vp]
        lib.pc_paged_attention_split_noalloc.restype = i32
        lib.pc_paged_attention_split_noalloc.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, vp, i32, vp, i32, i32,
                                                         i32, i32, i32, i32, f32, vp, i32, vp]
        lib.pc_stream_read.restype = i32
        lib.pc_stream_read.argtypes = [vp, i64, vp, i32, i32, vp]
        lib.pc_gather_read.restype = i32
        lib.pc_gather_read.argtypes = [vp, vp, i64, i64, i64, i64, vp, i32, vp, i32, i32, i32, i32, i32, vp, i32, vp]
        _lib = lib
    return _lib


def library():
    """The loaded ``ctypes.CDLL`` (raises if the library has not been built)."""
    return _load()


def abi_version() -> int:
    return _load().pc_abi_version()


def status_string(status: int) -> str:
    return _load().pc_status_string(status).decode()


def _check(fn: str, status: int):
    if status != PC_OK:
        raise PagedCacheError(fn, status)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype not in _DTYPES:
        raise TypeError(f"unsupported storage dtype {t.dtype}")
    return _DTYPES[t.dtype]


def _ptr(t, elem_offset: int = 0):
    if t is None:
        return None
    return t.data_ptr() + elem_offset * t.element_size()


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(t: torch.Tensor, stream):
    if stream is not None:
        return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    if _raw_stream is not None:  # the current stream's handle without building a Stream object
        return _raw_stream(t.device.index)
    return torch.cuda.current_stream(t.device).cuda_stream


def _same_device(*ts):
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("every tensor must live on the GPU")
        dev = dev or t.device
        if t.device != dev:
            raise ValueError("tensors on different devices")


def _pool_extent(num_blocks: int, block_stride: int, token_stride: int, head_stride: int, block_size: int,
                 num_kv_heads: int, head_size: int) -> int:
    """Elements a pool buffer must hold past its base: one past the largest element index
    the strides can reach (block num_blocks-1, row block_size-1, head num_kv_heads-1)."""
    return ((num_blocks - 1) * block_stride + (block_size - 1) * token_stride + (num_kv_heads - 1) * head_stride +
            head_size)


def _check_pool(k_pool, v_pool, v_offset: int, num_blocks: int, block_stride: int, token_stride: int,
                head_stride: int, block_size: int, num_kv_heads: int, head_size: int):
    """The pool buffers cover every element the layout can address, so no slot or block id
    the kernels accept can reach past them."""
    if num_blocks <= 0 or block_stride <= 0 or token_stride <= 0 or head_stride <= 0 or block_size <= 0:
        raise ValueError("num_blocks, the strides and block_size must be positive")
    if v_offset < 0:
        raise ValueError("v_offset must be non-negative")
    need = _pool_extent(num_blocks, block_stride, token_stride, head_stride, block_size, num_kv_heads, head_size)
    for t, off, nm in ((k_pool, 0, "k_pool"), (v_pool, v_offset, "v_pool")):
        if not t.is_contiguous():
            raise ValueError(f"{nm} must be contiguous")
        if t.numel() - off < need:
            raise ValueError(f"{nm} holds {t.numel() - off} elements past its base but the layout addresses {need}")


def _check_seq_inputs(S: int, block_tables, seq_lens):
    # (max_seq_len against the table width is the library's own check)
    if block_tables.shape[0] != S:
        raise ValueError(f"block_tables has {block_tables.shape[0]} rows for {S} sequences")
    if seq_lens.numel() != S:
        raise ValueError(f"seq_lens has {seq_lens.numel()} entries for {S} sequences")


def _check_partials(S: int, Hq: int, D: int, max_seq_len: int, partition_size: int, exp_sums, max_logits,
                    tmp_out):
    if partition_size == 0:
        if exp_sums is not None or max_logits is not None or tmp_out is not None:
            raise ValueError("the one-pass path takes no partials")
        return
    if exp_sums is None or max_logits is None or tmp_out is None:
        raise ValueError("the split path needs exp_sums, max_logits and tmp_out")
    # the decode lays partials out with P = ceil(max_seq_len / partition_size) per row and the
    # reduce reads them with tmp_out's P, so the two must agree (with max_seq_len 0 nothing
    # is written or read)
    P = -(-max_seq_len // partition_size) if partition_size > 0 else 0
    P = tmp_out.shape[2] if P == 0 and tmp_out.dim() == 4 else P
    if tuple(exp_sums.shape) != (S, Hq, P) or tuple(max_logits.shape) != (S, Hq, P) or \
            tuple(tmp_out.shape) != (S, Hq, P, D):
        raise ValueError(f"partials must be [S, Hq, P] and [S, Hq, P, D] with P = ceil(max_seq_len / "
                         f"partition_size) = {P}")


def reshape_and_cache(key: torch.Tensor, value: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                      slot_mapping: torch.Tensor, *, num_blocks: int, block_stride: int, token_stride: int,
                      head_stride: int, block_size: int = 16, v_offset: int = 0, stream=None) -> None:
    """Scatter ``key``/``value`` [T, Hkv, D] into the pool through ``slot_mapping`` (int64 [T]).
    ``v_offset`` places V that many elements past ``v_pool``'s start (one-buffer layouts)."""
    _same_device(key, value, k_pool, v_pool, slot_mapping)
    if key.dim() != 3 or value.shape != key.shape or key.stride(2) != 1 or value.stride(2) != 1 or \
            key.stride(1) != key.shape[2] or value.stride(1) != value.shape[2]:
        raise ValueError("key/value must be [T, Hkv, D] with contiguous rows")
    if slot_mapping.dtype != torch.int64 or not slot_mapping.is_contiguous() or slot_mapping.numel() != key.shape[0]:
        raise ValueError("slot_mapping must be a contiguous int64 [T]")
    dt = _dtype_code(key)
    for t in (value, k_pool, v_pool):
        if _DTYPES.get(t.dtype) != dt:
            raise TypeError("key, value and the pool must share one storage dtype")
    T, Hkv, D = key.shape
    _check_pool(k_pool, v_pool, v_offset, num_blocks, block_stride, token_stride, head_stride, block_size, Hkv, D)
    st = _load().pc_reshape_and_cache(_ptr(key), _ptr(value), key.stride(0), value.stride(0), _ptr(k_pool),
                                      _ptr(v_pool, v_offset), num_blocks, block_stride, token_stride, head_stride,
                                      _ptr(slot_mapping), T, Hkv, D, block_size, dt, _stream(key, stream))
    _check("pc_reshape_and_cache", st)


def paged_attention_decode(out, q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                           block_tables: torch.Tensor, seq_lens: torch.Tensor, max_seq_len: int, *,
                           num_kv_heads: int, scale: float, num_blocks: int, block_stride: int, token_stride: int,
                           head_stride: int, block_size: int = 16, v_offset: int = 0, partition_size: int = 0,
                           exp_sums=None, max_logits=None, tmp_out=None, alibi_slopes=None, stream=None) -> None:
    """Decode attention of ``q`` [S, Hq, D] over the paged pool.  ``partition_size`` 0 writes
    ``out``; 512 writes only the partials (``exp_sums``, ``max_logits`` [S, Hq, P], ``tmp_out``
    [S, Hq, P, D], fp32).  ``alibi_slopes``: optional fp32 [Hq] ALiBi slopes."""
    _same_device(out, q, k_pool, v_pool, block_tables, seq_lens, exp_sums, max_logits, tmp_out, alibi_slopes)
    _check_alibi(alibi_slopes, q)
    if q.dim() != 3 or not q.is_contiguous():
        raise ValueError("q must be a contiguous [S, Hq, D]")
    if out is not None and (out.shape != q.shape or not out.is_contiguous() or out.dtype != q.dtype):
        raise ValueError("out must be a contiguous tensor shaped and typed like q")
    if block_tables.dtype != torch.int32 or block_tables.dim() != 2 or not block_tables.is_contiguous():
        raise ValueError("block_tables must be a contiguous int32 [S, W]")
    if seq_lens.dtype != torch.int32 or not seq_lens.is_contiguous():
        raise ValueError("seq_lens must be a contiguous int32 [S]")
    for t in (exp_sums, max_logits, tmp_out):
        if t is not None and (t.dtype != torch.float32 or not t.is_contiguous()):
            raise ValueError("partials must be contiguous float32")
    dt = _dtype_code(q)
    if _DTYPES.get(k_pool.dtype) != dt or _DTYPES.get(v_pool.dtype) != dt:
        raise TypeError("q and the pool must share one storage dtype")
    S, Hq, D = q.shape
    _check_seq_inputs(S, block_tables, seq_lens)
    _check_partials(S, Hq, D, max_seq_len, partition_size, exp_sums, max_logits, tmp_out)
    _check_pool(k_pool, v_pool, v_offset, num_blocks, block_stride, token_stride, head_stride, block_size,
                num_kv_heads, D)
    st = _load().pc_paged_attention_decode(
        _ptr(out), _ptr(q), _ptr(k_pool), _ptr(v_pool, v_offset), num_blocks, block_stride, token_stride,
        head_stride, _ptr(block_tables), block_tables.shape[1], _ptr(seq_lens), S, max_seq_len, Hq, num_kv_heads,
        D, block_size, scale, partition_size, _ptr(exp_sums), _ptr(max_logits), _ptr(tmp_out), _ptr(alibi_slopes),
        dt, _stream(q, stream))
    _check("pc_paged_attention_decode", st)


def paged_attention_decode_prefix(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                                  block_tables: torch.Tensor, seq_lens: torch.Tensor, max_seq_len: int, *,
                                  num_kv_heads: int, scale: float, num_blocks: int, block_stride: int,
                                  token_stride: int, head_stride: int, exp_sums, max_logits, tmp_out,
                                  prefix_table, shared_lens, block_size: int = 16, v_offset: int = 0,
                                  alibi_slopes=None, stream=None) -> None:
    """The split path's partials for sequences sharing a prefix (pc_paged_attention_decode_prefix):
    ``prefix_table`` int32 [prefix_blocks] the shared blocks, ``shared_lens`` int32 [S] each
    sequence's tokens in them.  Follow with paged_attention_reduce."""
    _same_device(q, k_pool, v_pool, block_tables, seq_lens, exp_sums, max_logits, tmp_out, alibi_slopes,
                 prefix_table, shared_lens)
    _check_alibi(alibi_slopes, q)
    if q.dim() != 3 or not q.is_contiguous():
        raise ValueError("q must be a contiguous [S, Hq, D]")
    if block_tables.dtype != torch.int32 or block_tables.dim() != 2 or not block_tables.is_contiguous():
        raise ValueError("block_tables must be a contiguous int32 [S, W]")
    if seq_lens.dtype != torch.int32 or not seq_lens.is_contiguous():
        raise ValueError("seq_lens must be a contiguous int32 [S]")
    for t in (exp_sums, max_logits, tmp_out):
        if t is None or t.dtype != torch.float32 or not t.is_contiguous():
            raise ValueError("partials must be contiguous float32")
    dt = _dtype_code(q)
    if _DTYPES.get(k_pool.dtype) != dt or _DTYPES.get(v_pool.dtype) != dt:
        raise TypeError("q and the pool must share one storage dtype")
    S, Hq, D = q.shape
    if prefix_table.dtype != torch.int32 or prefix_table.dim() != 1 or not prefix_table.is_contiguous():
        raise ValueError("prefix_table must be a contiguous int32 [prefix_blocks]")
    if shared_lens.dtype != torch.int32 or not shared_lens.is_contiguous() or shared_lens.numel() != S:
        raise ValueError("shared_lens must be a contiguous int32 [S]")
    _check_seq_inputs(S, block_tables, seq_lens)
    _check_partials(S, Hq, D, max_seq_len, PARTITION_SIZE, exp_sums, max_logits, tmp_out)
    _check_pool(k_pool, v_pool, v_offset, num_blocks, block_stride, token_stride, head_stride, block_size,
                num_kv_heads, D)
    st = _load().pc_paged_attention_decode_prefix(
        _ptr(q), _ptr(k_pool), _ptr(v_pool, v_offset), num_blocks, block_stride, token_stride, head_stride,
        _ptr(block_tables), block_tables.shape[1], _ptr(seq_lens), S, max_seq_len, Hq, num_kv_heads, D, block_size,
        scale, _ptr(exp_sums), _ptr(max_logits), _ptr(tmp_out), _ptr(alibi_slopes), _ptr(prefix_table),
        prefix_table.numel(), _ptr(shared_lens), dt, _stream(q, stream))
    _check("pc_paged_attention_decode_prefix", st)


def paged_attention_split_noalloc(out: torch.Tensor, q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                                  block_tables: torch.Tensor, seq_lens: torch.Tensor, max_seq_len: int, *,
                                  num_kv_heads: int, scale: float, num_blocks: int, block_stride: int,
                                  token_stride: int, head_stride: int, block_size: int = 16, v_offset: int = 0,
                                  alibi_slopes=None, stream=None) -> None:
    """The split decode and its reduce into ``out`` [S, Hq, D] with the partials in the
    library's own device buffer (pc_paged_attention_split_noalloc): allocates nothing.
    Keyword arguments as for paged_attention_decode."""
    _same_device(out, q, k_pool, v_pool, block_tables, seq_lens, alibi_slopes)
    _check_alibi(alibi_slopes, q)
    if q.dim() != 3 or not q.is_contiguous():
        raise ValueError("q must be a contiguous [S, Hq, D]")
    if out is None or out.shape != q.shape or not out.is_contiguous() or out.dtype != q.dtype:
        raise ValueError("out must be a contiguous tensor shaped and typed like q")
    if block_tables.dtype != torch.int32 or block_tables.dim() != 2 or not block_tables.is_contiguous():
        raise ValueError("block_tables must be a contiguous int32 [S, W]")
    if seq_lens.dtype != torch.int32 or not seq_lens.is_contiguous():
        raise ValueError("seq_lens must be a contiguous int32 [S]")
    dt = _dtype_code(q)
    if _DTYPES.get(k_pool.dtype) != dt or _DTYPES.get(v_pool.dtype) != dt:
        raise TypeError("q and the pool must share one storage dtype")
    S, Hq, D = q.shape
    _check_seq_inputs(S, block_tables, seq_lens)
    _check_pool(k_pool, v_pool, v_offset, num_blocks, block_stride, token_stride, head_stride, block_size,
                num_kv_heads, D)
    st = _load().pc_paged_attention_split_noalloc(
        _ptr(out), _ptr(q), _ptr(k_pool), _ptr(v_pool, v_offset), num_blocks, block_stride, token_stride,
        head_stride, _ptr(block_tables), block_tables.shape[1], _ptr(seq_lens), S, max_seq_len, Hq, num_kv_heads,
        D, block_size, scale, _ptr(alibi_slopes), dt, _stream(q, stream))
    _check("pc_paged_attention_split_noalloc", st)


def reshape_and_cache_decode(out, q: torch.Tensor, key: torch.Tensor, value: torch.Tensor, k_pool: torch.Tensor,
                             v_pool: torch.Tensor, slot_mapping: torch.Tensor, block_tables: torch.Tensor,
                             seq_lens: torch.Tensor, max_seq_len: int, *, num_kv_heads: int, scale: float,
                             num_blocks: int, block_stride: int, token_stride: int, head_stride: int,
                             block_size: int = 16, v_offset: int = 0, partition_size: int = 0, exp_sums=None,
                             max_logits=None, tmp_out=None, alibi_slopes=None, stream=None) -> None:
    """One decode step in one launch: ``key``/``value`` [S, Hkv, D] of each sequence's newest
    token go to ``slot_mapping`` (int64 [S], the slot of position seq_len - 1, or outside the
    pool), then the decode of ``q`` [S, Hq, D] -- as reshape_and_cache followed by
    paged_attention_decode (same keyword arguments).  fp16 / bf16 only."""
    _same_device(out, q, key, value, k_pool, v_pool, slot_mapping, block_tables, seq_lens, exp_sums, max_logits,
                 tmp_out, alibi_slopes)
    _check_alibi(alibi_slopes, q)
    if q.dim() != 3 or not q.is_contiguous():
        raise ValueError("q must be a contiguous [S, Hq, D]")
    if out is not None and (out.shape != q.shape or not out.is_contiguous() or out.dtype != q.dtype):
        raise ValueError("out must be a contiguous tensor shaped and typed like q")
    S, Hq, D = q.shape
    if key.dim() != 3 or value.shape != key.shape or key.shape[0] != S or key.stride(2) != 1 or \
            value.stride(2) != 1 or key.stride(1) != key.shape[2] or value.stride(1) != value.shape[2]:
        raise ValueError("key/value must be [S, Hkv, D] with contiguous rows, one token per sequence")
    if slot_mapping.dtype != torch.int64 or not slot_mapping.is_contiguous() or slot_mapping.numel() != S:
        raise ValueError("slot_mapping must be a contiguous int64 [S]")
    if block_tables.dtype != torch.int32 or block_tables.dim() != 2 or not block_tables.is_contiguous():
        raise ValueError("block_tables must be a contiguous int32 [S, W]")
    if seq_lens.dtype != torch.int32 or not seq_lens.is_contiguous():
        raise ValueError("seq_lens must be a contiguous int32 [S]")
    for t in (exp_sums, max_logits, tmp_out):
        if t is not None and (t.dtype != torch.float32 or not t.is_contiguous()):
            raise ValueError("partials must be contiguous float32")
    dt = _dtype_code(q)
    for t in (key, value, k_pool, v_pool):
        if _DTYPES.get(t.dtype) != dt:
            raise TypeError("q, key, value and the pool must share one storage dtype")
    if key.shape[1] != num_kv_heads or key.shape[2] != D:
        raise ValueError("key/value rows must hold num_kv_heads x head_size elements")
    _check_seq_inputs(S, block_tables, seq_lens)
    _check_partials(S, Hq, D, max_seq_len, partition_size, exp_sums, max_logits, tmp_out)
    _check_pool(k_pool, v_pool, v_offset, num_blocks, block_stride, token_stride, head_stride, block_size,
                num_kv_heads, D)
    st = _load().pc_reshape_and_cache_decode(
        _ptr(out), _ptr(q), _ptr(key), _ptr(value), key.stride(0), value.stride(0), _ptr(slot_mapping), _ptr(k_pool),
        _ptr(v_pool, v_offset), num_blocks, block_stride, token_stride, head_stride, _ptr(block_tables),
        block_tables.shape[1], _ptr(seq_lens), S, max_seq_len, Hq, num_kv_heads, D, block_size, scale, partition_size,
        _ptr(exp_sums), _ptr(max_logits), _ptr(tmp_out), _ptr(alibi_slopes), dt, _stream(q, stream))
    _check("pc_reshape_and_cache_decode", st)


def _check_alibi(alibi_slopes, q):
    if alibi_slopes is not None and (alibi_slopes.dtype != torch.float32 or not alibi_slopes.is_contiguous()
                                     or alibi_slopes.numel() != q.shape[1]):
        raise ValueError("alibi_slopes must be a contiguous float32 [num_q_heads]")


def _check_kv_scales(k_scale, v_scale, num_kv_heads: int, kv_scale_stride: int):
    for t in (k_scale, v_scale):
        if t.dtype != torch.float32 or not t.is_contiguous():
            raise ValueError("k_scale / v_scale must be contiguous float32")
        if kv_scale_stride < 0 or t.numel() <= (num_kv_heads - 1) * kv_scale_stride:
            raise ValueError("k_scale / v_scale must hold an entry at h * kv_scale_stride for every kv head")


def reshape_and_cache_fp8(key: torch.Tensor, value: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                          slot_mapping: torch.Tensor, k_scale: torch.Tensor, v_scale: torch.Tensor, *,
                          num_blocks: int, block_stride: int, token_stride: int, head_stride: int,
                          kv_scale_stride: int = 1, block_size: int = 16, v_offset: int = 0, stream=None) -> None:
    """Quantise ``key``/``value`` [T, Hkv, D] (fp32/fp16/bf16) to OCP E4M3 codes in uint8 pools;
    head h divides by ``k_scale[h * kv_scale_stride]`` / ``v_scale[...]``.  Pool strides are bytes."""
    _same_device(key, value, k_pool, v_pool, slot_mapping, k_scale, v_scale)
    if key.dim() != 3 or value.shape != key.shape or key.stride(2) != 1 or value.stride(2) != 1 or \
            key.stride(1) != key.shape[2] or value.stride(1) != value.shape[2]:
        raise ValueError("key/value must be [T, Hkv, D] with contiguous rows")
    if slot_mapping.dtype != torch.int64 or not slot_mapping.is_contiguous() or slot_mapping.numel() != key.shape[0]:
        raise ValueError("slot_mapping must be a contiguous int64 [T]")
    if k_pool.dtype != torch.uint8 or v_pool.dtype != torch.uint8:
        raise TypeError("8-bit pools must be uint8")
    dt = _dtype_code(key)
    if _DTYPES.get(value.dtype) != dt:
        raise TypeError("key and value must share one dtype")
    T, Hkv, D = key.shape
    _check_kv_scales(k_scale, v_scale, Hkv, kv_scale_stride)
    _check_pool(k_pool, v_pool, v_offset, num_blocks, block_stride, token_stride, head_stride, block_size, Hkv, D)
    st = _load().pc_reshape_and_cache_fp8(_ptr(key), _ptr(value), key.stride(0), value.stride(0), _ptr(k_pool),
                                          _ptr(v_pool, v_offset), num_blocks, block_stride, token_stride,
                                          head_stride, _ptr(slot_mapping), T, Hkv, D, block_size, _ptr(k_scale),
                                          _ptr(v_scale), kv_scale_stride, dt, _stream(key, stream))
    _check("pc_reshape_and_cache_fp8", st)


def paged_attention_decode_fp8(out, q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                               block_tables: torch.Tensor, seq_lens: torch.Tensor, max_seq_len: int,
                               k_scale: torch.Tensor, v_scale: torch.Tensor, *, num_kv_heads: int, scale: float,
                               num_blocks: int, block_stride: int, token_stride: int, head_stride: int,
                               kv_scale_stride: int = 1, block_size: int = 16, v_offset: int = 0,
                               partition_size: int = 0, exp_sums=None, max_logits=None, tmp_out=None,
                               alibi_slopes=None, stream=None) -> None:
    """``paged_attention_decode`` over uint8 pools of E4M3 codes (strides in bytes); K and V are
    the codes times the kv head's ``k_scale`` / ``v_scale``.  ``q`` is fp16 or bf16."""
    _same_device(out, q, k_pool, v_pool, block_tables, seq_lens, exp_sums, max_logits, tmp_out, k_scale, v_scale,
                 alibi_slopes)
    _check_alibi(alibi_slopes, q)
    if q.dim() != 3 or not q.is_contiguous():
        raise ValueError("q must be a contiguous [S, Hq, D]")
    if out is not None and (out.shape != q.shape or not out.is_contiguous() or out.dtype != q.dtype):
        raise ValueError("out must be a contiguous tensor shaped and typed like q")
    if block_tables.dtype != torch.int32 or block_tables.dim() != 2 or not block_tables.is_contiguous():
        raise ValueError("block_tables must be a contiguous int32 [S, W]")
    if seq_lens.dtype != torch.int32 or not seq_lens.is_contiguous():
        raise ValueError("seq_lens must be a contiguous int32 [S]")
    for t in (exp_sums, max_logits, tmp_out):
        if t is not None and (t.dtype != torch.float32 or not t.is_contiguous()):
            raise ValueError("partials must be contiguous float32")
    if k_pool.dtype != torch.uint8 or v_pool.dtype != torch.uint8:
        raise TypeError("8-bit pools must be uint8")
    _check_kv_scales(k_scale, v_scale, num_kv_heads, kv_scale_stride)
    dt = _dtype_code(q)
    S, Hq, D = q.shape
    _check_seq_inputs(S, block_tables, seq_lens)
    _check_partials(S, Hq, D, max_seq_len, partition_size, exp_sums, max_logits, tmp_out)
    _check_pool(k_pool, v_pool, v_offset, num_blocks, block_stride, token_stride, head_stride, block_size,
                num_kv_heads, D)
    st = _load().pc_paged_attention_decode_fp8(
        _ptr(out), _ptr(q), _ptr(k_pool), _ptr(v_pool, v_offset), num_blocks, block_stride, token_stride,
        head_stride, _ptr(block_tables), block_tables.shape[1], _ptr(seq_lens), S, max_seq_len, Hq, num_kv_heads,
        D, block_size, scale, partition_size, _ptr(exp_sums), _ptr(max_logits), _ptr(tmp_out), _ptr(alibi_slopes),
        _ptr(k_scale), _ptr(v_scale), kv_scale_stride, dt, _stream(q, stream))
    _check("pc_paged_attention_decode_fp8", st)


def paged_attention_varlen(out: torch.Tensor, q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                           block_tables: torch.Tensor, query_start_loc: torch.Tensor, seq_lens: torch.Tensor,
                           max_query_len: int, *, num_kv_heads: int, scale: float, num_blocks: int,
                           block_stride: int, token_stride: int, head_stride: int, causal: bool = True,
                           alibi_slopes=None, block_size: int = 16, v_offset: int = 0, stream=None) -> None:
    """Attention of the packed multi-token queries ``q`` [total_q, Hq, D]: request r owns rows
    ``query_start_loc[r] .. query_start_loc[r+1]``, its newest tokens (causal by default)."""
    _same_device(out, q, k_pool, v_pool, block_tables, query_start_loc, seq_lens, alibi_slopes)
    if q.dim() != 3 or not q.is_contiguous():
        raise ValueError("q must be a contiguous [total_q, Hq, D]")
    if out.shape != q.shape or not out.is_contiguous() or out.dtype != q.dtype:
        raise ValueError("out must be a contiguous tensor shaped and typed like q")
    if block_tables.dtype != torch.int32 or block_tables.dim() != 2 or not block_tables.is_contiguous():
        raise ValueError("block_tables must be a contiguous int32 [R, W]")
    for t, nm in ((query_start_loc, "query_start_loc"), (seq_lens, "seq_lens")):
        if t.dtype != torch.int32 or not t.is_contiguous():
            raise ValueError(f"{nm} must be a contiguous int32 tensor")
    R = seq_lens.numel()
    if query_start_loc.numel() != R + 1:
        raise ValueError("query_start_loc must hold num_reqs + 1 entries")
    if block_tables.shape[0] != R:
        raise ValueError(f"block_tables has {block_tables.shape[0]} rows for {R} requests")
    _check_pool(k_pool, v_pool, v_offset, num_blocks, block_stride, token_stride, head_stride, block_size,
                num_kv_heads, q.shape[2])
    _check_alibi(alibi_slopes, q)
    dt = _dtype_code(q)
    if _DTYPES.get(k_pool.dtype) != dt or _DTYPES.get(v_pool.dtype) != dt:
        raise TypeError("q and the pool must share one storage dtype")
    T, Hq, D = q.shape
    st = _load().pc_paged_attention_varlen(
        _ptr(out), _ptr(q), _ptr(k_pool), _ptr(v_pool, v_offset), num_blocks, block_stride, token_stride,
        head_stride, _ptr(block_tables), block_tables.shape[1], _ptr(query_start_loc), _ptr(seq_lens), R, T,
        max_query_len, Hq, num_kv_heads, D, block_size, scale, int(bool(causal)), _ptr(alibi_slopes), dt,
        _stream(q, stream))
    _check("pc_paged_attention_varlen", st)


def paged_attention_reduce(out: torch.Tensor, exp_sums: torch.Tensor, max_logits: torch.Tensor,
                           tmp_out: torch.Tensor, seq_lens: torch.Tensor, *, partition_size: int = PARTITION_SIZE,
                           stream=None) -> None:
    """Merge partials [S, Hq, P(, D)] into ``out`` [S, Hq, D]."""
    _same_device(out, exp_sums, max_logits, tmp_out, seq_lens)
    if tmp_out.dim() != 4 or not (out.is_contiguous() and tmp_out.is_contiguous() and exp_sums.is_contiguous()
                                  and max_logits.is_contiguous()):
        raise ValueError("contiguous out [S,Hq,D] and partials [S,Hq,P(,D)] expected")
    S, Hq, P, D = tmp_out.shape
    if tuple(out.shape) != (S, Hq, D):
        raise ValueError("out must be [S, Hq, D] matching tmp_out [S, Hq, P, D]")
    if tuple(exp_sums.shape) != (S, Hq, P) or tuple(max_logits.shape) != (S, Hq, P):
        raise ValueError("exp_sums and max_logits must be [S, Hq, P] matching tmp_out")
    for t in (exp_sums, max_logits, tmp_out):
        if t.dtype != torch.float32:
            raise ValueError("partials must be float32")
    if seq_lens.dtype != torch.int32 or not seq_lens.is_contiguous() or seq_lens.numel() != S:
        raise ValueError("seq_lens must be a contiguous int32 [S]")
    st = _load().pc_paged_attention_reduce(_ptr(out), _ptr(exp_sums), _ptr(max_logits), _ptr(tmp_out),
                                           _ptr(seq_lens), S, Hq, D, P, partition_size, _dtype_code(out),
                                           _stream(out, stream))
    _check("pc_paged_attention_reduce", st)


def paged_attention_plan_lens(seq_lens, num_q_heads: int, num_kv_heads: int, head_size: int, head_stride: int,
                              dtype: torch.dtype, kv_fp8: bool = False, shared_lens=None):
    """(partition_size, max_num_partitions, workspace_bytes) for a batch whose lengths the
    host knows: ``seq_lens`` (and optional ``shared_lens``, the leading tokens of each
    sequence in blocks other sequences also read) are host sequences of ints (list, numpy
    array or CPU tensor)."""
    import numpy as np

    def host(x):
        return np.ascontiguousarray(np.asarray(x.cpu() if isinstance(x, torch.Tensor) else x, dtype=np.int32))
    lens = host(seq_lens)
    shared = None if shared_lens is None else host(shared_lens)
    if shared is not None and shared.shape != lens.shape:
        raise ValueError("shared_lens must have one entry per sequence")
    ps, mp, ws = ctypes.c_int(0), ctypes.c_int(0), ctypes.c_size_t(0)
    st = _load().pc_paged_attention_plan_lens(lens.ctypes.data if lens.size else None,
                                              shared.ctypes.data if shared is not None and shared.size else None,
                                              int(lens.size), num_q_heads, num_kv_heads, head_size, head_stride,
                                              int(bool(kv_fp8)), _DTYPES[dtype], ctypes.byref(ps), ctypes.byref(mp),
                                              ctypes.byref(ws))
    _check("pc_paged_attention_plan_lens", st)
    return ps.value, mp.value, ws.value


def paged_attention_plan(num_seqs: int, num_q_heads: int, num_kv_heads: int, head_size: int, max_seq_len: int,
                         dtype: torch.dtype):
    """(partition_size, max_num_partitions, workspace_bytes) chosen by the library's planner."""
    ps, mp, ws = ctypes.c_int(0), ctypes.c_int(0), ctypes.c_size_t(0)
    st = _load().pc_paged_attention_plan(num_seqs, num_q_heads, num_kv_heads, head_size, max_seq_len,
                                         _DTYPES[dtype], ctypes.byref(ps), ctypes.byref(mp), ctypes.byref(ws))
    _check("pc_paged_attention_plan", st)
    return ps.value, mp.value, ws.value


def stream_read(src: torch.Tensor, sink: torch.Tensor, *, cache_policy: int = 0, stream=None) -> None:
    """Measurement aid: read every byte of ``src`` once (pc_stream_read); ``sink`` is a uint32
    (int32) tensor with one entry per workgroup of the launch."""
    _same_device(src, sink)
    if not src.is_contiguous() or sink.dtype not in (torch.int32, torch.uint32) or not sink.is_contiguous():
        raise ValueError("src must be contiguous and sink a contiguous 32-bit integer tensor")
    st = _load().pc_stream_read(_ptr(src), src.numel() * src.element_size(), _ptr(sink), sink.numel(),
                                cache_policy, _stream(src, stream))
    _check("pc_stream_read", st)


GATHER_SINK_WORDS = 4096


def gather_read(k_pool: torch.Tensor, v_pool: torch.Tensor, block_tables: torch.Tensor, seq_lens: torch.Tensor,
                max_seq_len: int, sink: torch.Tensor, *, num_kv_heads: int, head_size: int, num_blocks: int,
                block_stride: int, token_stride: int, head_stride: int, block_size: int = 16, v_offset: int = 0,
                v_cache_policy: int = 0, stream=None) -> None:
    """Measurement aid: read every K/V tile a decode of this batch reads, loads only
    (pc_gather_read).  ``sink``: a zeroed 32-bit integer tensor of 4096 entries; the XOR of
    its entries afterwards is the XOR of every 32-bit word read."""
    _same_device(k_pool, v_pool, block_tables, seq_lens, sink)
    if block_size != 16:
        raise ValueError("pc_gather_read reads 16-token blocks")
    if sink.dtype not in (torch.int32, torch.uint32) or not sink.is_contiguous() or sink.numel() != GATHER_SINK_WORDS:
        raise ValueError(f"sink must be a contiguous 32-bit integer tensor of {GATHER_SINK_WORDS} entries")
    if block_tables.dtype != torch.int32 or block_tables.dim() != 2 or not block_tables.is_contiguous():
        raise ValueError("block_tables must be a contiguous int32 [S, max_blocks_per_seq]")
    if seq_lens.dtype != torch.int32 or not seq_lens.is_contiguous():
        raise ValueError("seq_lens must be a contiguous int32 [S]")
    if k_pool.dtype != v_pool.dtype:
        raise ValueError("k_pool and v_pool must share one element type")
    S = block_tables.shape[0]
    _check_seq_inputs(S, block_tables, seq_lens)
    _check_pool(k_pool, v_pool, v_offset, num_blocks, block_stride, token_stride, head_stride, block_size,
                num_kv_heads, head_size)
    st = _load().pc_gather_read(_ptr(k_pool), _ptr(v_pool, v_offset), num_blocks, block_stride, token_stride,
                                head_stride, _ptr(block_tables), block_tables.shape[1], _ptr(seq_lens), S,
                                max_seq_len, num_kv_heads, head_size, k_pool.element_size(), _ptr(sink),
                                v_cache_policy, _stream(k_pool, stream))
    _check("pc_gather_read", st)
