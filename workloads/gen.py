"""Seeded generator of paged-KV decode workloads.

Every workload is a decode step of a serving engine, as the pages describe it:
earlier tokens already sit in a pool of fixed 16-token physical blocks, the step
first writes one new token per sequence through ``slot_mapping`` (a negative slot
means "no destination"), then attention reads each sequence's history through its
``block_table``.

What this module produces is plain input data:

* ``seq_lens`` (int32), ``block_tables`` (int32, rows padded with -1),
* q, the pre-filled history rows ``pre_key``/``pre_value`` together with the slots
  a scheduler assigned them (``pre_slots``), and the step's new rows
  ``key``/``value`` with their ``slot_mapping`` (int64),
* the pool layout (element strides of a block, a token row and a head), and
* ``logical_src``: for every sequence, which drawn row holds position ``t`` -- the
  contiguous history that paging is supposed to reproduce.

Recipe (identical for every workload):

* ``rng = numpy.random.Generator(numpy.random.PCG64(seed))`` draws, in order, the
  sequence lengths, the block placement and the padding positions; the five named
  workloads use ``seed = workload index``.
* Bulk values come from five streams: q (0), K rows (1), V rows (2), new keys (3),
  new values (4); row chunk ``c`` (4096 rows) of stream ``k`` is drawn by
  ``Generator(PCG64(SeedSequence([seed, k, c])))``.
* Values are ``standard_normal`` in float32, rounded to nearest-even into the
  workload's storage type (fp32, bf16 or fp16); they are kept as raw bit patterns.
* Pool memory that no token occupies holds a quiet-NaN bit pattern.
* ``scale = float32(1 / sqrt(head_size))``.

The scheduler-side flattening ``slot = physical_block * block_size + offset`` is
applied here, once, to hand the write its destinations ("How vLLM CUDA Kernels
Write and Read the Paged KV Cache", section "Mapping one token to a physical
slot").  Decoding a slot back into (block, offset) and every address computation
belong to the consumers.
"""

from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace

import numpy as np

BLOCK_SIZE = 16

CONFIG_NAMES = {
    0: "tiny_mha_f32_s2",
    1: "gqa_bf16_s64_l512_2048",
    2: "combined_block_bf16_s128_l1_2048",
    3: "long_context_bf16_s4_l32768_split512",
    4: "mixed_serving_f16_s256_l16_8192_prefix1024",
}

_NAN_BITS = {"f32": 0x7FC00000, "bf16": 0x7FC0, "f16": 0x7E00}
_BITS_NP = {"f32": np.uint32, "bf16": np.uint16, "f16": np.uint16}


def dtype_nbytes(dtype: str) -> int:
    return 4 if dtype == "f32" else 2


def nan_bits(dtype: str) -> int:
    """Quiet-NaN bit pattern used to fill pool memory that no token occupies."""
    return _NAN_BITS[dtype]


def _to_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round finite float32 values to nearest-even in the storage type; return raw bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f32":
        return x.view(np.uint32).copy()
    if dtype == "f16":
        return x.astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        # round-to-nearest-even on the upper 16 bits; cannot overflow uint32 for finite x
        u = x.view(np.uint32).copy()
        lsb = u >> 16
        lsb &= 1
        u += np.uint32(0x7FFF)
        u += lsb
        u >>= 16
        return u.astype(np.uint16)
    raise ValueError(dtype)


_CHUNK_ROWS = 4096


def _normal_bits(seed: int, stream: int, shape, dtype: str, out: np.ndarray | None = None) -> np.ndarray:
    """standard_normal(float32) rounded into ``dtype`` bits.

    Rows are drawn in chunks of 4096; chunk ``c`` of bulk stream ``stream`` comes
    from ``Generator(PCG64(SeedSequence([seed, stream, c])))``, so the result does
    not depend on how many threads fill it.
    """
    shape = tuple(int(s) for s in shape)
    if out is None:
        out = np.empty(shape, dtype=_BITS_NP[dtype])
    if shape[0] == 0:
        return out
    row = int(np.prod(shape[1:])) if len(shape) > 1 else 1
    flat = out.reshape(shape[0], row)
    chunks = range(0, (shape[0] + _CHUNK_ROWS - 1) // _CHUNK_ROWS)

    def fill(c):
        r0 = c * _CHUNK_ROWS
        r1 = min(shape[0], r0 + _CHUNK_ROWS)
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, stream, c])))
        flat[r0:r1] = _to_bits(g.standard_normal((r1 - r0, row), dtype=np.float32), dtype)

    if len(chunks) == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as ex:
            list(ex.map(fill, chunks))
    return out


@dataclass
class Workload:
    name: str
    seed: int
    dtype: str  # 'f32' | 'bf16' | 'f16' -- q, pool, key/value and out share it
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_size: int
    block_size: int
    layout: str  # 'hnd' | 'nhd' | 'combined'
    num_blocks: int
    block_stride: int  # element strides inside one pool buffer; head_size has stride 1
    token_stride: int
    head_stride: int
    v_offset: int  # 'combined': V starts this many elements after K in one buffer
    pool_elems: int  # elements of one pool buffer (K and V each; the single buffer for 'combined')
    seq_lens: np.ndarray  # int32 [S]
    block_tables: np.ndarray  # int32 [S, W], -1 past each row's valid blocks
    scale: np.float32
    q: np.ndarray  # bits [S, Hq, D]
    pre_slots: np.ndarray  # int64 [Tp]
    pre_key: np.ndarray  # bits [Tp, Hkv, D]
    pre_value: np.ndarray
    slot_mapping: np.ndarray  # int64 [T]: the step's write, -1 = padding
    key: np.ndarray  # bits [T, Hkv, D]
    value: np.ndarray
    logical_src: list = field(repr=False, default_factory=list)  # per seq: int64 [L_s] rows of bank_k/bank_v
    bank_k: np.ndarray = field(repr=False, default=None)  # rows referenced by logical_src
    bank_v: np.ndarray = field(repr=False, default=None)
    prefix_blocks: int = 0
    notes: str = ""
    # 8-bit cache: kv_dtype 'fp8' stores OCP E4M3 codes; head h of K uses
    # k_scale[h * scale_stride] (scale_stride 0: one shared scale), V likewise
    kv_dtype: str = ""
    k_scale: np.ndarray = field(repr=False, default=None)  # float32
    v_scale: np.ndarray = field(repr=False, default=None)
    scale_stride: int = 0
    # ALiBi: one float32 slope per query head (None: no positional bias)
    alibi_slopes: np.ndarray = field(repr=False, default=None)

    # ----- sizes -------------------------------------------------------------------
    @property
    def esize(self) -> int:
        return dtype_nbytes(self.dtype)

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens.max()) if self.num_seqs else 0

    @property
    def bits_dtype(self):
        return _BITS_NP[self.dtype]

    @property
    def fp8(self) -> bool:
        return self.kv_dtype == "fp8"

    @property
    def kv_esize(self) -> int:
        return 1 if self.fp8 else self.esize

    def kv_bytes(self) -> int:
        """K and V bytes of exactly seq_len tokens per sequence (no block padding)."""
        return int(self.seq_lens.astype(np.int64).sum()) * self.num_kv_heads * self.head_size * 2 * self.kv_esize

    def qo_bytes(self) -> int:
        return self.num_seqs * self.num_q_heads * self.head_size * 2 * self.esize

    def effective_bytes(self) -> int:
        return self.kv_bytes() + self.qo_bytes()

    def unique_kv_bytes(self) -> int:
        """K/V bytes of distinct physical token rows read (shared prefix counted once)."""
        used = {}
        for s in range(self.num_seqs):
            L = int(self.seq_lens[s])
            nb = -(-L // self.block_size)
            for j in range(nb):
                b = int(self.block_tables[s, j])
                tok = min(self.block_size, L - j * self.block_size)
                used[b] = max(used.get(b, 0), tok)
        return sum(used.values()) * self.num_kv_heads * self.head_size * 2 * self.kv_esize

    def shared_lens(self) -> np.ndarray:
        """Per sequence: leading tokens in blocks that other sequences also read (the shared
        prefix's blocks; a sequence's last block is always its own).  All zero without one."""
        if not self.prefix_blocks:
            return np.zeros(self.num_seqs, np.int32)
        nb = -(-self.seq_lens.astype(np.int64) // self.block_size)
        sh = np.minimum(self.prefix_blocks, np.maximum(nb - 1, 0)) * self.block_size
        return np.minimum(sh, self.seq_lens).astype(np.int32)

    def prefix_table(self) -> np.ndarray:
        """The shared prefix's physical blocks in token order (empty without a prefix): the
        first prefix_blocks entries of a sequence that shares them all."""
        if not self.prefix_blocks:
            return np.zeros(0, np.int32)
        owner = int(np.argmax(self.shared_lens()))
        return np.ascontiguousarray(self.block_tables[owner, :self.prefix_blocks], np.int32)

    # ----- memory images ---------------------------------------------------------
    def nan_pool(self) -> np.ndarray:
        """One pool buffer (element bits) filled with the quiet-NaN pattern (0x7F for E4M3)."""
        if self.fp8:
            return np.full(self.pool_elems, 0x7F, dtype=np.uint8)
        return np.full(self.pool_elems, nan_bits(self.dtype), dtype=self.bits_dtype)

    def logical_k(self, s: int) -> np.ndarray:
        return self.bank_k[self.logical_src[s]]

    def logical_v(self, s: int) -> np.ndarray:
        return self.bank_v[self.logical_src[s]]


# ----------------------------------------------------------------------------------
# layouts
# ----------------------------------------------------------------------------------

def _layout(layout: str, num_blocks: int, Hkv: int, D: int, B: int):
    """Element strides (block, token, head), V offset and buffer size of a layout."""
    if layout == "hnd":  # [num_blocks, Hkv, B, D], K and V in separate buffers
        return Hkv * B * D, D, B * D, 0, num_blocks * Hkv * B * D
    if layout == "nhd":  # [num_blocks, B, Hkv, D], K and V in separate buffers
        return B * Hkv * D, Hkv * D, D, 0, num_blocks * B * Hkv * D
    if layout == "combined":  # one buffer; per block: K [B, Hkv, D] then V [B, Hkv, D]
        return 2 * B * Hkv * D, Hkv * D, D, B * Hkv * D, num_blocks * 2 * B * Hkv * D
    raise ValueError(layout)


# ----------------------------------------------------------------------------------
# assembly shared by every workload
# ----------------------------------------------------------------------------------

def _assemble(*, name, seed, rng, dtype, Hq, Hkv, D, layout, num_blocks, seq_lens, block_tables,
              prefix_blocks=0, pad_count=0, extra_pad_rows=0, notes="", contents=True,
              block_size=BLOCK_SIZE) -> Workload:
    """Draw contents and build the write lists for given lengths and block tables.

    Bulk draws use streams 0 (q), 1 (K rows), 2 (V rows), 3 (new keys), 4 (new
    values); the padding positions come from ``rng`` after the tables.  With
    ``contents=False`` the bulk arrays are left zero-filled (structure only); every
    other field is identical.
    """
    draw = _normal_bits if contents else (lambda seed_, stream_, shape_, dtype_, out=None:
                                           out if out is not None else np.zeros(shape_, _BITS_NP[dtype_]))
    B = block_size
    S = len(seq_lens)
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    block_tables = np.ascontiguousarray(block_tables, dtype=np.int32)
    bs, ts, hs, voff, pool_elems = _layout(layout, num_blocks, Hkv, D, B)
    prefix_len = prefix_blocks * B
    Ls = [int(L) for L in seq_lens]

    q = draw(seed, 0, (S, Hq, D), dtype)

    # blocks of the shared prefix that each sequence reads (its last block is private)
    shared = [min(prefix_blocks, max(-(-L // B) - 1, 0)) if prefix_blocks else 0 for L in Ls]
    # positions that need a freshly drawn row: the prefix, then per sequence the
    # private positions at or past the prefix, before the last one
    fresh_lo = [max(shared[s] * B, prefix_len) for s in range(S)]
    fresh_cnt = [max(Ls[s] - 1 - fresh_lo[s], 0) for s in range(S)]
    fresh_base = np.concatenate([[prefix_len], prefix_len + np.cumsum(fresh_cnt)]).astype(np.int64)
    n_rand = int(fresh_base[-1])

    # bank = drawn history rows followed by the step's new rows; logical_src indexes it
    T = S + extra_pad_rows
    alloc = np.empty if contents else np.zeros
    bank_k = alloc((n_rand + T, Hkv, D), dtype=_BITS_NP[dtype])
    bank_v = alloc((n_rand + T, Hkv, D), dtype=_BITS_NP[dtype])
    draw(seed, 1, (n_rand, Hkv, D), dtype, out=bank_k[:n_rand])
    draw(seed, 2, (n_rand, Hkv, D), dtype, out=bank_v[:n_rand])
    key = draw(seed, 3, (T, Hkv, D), dtype, out=bank_k[n_rand:])
    value = draw(seed, 4, (T, Hkv, D), dtype, out=bank_v[n_rand:])

    padded = np.zeros(S, dtype=bool)
    if pad_count:
        padded[rng.choice(S, size=pad_count, replace=False)] = True

    logical_src = []
    pre_rows = []
    pre_slots = []

    def slots_of(s, pos):
        return block_tables[s, pos // B].astype(np.int64) * B + pos % B

    if prefix_blocks:
        owner = next((s for s in range(S) if shared[s] == prefix_blocks), None)
        if owner is None:
            raise ValueError("no sequence spans the whole shared prefix")
        pos = np.arange(prefix_len, dtype=np.int64)
        pre_rows.append(pos)
        pre_slots.append(slots_of(owner, pos))

    slot_mapping = np.full(T, -1, dtype=np.int64)
    for s in range(S):
        L = Ls[s]
        pos = np.arange(L, dtype=np.int64)
        src = pos.copy()  # prefix rows (shared or private copies) are bank rows 0..prefix_len-1
        lo = fresh_lo[s]
        if L - 1 > lo:
            src[lo:L - 1] = fresh_base[s] + np.arange(L - 1 - lo)
        if L >= 1:
            src[L - 1] = n_rand + s
        logical_src.append(src)
        priv = pos[shared[s] * B:L - 1]
        pre_rows.append(src[priv])
        pre_slots.append(slots_of(s, priv))
        if L >= 1:
            last = np.array([L - 1], dtype=np.int64)
            if padded[s]:
                pre_rows.append(np.array([n_rand + s], dtype=np.int64))
                pre_slots.append(slots_of(s, last))
            else:
                slot_mapping[s] = int(slots_of(s, last)[0])

    pre_rows = np.concatenate(pre_rows) if pre_rows else np.empty(0, dtype=np.int64)
    pre_slots = np.concatenate(pre_slots) if pre_slots else np.empty(0, dtype=np.int64)
    return Workload(
        name=name, seed=seed, dtype=dtype, num_seqs=S, num_q_heads=Hq, num_kv_heads=Hkv, head_size=D,
        block_size=B, layout=layout, num_blocks=num_blocks, block_stride=bs, token_stride=ts, head_stride=hs,
        v_offset=voff, pool_elems=pool_elems, seq_lens=seq_lens, block_tables=block_tables,
        scale=np.float32(1.0 / math.sqrt(D)), q=q, pre_slots=pre_slots.astype(np.int64),
        pre_key=bank_k[pre_rows] if contents else np.zeros((len(pre_rows), Hkv, D), _BITS_NP[dtype]),
        pre_value=bank_v[pre_rows] if contents else np.zeros((len(pre_rows), Hkv, D), _BITS_NP[dtype]),
        slot_mapping=slot_mapping, key=key, value=value, logical_src=logical_src, bank_k=bank_k, bank_v=bank_v,
        prefix_blocks=prefix_blocks, notes=notes)


def _deal(perm: np.ndarray, nblocks, width: int) -> np.ndarray:
    """Give each sequence the next n_s ids of ``perm``, in order; pad rows with -1."""
    S = len(nblocks)
    table = np.full((S, width), -1, dtype=np.int32)
    off = 0
    for s, n in enumerate(nblocks):
        table[s, :n] = perm[off:off + n]
        off += n
    return table


def _nblocks(seq_lens, block_size=BLOCK_SIZE):
    return [-(-int(L) // block_size) for L in seq_lens]


# ----------------------------------------------------------------------------------
# the five named workloads
# ----------------------------------------------------------------------------------

def make_config(idx: int, seed: int | None = None, contents: bool = True, block_size: int = BLOCK_SIZE) -> Workload:
    """Build named workload ``idx`` (0..4) with ``seed`` (default: ``idx``).
    ``contents=False`` skips drawing values (lengths, tables and slots only).
    ``block_size`` (workloads 1 and 3 only) stores the same tokens in blocks of that
    many tokens; 16 draws exactly the named workload."""
    seed = idx if seed is None else seed
    rng = np.random.Generator(np.random.PCG64(seed))
    name = CONFIG_NAMES[idx]
    B = block_size
    if B != BLOCK_SIZE:
        if idx not in (1, 3):
            raise ValueError("other block sizes are offered for workloads 1 and 3")
        name = f"{name}_b{B}"
    if idx == 0:
        # tiny MHA fp32: 2 sequences of 20 and 37 tokens, 16-block pool; both tables
        # come from one permutation (disjoint), the step writes each last token and
        # one appended padding row (slot -1).
        seq_lens = np.array([20, 37], dtype=np.int32)
        nb = _nblocks(seq_lens)
        perm = rng.permutation(16)
        table = _deal(perm, nb, max(nb))
        return _assemble(name=name, seed=seed, rng=rng, dtype="f32", Hq=4, Hkv=4, D=64, layout="hnd",
                         num_blocks=16, seq_lens=seq_lens, block_tables=table, extra_pad_rows=1, contents=contents,
                         notes="single-pass path")
    if idx == 1:
        # GQA 32/8, D=128, bf16; L ~ U{512..2048}; pool = 2x the blocks needed,
        # a permutation of the pool dealt to the sequences in order.
        seq_lens = rng.integers(512, 2048, size=64, endpoint=True).astype(np.int32)
        nb = _nblocks(seq_lens, B)
        N = sum(nb)
        perm = rng.permutation(2 * N)
        table = _deal(perm, nb, 2048 // B)
        return _assemble(name=name, seed=seed, rng=rng, dtype="bf16", Hq=32, Hkv=8, D=128, layout="hnd",
                         num_blocks=2 * N, seq_lens=seq_lens, block_tables=table, notes="single-pass path",
                         contents=contents, block_size=B)
    if idx == 2:
        # combined K-then-V block (8 kv heads x 64 = 512 per token, bf16): a block is
        # 32 KiB, a 2 GiB pool is 65536 blocks; L ~ U{1..2048}; ids drawn without
        # replacement from the whole pool.
        seq_lens = rng.integers(1, 2048, size=128, endpoint=True).astype(np.int32)
        nb = _nblocks(seq_lens)
        ids = rng.choice(65536, size=sum(nb), replace=False)
        table = _deal(ids, nb, 2048 // B)
        return _assemble(name=name, seed=seed, rng=rng, dtype="bf16", Hq=32, Hkv=8, D=64, layout="combined",
                         num_blocks=65536, seq_lens=seq_lens, block_tables=table, notes="dispatcher decides",
                         contents=contents)
    if idx == 3:
        # long context: 4 x 32768 tokens, GQA 32/8, D=128, bf16, exactly 8192 blocks permuted
        seq_lens = np.full(4, 32768, dtype=np.int32)
        nb = _nblocks(seq_lens, B)
        perm = rng.permutation(sum(nb))  # exactly the blocks needed (8192 of 16 tokens)
        table = _deal(perm, nb, 32768 // B)
        return _assemble(name=name, seed=seed, rng=rng, dtype="bf16", Hq=32, Hkv=8, D=128, layout="hnd",
                         num_blocks=sum(nb), seq_lens=seq_lens, block_tables=table,
                         notes="split path, 512-token partitions, then the log-sum-exp reduce", contents=contents,
                         block_size=B)
    if idx == 4:
        # mixed serving step, fp16 MHA 32 heads x 128: L = floor(exp(U[ln 16, ln 8193)))
        # (log-uniform on [16, 8192]); a 1024-token prefix (64 blocks) is shared by all
        # sequences through identical leading table entries; a sequence shorter than
        # the prefix shares all but its last block, which is private.  The pool is the
        # 64 prefix blocks plus the private ones, permuted.  The step writes each
        # sequence's last token; 26 of the 256 slots (10%) are -1 padding, whose
        # tokens are already in the pool.
        S = 256
        u = rng.uniform(math.log(16), math.log(8193), size=S)
        seq_lens = np.clip(np.floor(np.exp(u)), 16, 8192).astype(np.int32)
        nb = _nblocks(seq_lens)
        P = 64
        priv = [n - min(P, n - 1) for n in nb]
        total = P + sum(priv)
        perm = rng.permutation(total)
        prefix = perm[:P]
        table = np.full((S, 8192 // B), -1, dtype=np.int32)
        off = P
        for s in range(S):
            sh = min(P, nb[s] - 1)
            table[s, :sh] = prefix[:sh]
            table[s, sh:nb[s]] = perm[off:off + priv[s]]
            off += priv[s]
        if not any(min(P, n - 1) == P for n in nb):
            raise RuntimeError("no sequence spans the prefix")
        return _assemble(name=name, seed=seed, rng=rng, dtype="f16", Hq=32, Hkv=32, D=128, layout="hnd",
                         num_blocks=total, seq_lens=seq_lens, block_tables=table, prefix_blocks=P,
                         pad_count=round(0.1 * S), notes="dispatcher decides", contents=contents)
    raise ValueError(idx)


# ----------------------------------------------------------------------------------
# free-form workloads for edge cases
# ----------------------------------------------------------------------------------

def custom(seed: int, dtype: str, num_q_heads: int, num_kv_heads: int, head_size: int, seq_lens,
           layout: str = "hnd", pool_factor: float = 2.0, table_width: int | None = None,
           extra_pad_rows: int = 0, pad_count: int = 0, prefix_blocks: int = 0, name: str = "custom",
           placement=None, block_size: int = BLOCK_SIZE) -> Workload:
    """A workload with given lengths; blocks are a permutation of a pool
    ``pool_factor`` times the blocks needed (at least 1), dealt in order.

    ``placement`` changes only where blocks go, never the contents: ``None`` uses
    the permutation drawn from ``seed``, ``"identity"`` deals blocks 0, 1, 2, ... in
    order, an int draws the permutation from ``PCG64(placement)`` instead.
    """
    rng = np.random.Generator(np.random.PCG64(seed))

    def _perm(n):
        p = rng.permutation(n)  # always drawn, so later draws from rng do not move
        if placement is None:
            return p
        if isinstance(placement, str) and placement == "identity":
            return np.arange(n)
        return np.random.Generator(np.random.PCG64(int(placement))).permutation(n)

    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    nb = _nblocks(seq_lens, block_size)
    width = table_width if table_width is not None else max(max(nb) if len(nb) else 1, 1)
    if prefix_blocks:
        P = prefix_blocks
        priv = [n - min(P, max(n - 1, 0)) for n in nb]
        total = P + sum(priv)
        total = max(total, int(math.ceil(total * pool_factor)))
        perm = _perm(total)
        prefix = perm[:P]
        table = np.full((len(nb), width), -1, dtype=np.int32)
        off = P
        for s, n in enumerate(nb):
            sh = min(P, max(n - 1, 0))
            table[s, :sh] = prefix[:sh]
            table[s, sh:n] = perm[off:off + priv[s]]
            off += priv[s]
        num_blocks = total
    else:
        N = sum(nb)
        num_blocks = max(1, int(math.ceil(N * pool_factor)))
        perm = _perm(num_blocks)
        table = _deal(perm, nb, width)
    return _assemble(name=name, seed=seed, rng=rng, dtype=dtype, Hq=num_q_heads, Hkv=num_kv_heads, D=head_size,
                     layout=layout, num_blocks=num_blocks, seq_lens=seq_lens, block_tables=table,
                     prefix_blocks=prefix_blocks, pad_count=pad_count, extra_pad_rows=extra_pad_rows,
                     block_size=block_size)


def fp8_variant(wl: Workload, per_head: bool = True, lo: float = 0.008, hi: float = 0.03) -> Workload:
    """The same workload over an 8-bit (OCP E4M3) cache: the history and the step's
    rows (still in ``wl.dtype``) are quantised by the write.  Scales are float32 drawn
    uniformly in [lo, hi) from stream 5 -- one per kv head (per_head) or one shared;
    with standard-normal values a few |x| / scale exceed 448 and saturate."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([wl.seed, 5])))
    n = wl.num_kv_heads if per_head else 1
    ks = rng.uniform(lo, hi, size=n).astype(np.float32)
    vs = rng.uniform(lo, hi, size=n).astype(np.float32)
    name = wl.name.replace(wl.dtype, f"{wl.dtype}q_fp8e4m3", 1) if wl.dtype in wl.name else wl.name + "_fp8e4m3"
    return replace(wl, name=name, kv_dtype="fp8", k_scale=ks, v_scale=vs, scale_stride=1 if per_head else 0)


def alibi_variant(wl: Workload, slopes=None) -> Workload:
    """The same workload with an ALiBi bias.  ``slopes`` (one per query head) default
    to the geometric sequence 2^(-8 (h + 1) / Hq), the usual recipe for Hq heads;
    they are inputs here, not part of the method."""
    H = wl.num_q_heads
    if slopes is None:
        slopes = 2.0 ** (-8.0 * (np.arange(H) + 1) / H)
    slopes = np.ascontiguousarray(slopes, dtype=np.float32)
    if slopes.shape != (H,):
        raise ValueError("one slope per query head")
    return replace(wl, name=wl.name + "_alibi", alibi_slopes=slopes)


@dataclass
class VarlenStep:
    """Several query tokens per request (chunked prefill, speculative decode) over a
    workload's history.  Request r owns rows [query_start_loc[r], query_start_loc[r+1])
    of the packed query; they are its newest n_r tokens (positions L_r - n_r .. L_r - 1),
    whose K/V rows the step writes first (``key``/``value`` through ``slot_mapping``)."""
    q: np.ndarray = field(repr=False)                  # bits [total_q, Hq, D]
    query_start_loc: np.ndarray = field(repr=False)    # int32 [R + 1]
    query_lens: np.ndarray = field(repr=False)         # int32 [R]
    key: np.ndarray = field(repr=False)                # bits [total_q, Hkv, D]
    value: np.ndarray = field(repr=False)
    slot_mapping: np.ndarray = field(repr=False)       # int64 [total_q]
    causal: bool = True

    @property
    def total_q(self) -> int:
        return int(self.query_start_loc[-1])

    @property
    def max_query_len(self) -> int:
        return int(self.query_lens.max()) if len(self.query_lens) else 0


def varlen_variant(wl: Workload, query_lens, causal: bool = True) -> VarlenStep:
    """Queries of ``query_lens[r]`` (<= seq_lens[r]) tokens per request of ``wl``.  The
    packed q is drawn from stream 6; the step's K/V rows are the requests' own newest
    logical rows, so writing them leaves the pool unchanged."""
    n = np.asarray(query_lens, dtype=np.int32)
    if n.shape != (wl.num_seqs,) or (n < 0).any() or (n > wl.seq_lens).any():
        raise ValueError("one query length per request, 0 <= n_r <= seq_len_r")
    qs = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    total = int(qs[-1])
    q = _normal_bits(wl.seed, 6, (total, wl.num_q_heads, wl.head_size), wl.dtype)
    keys, values, slots = [], [], []
    B = wl.block_size
    for r in range(wl.num_seqs):
        L, k = int(wl.seq_lens[r]), int(n[r])
        pos = np.arange(L - k, L, dtype=np.int64)
        keys.append(wl.logical_k(r)[L - k:L])
        values.append(wl.logical_v(r)[L - k:L])
        slots.append(wl.block_tables[r, pos // B].astype(np.int64) * B + pos % B)
    shape = (0, wl.num_kv_heads, wl.head_size)
    cat = lambda xs: np.concatenate(xs) if xs else np.zeros(shape, _BITS_NP[wl.dtype])
    return VarlenStep(q=q, query_start_loc=qs, query_lens=n, key=cat(keys), value=cat(values),
                      slot_mapping=np.concatenate(slots) if slots else np.zeros(0, np.int64), causal=causal)


VARLEN_CONFIGS = {
    # chunked prefill: 8 requests whose newest 512 tokens form the query, histories of
    # 1024..4096 tokens (chunk included), GQA 32/8, D = 128, bf16
    "prefill": dict(name="chunked_prefill_bf16_r8_q512_l1024_4096", seed=21, S=8, lo=1024, hi=4096, n=512),
    # speculative decode: 64 requests verifying 4 draft tokens each over 512..2048 tokens
    "spec": dict(name="spec_decode_bf16_s64_q4_l512_2048", seed=22, S=64, lo=512, hi=2048, n=4),
}


def varlen_config(kind: str, contents: bool = True):
    """(workload, VarlenStep) of a named multi-token workload (see VARLEN_CONFIGS)."""
    c = VARLEN_CONFIGS[kind]
    rng = np.random.Generator(np.random.PCG64(c["seed"]))
    lengths = rng.integers(c["lo"], c["hi"] + 1, size=c["S"]).astype(np.int32)
    wl = custom(c["seed"], "bf16", 32, 8, 128, lengths, name=c["name"])
    return wl, varlen_variant(wl, np.full(c["S"], c["n"], np.int32))
