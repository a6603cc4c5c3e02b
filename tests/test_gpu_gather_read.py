"""pc_gather_read, the benchmark's gather yardstick, reads exactly the decode's tiles: for
every sequence, kv head and block covering its tokens, the 16 token rows of that head
from the K pool and from the V pool.  The XOR of its sink must equal the XOR of every
32-bit word of those rows, computed on the host from the same pool bytes."""

import numpy as np
import pytest
import torch

import gpu_harness as gh
import paged_kv_cache_reshape_amd as pc
from workloads import custom, fp8_variant

pytestmark = pytest.mark.gpu

LENGTHS = [1, 15, 16, 17, 300, 511, 512, 513, 1100, 2050]


def host_xor(wl, pool, block_tables, seq_lens):
    """XOR of every 32-bit word of the tiles the decode reads, from the pool's bytes."""
    esz = 1 if pool.fp8 else (4 if wl.dtype == "f32" else 2)
    bufs = [b.view(np.uint8).reshape(-1) for b in pool.bits()]
    kb = bufs[0]
    vb, voff = (bufs[0], wl.v_offset * esz) if len(bufs) == 1 else (bufs[1], 0)
    rows = []
    for s, L in enumerate(seq_lens):
        for j in range(-(-int(L) // 16)):
            b = int(block_tables[s, j])
            if not 0 <= b < wl.num_blocks:
                continue
            for h in range(wl.num_kv_heads):
                for r in range(16):
                    rows.append((b * wl.block_stride + r * wl.token_stride + h * wl.head_stride) * esz)
    if not rows:
        return 0
    starts = np.asarray(rows, np.int64)[:, None] + np.arange(wl.head_size * esz, dtype=np.int64)[None, :]
    x = np.bitwise_xor.reduce(kb[starts].reshape(-1).view(np.uint32))
    return int(x ^ np.bitwise_xor.reduce(vb[starts + voff].reshape(-1).view(np.uint32)))


def gpu_xor(pool, wl, block_tables, seq_lens, policy):
    sink = torch.zeros(pc.GATHER_SINK_WORDS, dtype=torch.int32, device="cuda")
    bt = torch.from_numpy(np.ascontiguousarray(block_tables, np.int32)).cuda()
    sl = torch.from_numpy(np.ascontiguousarray(seq_lens, np.int32)).cuda()
    msl = int(max(seq_lens)) if len(seq_lens) else 0
    kw = pool.layout_kwargs()
    pc.gather_read(pool.k, pool.v, bt, sl, msl, sink, num_kv_heads=wl.num_kv_heads, head_size=wl.head_size,
                   num_blocks=kw["num_blocks"], block_stride=kw["block_stride"], token_stride=kw["token_stride"],
                   head_stride=kw["head_stride"], v_offset=kw.get("v_offset", 0), v_cache_policy=policy)
    torch.cuda.synchronize()
    return int(np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32)))


CASES = [("bf16", "hnd", 128, False), ("f16", "nhd", 128, False), ("bf16", "combined", 64, False),
         ("f32", "hnd", 128, False), ("bf16", "hnd", 128, True), ("f16", "nhd", 128, True)]


@pytest.mark.parametrize("dt,layout,D,fp8", CASES, ids=[f"{a}-{b}-d{c}{'-fp8' if d else ''}" for a, b, c, d in CASES])
@pytest.mark.parametrize("policy", [0, 2])
def test_gather_reads_exactly_the_decode_tiles(dt, layout, D, fp8, policy):
    wl = custom(900 + D, dt, 8, 4, D, LENGTHS, layout=layout)
    if fp8:
        wl = fp8_variant(wl)
    pool = gh.filled_pool(wl)
    assert gpu_xor(pool, wl, wl.block_tables, wl.seq_lens, policy) == host_xor(wl, pool, wl.block_tables, wl.seq_lens)


def test_gather_with_shared_blocks_and_a_bad_id():
    """Blocks shared by several sequences are read once per sequence; an id outside the
    pool is not read at all."""
    wl = custom(950, "bf16", 8, 2, 128, LENGTHS, prefix_blocks=40)
    pool = gh.filled_pool(wl)
    bt = wl.block_tables.copy()
    bt[8, 3] = wl.num_blocks + 5
    assert gpu_xor(pool, wl, bt, wl.seq_lens, 2) == host_xor(wl, pool, bt, wl.seq_lens)
