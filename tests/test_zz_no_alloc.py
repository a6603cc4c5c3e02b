"""pc_paged_attention_split_noalloc: the split decode and its reduce, with the partials
in the library's own device buffer instead of a caller's workspace.

Its output must equal, bit for bit, that of the split path with a caller-allocated
workspace (pc_paged_attention_decode with 512-token partitions, then
pc_paged_attention_reduce): the same kernels on the same inputs.  Calls come in a row,
each later one smaller than the one before, so that what an earlier call left in the
buffer would show if a later call read it.  The first small case is also held to the
fp64 oracle, and no call after a GPU's first may change the device's free memory.
"""

import numpy as np
import pytest
import torch

import gpu_harness as gh
import oracle
import paged_kv_cache_reshape_amd as pc
from test_gpu_parity import check_attention
from workloads import alibi_variant, custom, make_config

pytestmark = pytest.mark.gpu

_BITS = {torch.float32: torch.int32, torch.float16: torch.int16, torch.bfloat16: torch.int16}


def noalloc(pool, inp, msl=None):
    wl = pool.wl
    out = torch.full_like(inp.q, float("nan"))
    pc.paged_attention_split_noalloc(out, inp.q, pool.k, pool.v, inp.block_tables, inp.seq_lens,
                                     inp.max_seq_len if msl is None else msl, num_kv_heads=wl.num_kv_heads,
                                     scale=float(wl.scale), alibi_slopes=inp.alibi, **pool.layout_kwargs())
    return out


def with_workspace(pool, inp):
    out, path = gh.decode(pool, inp, "split")
    assert path == "split"
    return out


def assert_same_bits(a, b, what):
    torch.cuda.synchronize()
    assert a.shape == b.shape and a.dtype == b.dtype
    same = torch.equal(a.view(_BITS[a.dtype]), b.view(_BITS[b.dtype]))
    print(f"{what}: {'identical' if same else 'DIFFERENT'} bits over {a.numel()} outputs", flush=True)
    assert same, what


def free_bytes():
    torch.cuda.synchronize()
    return torch.cuda.mem_get_info()[0]


class RandomPool:
    """A pool of random 16-bit values on the device, laid out as the workload says (no
    host copy: only the two GPU paths are compared on it)."""

    def __init__(self, wl, dtype):
        g = torch.Generator(device="cuda").manual_seed(1234)
        self.wl = wl
        self.k = torch.randn(wl.pool_elems, dtype=dtype, device="cuda", generator=g)
        self.v = self.k if wl.layout == "combined" else torch.randn(wl.pool_elems, dtype=dtype, device="cuda",
                                                                      generator=g)
        self.fp8 = False
        self.v_offset = wl.v_offset if wl.layout == "combined" else 0

    def layout_kwargs(self):
        w = self.wl
        return dict(num_blocks=w.num_blocks, block_stride=w.block_stride, token_stride=w.token_stride,
                    head_stride=w.head_stride, block_size=w.block_size, v_offset=self.v_offset)


class RandomInputs:
    def __init__(self, wl, dtype):
        g = torch.Generator(device="cuda").manual_seed(99)
        self.q = torch.randn(wl.num_seqs, wl.num_q_heads, wl.head_size, dtype=dtype, device="cuda", generator=g)
        self.seq_lens_host = np.asarray(wl.seq_lens, np.int32)
        self.seq_lens = torch.from_numpy(self.seq_lens_host.copy()).cuda()
        self.block_tables = torch.from_numpy(np.ascontiguousarray(wl.block_tables, np.int32)).cuda()
        self.max_seq_len = int(self.seq_lens_host.max())
        self.alibi = None


def test_noalloc_matches_workspace_path_over_calls_in_a_row():
    # 1: the mixed-serving workload at full size (256 sequences up to 8192 tokens, 32
    #    heads of 128, fp16, a 1024-token shared prefix): 68 MB of partials
    big = make_config(4, contents=False)
    bpool, binp = RandomPool(big, torch.float16), RandomInputs(big, torch.float16)
    print(f"call 1: {big.name}, partitions {-(-binp.max_seq_len // 512)}", flush=True)
    got1 = noalloc(bpool, binp)
    assert_same_bits(got1, with_workspace(bpool, binp), "call 1 (mixed serving, full size)")
    del bpool, binp

    # 2: smaller, bf16, head size 128, GQA 4, lengths across partition edges, empty ones
    wl2 = custom(71, "bf16", 16, 4, 128, [0, 1, 511, 512, 513, 1024, 1500, 0, 3000], layout="hnd")
    pool2, inp2 = gh.filled_pool(wl2), gh.DecodeInputs(wl2)
    free0 = free_bytes()
    got2 = noalloc(pool2, inp2)
    assert free_bytes() == free0, "the call changed the device's free memory"
    assert_same_bits(got2, with_workspace(pool2, inp2), "call 2 (bf16 D128 G4)")
    check_attention(gh.out_f64(got2), oracle.decode(wl2, oracle.filled_pool(wl2)), "bf16", "call 2 against the oracle")

    # 3: smaller still, fp16, head size 64 in the combined-block layout, ALiBi
    rng = np.random.default_rng(3)
    wl3 = alibi_variant(custom(72, "f16", 8, 2, 64, [700, 5, 1030], layout="combined"),
                        slopes=rng.uniform(-0.2, 0.2, 8).astype(np.float32))
    pool3, inp3 = gh.filled_pool(wl3), gh.DecodeInputs(wl3)
    free0 = free_bytes()
    got3 = noalloc(pool3, inp3)
    assert free_bytes() == free0, "the call changed the device's free memory"
    assert_same_bits(got3, with_workspace(pool3, inp3), "call 3 (f16 D64 combined, ALiBi)")
    check_attention(gh.out_f64(got3), oracle.decode(wl3, oracle.filled_pool(wl3)), "f16", "call 3 against the oracle")


def test_noalloc_fp32_and_a_single_partition():
    for seed, lens in ((73, [1, 200, 511]), (74, [512, 600])):  # P = 1, then P = 2
        wl = custom(seed, "f32", 4, 2, 128, lens)
        pool, inp = gh.filled_pool(wl), gh.DecodeInputs(wl)
        assert_same_bits(noalloc(pool, inp), with_workspace(pool, inp), f"fp32 {lens}")


def test_noalloc_refuses_what_does_not_fit():
    """Partials beyond the buffer: PC_ERR_TOO_LARGE before anything is enqueued (out keeps
    its NaNs); the largest request that fits runs."""
    S, Hq, D = 64, 64, 128
    msl = 32768  # 64 partitions: 64 * 64 * 64 * 130 * 4 bytes = 136 MB > 128 MiB
    rows = S * Hq * (msl // 512)
    assert 4 * (rows * D + 2 * rows) > pc.NOALLOC_SCRATCH_BYTES
    q = torch.zeros(S, Hq, D, dtype=torch.bfloat16, device="cuda")
    out = torch.full_like(q, float("nan"))
    pool = torch.zeros(8 * 16 * D * 8, dtype=torch.bfloat16, device="cuda")  # 8 blocks, 8 kv heads, HND
    tables = torch.zeros(S, msl // 16, dtype=torch.int32, device="cuda")
    lens = torch.ones(S, dtype=torch.int32, device="cuda")
    lay = dict(num_kv_heads=8, scale=D ** -0.5, num_blocks=8, block_stride=8 * 16 * D, token_stride=D,
               head_stride=16 * D, block_size=16)
    with pytest.raises(pc.PagedCacheError) as e:
        pc.paged_attention_split_noalloc(out, q, pool, pool, tables, lens, msl, **lay)
    assert e.value.status == -4
    torch.cuda.synchronize()
    assert torch.isnan(out).all()
    # 60 partitions fit (64 * 64 * 60 * 130 * 4 bytes = 128 MB): every sequence holds one token
    pc.paged_attention_split_noalloc(out, q, pool, pool, tables, lens, 60 * 512, **lay)
    torch.cuda.synchronize()
    assert torch.equal(out, torch.zeros_like(out))  # q = 0 and K = V = 0 everywhere: zeros


def test_noalloc_under_graph_capture():
    """The entry point's reason to exist: it can be recorded into a HIP graph (it allocates
    nothing and enqueues only kernels).  The graph is replayed several times with eager
    work and synchronisations between the replays; every replay equals the eager call."""
    wl = custom(75, "bf16", 16, 4, 128, [1, 300, 513, 1400, 2000], layout="hnd")
    pool, inp = gh.filled_pool(wl), gh.DecodeInputs(wl)
    ref = noalloc(pool, inp)  # eager (also the device's first call, outside the capture)
    torch.cuda.synchronize()
    out = torch.full_like(inp.q, float("nan"))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm the capture stream outside the graph
        pc.paged_attention_split_noalloc(out, inp.q, pool.k, pool.v, inp.block_tables, inp.seq_lens,
                                         inp.max_seq_len, num_kv_heads=wl.num_kv_heads, scale=float(wl.scale),
                                         **pool.layout_kwargs())
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        pc.paged_attention_split_noalloc(out, inp.q, pool.k, pool.v, inp.block_tables, inp.seq_lens,
                                         inp.max_seq_len, num_kv_heads=wl.num_kv_heads, scale=float(wl.scale),
                                         **pool.layout_kwargs())
    for r in range(4):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert_same_bits(out, ref, f"graph replay {r}")
        noalloc(pool, inp)  # eager work on the same buffer between replays
        torch.cuda.synchronize()
