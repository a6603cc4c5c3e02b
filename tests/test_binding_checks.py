"""The binding's host-side shape and extent checks: a mismatch raises ValueError
before anything reaches the library (so no kernel can read or write past a buffer).

The check helpers only look at shapes, so they run here on CPU tensors; the GPU test
drives the public functions with device tensors and mismatched shapes.
"""

import pytest
import torch

from paged_kv_cache_reshape_amd import _native as N

HND = dict(num_blocks=4, block_stride=2 * 16 * 64, token_stride=64, head_stride=16 * 64, block_size=16,
           num_kv_heads=2, head_size=64)


def test_pool_extent_is_one_past_the_last_element():
    # block 3, row 15, head 1, dim 63 of an HND pool of 4 blocks is its last element
    assert N._pool_extent(**HND) == 4 * 2 * 16 * 64


def test_pool_too_small_is_refused():
    ok = torch.empty(4 * 2 * 16 * 64)
    N._check_pool(ok, ok, 0, **HND)
    with pytest.raises(ValueError, match="k_pool"):
        N._check_pool(torch.empty(ok.numel() - 1), ok, 0, **HND)
    with pytest.raises(ValueError, match="v_pool"):
        N._check_pool(ok, ok, 1, **HND)  # V one element further in: its last element is out


def test_combined_block_extent():
    # one buffer, K for 16 tokens then V at +16*Hkv*D: strides {2*16*Hkv*D, Hkv*D, D}
    Hkv, D, nb = 8, 64, 3
    lay = dict(num_blocks=nb, block_stride=2 * 16 * Hkv * D, token_stride=Hkv * D, head_stride=D, block_size=16,
               num_kv_heads=Hkv, head_size=D)
    buf = torch.empty(nb * 2 * 16 * Hkv * D)
    N._check_pool(buf, buf, 16 * Hkv * D, **lay)
    with pytest.raises(ValueError):
        N._check_pool(buf[:-1], buf[:-1], 16 * Hkv * D, **lay)


def test_sequence_inputs_must_match_num_seqs():
    N._check_seq_inputs(3, torch.empty(3, 5), torch.empty(3))
    with pytest.raises(ValueError, match="block_tables"):
        N._check_seq_inputs(3, torch.empty(2, 5), torch.empty(3))
    with pytest.raises(ValueError, match="seq_lens"):
        N._check_seq_inputs(3, torch.empty(3, 5), torch.empty(4))


def test_partials_shape_follows_max_seq_len():
    S, Hq, D = 2, 8, 128
    good = (torch.empty(S, Hq, 3), torch.empty(S, Hq, 3), torch.empty(S, Hq, 3, D))
    N._check_partials(S, Hq, D, 1025, 512, *good)  # ceil(1025 / 512) = 3
    with pytest.raises(ValueError):
        N._check_partials(S, Hq, D, 1024, 512, *good)  # the decode would lay them out with P = 2
    with pytest.raises(ValueError):
        N._check_partials(S, Hq, D, 1025, 512, good[0], good[1], torch.empty(S, Hq, 3, 64))
    with pytest.raises(ValueError):
        N._check_partials(S, Hq, D, 1025, 0, *good)  # the one-pass path takes none
    with pytest.raises(ValueError):
        N._check_partials(S, Hq, D, 1025, 512, None, good[1], good[2])
    N._check_partials(S, Hq, D, 0, 512, *good)  # nothing is written or read


@pytest.mark.gpu
def test_public_calls_refuse_mismatched_shapes():
    import paged_kv_cache_reshape_amd as pc
    dev = "cuda"
    S, Hq, Hkv, D, nb = 2, 8, 2, 64, 4
    lay = dict(num_blocks=nb, block_stride=Hkv * 16 * D, token_stride=D, head_stride=16 * D, block_size=16)
    pool = torch.zeros(nb * Hkv * 16 * D, dtype=torch.bfloat16, device=dev)
    small = pool[:-8]
    q = torch.zeros(S, Hq, D, dtype=torch.bfloat16, device=dev)
    out = torch.empty_like(q)
    bt = torch.zeros(S, 2, dtype=torch.int32, device=dev)
    sl = torch.full((S,), 20, dtype=torch.int32, device=dev)
    kw = dict(num_kv_heads=Hkv, scale=0.125, **lay)
    pc.paged_attention_decode(out, q, pool, pool, bt, sl, 20, **kw)  # well-formed: runs
    with pytest.raises(ValueError):
        pc.paged_attention_decode(out, q, small, pool, bt, sl, 20, **kw)
    with pytest.raises(ValueError):
        pc.paged_attention_decode(out, q, pool, pool, bt[:1], sl, 20, **kw)
    with pytest.raises(ValueError):
        pc.paged_attention_decode(out, q, pool, pool, bt, sl[:1], 20, **kw)
    key = torch.zeros(3, Hkv, D, dtype=torch.bfloat16, device=dev)
    slots = torch.zeros(3, dtype=torch.int64, device=dev)
    with pytest.raises(ValueError):
        pc.reshape_and_cache(key, key, small, pool, slots, **lay)
    es = torch.empty(S, Hq, 2, device=dev)
    tmp = torch.empty(S, Hq, 2, D, device=dev)
    with pytest.raises(ValueError):  # the reduce's out must match the partials
        pc.paged_attention_reduce(out[:1], es, es, tmp, sl)
    torch.cuda.synchronize()


@pytest.mark.gpu
def test_prefix_and_noalloc_calls_refuse_mismatched_shapes():
    import paged_kv_cache_reshape_amd as pc
    dev = "cuda"
    S, Hq, Hkv, D, nb = 2, 8, 2, 64, 40
    lay = dict(num_blocks=nb, block_stride=Hkv * 16 * D, token_stride=D, head_stride=16 * D, block_size=16)
    pool = torch.zeros(nb * Hkv * 16 * D, dtype=torch.bfloat16, device=dev)
    q = torch.zeros(S, Hq, D, dtype=torch.bfloat16, device=dev)
    bt = torch.arange(S * 20, dtype=torch.int32, device=dev).reshape(S, 20) % nb
    bt[1, :16] = bt[0, :16]  # the first 16 blocks shared
    sl = torch.full((S,), 300, dtype=torch.int32, device=dev)
    P = 1
    es, ml, tmp = (torch.empty(S, Hq, P, device=dev), torch.empty(S, Hq, P, device=dev),
                   torch.empty(S, Hq, P, D, device=dev))
    pt = bt[0, :16].contiguous()
    shared = torch.full((S,), 256, dtype=torch.int32, device=dev)
    kw = dict(num_kv_heads=Hkv, scale=0.125, exp_sums=es, max_logits=ml, tmp_out=tmp, **lay)
    pc.paged_attention_decode_prefix(q, pool, pool, bt, sl, 300, prefix_table=pt, shared_lens=shared, **kw)  # runs
    with pytest.raises(ValueError):  # one shared count per sequence
        pc.paged_attention_decode_prefix(q, pool, pool, bt, sl, 300, prefix_table=pt, shared_lens=shared[:1], **kw)
    with pytest.raises(ValueError):  # block ids are int32
        pc.paged_attention_decode_prefix(q, pool, pool, bt, sl, 300, prefix_table=pt.long(), shared_lens=shared, **kw)
    with pytest.raises(ValueError):  # partials sized for the decode's partitions
        pc.paged_attention_decode_prefix(q, pool, pool, bt, sl, 600, prefix_table=pt, shared_lens=shared, **kw)
    out = torch.empty_like(q)
    nkw = dict(num_kv_heads=Hkv, scale=0.125, **lay)
    pc.paged_attention_split_noalloc(out, q, pool, pool, bt, sl, 300, **nkw)  # runs
    with pytest.raises(ValueError):
        pc.paged_attention_split_noalloc(out[:1], q, pool, pool, bt, sl, 300, **nkw)
    with pytest.raises(ValueError):
        pc.paged_attention_split_noalloc(out, q, pool[:-8], pool, bt, sl, 300, **nkw)
    torch.cuda.synchronize()
