"""The planner against its measured table (profiles/planner_table.md): for every batch
shape there, pc_paged_attention_plan_lens must pick a path whose measured time is close
to the faster of what the library can run -- the one-pass kernel the decode picks for
that batch, or the split path with its reduce.  CPU only: the planner is host code.
"""

import os
import re

import pytest
import torch

import bench
import paged_kv_cache_reshape_amd as pc

TABLE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "profiles", "planner_table.md")
CUS = 256  # MI355X; the planner's fallback when no device is visible


def onepass_grid(units, max_len):
    """The decode's one-pass kernel choice as pc.h documents it (16-bit pools)."""
    return max_len <= 512 or (units >= 32 * CUS and max_len <= 2048)


def rows():
    out = []
    for line in open(TABLE):
        m = re.match(r"\| (\d+) \| (\d+) \| (\d+) \| (\d+) \| (\w+) \| (\d+) \| [\d.]+ \| ([\d.]+) \| ([\d.]+) "
                     r"\| ([\d.]+) \|", line)
        if m:
            Hq, Hkv, U, ml = (int(m.group(i)) for i in range(1, 5))
            out.append((Hq, Hkv, U, ml, m.group(5), int(m.group(6)), float(m.group(7)), float(m.group(8)),
                        float(m.group(9))))
    return out


def test_table_is_complete():
    r = rows()
    assert len(r) >= 210
    assert {x[1] for x in r} == {8, 32}
    assert sum(1 for x in r if x[5]) >= 24  # batches with a shared prefix


def test_planner_picks_the_faster_path():
    losses = []
    for Hq, Hkv, U, ml, mix, prefix, t_pers, t_grid, t_split in rows():
        lens = bench.grid_lengths(U // Hkv, ml, mix, Hkv)
        ps, P, ws = pc.paged_attention_plan_lens(lens, Hq, Hkv, 128, 16 * 128, torch.bfloat16,
                                                 shared_lens=bench.grid_shared_lens(lens, prefix))
        assert ps in (0, pc.PARTITION_SIZE) and P == (-(-ml // 512) if ps else 1)
        t_one = t_grid if onepass_grid(U, ml) else t_pers
        chosen = t_split if ps else t_one
        losses.append((chosen / min(t_one, t_split), chosen / min(t_pers, t_grid, t_split), (Hq, Hkv, U, ml, mix, prefix)))
    within = sum(1 for l2, _, _ in losses if l2 <= 1.05)
    worst = max(losses)
    print(f"planner: {within}/{len(losses)} within 5% of the faster path, worst {worst[0]:.3f} at {worst[2]}; "
          f"against the fastest of the three kernels: worst {max(l3 for _, l3, _ in losses):.3f}")
    assert within >= 0.97 * len(losses)
    assert worst[0] <= 1.12


def test_planner_without_lengths_on_the_workloads():
    """pc_paged_attention_plan takes every sequence at max_seq_len: the measured winners
    of uniform-length batches."""
    bf16 = torch.bfloat16
    assert pc.paged_attention_plan(64, 32, 8, 128, 2048, bf16)[0] == 0  # 512 units x 2048: one pass
    assert pc.paged_attention_plan(4, 32, 8, 128, 32768, bf16)[0] == 512  # 32 units x 32768: split
    assert pc.paged_attention_plan(16, 32, 8, 128, 8192, bf16)[0] == 512  # 128 units x 8192: split
    assert pc.paged_attention_plan(512, 32, 8, 128, 8192, bf16)[0] == 0  # 4096 units x 8192: one pass


def workload_rows():
    out = []
    for line in open(TABLE):
        m = re.match(r"\| (\d) \| `(\w+)` \| ([\d.]+) \| ([\d.]+) \|", line)
        if m:
            out.append((int(m.group(1)), m.group(2), float(m.group(3)), float(m.group(4))))
    return out


def test_planner_on_the_five_workloads():
    """Each workload, timed on both paths (the table's last section): the planner, given
    its lengths and its shared prefix tokens, picks the faster."""
    from workloads import make_config
    rows = workload_rows()
    assert [r[0] for r in rows] == [0, 1, 2, 3, 4]
    dt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
    for idx, name, t_one, t_split in rows:
        wl = make_config(idx, contents=False)
        assert wl.name == name
        ps, _, _ = pc.paged_attention_plan_lens(wl.seq_lens, wl.num_q_heads, wl.num_kv_heads, wl.head_size,
                                                 wl.head_stride, dt[wl.dtype], shared_lens=wl.shared_lens())
        faster_split = t_split < t_one
        assert bool(ps) == faster_split, (name, ps, t_one, t_split)


def test_plan_lens_refuses_inconsistent_shared_counts():
    lens = [600, 1100]
    with pytest.raises(pc.PagedCacheError):  # more shared tokens than the sequence has
        pc.paged_attention_plan_lens(lens, 32, 8, 128, 16 * 128, torch.bfloat16, shared_lens=[700, 1024])
    with pytest.raises(pc.PagedCacheError):
        pc.paged_attention_plan_lens(lens, 32, 8, 128, 16 * 128, torch.bfloat16, shared_lens=[-16, 0])
    with pytest.raises(ValueError):  # one entry per sequence
        pc.paged_attention_plan_lens(lens, 32, 8, 128, 16 * 128, torch.bfloat16, shared_lens=[0])
    pc.paged_attention_plan_lens(lens, 32, 8, 128, 16 * 128, torch.bfloat16, shared_lens=[592, 1024])
