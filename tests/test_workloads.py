"""Seeded input generators: shapes, disjointness and the pages' counts (CPU only)."""
import numpy as np
import pytest

import oracle
from paged_kv_cache_kvm_amd import workloads as wl


def test_block_tables_disjoint_and_sized():
    w = wl.LLAMA8B
    per = [wl.blocks_needed(t, w.shape.block_tokens) for t in w.t_all]
    assert per == [2080] * 8
    tabs = wl.block_tables(w.seed, 1, w.pool_blocks, per)
    oracle.check_block_tables(tabs, w.pool_blocks)
    again = wl.block_tables(w.seed, 1, w.pool_blocks, per)
    assert all(np.array_equal(a, b) for a, b in zip(tabs, again)), "not reproducible"
    with pytest.raises(ValueError):
        wl.block_tables(1, 1, 10, [6, 5])


def test_placements_disjoint():
    rng = np.random.default_rng(0)
    lens = 256 * rng.integers(1, 50, size=5000)
    off = wl.placements(3, 4, lens, int(lens.sum()) + 256 * 777, 256)
    assert np.all(off % 256 == 0)
    order = np.argsort(off)
    ends = off[order] + lens[order]
    assert np.all(off[order][1:] >= ends[:-1]), "overlap"
    assert ends[-1] <= int(lens.sum()) + 256 * 777
    # exact fit: no slack at all
    tight = wl.placements(3, 5, lens, int(lens.sum()), 256)
    o = np.argsort(tight)
    assert tight[o][0] == 0 and np.all(tight[o][1:] == (tight[o] + lens[o])[:-1])


def test_small_objects_workload():
    w = wl.SMALL_OBJS
    d = wl.small_object_descs(w)
    assert d.shape == (200000, 3)
    lens = d[:, 2].astype(np.int64)
    assert lens.min() >= 4096 and lens.max() <= 131072 and np.all(lens % 256 == 0)
    for col, arena in ((0, w.src_arena), (1, w.dst_arena)):
        off = d[:, col].astype(np.int64)
        o = np.argsort(off)
        assert np.all(off[o][1:] >= (off[o] + lens[o])[:-1])
        assert (off + lens).max() <= arena
    # about 13.5 GB each way, as sized
    assert 12.5e9 < lens.sum() < 14.5e9


def test_qwen32b_objects_match_page_counts():
    """The restore list of one 128000-token sequence has the 2,000 blocks and
    256,000 objects that the Tutti reading notes print (prerequisites 5, eq. 3-4)."""
    descs, bt, pool_bytes = wl.qwen32b_object_descs()
    sh = wl.QWEN32B_SHAPE
    assert len(bt) == oracle.blocks_for_tokens(wl.QWEN32B_TOKENS, sh.block_tokens) == 2000
    n = oracle.objects_for_tokens(wl.QWEN32B_TOKENS, sh.block_tokens, sh.layers, sh.sides)
    assert descs.shape[0] == n == 256000
    assert np.all(descs[:, 2] == 64 * 8 * 128 * 2)  # 128 KiB objects
    # destinations tile the pool exactly once
    dst = np.sort(descs[:, 1].astype(np.int64))
    assert dst[0] == 0 and np.all(np.diff(dst) == 131072) and dst[-1] + 131072 == pool_bytes
    src = descs[:, 0].astype(np.int64)
    o = np.argsort(src)
    assert np.all(src[o][1:] >= src[o][:-1] + 131072) and src.max() + 131072 <= wl.QWEN32B_STAGING


def test_mla_agentic_draws():
    w = wl.mla_agentic()
    assert len(w.t_hit) == 64 and len(w.t_miss) == 64
    assert min(w.t_hit) >= 16384 and max(w.t_hit) <= 65536
    assert min(w.t_miss) >= 128 and max(w.t_miss) <= 1024
    assert w.shape.row_bytes == 1152 and w.shape.sides == 1 and w.slot_pool
    assert wl.mla_agentic().t_hit == w.t_hit


def test_bf16_rounding_matches_torch():
    import torch
    bits = wl.bf16_normal_bits(5, 6, 100000)
    x = np.random.default_rng([5, 6]).standard_normal(100000, dtype=np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bits, ref)
