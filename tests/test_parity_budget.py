"""GPU parity under a workgroup budget (kvm_ctx_set_max_workgroups): with the
grid capped below the tile count every workgroup loops over several tiles,
and every byte must still equal the oracle's. Budgets of 1 (one workgroup
walks every tile), small odd counts (uneven strides over the tiles) and one
above the tile count (the budget has no effect) are covered for every
operation, plus bad block ids met inside a workgroup's loop."""
import numpy as np
import pytest
import torch

from gpu_util import (SENTINEL, case_seed, down, run_batch_copy, run_merge,
                      run_pack_unpack, run_unpack_merge, say, up)
from paged_kv_cache_kvm_amd import kvmove as kv
from paged_kv_cache_kvm_amd import workloads as wl

pytestmark = pytest.mark.gpu

BUDGETS = [1, 3, 7, 100000]


@pytest.fixture(scope="module")
def ctx(gpu):
    c = kv.Context(0)
    yield c
    c.close()


@pytest.fixture
def budget_ctx(ctx, request):
    say(f"  workgroup budget {request.param}")
    ctx.set_max_workgroups(request.param)
    yield ctx
    ctx.set_max_workgroups(0)


@pytest.mark.parametrize("budget_ctx", BUDGETS, indirect=True)
@pytest.mark.parametrize("case", [
    # (L, S, N, B, rb, Ts, kind)
    (4, 2, 64, 16, 256, [240, 17, 1], "dense"),
    (5, 2, 500, 3, 48, [2, 1] * 70, "dense"),        # 140 sequences: two launches
    (3, 1, 300, 64, 1152, [700, 65, 0], "slot"),
    (2, 2, 30, 4, 5, [23, 9], "block_major"),         # byte moves
    (3, 3, 50, 8, 64, [40, 9], "block_major"),        # three sides
], ids=["dense", "many-seqs", "mla-slot", "bytes", "three-sides"])
def test_budget_pack_unpack(budget_ctx, gpu, case):
    L, S, N, B, rb, Ts, kind = case
    run_pack_unpack(budget_ctx, gpu, L, S, N, B, rb, Ts, kind=kind,
                    seed=case_seed(case))


@pytest.mark.parametrize("budget_ctx", BUDGETS, indirect=True)
@pytest.mark.parametrize("case", [
    # (C, reqs, L, hit_pad, miss_pad, out_pad, offset)
    (4096, [(300, 20), (0, 9), (13, 0), (0, 0), (64, 64)], 32, 0, 0, 0, 0),
    (36, [(5, 3)] * 90, 3, 4, 12, 28, 0),
    (1152, [(1000, 77), (300, 5)], 61, 0, 0, 0, 0),  # short 16-byte rows: ~50 KiB tiles
], ids=["llama-rows", "many-reqs", "mla-rows"])
def test_budget_merge(budget_ctx, gpu, case):
    C, reqs, L, hp, mp, op, off = case
    run_merge(budget_ctx, gpu, C, reqs, L=L, hit_pad=hp, miss_pad=mp, out_pad=op, offset=off,
              seed=case_seed(case))


@pytest.mark.parametrize("budget_ctx", BUDGETS, indirect=True)
@pytest.mark.parametrize("case", [
    # (L, S, N, B, rb, reqs, kind)
    (3, 2, 200, 16, 512, [(300, 20), (0, 9), (13, 0), (0, 0), (64, 64)], "dense"),
    (2, 2, 700, 3, 48, [(5, 2), (1, 1)] * 70, "block_major"),
    (2, 3, 100, 4, 32, [(23, 5), (9, 0), (0, 3)], "dense"),     # three sides
    (3, 1, 300, 64, 1152, [(700, 77), (65, 3)], "slot"),        # wide items: split stores
], ids=["mixed", "many-reqs", "three-sides", "mla-slot"])
def test_budget_unpack_merge(budget_ctx, gpu, case):
    L, S, N, B, rb, reqs, kind = case
    run_unpack_merge(budget_ctx, gpu, L, S, N, B, rb, reqs, kind=kind,
                     seed=case_seed(case))


@pytest.mark.parametrize("budget_ctx", BUDGETS, indirect=True)
def test_budget_batch_copy(budget_ctx, gpu):
    rng = np.random.default_rng(77)
    lens = np.concatenate([256 * rng.integers(16, 512, endpoint=True, size=500),
                           rng.integers(0, 300, size=500)])
    slots = (lens + 255) // 256 * 256            # placements take whole 256-byte granules
    arena = int(slots.sum()) + (8 << 20)
    src_off = wl.placements(77, 1, slots, arena) + rng.integers(0, 16, size=lens.size)
    dst_off = wl.placements(77, 2, slots, arena)
    descs = np.stack([src_off.astype(np.uint64), dst_off.astype(np.uint64),
                      lens.astype(np.uint64)], axis=1)
    run_batch_copy(budget_ctx, gpu, rng.integers(0, 256, arena + 16, dtype=np.uint8),
                   np.full(arena, SENTINEL, np.uint8), descs, label="mixed sizes, budget")


@pytest.mark.parametrize("budget_ctx", BUDGETS, indirect=True)
@pytest.mark.parametrize("kind", ["one-piece", "multi-piece"])
def test_budget_batch_copy_pieces(budget_ctx, gpu, kind):
    """Aligned objects cut into pieces (16-128 KiB: one piece each; 16-512 KiB:
    up to four), so that a budgeted grid walks several pieces per workgroup;
    each list copied twice, the second time with its shape known (one
    workgroup per object only where the budget allows a grid that large)."""
    rng = np.random.default_rng(79 if kind == "one-piece" else 80)
    hi = 8 if kind == "one-piece" else 32
    lens = 16384 * rng.integers(1, hi + 1, size=300)
    arena = int(lens.sum()) + (8 << 20)
    descs = np.stack([wl.placements(79, 1, lens, arena), wl.placements(79, 2, lens, arena),
                      lens], axis=1).astype(np.uint64)
    src_np = rng.integers(0, 256, arena, dtype=np.uint8)
    for call in range(2):
        run_batch_copy(budget_ctx, gpu, src_np, np.full(arena, SENTINEL, np.uint8), descs,
                       label=f"{kind}, budget, call {call}")


@pytest.mark.parametrize("budget_ctx", BUDGETS, indirect=True)
def test_budget_batch_copy_short_list(budget_ctx, gpu):
    """40 objects (one launch, shares found by each wavefront's own scan), one
    of them 4 MiB so that it spans many shares, and one out of range."""
    rng = np.random.default_rng(78)
    lens = rng.integers(0, 5000, size=40)
    lens[7] = 4 << 20
    arena = int(lens.sum()) + (1 << 16)
    src_off = wl.placements(78, 1, lens, arena, 1)
    dst_off = wl.placements(78, 2, lens, arena, 1)
    descs = np.stack([src_off.astype(np.uint64), dst_off.astype(np.uint64),
                      lens.astype(np.uint64)], axis=1)
    descs[30] = (arena - 3, 0, 9)                 # source runs past its buffer
    run_batch_copy(budget_ctx, gpu, rng.integers(0, 256, arena, dtype=np.uint8),
                   np.full(arena, SENTINEL, np.uint8), descs, expect_skipped=1,
                   label="short list, budget")


@pytest.mark.parametrize("budget_ctx", [1, 2], indirect=True)
def test_budget_bad_block_ids(budget_ctx, gpu):
    """A bad id skips its tile inside a workgroup's loop; the tiles after it in
    the same workgroup are still moved."""
    L, S, N, B, RB = 3, 2, 8, 4, 16
    layout = kv.pool_layout(S, B, RB, B * RB, N * B * RB, S * N * B * RB, N)
    pool = up(np.full(L * S * N * B * RB, SENTINEL, np.uint8), gpu)
    full_np = (np.arange(16 * L * S * RB, dtype=np.uint32) % 251).astype(np.uint8)
    full = up(full_np, gpu)
    bt = up(np.array([3, N, -1, 1], np.int32), gpu)          # entries 1 and 2 out of range
    kv.kvm_unpack_layer(budget_ctx.handle, layout, pool, L, 1, [kv.seq(bt, full, 16)])
    assert budget_ctx.take_device_errors() == 2
    p = down(pool).reshape(L, S, N, B, RB)
    rows = full_np.reshape(16, L, S, RB)
    for b, n in ((0, 3), (3, 1)):
        for s in range(S):
            assert np.array_equal(p[1, s, n], rows[b * B:(b + 1) * B, 1, s])
    touched = {n for n in range(N) if not np.all(p[1, :, n] == SENTINEL)}
    assert touched == {3, 1}
    assert np.all(np.delete(p, 1, axis=0) == SENTINEL)

    packed = up(np.full(16 * L * S * RB, SENTINEL, np.uint8), gpu)
    kv.kvm_pack_full(budget_ctx.handle, layout, pool, L, [kv.seq(bt, packed, 16)])
    assert budget_ctx.take_device_errors() == 2 * L
    got = down(packed).reshape(16, L, S, RB)
    for b, n in ((0, 3), (3, 1)):
        assert np.array_equal(got[b * B:(b + 1) * B].transpose(1, 2, 0, 3), p[:, :, n])
    assert np.all(got[B:3 * B] == SENTINEL)


def test_budget_rejects_negative(ctx, gpu):
    with pytest.raises(kv.KvmError):
        ctx.set_max_workgroups(-1)
    ctx.set_max_workgroups(0)
    torch.cuda.synchronize()
