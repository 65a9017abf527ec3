"""GPU parity on a seeded random sweep of small shapes (every byte against the
oracle): random layers, sides (1-4), block sizes, row sizes (any byte count,
so every move width), pool layouts, block and token-stride padding, base
offsets, request counts and token counts, including empty requests; random
merge row sizes and paddings; random copy lists with zero-length objects and
arbitrary alignment, and lists on 16-byte granules whose objects are cut into
pieces, each copied twice. The oracle runs first in every runner, so a case that
does not fit its buffers fails on the CPU before any kernel runs."""
import os

import numpy as np
import pytest

from gpu_util import SENTINEL, run_batch_copy, run_merge, run_pack_unpack, run_unpack_merge, say
from paged_kv_cache_kvm_amd import kvmove as kv
from paged_kv_cache_kvm_amd import workloads as wl

pytestmark = pytest.mark.gpu

# cases per operation; a longer sweep: KVM_RANDOM_CASES=500
CASES = int(os.environ.get("KVM_RANDOM_CASES", "40"))
ROW_BYTES = [1, 2, 3, 5, 8, 12, 16, 24, 48, 64, 100, 256, 576, 1152, 2048]
KINDS = ["dense", "block_major", "slot"]


def _paged_case(i):
    r = np.random.default_rng([2024, i])
    L, S = int(r.integers(1, 6)), int(r.integers(1, 5))
    B, rb = int(r.choice([*range(1, 21), 32, 64])), int(r.choice(ROW_BYTES))
    n = int(r.integers(1, 7))
    Ts = [int(t) for t in r.integers(0, 200, size=n)]
    N = sum(wl.blocks_needed(t, B) for t in Ts) + int(r.integers(1, 20))
    kind = KINDS[int(r.integers(0, 3))]
    block_pad = int(r.choice([0, 0, 0, 3, 8, 16]))
    ts_pad = int(r.choice([0, 0, 5, 16]))
    offset = int(r.choice([0, 0, 1, 4, 8]))
    return L, S, N, B, rb, Ts, kind, block_pad, ts_pad, offset


@pytest.fixture(scope="module")
def ctx(gpu):
    c = kv.Context(0)
    yield c
    c.close()


@pytest.mark.parametrize("i", range(CASES))
def test_random_pack_unpack(ctx, gpu, i):
    L, S, N, B, rb, Ts, kind, bp, tp, off = _paged_case(i)
    run_pack_unpack(ctx, gpu, L, S, N, B, rb, Ts, kind=kind, block_pad=bp, ts_pad=tp, offset=off,
                    seed=3000 + i)


@pytest.mark.parametrize("i", range(CASES))
def test_random_unpack_merge(ctx, gpu, i):
    L, S, N, B, rb, Ts, kind, _, tp, off = _paged_case(100_000 + i)
    r = np.random.default_rng([2025, i])
    reqs = [(t, int(r.integers(0, 60))) for t in Ts]
    N = sum(wl.blocks_needed(h + m, B) for h, m in reqs) + 1
    run_unpack_merge(ctx, gpu, L, S, N, B, rb, reqs, kind=kind, ts_pad=tp,
                     miss_pad=int(r.choice([0, 0, 7, 16])), out_pad=int(r.choice([0, 0, 3, 32])),
                     offset=off, seed=4000 + i)


@pytest.mark.parametrize("i", range(CASES))
def test_random_merge(ctx, gpu, i):
    r = np.random.default_rng([2026, i])
    C = int(r.choice([1, 3, 16, 36, 100, 512, 1152, 4096, 5000]))
    reqs = [(int(r.integers(0, 300)), int(r.integers(0, 100))) for _ in range(int(r.integers(1, 9)))]
    run_merge(ctx, gpu, C, reqs, L=int(r.integers(1, 7)), hit_pad=int(r.choice([0, 0, 3, 16])),
              miss_pad=int(r.choice([0, 0, 5, 16])), out_pad=int(r.choice([0, 0, 1, 32])),
              offset=int(r.choice([0, 0, 1, 8])), seed=5000 + i)


@pytest.mark.parametrize("i", range(CASES))
def test_random_batch_copy(ctx, gpu, i):
    r = np.random.default_rng([2027, i])
    n = int(r.integers(1, 3000))
    lens = r.integers(0, 20000, size=n)
    lens[r.random(n) < 0.05] = 0
    dst_size = int(lens.sum()) + int(r.integers(0, 1 << 16)) + 1
    src_size = int(r.integers(20000, 1 << 22))
    dst_off = wl.placements(6000 + i, 1, lens, dst_size, granule=1)
    src_off = r.integers(0, src_size - lens + 1)
    descs = np.stack([src_off.astype(np.uint64), dst_off.astype(np.uint64),
                      lens.astype(np.uint64)], axis=1)
    say(f"  random copy case {i}")
    run_batch_copy(ctx, gpu, r.integers(0, 256, src_size, dtype=np.uint8),
                   np.full(dst_size, SENTINEL, np.uint8), descs, label=f"random {i}")


@pytest.mark.parametrize("i", range(CASES))
def test_random_batch_copy_pieces(ctx, gpu, i):
    """Lists on 16-byte granules, objects up to 512 KiB (zero to four pieces,
    ragged last pieces), with a share of unaligned, short and empty objects,
    and sometimes nothing but one-piece objects; each list is copied twice, the
    second call with the list's shape known (its grid from the piece count, or
    one workgroup per object)."""
    r = np.random.default_rng([2028, i])
    n = int(r.integers(1, 400))
    lens = 16 * r.integers(1, 32768, size=n)
    uniform = r.random() < 0.3
    if uniform:                                    # every object one piece
        lens = 16 * r.integers(1024, 8193, size=n)
    else:
        odd = r.random(n) < 0.15
        lens[odd] = r.integers(0, 70000, size=int(odd.sum()))       # any length, any size
    slots = (lens + 15) // 16 * 16 + 16          # whole granules, room for a shifted source
    dst_size = int(slots.sum()) + int(r.integers(0, 1 << 16)) + 16
    src_size = int(slots.sum()) + int(r.integers(0, 1 << 16)) + 16
    dst_off = wl.placements(7000 + i, 1, slots, dst_size, granule=16)
    src_off = wl.placements(7000 + i, 2, slots, src_size, granule=16)
    if not uniform:
        shift = r.random(n) < 0.1
        src_off[shift] += r.integers(1, 16, size=int(shift.sum()))   # unaligned sources
    descs = np.stack([src_off.astype(np.uint64), dst_off.astype(np.uint64),
                      lens.astype(np.uint64)], axis=1)
    src_np = r.integers(0, 256, src_size, dtype=np.uint8)
    say(f"  random piece copy case {i} ({n} objects{', one piece each' if uniform else ''})")
    for call in range(2):
        run_batch_copy(ctx, gpu, src_np, np.full(dst_size, SENTINEL, np.uint8), descs,
                       label=f"random pieces {i} call {call}")


@pytest.mark.parametrize("i", range(CASES))
def test_random_batch_copy_one_object(gpu, i):
    """Lists of one object: lengths from 0 to 2 MiB (none to 16 pieces, ragged
    last pieces, often on 16-byte granules, sometimes any length), sources and
    destinations at any alignment inside buffers of random size, sometimes an
    object past a buffer's end (skipped and counted), and workgroup budgets
    from none to below the piece count. Each list is copied twice: the first
    call sizes its grid from the buffers, the second from the piece count the
    first left."""
    r = np.random.default_rng([2029, i])
    ln = int(16 * r.integers(0, 131073)) if r.random() < 0.7 else int(r.integers(0, 1 << 21))
    src_size = ln + int(r.integers(1, 1 << 20))
    dst_size = ln + int(r.integers(1, 1 << 20))
    so = int(r.integers(0, src_size - ln + 1))
    do = int(r.integers(0, dst_size - ln + 1))
    if r.random() < 0.4:                            # both 16-byte aligned
        so, do = so // 16 * 16, do // 16 * 16
    bad = 0
    if r.random() < 0.1:                            # past the end of one buffer
        if r.random() < 0.5:
            so = src_size - max(ln, 1) + int(r.integers(1, 64))
        else:
            do = dst_size - max(ln, 1) + int(r.integers(1, 64))
        ln = max(ln, 1)
        bad = 1
    budget = int(r.choice([0, 0, 0, 1, 3, 7, 64]))
    descs = np.array([[so, do, ln]], np.uint64)
    src_np = r.integers(0, 256, src_size, dtype=np.uint8)
    say(f"  random one-object copy case {i}: {ln} B, src+{so % 16} dst+{do % 16}, budget {budget}")
    c = kv.Context(0)
    try:
        c.set_max_workgroups(budget)
        for call in range(2):
            run_batch_copy(c, gpu, src_np, np.full(dst_size, SENTINEL, np.uint8), descs,
                           expect_skipped=bad, label=f"random one object {i} call {call}")
    finally:
        c.close()
