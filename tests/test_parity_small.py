"""GPU parity at oracle-friendly sizes: every byte of every output of the HIP
library (called through the C ABI) equals the oracle's on the same seeded
inputs. Shapes span several tiles, ragged tails, every move width, every
layout the pool descriptor allows, and the degenerate cases."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import (SENTINEL, case_seed, down, run_batch_copy, run_merge,
                      run_pack_unpack, run_unpack_merge, say, up)
from paged_kv_cache_kvm_amd import kvmove as kv
from paged_kv_cache_kvm_amd import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ctx(gpu):
    c = kv.Context(0)
    yield c
    c.close()


def test_tiny_workload(ctx, gpu):
    """The tiny workload end to end with its bf16 payload: pack_full(T_all),
    unpack of the 240 hit tokens for every layer, merge for every layer."""
    w = wl.TINY
    sh = w.shape
    L, S, B, rb, N = sh.layers, sh.sides, sh.block_tokens, sh.row_bytes, w.pool_blocks
    C = sh.c_kv_bytes
    t_hit, t_miss = w.t_hit[0], w.t_miss[0]
    t_all = t_hit + t_miss
    say(f"  tiny workload seed={w.seed}")
    pool_np = wl.bf16_normal_bits(w.seed, 1, L * S * N * B * rb // 2).view(np.uint8)
    bt_np = wl.block_tables(w.seed, 2, N, [wl.blocks_needed(t_all, B)])[0]
    layout = kv.pool_layout(S, B, rb, B * rb, N * B * rb, S * N * B * rb, N)
    ref = oracle.pool_struct(S, B, rb, B * rb, N * B * rb, S * N * B * rb, N)
    pool, bt = up(pool_np, gpu), up(bt_np, gpu)
    full = torch.zeros(t_all * L * C, dtype=torch.uint8, device=gpu)
    kv.kvm_pack_full(ctx.handle, layout, pool, L, [kv.seq(bt, full, t_all)])
    full_ref = np.zeros(t_all * L * C, np.uint8)
    oracle.pack_full(pool_np, ref, L, bt_np, t_all, full_ref)
    torch.cuda.synchronize()
    assert np.array_equal(down(full), full_ref)

    miss_np = wl.bf16_normal_bits(w.seed, 3, L * t_miss * C // 2).view(np.uint8)
    miss = up(miss_np, gpu)
    pool_b = up(np.full(pool_np.size, SENTINEL, np.uint8), gpu)
    pool_b_ref = np.full(pool_np.size, SENTINEL, np.uint8)
    for l in range(L):
        kv.kvm_unpack_layer(ctx.handle, layout, pool_b, L, l, [kv.seq(bt, full, t_hit)])
        oracle.unpack_layer(pool_b_ref, ref, L, l, bt_np, t_hit, full_ref)
        out = torch.full((t_all * C,), SENTINEL, dtype=torch.uint8, device=gpu)
        kv.kvm_merge_layer(ctx.handle, C, [kv.merge_seq(full.data_ptr() + l * C, L * C, t_hit,
                                                        miss.data_ptr() + l * t_miss * C, C,
                                                        t_miss, out, C)])
        out_ref = np.full(t_all * C, SENTINEL, np.uint8)
        oracle.merge_layer(C, full_ref[l * C:], L * C, t_hit, miss_np[l * t_miss * C:], C,
                           t_miss, out_ref, C)
        torch.cuda.synchronize()
        assert np.array_equal(down(out), out_ref), f"merge layer {l}"
        assert np.array_equal(down(pool_b), pool_b_ref), f"unpack layer {l}"
    assert ctx.take_device_errors() == 0


PACK_CASES = [
    # (L, S, N, B, rb, Ts, kind, block_pad, ts_pad, offset)
    (4, 2, 64, 16, 256, [256], "dense", 0, 0, 0),
    (4, 2, 64, 16, 256, [240, 17, 1], "dense", 0, 0, 0),
    (3, 1, 300, 64, 1152, [700, 64, 65, 0, 1], "dense", 0, 0, 0),      # MLA-like rows
    (2, 2, 40, 1, 2048, [33, 7], "dense", 0, 0, 0),                      # B = 1
    (5, 2, 500, 3, 48, [2, 1] * 70, "dense", 0, 0, 0),                  # 140 sequences
    (4, 2, 64, 16, 256, [200, 31], "block_major", 0, 0, 0),
    (4, 2, 64, 16, 256, [200, 31], "slot", 0, 0, 0),
    (3, 2, 50, 5, 80, [44, 13], "dense", 48, 96, 0),                     # padded blocks/tokens
    (2, 2, 30, 4, 24, [23, 9], "dense", 8, 8, 8),                        # 8-byte moves
    (2, 2, 30, 4, 12, [23, 9], "dense", 4, 4, 4),                        # 4-byte moves
    (2, 2, 30, 4, 6, [23, 9], "dense", 2, 2, 2),                         # 2-byte moves
    (2, 2, 30, 4, 5, [23, 9], "dense", 1, 3, 1),                         # byte moves
    (2, 2, 64, 16, 256, [100, 50], "dense", 0, 0, 1),                    # odd base address
    (1, 1, 8, 7, 16, [0, 0, 5], "slot", 0, 0, 0),
    (2, 2, 70000, 1, 16, [10, 3], "dense", 0, 0, 0),                    # pool >> tiles: own order
    (2, 3, 40, 4, 48, [33, 7], "dense", 0, 0, 0),                       # three sides
    (3, 5, 30, 2, 32, [19, 4, 1], "block_major", 0, 16, 0),             # five sides, padded tokens
    (2, 2, 20, 256, 100, [1000, 257, 3], "dense", 0, 0, 0),              # 256-token blocks, 4-byte moves
    (1, 1, 8, 1024, 16, [3000, 1025], "slot", 0, 0, 0),                 # 1024-token blocks
    (2, 2, 64, 16, 1024, [300, 77], "dense", 0, 0, 0),                   # 2048-unit pack tiles
    (3, 1, 80, 16, 1152, [301, 45], "slot", 0, 0, 0),                    # MLA rows, 16-token blocks
]


@pytest.mark.parametrize("case", PACK_CASES, ids=[f"pack{i}" for i in range(len(PACK_CASES))])
def test_pack_unpack(ctx, gpu, case):
    L, S, N, B, rb, Ts, kind, bp, tp, off = case
    run_pack_unpack(ctx, gpu, L, S, N, B, rb, Ts, kind=kind, block_pad=bp, ts_pad=tp, offset=off,
                    seed=case_seed(case))


MERGE_CASES = [
    # (C, reqs, L, hit_pad, miss_pad, out_pad, offset)
    (512, [(240, 16)], 4, 0, 0, 0, 0),
    (4096, [(300, 20), (0, 9), (13, 0), (0, 0), (64, 64)], 32, 0, 0, 0, 0),
    (1152, [(1000, 77)], 61, 0, 0, 128, 0),
    (36, [(5, 3)] * 90, 3, 4, 12, 28, 0),                 # 90 requests, 4-byte moves
    (10, [(17, 5), (1, 1)], 2, 2, 6, 2, 2),               # 2-byte moves
    (7, [(9, 4)], 2, 1, 3, 5, 1),                         # byte moves
    (65536 * 2, [(3, 2)], 2, 0, 0, 0, 0),                 # rows above the tile target
]


@pytest.mark.parametrize("case", MERGE_CASES, ids=[f"merge{i}" for i in range(len(MERGE_CASES))])
def test_merge(ctx, gpu, case):
    C, reqs, L, hp, mp, op, off = case
    run_merge(ctx, gpu, C, reqs, L=L, hit_pad=hp, miss_pad=mp, out_pad=op, offset=off,
              seed=case_seed(case))


def _descs(src_off, dst_off, lens):
    cols = [np.array([int(v) for v in (c.tolist() if isinstance(c, np.ndarray) else c)],
                     dtype=object).astype(np.uint64)
            for c in (src_off, dst_off, lens)]
    return np.stack(cols, axis=1)


def test_batch_copy_random(ctx, gpu):
    rng = np.random.default_rng(21)
    lens = 256 * rng.integers(16, 512, endpoint=True, size=3000)
    arena = int(lens.sum()) + (64 << 20)
    d = _descs(wl.placements(21, 1, lens, arena), wl.placements(21, 2, lens, arena), lens)
    run_batch_copy(ctx, gpu, rng.integers(0, 256, arena, dtype=np.uint8),
                   np.full(arena, SENTINEL, np.uint8), d, label="4K-128K objects")


@pytest.mark.parametrize("n", [5, 300, 70_000], ids=["one-group", "meta", "three-pass"])
def test_batch_copy_huge_objects(ctx, gpu, n):
    """Objects of many pieces (up to 3 MiB, with ragged last pieces) mixed with
    one-piece, short and unaligned ones: one group, the one-workgroup metadata
    pass, and the three-launch metadata pass. Sizes straddle the 16 KiB,
    64 KiB (piece layout) and 128 KiB (piece) boundaries."""
    rng = np.random.default_rng(90 + n)
    edge = [1 << 20, (1 << 20) - 16, (1 << 20) + 16, (3 << 20) + 4080, (64 << 10) * 17,
            (128 << 10) + 16, 16 << 10, 5000]
    lens = np.array([edge[i % len(edge)] for i in range(min(n, 40))], np.int64)
    if n > 40:
        rest = 256 * rng.integers(1, 64, size=n - 40)             # short objects, 256 B - 16 KiB
        lens = np.concatenate([lens, rest])
        rng.shuffle(lens)
    slots = -(-lens // 256) * 256
    arena = int(slots.sum()) + (8 << 20)
    d = _descs(wl.placements(91, 1, slots, arena), wl.placements(91, 2, slots, arena), lens)
    shift = np.zeros(len(lens), bool)
    shift[3::7] = True
    shift &= (slots - lens) >= 8                                   # room in the source slot
    d[shift, 0] += 8                                               # some sources unaligned
    run_batch_copy(ctx, gpu, rng.integers(0, 256, arena, dtype=np.uint8),
                   np.full(arena, SENTINEL, np.uint8), d, label=f"huge objects n={n}")


def test_batch_copy_alignment_matrix(ctx, gpu):
    """Every (src % 16, dst % 16) pair, with lengths 0..300 and one 1 MiB object."""
    rng = np.random.default_rng(22)
    rows, at_s, at_d = [], 0, 0
    for sa in range(16):
        for da in range(16):
            for ln in (0, 1, 15, 16, 17, 63, 64, 255, 300, int(rng.integers(0, 301))):
                s = at_s + sa
                dd = at_d + da
                rows.append((s, dd, ln))
                at_s = (s + ln + 31) // 16 * 16
                at_d = (dd + ln + 31) // 16 * 16
    rows.append((at_s + 3, at_d + 3, 1 << 20))
    rows.append((at_s + (1 << 20) + 64, at_d + (1 << 20) + 67, (1 << 20) + 5))
    d = np.array(rows, np.uint64)
    size = int(max(d[:, 0].max(), d[:, 1].max())) + (2 << 20) + 256
    run_batch_copy(ctx, gpu, rng.integers(0, 256, size, dtype=np.uint8),
                   np.full(size, SENTINEL, np.uint8), d, label="alignment matrix")


def test_batch_copy_one_large_object(ctx, gpu):
    """A 96 MiB object is split across many wavefronts."""
    rng = np.random.default_rng(23)
    n = 96 << 20
    src = rng.integers(0, 256, n + 4096, dtype=np.uint8)
    d = _descs([4096], [256], [n])
    run_batch_copy(ctx, gpu, src, np.full(n + 512, SENTINEL, np.uint8), d, label="one large")


ONE_OBJECT_CASES = {
    # (source offset, destination offset, length, source bytes, workgroup budget)
    "pieces+ragged": (4096, 256, 5 * (128 << 10) + 4080, 6 << 20, 0),
    "one-piece": (0, 1 << 20, 128 << 10, 2 << 20, 0),
    "short-piece": (16, 32, (48 << 10) + 16, 1 << 20, 0),
    "below-16KiB": (64, 128, (16 << 10) - 16, 1 << 20, 0),
    "unaligned-big": (8, 3, (3 << 20) + 5, 4 << 20, 0),
    "empty": (100, 200, 0, 1 << 20, 0),
    "past-source-end": ((1 << 20) - 64, 0, 128, 1 << 20, 0),
    "budget-3": (4096, 256, 40 * (128 << 10) + 512, 6 << 20, 3),
}


@pytest.mark.parametrize("case", list(ONE_OBJECT_CASES))
def test_batch_copy_one_object(gpu, case):
    """A list of one object (its own launch): full pieces, a ragged last piece,
    a piece-sized and a sub-piece object, an object just under the 16 KiB
    piece threshold, an unaligned big object (wavefront shares), an empty one,
    one outside the source (skipped and counted) and a workgroup budget below
    the piece count. Each list is copied twice: the second call sizes its grid
    from the piece count the first one left."""
    so, do, ln, sb, budget = ONE_OBJECT_CASES[case]
    rng = np.random.default_rng(2900 + len(case))
    src_np = rng.integers(0, 256, sb, dtype=np.uint8)
    db = max(do + ln, 1 << 16) + 4096
    d = _descs([so], [do], [ln])
    bad = 1 if so + ln > sb else 0
    c = kv.Context(0)
    try:
        c.set_max_workgroups(budget)
        for call in range(2):
            run_batch_copy(c, gpu, src_np, np.full(db, SENTINEL, np.uint8), d, expect_skipped=bad,
                           label=f"one object {case} call {call}")
    finally:
        c.close()


def test_batch_copy_many_tiny_objects(ctx, gpu):
    rng = np.random.default_rng(24)
    lens = rng.integers(0, 65, size=100000)
    arena = int(lens.sum()) + 200000
    d = _descs(wl.placements(24, 1, lens, arena, 1), wl.placements(24, 2, lens, arena, 1), lens)
    run_batch_copy(ctx, gpu, rng.integers(0, 256, arena, dtype=np.uint8),
                   np.full(arena, SENTINEL, np.uint8), d, label="100k tiny")


def test_batch_copy_same_buffer(ctx, gpu):
    rng = np.random.default_rng(25)
    buf = rng.integers(0, 256, 1 << 22, dtype=np.uint8)
    lens = 64 * rng.integers(1, 100, size=200)
    offs = wl.placements(25, 1, np.concatenate([lens, lens]), 1 << 22, 64)
    d = _descs(offs[:200], offs[200:], lens)
    run_batch_copy(ctx, gpu, buf, buf, d, same_buffer=True, label="same buffer")


def test_batch_copy_skips_out_of_range(ctx, gpu):
    rng = np.random.default_rng(26)
    size = 1 << 20
    d = _descs([0, 100, size - 10, 5, 2**63, 7000], [0, 5000, 20000, size - 3, 30000, 2**64 - 8],
               [64, 300, 11, 4, 8, 9])
    run_batch_copy(ctx, gpu, rng.integers(0, 256, size, dtype=np.uint8),
                   np.full(size, SENTINEL, np.uint8), d, expect_skipped=4, label="out of range")


@pytest.mark.parametrize("n", [1, 2, 63, 64, 65, 129])
def test_batch_copy_short_lists(ctx, gpu, n):
    """Lists around the one-group limit (64 objects: one launch, no scratch),
    with mixed alignments, zero lengths and two objects outside a buffer."""
    rng = np.random.default_rng(27 + n)
    lens = rng.integers(0, 20000, size=n)
    lens[rng.integers(0, n)] = 0
    arena = int(lens.sum()) + 64 * n + 4096
    src_off = wl.placements(27, n, lens, arena, 1)
    dst_off = wl.placements(28, n, lens, arena, 1)
    d = _descs(src_off, dst_off, lens)
    bad = 0
    if n >= 2:
        d[n - 1] = (arena - 5, 0, 6)             # source runs past its buffer
        d[0] = (0, 2**64 - 16, 32)               # destination offset far out of range
        bad = 2
    run_batch_copy(ctx, gpu, rng.integers(0, 256, arena, dtype=np.uint8),
                   np.full(arena, SENTINEL, np.uint8), d, expect_skipped=bad,
                   label=f"short list n={n}")


def test_batch_copy_short_list_uses_no_scratch(gpu):
    """A list of at most 64 objects allocates nothing on a fresh context and
    runs on a second stream beside a long list's copy on the first."""
    c = kv.Context(0)
    try:
        before = c.device_bytes()
        rng = np.random.default_rng(29)
        src_np = rng.integers(0, 256, 1 << 20, dtype=np.uint8)
        lens = np.full(64, 4096)
        offs = 4096 * np.arange(64)
        short = up(_descs(offs, offs[::-1].copy(), lens).view(np.uint8), gpu)
        src = up(src_np, gpu)
        dst = torch.full((1 << 20,), SENTINEL, dtype=torch.uint8, device=gpu)
        kv.kvm_batch_copy(c.handle, dst, 1 << 20, src, 1 << 20, short, 64)
        torch.cuda.synchronize()
        assert c.device_bytes() == before
        want = np.full(1 << 20, SENTINEL, np.uint8)
        oracle.batch_copy(want, src_np, _descs(offs, offs[::-1].copy(), lens))
        assert np.array_equal(down(dst), want)

        long_lens = 256 * rng.integers(1, 64, size=3000)
        arena = int(long_lens.sum()) + (1 << 20)
        lsrc_np = rng.integers(0, 256, arena, dtype=np.uint8)
        ld = _descs(wl.placements(30, 1, long_lens, arena), wl.placements(30, 2, long_lens, arena),
                    long_lens)
        lsrc, ldst = up(lsrc_np, gpu), torch.full((arena,), SENTINEL, dtype=torch.uint8, device=gpu)
        ldesc = up(ld.view(np.uint8), gpu)
        dst.fill_(SENTINEL)
        a, b = torch.cuda.Stream(gpu), torch.cuda.Stream(gpu)
        a.wait_stream(torch.cuda.current_stream())
        b.wait_stream(torch.cuda.current_stream())
        kv.kvm_batch_copy(c.handle, ldst, arena, lsrc, arena, ldesc, len(ld), stream=a)
        kv.kvm_batch_copy(c.handle, dst, 1 << 20, src, 1 << 20, short, 64, stream=b)
        torch.cuda.synchronize()
        lwant = np.full(arena, SENTINEL, np.uint8)
        oracle.batch_copy(lwant, lsrc_np, ld)
        assert np.array_equal(down(ldst), lwant)
        assert np.array_equal(down(dst), want)
        assert c.take_device_errors() == 0
    finally:
        c.close()


def test_raw_bits_survive(ctx, gpu):
    """bf16 NaN payloads, infinities, -0 and denormals come out bit-identical."""
    specials = np.array([0x7FC1, 0xFFFF, 0x7F80, 0xFF80, 0x8000, 0x0001, 0x807F, 0x7FBF],
                        np.uint16)
    L, S, N, B, hd = 2, 2, 8, 4, 32
    rb = hd * 2
    pool16 = np.resize(specials, L * S * N * B * hd)
    pool_np = pool16.view(np.uint8)
    bt_np = np.array([5, 2, 7], np.int32)
    layout = kv.pool_layout(S, B, rb, B * rb, N * B * rb, S * N * B * rb, N)
    ref = oracle.pool_struct(S, B, rb, B * rb, N * B * rb, S * N * B * rb, N)
    T = 11
    pool, bt = up(pool_np, gpu), up(bt_np, gpu)
    full = torch.zeros(T * L * S * rb, dtype=torch.uint8, device=gpu)
    kv.kvm_pack_full(ctx.handle, layout, pool, L, [kv.seq(bt, full, T)])
    want = np.zeros(T * L * S * rb, np.uint8)
    oracle.pack_full(pool_np, ref, L, bt_np, T, want)
    torch.cuda.synchronize()
    got = down(full)
    assert np.array_equal(got, want)
    assert set(np.unique(got.view(np.uint16))) <= set(specials.tolist())
    d = up(np.array([[0, 0, pool_np.size]], np.uint64).view(np.uint8), gpu)
    dst = torch.zeros(pool_np.size, dtype=torch.uint8, device=gpu)
    kv.kvm_batch_copy(ctx.handle, dst, pool_np.size, pool, pool_np.size, d, 1)
    torch.cuda.synchronize()
    assert np.array_equal(down(dst), pool_np)


def test_repeated_and_changing_records(ctx, gpu):
    """Back-to-back calls with identical records reuse staged records; a change
    in any field (token count, pointer) must be seen by the next launch."""
    L, S, N, B, rb = 3, 2, 32, 4, 64
    layout = kv.pool_layout(S, B, rb, B * rb, N * B * rb, S * N * B * rb, N)
    ref = oracle.pool_struct(S, B, rb, B * rb, N * B * rb, S * N * B * rb, N)
    rng = np.random.default_rng(27)
    bt_np = wl.block_tables(27, 1, N, [8])[0]
    bt = up(bt_np, gpu)
    fb_np = [rng.integers(0, 256, 32 * L * S * rb, dtype=np.uint8) for _ in range(2)]
    fbs = [up(f, gpu) for f in fb_np]
    pool = up(np.full(L * S * N * B * rb, SENTINEL, np.uint8), gpu)
    want = np.full(L * S * N * B * rb, SENTINEL, np.uint8)
    side = torch.cuda.Stream()
    plan = [(0, 32, 0, None), (1, 32, 0, None), (1, 32, 1, None), (2, 5, 1, None), (2, 5, 1, side),
            (0, 31, 0, side), (1, 32, 1, None), (2, 32, 0, None)]
    for layer, T, which, stream in plan:
        if stream is not None:
            stream.wait_stream(torch.cuda.current_stream())
        kv.kvm_unpack_layer(ctx.handle, layout, pool, L, layer, [kv.seq(bt, fbs[which], T)],
                            stream=stream)
        if stream is not None:
            torch.cuda.current_stream().wait_stream(stream)
        oracle.unpack_layer(want, ref, L, layer, bt_np, T, fb_np[which])
    torch.cuda.synchronize()
    assert np.array_equal(down(pool), want)


def test_unpack_order_survives_table_rewrite(ctx, gpu):
    """The unpack tile order is cached per record set. Rewriting a block table
    in place (same pointer, same token count) leaves a stale order, which is
    still a permutation of the same tiles: results must follow the new table."""
    L, S, N, B, rb, T = 2, 2, 96, 4, 64, 90
    layout = kv.pool_layout(S, B, rb, B * rb, N * B * rb, S * N * B * rb, N)
    ref = oracle.pool_struct(S, B, rb, B * rb, N * B * rb, S * N * B * rb, N)
    rng = np.random.default_rng(31)
    fb_np = rng.integers(0, 256, T * L * S * rb, dtype=np.uint8)
    fb = up(fb_np, gpu)
    tab1 = wl.block_tables(31, 1, N, [wl.blocks_needed(T, B)])[0]
    tab2 = wl.block_tables(31, 2, N, [wl.blocks_needed(T, B)])[0]
    bt = up(tab1, gpu)
    want = np.full(L * S * N * B * rb, SENTINEL, np.uint8)
    pool = up(want, gpu)
    for l, tab in ((0, tab1), (1, tab1), (0, tab2), (1, tab2)):
        oracle.unpack_layer(want, ref, L, l, tab, T, fb_np)
        bt.copy_(torch.from_numpy(tab.view(np.uint8)).to(gpu))   # in place, same pointer
        kv.kvm_unpack_layer(ctx.handle, layout, pool, L, l, [kv.seq(bt, fb, T)])
        torch.cuda.synchronize()
        assert np.array_equal(down(pool), want), f"layer {l}"


def test_unpack_order_cache_eviction(ctx, gpu):
    """More distinct record sets than the context caches: evicted orders are
    rebuilt and every call still matches the oracle."""
    L, S, N, B, rb = 2, 2, 64, 4, 32
    layout = kv.pool_layout(S, B, rb, B * rb, N * B * rb, S * N * B * rb, N)
    ref = oracle.pool_struct(S, B, rb, B * rb, N * B * rb, S * N * B * rb, N)
    rng = np.random.default_rng(32)
    fb_np = rng.integers(0, 256, 200 * L * S * rb, dtype=np.uint8)
    fb = up(fb_np, gpu)
    tab = wl.block_tables(32, 1, N, [50])[0]
    bt = up(tab, gpu)
    want = np.full(L * S * N * B * rb, SENTINEL, np.uint8)
    pool = up(want, gpu)
    for i, T in enumerate(list(range(100, 140)) + list(range(100, 110))):   # 40 sets, then reuse
        l = i % L
        oracle.unpack_layer(want, ref, L, l, tab, T, fb_np)
        kv.kvm_unpack_layer(ctx.handle, layout, pool, L, l, [kv.seq(bt, fb, T)])
    torch.cuda.synchronize()
    assert np.array_equal(down(pool), want)


FUSED_CASES = [
    # (L, S, N, B, rb, reqs, kind, ts_pad, miss_pad, out_pad, offset)
    (4, 2, 64, 16, 256, [(240, 16)], "dense", 0, 0, 0, 0),
    (3, 2, 200, 16, 512, [(300, 20), (0, 9), (13, 0), (0, 0), (64, 64)], "dense", 0, 0, 0, 0),
    (3, 1, 300, 64, 1152, [(700, 77), (65, 3)], "slot", 0, 0, 128, 0),
    (2, 2, 700, 3, 48, [(5, 2), (1, 1)] * 70, "block_major", 0, 0, 0, 0),   # 140 requests
    (2, 2, 60, 4, 12, [(23, 5), (9, 0)], "dense", 4, 4, 4, 4),               # 4-byte moves
    (2, 2, 60, 4, 5, [(23, 5), (9, 2)], "dense", 3, 1, 5, 1),                # byte moves
    (2, 3, 60, 4, 32, [(23, 5), (9, 0), (0, 3)], "dense", 0, 0, 16, 0),     # three sides
    (3, 5, 40, 2, 16, [(13, 2), (6, 1)], "slot", 16, 0, 0, 0),              # five sides
    (2, 2, 24, 256, 100, [(1000, 30), (257, 0), (3, 5)], "dense", 0, 0, 0, 0),  # 256-token blocks
    (1, 1, 10, 1024, 16, [(3000, 100), (1025, 1)], "slot", 0, 0, 16, 0),     # 1024-token blocks
    (2, 2, 64, 16, 1024, [(300, 20), (77, 3)], "dense", 0, 0, 0, 0),           # 64-wide heads
    # miss rows in the fused launch, several 64 KiB tiles of them per request
    # (1 KiB rows), beside a request with miss rows only (its own merge launch)
    (2, 2, 100, 16, 512, [(300, 200), (0, 70), (50, 130)], "dense", 0, 0, 0, 0),
    # miss rows 8 bytes off the hit rows' 16-byte unit: a merge launch of their own
    (2, 2, 100, 16, 512, [(300, 200), (50, 130)], "dense", 0, 8, 0, 0),
]


@pytest.mark.parametrize("case", FUSED_CASES, ids=[f"fused{i}" for i in range(len(FUSED_CASES))])
def test_unpack_merge(ctx, gpu, case):
    L, S, N, B, rb, reqs, kind, tp, mp, op, off = case
    run_unpack_merge(ctx, gpu, L, S, N, B, rb, reqs, kind=kind, ts_pad=tp, miss_pad=mp,
                     out_pad=op, offset=off, seed=case_seed(case))


def test_one_context_on_two_streams(gpu):
    """One context used on two streams with no host synchronisation between
    calls: the destination order sorted on stream A is reused by stream B (which
    must wait for the sort), and batched copies alternate streams over the
    shared group scratch (each must wait for the previous call's kernels)."""
    say("  two streams, one context")
    c = kv.Context(0)
    try:
        L, S, N, B, rb = 4, 2, 300, 16, 256
        layout = kv.pool_layout(S, B, rb, B * rb, N * B * rb, S * N * B * rb, N)
        ref = oracle.pool_struct(S, B, rb, B * rb, N * B * rb, S * N * B * rb, N)
        rng = np.random.default_rng(61)
        Ts = [700, 333, 1201]
        tables = wl.block_tables(61, 1, N, [wl.blocks_needed(t, B) for t in Ts])
        fb_np = [rng.integers(0, 256, T * L * S * rb, dtype=np.uint8) for T in Ts]
        want = np.full(L * S * N * B * rb, SENTINEL, np.uint8)
        for layer in range(L):
            for i, T in enumerate(Ts):
                oracle.unpack_layer(want, ref, L, layer, tables[i], T, fb_np[i])
        bts = [up(t, gpu) for t in tables]
        fbs = [up(f, gpu) for f in fb_np]
        pool = up(np.full(L * S * N * B * rb, SENTINEL, np.uint8), gpu)
        seqs = [kv.seq(bts[i], fbs[i], T) for i, T in enumerate(Ts)]
        a, b = torch.cuda.Stream(), torch.cuda.Stream()
        torch.cuda.synchronize()
        for layer in range(L):            # the sort runs on a; layers alternate a, b
            kv.kvm_unpack_layer(c.handle, layout, pool, L, layer, seqs, stream=a if layer % 2 == 0 else b)
        torch.cuda.synchronize()
        assert np.array_equal(down(pool), want)

        # batched copies alternating streams
        src_np = rng.integers(0, 256, 1 << 22, dtype=np.uint8)
        src = up(src_np, gpu)
        dst = up(np.full(1 << 22, SENTINEL, np.uint8), gpu)
        lists, dlists = [], []
        region = (1 << 22) // 6                  # list k writes only its own region of dst
        region -= region % 256
        for k in range(6):
            lens = 256 * rng.integers(1, 16, size=200)
            d = np.stack([wl.placements(70 + k, 1, lens, 1 << 22),
                          k * region + wl.placements(70 + k, 2, lens, region), lens],
                         axis=1).astype(np.uint64)
            lists.append(d)
            dlists.append(up(d.view(np.uint8), gpu))
        want_dst = np.full(1 << 22, SENTINEL, np.uint8)
        for d in lists:
            oracle.batch_copy(want_dst, src_np, d)
        torch.cuda.synchronize()
        for k, d in enumerate(dlists):     # no waits between the calls: the library's own
            kv.kvm_batch_copy(c.handle, dst, 1 << 22, src, 1 << 22, d, len(lists[k]),
                              stream=a if k % 2 == 0 else b)
        torch.cuda.synchronize()
        assert np.array_equal(down(dst), want_dst)
        assert c.take_device_errors() == 0
    finally:
        c.close()


def test_copy_scratch_second_stream_waits(gpu):
    """Two lists that share the group scratch: the first, slow (one
    workgroup), on stream a as the context's first copy, so it records no
    event; the second on stream b right after it. The first call on b must
    wait for a's copy before the scratch is rewritten."""
    say("  batched copy: a second stream after a slow first copy")
    c = kv.Context(0)
    try:
        rng = np.random.default_rng(73)
        size = 1 << 24
        src_np = rng.integers(0, 256, size, dtype=np.uint8)
        src = up(src_np, gpu)
        half = size // 2
        lists = []
        for k in range(2):
            lens = 256 * rng.integers(1, 16, size=1500)
            d = np.stack([wl.placements(73, 1 + k, lens, size),
                          k * half + wl.placements(73, 3 + k, lens, half), lens],
                         axis=1).astype(np.uint64)
            lists.append(d)
        want = np.full(size, SENTINEL, np.uint8)
        for d in lists:
            oracle.batch_copy(want, src_np, d)
        dst = up(np.full(size, SENTINEL, np.uint8), gpu)
        dd = [up(d.view(np.uint8), gpu) for d in lists]
        a, b = torch.cuda.Stream(), torch.cuda.Stream()
        torch.cuda.synchronize()
        c.set_max_workgroups(1)
        kv.kvm_batch_copy(c.handle, dst, size, src, size, dd[0], len(lists[0]), stream=a)
        c.set_max_workgroups(0)
        kv.kvm_batch_copy(c.handle, dst, size, src, size, dd[1], len(lists[1]), stream=b)
        torch.cuda.synchronize()
        assert np.array_equal(down(dst), want)
        assert c.take_device_errors() == 0
    finally:
        c.close()


def test_move_calls_do_not_wait_for_the_device(gpu):
    """No move call waits for the whole device. While a slow batched copy
    (one workgroup, 1 GiB) runs on stream a, calls on stream b grow the unpack
    order (a bigger record set), grow the batched-copy scratch as the first
    copy on a second stream, and an unpack on a takes the order cache's second
    stream: all of them return while a's copy is still running (its event is
    not complete). Every result is then compared with the oracle."""
    say("  move calls beside a slow copy on another stream")
    c = kv.Context(0)
    try:
        L, S, N, B, rb = 2, 2, 2000, 16, 256
        layout = kv.pool_layout(S, B, rb, B * rb, N * B * rb, S * N * B * rb, N)
        ref = oracle.pool_struct(S, B, rb, B * rb, N * B * rb, S * N * B * rb, N)
        rng = np.random.default_rng(83)
        Ts = [1000, 20000]
        tables = wl.block_tables(83, 1, N, [wl.blocks_needed(t, B) for t in Ts])
        fb_np = [rng.integers(0, 256, t * L * S * rb, dtype=np.uint8) for t in Ts]
        want_pool = np.full(L * S * N * B * rb, SENTINEL, np.uint8)
        bts, fbs = [up(t, gpu) for t in tables], [up(f, gpu) for f in fb_np]
        pool = up(want_pool, gpu)

        big = 1 << 30                               # the slow copy: 16,384 objects of 64 KiB
        slow_lens = np.full(big >> 16, 1 << 16, np.int64)
        slow_d = np.stack([np.arange(len(slow_lens)) << 16,
                           np.arange(len(slow_lens))[::-1].copy() << 16, slow_lens],
                          axis=1).astype(np.uint64)
        slow_src = torch.randint(0, 256, (big,), dtype=torch.uint8, device=gpu)
        slow_dst = torch.empty(big, dtype=torch.uint8, device=gpu)
        arena = 1 << 26                             # a list that outgrows the scratch
        lens = 256 * rng.integers(1, 4, size=40_000)
        fast_d = np.stack([wl.placements(84, 1, lens, arena), wl.placements(84, 2, lens, arena),
                           lens], axis=1).astype(np.uint64)
        src_np = rng.integers(0, 256, arena, dtype=np.uint8)
        src, dst = up(src_np, gpu), up(np.full(arena, SENTINEL, np.uint8), gpu)
        dd_slow, dd_fast = up(slow_d.view(np.uint8), gpu), up(fast_d.view(np.uint8), gpu)
        a, b = torch.cuda.Stream(), torch.cuda.Stream()
        done_a = torch.cuda.Event()
        torch.cuda.synchronize()

        kv.kvm_unpack_layer(c.handle, layout, pool, L, 0, [kv.seq(bts[0], fbs[0], Ts[0])], stream=b)
        oracle.unpack_layer(want_pool, ref, L, 0, tables[0], Ts[0], fb_np[0])
        torch.cuda.synchronize()
        c.set_max_workgroups(1)
        kv.kvm_batch_copy(c.handle, slow_dst, big, slow_src, big, dd_slow, len(slow_d), stream=a)
        c.set_max_workgroups(0)
        done_a.record(a)
        before = c.device_bytes()
        kv.kvm_unpack_layer(c.handle, layout, pool, L, 1, [kv.seq(bts[1], fbs[1], Ts[1])], stream=b)
        kv.kvm_batch_copy(c.handle, dst, arena, src, arena, dd_fast, len(fast_d), stream=b)
        kv.kvm_unpack_layer(c.handle, layout, pool, L, 0, [kv.seq(bts[1], fbs[1], Ts[1])], stream=a)
        still_running = not done_a.query()
        grown = c.device_bytes() > before
        torch.cuda.synchronize()
        assert still_running, "a move call on stream b waited for stream a's copy"
        assert grown, "the calls were meant to grow the scratch"
        oracle.unpack_layer(want_pool, ref, L, 1, tables[1], Ts[1], fb_np[1])
        oracle.unpack_layer(want_pool, ref, L, 0, tables[1], Ts[1], fb_np[1])
        assert np.array_equal(down(pool), want_pool)
        want_dst = np.full(arena, SENTINEL, np.uint8)
        oracle.batch_copy(want_dst, src_np, fast_d)
        assert np.array_equal(down(dst), want_dst)
        assert torch.equal(slow_dst.view(-1, 1 << 16).flip(0).reshape(-1), slow_src)
        assert c.take_device_errors() == 0
        assert c.device_bytes() <= before + (64 << 20)   # set-aside scratch freed again
    finally:
        c.close()


def test_more_items_than_one_dispatch_holds(ctx, gpu):
    """4.3 M one-token blocks of 16 bytes: pack, unpack and fused items beyond
    the 4,194,303 workgroups of 1024 threads a dispatch can count, so the
    grid is capped and workgroups take several items each."""
    T = 4_300_000
    run_pack_unpack(ctx, gpu, 1, 1, T, 1, 16, [T], seed=11)
    run_unpack_merge(ctx, gpu, 1, 1, T + 100, 1, 16, [(T, 100)], kind="slot", seed=12)


@pytest.mark.parametrize("warm", [True, False], ids=["multi-stream", "second-stream"])
def test_order_eviction_waits_for_every_stream(gpu, warm):
    """A cached unpack order read on two streams, then evicted: the eviction
    must wait for both readers. Stream a reads it slowly (a budget of one
    workgroup), stream b reads it quickly and then brings 16 new record sets,
    the last of which evicts the order while a may still be reading it.
    multi-stream: the context has already seen both streams, so each read
    records its event; second-stream: the slow read is the context's first
    call, recorded by no event, and the first call on b must wait for it."""
    say(f"  order eviction with readers on two streams ({'warm' if warm else 'cold'})")
    c = kv.Context(0)
    try:
        L, S, N, B, rb = 2, 2, 1200, 4, 64
        layout = kv.pool_layout(S, B, rb, B * rb, N * B * rb, S * N * B * rb, N)
        ref = oracle.pool_struct(S, B, rb, B * rb, N * B * rb, S * N * B * rb, N)
        rng = np.random.default_rng(71)
        T = 4000                                   # 1000 blocks, read by one workgroup on a
        tab = wl.block_tables(71, 1, N, [wl.blocks_needed(T, B)])[0]
        fb_np = rng.integers(0, 256, T * L * S * rb, dtype=np.uint8)
        small = [100 + i for i in range(16)]       # 16 other record sets, fewer tiles
        want_a = np.full(L * S * N * B * rb, SENTINEL, np.uint8)
        oracle.unpack_layer(want_a, ref, L, 0, tab, T, fb_np)
        want_c = np.full(L * S * N * B * rb, SENTINEL, np.uint8)
        for t in small:
            oracle.unpack_layer(want_c, ref, L, 1, tab, t, fb_np)
        bt, fb = up(tab, gpu), up(fb_np, gpu)
        pool_a = up(np.full(L * S * N * B * rb, SENTINEL, np.uint8), gpu)
        pool_b = up(np.full(L * S * N * B * rb, SENTINEL, np.uint8), gpu)
        pool_c = up(np.full(L * S * N * B * rb, SENTINEL, np.uint8), gpu)
        a, b = torch.cuda.Stream(), torch.cuda.Stream()
        torch.cuda.synchronize()
        if warm:
            for st in (a, b):
                kv.kvm_unpack_layer(c.handle, layout, pool_c, L, 1, [kv.seq(bt, fb, 0)], stream=st)
                kv.kvm_unpack_layer(c.handle, layout, pool_c, L, 1, [kv.seq(bt, fb, 8)], stream=st)
            torch.cuda.synchronize()
        c.set_max_workgroups(1)
        kv.kvm_unpack_layer(c.handle, layout, pool_a, L, 0, [kv.seq(bt, fb, T)], stream=a)
        c.set_max_workgroups(0)
        kv.kvm_unpack_layer(c.handle, layout, pool_b, L, 0, [kv.seq(bt, fb, T)], stream=b)
        for t in small:
            kv.kvm_unpack_layer(c.handle, layout, pool_c, L, 1, [kv.seq(bt, fb, t)], stream=b)
        torch.cuda.synchronize()
        assert np.array_equal(down(pool_a), want_a), "slow reader on stream a"
        assert np.array_equal(down(pool_b), want_a), "reader on stream b"
        assert np.array_equal(down(pool_c), want_c), "the 16 evicting record sets"
        assert c.take_device_errors() == 0
    finally:
        c.close()


def test_batch_copy_list_shape_changes(ctx, gpu):
    """The grid of a batched copy comes from the piece count the previous call
    of the same list shape (object count and buffers) measured; a shape whose
    objects were all one piece is next copied one workgroup per object with
    no metadata pass. Every call must equal the oracle whatever the previous
    call saw: the same buffers and object count with a uniform list (twice,
    the second taking one workgroup per object), then a changed list (short,
    misaligned and multi-piece objects) under the same shape, then again."""
    rng = np.random.default_rng(77)
    arena = 64 << 20
    n = 300
    src_np = rng.integers(0, 256, arena, dtype=np.uint8)
    src = up(src_np, gpu)
    dst = up(np.full(arena, SENTINEL, np.uint8), gpu)
    want = np.full(arena, SENTINEL, np.uint8)
    uniform = np.full(n, 128 << 10, np.int64)
    changed = 256 * rng.integers(1, 2048, size=n).astype(np.int64)    # up to 512 KiB
    changed[::7] = rng.integers(1, 5000, size=len(changed[::7]))       # short, any length
    for call, lens in enumerate((uniform, uniform, changed, changed, uniform)):
        slots = -(-lens // 256) * 256                                  # whole granules
        d = np.stack([wl.placements(300 + call, 1, slots, arena),
                      wl.placements(300 + call, 2, slots, arena), lens], axis=1).astype(np.uint64)
        if call >= 2:
            d[1::5, 0] += 3                                            # source misaligned
            d[1::5, 2] = np.minimum(d[1::5, 2], 1000)
        say(f"  call {call}: {n} objects, {int(d[:, 2].sum())} bytes")
        dd = up(d.view(np.uint8), gpu)
        kv.kvm_batch_copy(ctx.handle, dst, arena, src, arena, dd, n)
        torch.cuda.synchronize()                                       # the count comes back
        oracle.batch_copy(want, src_np, d)
        assert np.array_equal(down(dst), want), f"call {call} differs"
    assert ctx.take_device_errors() == 0
