"""kvm_batch_copy_noalloc against kvm_batch_copy (GPU, through the C ABI).

The no-alloc entry point keeps its scratch in the device's static array; its
output must equal the allocating entry point's, byte for byte, and the
oracle's, on two calls in a row (the second with a smaller list), while the
context's device memory stays where it was. It is also replayed from a HIP
graph capture, for the callers it is for.
"""

import numpy as np
import pytest
import torch

import oracle
from gpu_util import SENTINEL, down, say, up
from paged_kv_cache_kvm_amd import kvmove as kv
from paged_kv_cache_kvm_amd import workloads as wl

pytestmark = pytest.mark.gpu


def _list(seed, n, arena):
    """n objects at random non-overlapping places in both arenas: most of
    them 16-byte friendly (256-byte granules), some with odd offsets and
    lengths, one empty and one past the end of the source (skipped)."""
    rng = np.random.default_rng(seed)
    lens = 256 * rng.integers(1, 9, size=n).astype(np.int64)
    src = wl.placements(seed, 1, lens, arena)
    dst = wl.placements(seed, 2, lens, arena)
    d = np.stack([src, dst, lens], axis=1).astype(np.uint64)
    odd = rng.choice(n, size=max(1, n // 10), replace=False)
    d[odd, 0] += rng.integers(0, 16, size=len(odd)).astype(np.uint64)   # source shifted
    d[odd, 2] -= rng.integers(16, 200, size=len(odd)).astype(np.uint64)  # shorter, any length
    d[odd[0], 2] = 0                                                     # an empty object
    bad = d.copy()
    bad[-1] = [arena - 8, 0, 64]                                         # past the source end
    return bad


def _copy(entry, ctx, src, dst, arena, descs_np, dev):
    d = up(descs_np.view(np.uint8), dev)
    lib = kv.load()
    rc = getattr(lib, entry)(ctx.handle, dst.data_ptr(), arena, src.data_ptr(), arena,
                            d.data_ptr(), len(descs_np), torch.cuda.current_stream().cuda_stream)
    assert rc == kv.KVM_OK, (entry, rc, kv.kvm_ctx_last_error(ctx.handle))
    torch.cuda.synchronize()
    return down(dst)


def test_noalloc_matches_batch_copy_on_two_calls(gpu):
    arena = 128 << 20
    ctx = kv.Context(0)
    try:
        # more than 65,536 objects takes the three-launch path; the second,
        # smaller list the one-workgroup metadata path
        for call, n in enumerate((70000, 3000)):
            descs = _list(1000 + call, n, arena)
            say(f"  call {call}: {n} objects in {arena >> 20} MiB arenas")
            rng = np.random.default_rng(2000 + call)
            src_np = rng.integers(0, 256, arena, dtype=np.uint8)
            src = up(src_np, gpu)
            dst_a = up(np.full(arena, SENTINEL, np.uint8), gpu)
            dst_b = up(np.full(arena, SENTINEL, np.uint8), gpu)
            before = ctx.device_bytes()
            got_b = _copy("kvm_batch_copy_noalloc", ctx, src, dst_b, arena, descs, gpu)
            assert ctx.device_bytes() == before, "the no-alloc call changed the context's memory"
            assert ctx.take_device_errors() == 1   # the object past the source end
            got_a = _copy("kvm_batch_copy", ctx, src, dst_a, arena, descs, gpu)
            assert ctx.take_device_errors() == 1
            assert np.array_equal(got_a, got_b), f"call {call}: no-alloc differs from kvm_batch_copy"
            want = np.full(arena, SENTINEL, np.uint8)
            oracle.batch_copy(want, src_np, descs[:-1])
            assert np.array_equal(got_b, want), f"call {call}: no-alloc differs from the oracle"
    finally:
        ctx.close()


@pytest.mark.parametrize("n", [3000, 70000], ids=["meta", "three-pass"])
def test_noalloc_pieces(gpu, n):
    """Objects of 1 KiB to 384 KiB (one to three pieces, ragged last pieces, the
    short ones to the wavefront shares): the piece records then live in the
    static array. Two calls in a row, the second once the shape's piece count
    is known; each equals kvm_batch_copy's output and the oracle's."""
    rng = np.random.default_rng(3000 + n)
    lens = 256 * rng.integers(16, 1537, size=n).astype(np.int64)       # 4 KiB - 384 KiB
    if n > 10000:                                  # keep the arena near 1 GiB: mostly 1-16 KiB
        short = np.ones(n, bool)
        short[::50] = False
        lens[short] = 256 * rng.integers(4, 65, size=int(short.sum()))
    arena = int(lens.sum()) + (64 << 20)
    descs = np.stack([wl.placements(3000 + n, 1, lens, arena), wl.placements(3000 + n, 2, lens, arena),
                      lens], axis=1).astype(np.uint64)
    ctx = kv.Context(0)
    try:
        src_np = rng.integers(0, 256, arena, dtype=np.uint8)
        src = up(src_np, gpu)
        want = np.full(arena, SENTINEL, np.uint8)
        oracle.batch_copy(want, src_np, descs)
        for call in range(2):
            say(f"  call {call}: {n} objects, {int(lens.sum()) >> 20} MiB")
            dst_b = up(np.full(arena, SENTINEL, np.uint8), gpu)
            before = ctx.device_bytes()
            got_b = _copy("kvm_batch_copy_noalloc", ctx, src, dst_b, arena, descs, gpu)
            assert ctx.device_bytes() == before, "the no-alloc call changed the context's memory"
            del dst_b
            dst_a = up(np.full(arena, SENTINEL, np.uint8), gpu)
            got_a = _copy("kvm_batch_copy", ctx, src, dst_a, arena, descs, gpu)
            del dst_a
            assert np.array_equal(got_b, want), f"call {call}: no-alloc differs from the oracle"
            assert np.array_equal(got_a, got_b), f"call {call}: no-alloc differs from kvm_batch_copy"
        assert ctx.take_device_errors() == 0
    finally:
        ctx.close()


def test_noalloc_short_list_and_limits(gpu):
    """A one-group list (at most 64 objects) and the length limit."""
    arena = 1 << 20
    ctx = kv.Context(0)
    try:
        descs = _list(7, 64, arena)[:-1]           # 63 valid objects, one group
        rng = np.random.default_rng(8)
        src_np = rng.integers(0, 256, arena, dtype=np.uint8)
        src = up(src_np, gpu)
        dst = up(np.full(arena, SENTINEL, np.uint8), gpu)
        got = _copy("kvm_batch_copy_noalloc", ctx, src, dst, arena, descs, gpu)
        want = np.full(arena, SENTINEL, np.uint8)
        oracle.batch_copy(want, src_np, descs)
        assert np.array_equal(got, want)
        lib = kv.load()
        st = torch.cuda.current_stream().cuda_stream
        rc = lib.kvm_batch_copy_noalloc(ctx.handle, dst.data_ptr(), arena, src.data_ptr(), arena,
                                        dst.data_ptr(), kv.KVM_NOALLOC_MAX_DESCS + 1, st)
        assert rc == kv.KVM_ERANGE   # refused before anything is enqueued
        assert lib.kvm_batch_copy_noalloc(ctx.handle, dst.data_ptr(), arena, src.data_ptr(), arena,
                                          dst.data_ptr(), 0, st) == kv.KVM_OK
        assert ctx.take_device_errors() == 0
    finally:
        ctx.close()


def test_noalloc_one_object(gpu):
    """A list of one object (full pieces and a ragged last one; then a shorter
    one): no scratch at all, the same bytes as kvm_batch_copy and the oracle,
    on two calls in a row."""
    arena = 8 << 20
    ctx = kv.Context(0)
    try:
        rng = np.random.default_rng(31)
        src_np = rng.integers(0, 256, arena, dtype=np.uint8)
        src = up(src_np, gpu)
        for call, ln in enumerate((5 * (128 << 10) + 4080, (48 << 10) + 16)):
            descs = np.array([[4096, 512, ln]], np.uint64)
            say(f"  call {call}: one object of {ln} bytes")
            before = ctx.device_bytes()
            got_b = _copy("kvm_batch_copy_noalloc", ctx, src, up(np.full(arena, SENTINEL, np.uint8), gpu),
                          arena, descs, gpu)
            assert ctx.device_bytes() == before, "the no-alloc call changed the context's memory"
            got_a = _copy("kvm_batch_copy", ctx, src, up(np.full(arena, SENTINEL, np.uint8), gpu),
                          arena, descs, gpu)
            want = np.full(arena, SENTINEL, np.uint8)
            oracle.batch_copy(want, src_np, descs)
            assert np.array_equal(got_b, want), f"call {call}: no-alloc differs from the oracle"
            assert np.array_equal(got_a, got_b), f"call {call}: no-alloc differs from kvm_batch_copy"
        assert ctx.take_device_errors() == 0
    finally:
        ctx.close()


def _graph_list(seed, lens, arena):
    return np.stack([wl.placements(seed, 1, lens, arena), wl.placements(seed, 2, lens, arena),
                     lens], axis=1).astype(np.uint64)


@pytest.mark.parametrize("kind", ["short", "pieces", "one"])
def test_noalloc_in_a_graph(gpu, kind):
    """Captured into a HIP graph: the call allocates nothing, records no event
    and clears nothing with a memset, so the capture holds only its kernels.
    The graph is replayed six times with eager work in between that rewrites
    the source, the destination and the descriptors (same count); every
    replay equals the oracle on the buffers as they are then."""
    say(f"  no-alloc batched copy under graph capture ({kind})")
    ctx = kv.Context(0)
    try:
        rng = np.random.default_rng(111)
        arena, n = 32 << 20, 700
        if kind == "short":
            lens = 256 * rng.integers(1, 9, size=n).astype(np.int64)
        elif kind == "one":                      # one object: 24 full pieces and a ragged one
            n = 1
            lens = np.array([24 * (128 << 10) + 3840], np.int64)
        else:
            lens = 16384 * rng.integers(1, 9, size=n).astype(np.int64)   # 16-128 KiB
            arena = 256 << 20
        src = torch.empty(arena, dtype=torch.uint8, device=gpu)
        dst = torch.empty(arena, dtype=torch.uint8, device=gpu)
        descs = torch.empty(n * 24, dtype=torch.uint8, device=gpu)
        lists = [_graph_list(120 + k, lens, arena) for k in range(3)]
        s = torch.cuda.Stream()
        g = torch.cuda.CUDAGraph()
        descs.copy_(torch.from_numpy(lists[0].view(np.uint8).reshape(-1)))
        # two eager calls first: the kernels are loaded before the capture, and
        # the list shape's piece count is known, so a one-piece-per-object list
        # is captured as one workgroup per object
        for _ in range(2):
            kv.kvm_batch_copy_noalloc(ctx.handle, dst, arena, src, arena, descs, n)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            kv.kvm_batch_copy_noalloc(ctx.handle, dst, arena, src, arena, descs, n,
                                      stream=torch.cuda.current_stream())
        for rep in range(6):
            d = lists[rep % 3]
            src_np = wl.random_bytes(200 + rep, 1, arena)
            src.copy_(torch.from_numpy(src_np))                 # eager work between replays
            dst.fill_(SENTINEL)
            descs.copy_(torch.from_numpy(d.view(np.uint8).reshape(-1)))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            want = np.full(arena, SENTINEL, np.uint8)
            oracle.batch_copy(want, src_np, d)
            assert np.array_equal(down(dst), want), f"replay {rep}"
        assert ctx.take_device_errors() == 0
        del g
    finally:
        ctx.close()
