"""Calls interleaved over several streams, checked against the oracle. A
context relies on stream order while it has seen one stream and switches to
per-call events at the first call on a second stream; the tile-order cache
(16 record sets) and the batched copy's scratch must stay correct across
that switch, under eviction and with slow launches (a one-workgroup budget)
still reading on another stream. Every record set writes its own pool blocks
and its own output rows, and repeating a call writes the same bytes, so the
final state does not depend on how the streams interleave."""
import os

import numpy as np
import pytest
import torch

import oracle
from gpu_util import SENTINEL, down, say, up
from paged_kv_cache_kvm_amd import kvmove as kv
from paged_kv_cache_kvm_amd import workloads as wl

pytestmark = pytest.mark.gpu


SEEDS = int(os.environ.get("KVM_STREAM_SEEDS", "3"))


@pytest.mark.parametrize("seed", range(1, SEEDS + 1))
def test_interleaved_streams(gpu, seed):
    rng = np.random.default_rng(500 + seed)
    L, S, B, rb = 2, 2, 4, 64
    C = S * rb
    SETS = 20                                   # more than the 16 cached orders
    Ts = rng.integers(1, 60, size=SETS)
    nbs = [wl.blocks_needed(int(t) + 8, B) for t in Ts]
    N = int(sum(nbs)) + 7
    tables = wl.block_tables(600 + seed, 1, N, nbs)   # disjoint: one block range per set
    layout = kv.pool_layout(S, B, rb, B * rb, N * B * rb, S * N * B * rb, N)
    ref = oracle.pool_struct(S, B, rb, B * rb, N * B * rb, S * N * B * rb, N)
    fb_np = [rng.integers(0, 256, int(t) * L * C, dtype=np.uint8) for t in Ts]
    miss_np = [rng.integers(0, 256, 8 * C, dtype=np.uint8) for _ in range(SETS)]
    bts = [up(t, gpu) for t in tables]
    fbs = [up(f, gpu) for f in fb_np]
    misses = [up(m, gpu) for m in miss_np]
    outs = [[torch.full(((int(t) + 8) * C,), SENTINEL, dtype=torch.uint8, device=gpu)
             for _ in range(L)] for t in Ts]
    pool = up(np.full(L * S * N * B * rb, SENTINEL, np.uint8), gpu)
    want_pool = np.full(L * S * N * B * rb, SENTINEL, np.uint8)
    want_out = [[None] * L for _ in range(SETS)]

    # copy lists, each writing its own region of dst, all of more than 64 objects:
    # short objects (wavefront shares, with scratch), one-piece objects (one
    # workgroup per object once the list's shape is known) and objects of up to
    # two pieces (piece records in the scratch)
    CP, region, src_bytes = 6, 1 << 25, 1 << 26
    src_np = rng.integers(0, 256, src_bytes, dtype=np.uint8)
    src = up(src_np, gpu)
    dst = up(np.full(CP * region, SENTINEL, np.uint8), gpu)
    want_dst = np.full(CP * region, SENTINEL, np.uint8)
    lists, dlists = [], []
    for k in range(CP):
        n = int(rng.integers(65, 120))
        if k % 3 == 0:
            lens = 256 * rng.integers(1, 4, size=n)
        elif k % 3 == 1:
            lens = 16384 * rng.integers(1, 9, size=n)          # 16-128 KiB, one piece
        else:
            lens = 4096 * rng.integers(4, 65, size=n)          # 16-256 KiB, up to two pieces
        d = np.stack([wl.placements(700 + k, seed, lens, src_bytes),
                      k * region + wl.placements(710 + k, seed, lens, region), lens],
                     axis=1).astype(np.uint64)
        lists.append(d)
        dlists.append(up(d.view(np.uint8), gpu))

    c = kv.Context(0)
    streams = [torch.cuda.Stream(), torch.cuda.Stream(), torch.cuda.current_stream()]
    torch.cuda.synchronize()
    try:
        plan = []
        for step in range(90):
            plan.append((int(rng.integers(0, 3)), int(rng.integers(0, SETS)),
                         int(rng.integers(0, L)), int(rng.integers(0, 3)),
                         int(rng.integers(0, CP)), bool(rng.random() < 0.15)))
        say(f"  interleaved streams seed={seed}: {len(plan)} calls on 3 streams")
        for op, k, l, si, ck, slow in plan:
            st = streams[si]
            c.set_max_workgroups(1 if slow else 0)
            T = int(Ts[k])
            if op == 0:
                kv.kvm_unpack_layer(c.handle, layout, pool, L, l, [kv.seq(bts[k], fbs[k], T)],
                                    stream=st)
                oracle.unpack_layer(want_pool, ref, L, l, tables[k], T, fb_np[k])
            elif op == 1:
                kv.kvm_unpack_merge_layer(c.handle, layout, pool, L, l, [
                    kv.layer_seq(bts[k], fbs[k], T, misses[k], C, 8, outs[k][l], C)], stream=st)
                oracle.unpack_layer(want_pool, ref, L, l, tables[k], T, fb_np[k])
                o = np.full((T + 8) * C, SENTINEL, np.uint8)
                oracle.merge_layer(C, fb_np[k][l * C:], L * C, T, miss_np[k], C, 8, o, C)
                want_out[k][l] = o
            else:
                kv.kvm_batch_copy(c.handle, dst, CP * region, src, src_bytes, dlists[ck],
                                  len(lists[ck]), stream=st)
                oracle.batch_copy(want_dst, src_np, lists[ck])
        c.set_max_workgroups(0)
        torch.cuda.synchronize()
        assert np.array_equal(down(pool), want_pool), "pool"
        for k in range(SETS):
            for l in range(L):
                if want_out[k][l] is not None:
                    assert np.array_equal(down(outs[k][l]), want_out[k][l]), f"out {k} {l}"
        assert np.array_equal(down(dst), want_dst), "batched copies"
        assert c.take_device_errors() == 0
    finally:
        c.close()
