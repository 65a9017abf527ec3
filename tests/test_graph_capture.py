"""pack_full and merge_layer captured into a HIP graph (GPU, through the C ABI).

Neither call reads state the context keeps between calls (their records travel
as kernel arguments), allocates, records an event or clears memory with a
memset, so a capture holds only their kernels. Each graph is replayed four
times with eager work in between that rewrites the buffers the launches read
(the pool, the Full Block hit rows, the miss rows) and refills the outputs with
the sentinel; every replay must equal the oracle on the buffers as they are
then.
"""

import numpy as np
import pytest
import torch

import oracle
from gpu_util import SENTINEL, down, say
from paged_kv_cache_kvm_amd import kvmove as kv
from paged_kv_cache_kvm_amd import workloads as wl

pytestmark = pytest.mark.gpu


def _capture(call):
    """Two eager calls (kernels loaded), then the call captured on a side stream."""
    for _ in range(2):
        call(torch.cuda.current_stream())
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.graph(g, stream=s):
        call(torch.cuda.current_stream())
    return g


def test_merge_layer_in_a_graph(gpu):
    say("  merge_layer under graph capture")
    L, C, layer = 4, 1024, 2
    reqs = [(300, 40), (0, 17), (129, 0), (64, 64)]
    hs, ms, os_ = L * C, C, C
    ctx = kv.Context(0)
    try:
        hits = [torch.empty(max(h, 1) * hs, dtype=torch.uint8, device=gpu) for h, _ in reqs]
        misses = [torch.empty(max(m, 1) * ms, dtype=torch.uint8, device=gpu) for _, m in reqs]
        outs = [torch.empty(max(h + m, 1) * os_, dtype=torch.uint8, device=gpu) for h, m in reqs]
        seqs = [kv.merge_seq(hits[i].data_ptr() + layer * C if h else 0, hs, h,
                             misses[i].data_ptr() if m else 0, ms, m, outs[i].data_ptr(), os_)
                for i, (h, m) in enumerate(reqs)]
        recs = kv.records(seqs)
        g = _capture(lambda st: kv.kvm_merge_layer(ctx.handle, C, recs, stream=st))
        for rep in range(4):
            hit_np = [wl.random_bytes(300 + rep, i, t.numel()) for i, t in enumerate(hits)]
            miss_np = [wl.random_bytes(400 + rep, i, t.numel()) for i, t in enumerate(misses)]
            for t, a in zip(hits + misses, hit_np + miss_np):
                t.copy_(torch.from_numpy(a))
            for o in outs:
                o.fill_(SENTINEL)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            for i, (h, m) in enumerate(reqs):
                want = np.full(outs[i].numel(), SENTINEL, np.uint8)
                oracle.merge_layer(C, hit_np[i][layer * C:] if h else None, hs, h,
                                   miss_np[i] if m else None, ms, m, want, os_)
                assert np.array_equal(down(outs[i]), want), f"replay {rep}, request {i}"
        assert ctx.take_device_errors() == 0
        del g
    finally:
        ctx.close()


def test_pack_full_in_a_graph(gpu):
    say("  pack_full under graph capture")
    L, S, N, B, rb = 3, 2, 40, 16, 512
    Ts = [200, 17, 96]
    layout = kv.pool_layout(S, B, rb, B * rb, N * B * rb, S * N * B * rb, N)
    ref = oracle.pool_struct(S, B, rb, B * rb, N * B * rb, S * N * B * rb, N)
    C = S * rb
    tables = wl.block_tables(77, 1, N, [wl.blocks_needed(t, B) for t in Ts])
    ctx = kv.Context(0)
    try:
        pool = torch.empty(L * S * N * B * rb, dtype=torch.uint8, device=gpu)
        bts = [torch.from_numpy(t).to(gpu) for t in tables]
        fulls = [torch.empty(t * L * C, dtype=torch.uint8, device=gpu) for t in Ts]
        recs = kv.records([kv.seq(bts[i], fulls[i], Ts[i]) for i in range(len(Ts))])
        g = _capture(lambda st: kv.kvm_pack_full(ctx.handle, layout, pool, L, recs, stream=st))
        for rep in range(4):
            pool_np = wl.random_bytes(500 + rep, 1, pool.numel())
            pool.copy_(torch.from_numpy(pool_np))
            for f in fulls:
                f.fill_(SENTINEL)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            for i, t in enumerate(Ts):
                want = np.full(fulls[i].numel(), SENTINEL, np.uint8)
                oracle.pack_full(pool_np, ref, L, tables[i], t, want)
                assert np.array_equal(down(fulls[i]), want), f"replay {rep}, sequence {i}"
        assert ctx.take_device_errors() == 0
        del g
    finally:
        ctx.close()
