"""GPU parity with the Full Block and complete_layer in pinned host memory (the
pages' host-DRAM prompt buffers): the same kernels read and write them over
PCIe through their device-visible addresses. Every byte is compared with the
oracle on the same inputs."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import SENTINEL, down, say, up
from paged_kv_cache_kvm_amd import kvmove as kv
from paged_kv_cache_kvm_amd import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ctx(gpu):
    c = kv.Context(0)
    yield c
    c.close()


def pinned(a: np.ndarray) -> torch.Tensor:
    t = torch.empty(a.size, dtype=torch.uint8, pin_memory=True)
    t.copy_(torch.from_numpy(np.ascontiguousarray(a).view(np.uint8).ravel()))
    return t


@pytest.mark.parametrize("L,S,N,B,rb,reqs", [
    (4, 2, 64, 16, 256, [(240, 16)]),
    (3, 1, 200, 64, 1152, [(700, 77), (65, 3), (0, 5)]),
    (2, 2, 300, 16, 2048, [(511, 33), (64, 0)]),
], ids=["tiny", "mla-like", "llama-like"])
def test_host_full_block(ctx, gpu, L, S, N, B, rb, reqs):
    """pack_full into, and unpack / merge / unpack_merge from, pinned host Full
    Blocks; merge and unpack_merge into pinned host complete_layer buffers."""
    C = S * rb
    say(f"  host tier L={L} S={S} N={N} B={B} rb={rb} reqs={reqs}")
    layout = kv.pool_layout(S, B, rb, B * rb, N * B * rb, S * N * B * rb, N)
    ref = oracle.pool_struct(S, B, rb, B * rb, N * B * rb, S * N * B * rb, N)
    rng = np.random.default_rng(L * 1000 + N)
    tables = wl.block_tables(41, N, N, [wl.blocks_needed(h + m, B) for h, m in reqs])
    bts = [up(t, gpu) for t in tables]
    pool_np = rng.integers(0, 256, L * S * N * B * rb, dtype=np.uint8)
    pool = up(pool_np, gpu)

    # pack_full into host Full Blocks (all T_all tokens)
    wants, fulls = [], []
    for i, (h, m) in enumerate(reqs):
        w = np.full(max(h + m, 1) * L * C, SENTINEL, np.uint8)
        oracle.pack_full(pool_np, ref, L, tables[i], h + m, w)
        wants.append(w)
        fulls.append(pinned(np.full(w.size, SENTINEL, np.uint8)))
    kv.kvm_pack_full(ctx.handle, layout, pool, L, [kv.seq(bts[i], fulls[i], h + m)
                                                  for i, (h, m) in enumerate(reqs)])
    torch.cuda.synchronize()
    for i in range(len(reqs)):
        assert np.array_equal(fulls[i].numpy(), wants[i]), f"pack_full to host, request {i}"

    # unpack, merge and the fused call from host Full Blocks into device / host buffers
    fb_np = [rng.integers(0, 256, max(h, 1) * L * C, dtype=np.uint8) for h, _ in reqs]
    miss_np = [rng.integers(0, 256, max(m, 1) * C, dtype=np.uint8) for _, m in reqs]
    fbs = [pinned(a) for a in fb_np]
    misses = [pinned(a) for a in miss_np]
    want_pool = pool_np.copy()
    for layer in sorted({0, L - 1}):
        want_out = []
        for i, (h, m) in enumerate(reqs):
            oracle.unpack_layer(want_pool, ref, L, layer, tables[i], h, fb_np[i])
            o = np.full(max(h + m, 1) * C, SENTINEL, np.uint8)
            oracle.merge_layer(C, fb_np[i][layer * C:] if h else None, L * C, h,
                               miss_np[i] if m else None, C, m, o, C)
            want_out.append(o)
        for fused in (False, True):
            pool_l = up(pool_np if layer == 0 else pool_after, gpu)
            outs = [pinned(np.full(max(h + m, 1) * C, SENTINEL, np.uint8)) for h, m in reqs]
            if fused:
                kv.kvm_unpack_merge_layer(ctx.handle, layout, pool_l, L, layer, [
                    kv.layer_seq(bts[i] if h else 0, fbs[i] if h else 0, h,
                                 misses[i] if m else 0, C, m, outs[i], C)
                    for i, (h, m) in enumerate(reqs)])
            else:
                kv.kvm_unpack_layer(ctx.handle, layout, pool_l, L, layer,
                                    [kv.seq(bts[i], fbs[i], h) for i, (h, _) in enumerate(reqs)])
                kv.kvm_merge_layer(ctx.handle, C, [
                    kv.merge_seq(fbs[i].data_ptr() + layer * C if h else 0, L * C, h,
                                 misses[i] if m else 0, C, m, outs[i], C)
                    for i, (h, m) in enumerate(reqs)])
            torch.cuda.synchronize()
            assert np.array_equal(down(pool_l), want_pool), f"unpack from host, layer {layer}"
            for i in range(len(reqs)):
                assert np.array_equal(outs[i].numpy(), want_out[i]), \
                    f"merge into host, layer {layer}, request {i}, fused={fused}"
        pool_after = want_pool.copy()
    assert ctx.take_device_errors() == 0


@pytest.mark.parametrize("direction", ["host-to-device", "device-to-host"])
@pytest.mark.parametrize("kind", ["pieces", "short", "one"])
def test_host_batch_copy(ctx, gpu, direction, kind):
    """The batched copy with its source (a restore from a host-DRAM staging
    buffer) or its destination in pinned host memory; the descriptors stay in
    device memory. Each list copied twice (the second time with its shape
    known), every byte against the oracle."""
    rng = np.random.default_rng({"pieces": 41, "short": 42, "one": 44}[kind])
    n = 1 if kind == "one" else 600
    if kind == "one":                           # 40 full pieces and a ragged last one
        lens = np.array([40 * (128 << 10) + 3840], np.int64)
    else:
        lens = (16384 * rng.integers(1, 17, size=n) if kind == "pieces"
                else 256 * rng.integers(1, 9, size=n)).astype(np.int64)
    arena = int(lens.sum()) + (4 << 20)
    descs = np.stack([wl.placements(43, 1, lens, arena), wl.placements(43, 2, lens, arena),
                      lens], axis=1).astype(np.uint64)
    say(f"  host batch copy {direction} {kind}: {n} objects, {int(lens.sum()) >> 20} MiB")
    src_np = rng.integers(0, 256, arena, dtype=np.uint8)
    want = np.full(arena, SENTINEL, np.uint8)
    oracle.batch_copy(want, src_np, descs)
    dd = up(descs.view(np.uint8), gpu)
    if direction == "host-to-device":
        src = pinned(src_np)
    else:
        src = up(src_np, gpu)
    for call in range(2):
        if direction == "host-to-device":
            dst = up(np.full(arena, SENTINEL, np.uint8), gpu)
        else:
            dst = pinned(np.full(arena, SENTINEL, np.uint8))
        kv.kvm_batch_copy(ctx.handle, dst, arena, src, arena, dd, n)
        torch.cuda.synchronize()
        got = down(dst) if direction == "host-to-device" else dst.numpy()
        assert np.array_equal(got, want), f"call {call}"
    assert ctx.take_device_errors() == 0
