"""GPU parity at the full workload sizes, in the launch configuration the bench
times (all requests in one call per op and layer, 16-byte moves), checked on
sampled outputs that the oracle computes from the same bytes.

The oracle is run on sub-problems it defines exactly: one layer slab of the
pool described as a one-layer slot pool, and one layer slice of a Full Block
described as a one-layer Full Block. Sampled layers and requests are fixed
below; every byte of each sampled output is compared.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import SENTINEL, say
from paged_kv_cache_kvm_amd import kvmove as kv
from paged_kv_cache_kvm_amd import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ctx(gpu):
    c = kv.Context(0)
    yield c
    c.close()
    torch.cuda.empty_cache()


def host(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(-1).view(torch.uint8).cpu().numpy()


def layer_slice(full: torch.Tensor, T: int, L: int, C: int, l: int) -> np.ndarray:
    """Rows [0, T) of layer l of a token-major [T][L][C] byte buffer, as [T][C]."""
    return host(full[:T * L * C].view(T, L, C)[:, l, :])


def need_free(nbytes):
    free, _ = torch.cuda.mem_get_info()
    if free < nbytes:
        pytest.fail(f"workload needs {nbytes / 2**30:.1f} GiB, {free / 2**30:.1f} GiB free")


@pytest.mark.parametrize("fused", [False, True], ids=["separate", "fused"])
def test_llama8b_layer_loop(ctx, gpu, fused):
    """8 x (32768 hit + 512 miss) tokens, 32 layers, B=16, 24576-block pool:
    unpack_layer + merge_layer for every layer (or unpack_merge_layer), then
    pack_full(T_all)."""
    w = wl.LLAMA8B
    sh = w.shape
    L, S, B, rb, N = sh.layers, sh.sides, sh.block_tokens, sh.row_bytes, w.pool_blocks
    C = sh.c_kv_bytes
    R, t_hit, t_miss = len(w.t_hit), w.t_hit[0], w.t_miss[0]
    t_all = t_hit + t_miss
    slab = S * N * B * rb
    need_free(L * slab + R * (t_hit * L * C + t_miss * L * C + 2 * t_all * L * C) + (1 << 30))
    say(f"  {w.name} seed={w.seed} fused={fused}")
    u8 = dict(dtype=torch.uint8, device=gpu)
    pool = torch.empty(L * slab, **u8)
    wl.fill_bf16_normal_(pool, w.seed, 1)
    tables = wl.block_tables(w.seed, 2, N, [wl.blocks_needed(t_all, B)] * R)
    bts = [torch.from_numpy(t).to(gpu) for t in tables]
    fbs = [torch.empty(t_hit * L * C, **u8) for _ in range(R)]
    misses = [torch.empty(t_miss * L * C, **u8) for _ in range(R)]
    for r in range(R):
        wl.fill_bf16_normal_(fbs[r], w.seed, 10 + r)
        wl.fill_bf16_normal_(misses[r], w.seed, 30 + r)
    complete = torch.full((R * L * t_all * C,), SENTINEL, **u8)
    packed = [torch.full((t_all * L * C,), SENTINEL, **u8) for _ in range(R)]
    layout = kv.pool_layout(S, B, rb, B * rb, N * B * rb, S * N * B * rb, N)
    unpack_seqs = [kv.seq(bts[r], fbs[r], t_hit) for r in range(R)]
    sample_layers = (0, 17, L - 1)
    pre = {}
    for l in range(L):
        if l in sample_layers:
            pre[l] = host(pool[l * slab:(l + 1) * slab])
        if fused:
            kv.kvm_unpack_merge_layer(ctx.handle, layout, pool, L, l, [
                kv.layer_seq(bts[r], fbs[r], t_hit, misses[r].data_ptr() + l * C, L * C, t_miss,
                             complete.data_ptr() + (r * L + l) * t_all * C, C)
                for r in range(R)])
            continue
        kv.kvm_unpack_layer(ctx.handle, layout, pool, L, l, unpack_seqs)
        kv.kvm_merge_layer(ctx.handle, C, [
            kv.merge_seq(fbs[r].data_ptr() + l * C, L * C, t_hit, misses[r].data_ptr() + l * C,
                         L * C, t_miss, complete.data_ptr() + (r * L + l) * t_all * C, C)
            for r in range(R)])
    kv.kvm_pack_full(ctx.handle, layout, pool, L, [kv.seq(bts[r], packed[r], t_all)
                                                  for r in range(R)])
    torch.cuda.synchronize()
    assert ctx.take_device_errors() == 0

    slot = oracle.pool_struct(S, B, rb, B * rb, N * B * rb, 0, N)  # one layer slab
    for l in sample_layers:
        say(f"  checking layer {l}")
        want = pre[l]
        hits = [layer_slice(fbs[r], t_hit, L, C, l) for r in range(R)]
        for r in range(R):
            oracle.unpack_layer(want, slot, 1, 0, tables[r], t_hit, hits[r])
        got_slab = host(pool[l * slab:(l + 1) * slab])
        assert np.array_equal(got_slab, want), f"unpack_layer {l}"
        for r in range(R):
            miss = layer_slice(misses[r], t_miss, L, C, l)
            exp = np.zeros(t_all * C, np.uint8)
            oracle.merge_layer(C, hits[r], C, t_hit, miss, C, t_miss, exp, C)
            got = host(complete[(r * L + l) * t_all * C:(r * L + l + 1) * t_all * C])
            assert np.array_equal(got, exp), f"merge_layer {l} request {r}"
        for r in (0, R - 1):
            exp = np.zeros(t_all * C, np.uint8)
            oracle.pack_full(got_slab, slot, 1, tables[r], t_all, exp)
            assert np.array_equal(layer_slice(packed[r], t_all, L, C, l), exp), \
                f"pack_full layer {l} request {r}"
    # Every layer and request, by a property of the three operations: a hit token's
    # row in the packed Full Block (read back from its slot after unpack) equals
    # its row in complete_layer (merged from the same hit slice).
    say("  checking pack_full == complete_layer on the hit rows of every layer")
    for r in range(R):
        pk = packed[r].view(t_all, L, C)
        cm = complete[r * L * t_all * C:(r + 1) * L * t_all * C].view(L, t_all, C)
        for l in range(L):
            assert torch.equal(pk[:t_hit, l], cm[l, :t_hit]), f"layer {l} request {r}"
    # Every layer, side and request, every token (the miss tokens t >= T_hit too),
    # by pack's definition on the final pool: packed[r][t][l][s] is the slot row
    # pool[l][s][bt[t / B]][t % B], gathered with torch from the block table.
    say("  checking pack_full == pool[l][s][bt[t/B]][t%B] for every token, layer and side")
    pv = pool.view(L, S, N, B, rb)
    for r in range(R):
        pk = packed[r].view(t_all, L, S, rb)
        bt_l = bts[r].long()
        for t0 in range(0, t_all, 4096):
            t = torch.arange(t0, min(t_all, t0 + 4096), device=gpu)
            rows = pv[:, :, bt_l[t // B], t % B]            # [L][S][tokens][rb]
            assert torch.equal(pk[t0:t0 + len(t)], rows.permute(2, 0, 1, 3)), \
                f"pack_full request {r} tokens [{t0}, {t0 + len(t)})"
            del rows
    del pool, pv, fbs, misses, complete, packed
    torch.cuda.empty_cache()


def _check_all_objects(src, dst, descs, granule=256, batch=2048):
    """Every object, on the device: dst[dst_off, +n) == src[src_off, +n). All
    offsets are multiples of `granule`, so each length class is compared through
    strided windows of the two buffers."""
    descs_t = torch.from_numpy(descs.astype(np.int64)).to(src.device)
    for n in np.unique(descs[:, 2]):
        n = int(n)
        sel = descs_t[descs_t[:, 2] == n]
        ws = src.unfold(0, n, granule)
        wd = dst.unfold(0, n, granule)
        for a in range(0, len(sel), batch):
            part = sel[a:a + batch]
            assert torch.equal(wd[part[:, 1] // granule], ws[part[:, 0] // granule]), \
                f"an object of {n} bytes differs"


def _check_untouched(dst, descs, granule=256, chunk=1 << 22):
    """Every granule of dst that no object covers still holds the sentinel."""
    covered = torch.zeros(dst.numel() // granule, dtype=torch.bool, device=dst.device)
    d = torch.from_numpy(descs.astype(np.int64)).to(dst.device)
    first, count = d[:, 1] // granule, d[:, 2] // granule
    idx = torch.repeat_interleave(first, count) + (
        torch.arange(int(count.sum().item()), device=dst.device)
        - torch.repeat_interleave(torch.cumsum(count, 0) - count, count))
    covered[idx] = True
    g = dst.view(-1, granule)
    for a in range(0, g.shape[0], chunk):
        free = ~covered[a:a + chunk]
        assert bool((g[a:a + chunk][free] == SENTINEL).all().item()), "a byte outside every object was written"


def _check_copies(src, dst, descs, sample, gaps=None):
    for k in sample:
        so, do, n = (int(x) for x in descs[k])
        exp = np.full(n, SENTINEL, np.uint8)
        oracle.batch_copy(exp, host(src[so:so + n]), np.array([[0, 0, n]], np.uint64))
        assert np.array_equal(host(dst[do:do + n]), exp), f"object {k}"
    if gaps is not None:
        for a, b in gaps:
            assert np.all(host(dst[a:b]) == SENTINEL), f"gap [{a}, {b}) written"


def test_qwen32b_object_restore(ctx, gpu):
    """One 128000-token sequence as 256000 K/V objects of 128 KiB scattered in a
    36 GiB staging arena, restored into the paged pool: one call of all
    objects (its first call, which runs the metadata pass, and a later one,
    which the list's known shape makes one workgroup per object, as the bench
    times it), then 64 per-layer calls of 4000."""
    descs_np, bt, pool_bytes = wl.qwen32b_object_descs()
    n = len(descs_np)
    need_free(wl.QWEN32B_STAGING + pool_bytes + (1 << 30))
    say(f"  qwen3-32b-like restore: {n} objects, pool {pool_bytes / 2**30:.2f} GiB")
    u8 = dict(dtype=torch.uint8, device=gpu)
    staging = torch.empty(wl.QWEN32B_STAGING, **u8)
    wl.fill_random_bytes_(staging, 1003, 5)
    descs = torch.from_numpy(descs_np.view(np.uint8).reshape(-1)).to(gpu)
    rng = np.random.default_rng(3)
    sample = np.concatenate([[0, n - 1], rng.choice(n, 3000, replace=False)])
    for mode in ("one call", "one call, shape known", "per layer"):
        pool = torch.full((pool_bytes,), SENTINEL, **u8)
        if mode.startswith("one call"):
            kv.kvm_batch_copy(ctx.handle, pool, pool_bytes, staging, wl.QWEN32B_STAGING, descs, n)
            if mode == "one call, shape known":   # the first call above left the shape's count
                torch.cuda.synchronize()
                pool.fill_(SENTINEL)
                kv.kvm_batch_copy(ctx.handle, pool, pool_bytes, staging, wl.QWEN32B_STAGING,
                                  descs, n)
        else:
            per = n // wl.QWEN32B_SHAPE.layers
            for l in range(wl.QWEN32B_SHAPE.layers):
                kv.kvm_batch_copy(ctx.handle, pool, pool_bytes, staging, wl.QWEN32B_STAGING,
                                  descs.data_ptr() + l * per * 24, per)
        torch.cuda.synchronize()
        say(f"  checking {mode}")
        assert ctx.take_device_errors() == 0
        _check_copies(staging, pool, descs_np, sample)
        _check_all_objects(staging, pool, descs_np)
        # the objects tile the pool exactly: the first 64 bytes of every object
        # were overwritten (64 random bytes all equal to the sentinel: p = 2^-512)
        heads = pool.view(-1, 131072)[:, :64]
        assert int((heads == SENTINEL).all(dim=1).sum().item()) == 0, "an object was not restored"
        del pool, heads
    del staging, descs
    torch.cuda.empty_cache()


@pytest.mark.parametrize("fused", [False, True], ids=["separate", "fused"])
def test_mla_agentic_layer_loop(ctx, gpu, fused):
    """64 requests, T_hit ~ U{16384..65536}, T_miss ~ U{128..1024}, 61 layers of
    one 576-element latent, B=64, one-layer slot pool: per layer unpack of the
    hit slice, then merge with that layer's miss rows into a 2-deep ring (or
    both in one unpack_merge_layer call)."""
    w = wl.mla_agentic()
    sh = w.shape
    L, S, B, rb, C = sh.layers, sh.sides, sh.block_tokens, sh.row_bytes, sh.c_kv_bytes
    R = len(w.t_hit)
    per_req = [wl.blocks_needed(t, B) for t in w.t_all]
    N = sum(per_req)
    fb_bytes = [t * L * C for t in w.t_hit]
    miss_bytes = [t * C for t in w.t_miss]
    slot_bytes = N * B * rb
    ring = [sum(t * C for t in w.t_all)] * 2
    need_free(sum(fb_bytes) + L * sum(miss_bytes) + slot_bytes + sum(ring) + (2 << 30))
    say(f"  {w.name}: sum T_hit={sum(w.t_hit)}, Full Blocks {sum(fb_bytes) / 2**30:.1f} GiB, "
        f"slot pool {N} blocks, fused={fused}")
    u8 = dict(dtype=torch.uint8, device=gpu)
    tables = wl.block_tables(w.seed, 2, N, per_req)
    bts = [torch.from_numpy(t).to(gpu) for t in tables]
    fbs = []
    for r in range(R):
        fbs.append(torch.empty(fb_bytes[r], **u8))
        wl.fill_bf16_normal_(fbs[r], w.seed, 100 + r)
    misses = torch.empty(L * sum(miss_bytes), **u8)       # [L][request][T_miss][C]
    wl.fill_bf16_normal_(misses, w.seed, 7)
    moff = np.concatenate([[0], np.cumsum(miss_bytes)])
    slot = torch.empty(slot_bytes, **u8)
    wl.fill_bf16_normal_(slot, w.seed, 8)
    rings = [torch.full((ring[0],), SENTINEL, **u8) for _ in range(2)]
    roff = np.concatenate([[0], np.cumsum([t * C for t in w.t_all])])
    layout = kv.pool_layout(S, B, rb, B * rb, N * B * rb, 0, N)
    seqs = [kv.seq(bts[r], fbs[r], w.t_hit[r]) for r in range(R)]
    sample_layers = (0, L // 2, L - 1)
    ref = oracle.pool_struct(S, B, rb, B * rb, N * B * rb, 0, N)
    for l in range(L):
        pre = host(slot) if l in sample_layers else None
        mbase = misses.data_ptr() + l * int(moff[-1])
        out = rings[l % 2]
        if fused:
            kv.kvm_unpack_merge_layer(ctx.handle, layout, slot, L, l, [
                kv.layer_seq(bts[r], fbs[r], w.t_hit[r], mbase + int(moff[r]), C, w.t_miss[r],
                             out.data_ptr() + int(roff[r]), C) for r in range(R)])
        else:
            kv.kvm_unpack_layer(ctx.handle, layout, slot, L, l, seqs)
            kv.kvm_merge_layer(ctx.handle, C, [
                kv.merge_seq(fbs[r].data_ptr() + l * C, L * C, w.t_hit[r], mbase + int(moff[r]),
                             C, w.t_miss[r], out.data_ptr() + int(roff[r]), C) for r in range(R)])
        # Every layer and request, by the operations' defining properties (on the
        # device, after the moves on the same stream): complete_layer is the layer's
        # hit slice then its miss rows, and hit token t sits in slot (bt[t / B], t % B).
        slots = slot.view(N, B, C)
        for r in range(R):
            th = w.t_hit[r]
            fbl = fbs[r].view(th, L, C)[:, l]
            o = out[int(roff[r]):int(roff[r + 1])].view(-1, C)
            mr = misses[l * int(moff[-1]) + int(moff[r]):l * int(moff[-1]) + int(moff[r + 1])]
            assert torch.equal(o[:th], fbl), f"complete_layer hit rows, layer {l} request {r}"
            assert torch.equal(o[th:], mr.view(-1, C)), f"complete_layer miss rows, layer {l}"
            t = torch.arange(th, device=gpu)
            assert torch.equal(slots[bts[r].long()[t // B], t % B], fbl), \
                f"slot rows, layer {l} request {r}"
        if pre is None:
            continue
        torch.cuda.synchronize()
        say(f"  checking layer {l}")
        hits = [layer_slice(fbs[r], w.t_hit[r], L, C, l) for r in range(R)]
        for r in range(R):
            oracle.unpack_layer(pre, ref, 1, 0, tables[r], w.t_hit[r], hits[r])
        assert np.array_equal(host(slot), pre), f"unpack_layer {l}"
        got = host(out)
        ml = host(misses[l * int(moff[-1]):(l + 1) * int(moff[-1])])
        for r in range(R):
            exp = np.zeros(w.t_all[r] * C, np.uint8)
            oracle.merge_layer(C, hits[r], C, w.t_hit[r], ml[int(moff[r]):], C, w.t_miss[r],
                               exp, C)
            assert np.array_equal(got[int(roff[r]):int(roff[r + 1])], exp), \
                f"merge_layer {l} request {r}"
    torch.cuda.synchronize()
    assert ctx.take_device_errors() == 0
    del fbs, misses, slot, rings
    torch.cuda.empty_cache()


def test_small_objects(ctx, gpu):
    """200000 objects of 256*U{16..512} bytes between two 16 GiB arenas: the
    first call (grid guessed), then a later one with the grid sized from the
    piece count the first left, as the bench times it; each checked whole."""
    w = wl.SMALL_OBJS
    descs_np = wl.small_object_descs(w)
    n = len(descs_np)
    need_free(w.src_arena + w.dst_arena + (1 << 30))
    say(f"  {w.name}")
    u8 = dict(dtype=torch.uint8, device=gpu)
    src = torch.empty(w.src_arena, **u8)
    wl.fill_random_bytes_(src, w.seed, 1)
    dst = torch.full((w.dst_arena,), SENTINEL, **u8)
    descs = torch.from_numpy(descs_np.view(np.uint8).reshape(-1)).to(gpu)
    rng = np.random.default_rng(5)
    sample = np.concatenate([[0, n - 1], rng.choice(n, 3000, replace=False)])
    order = np.argsort(descs_np[:, 1])
    ends = descs_np[order, 1] + descs_np[order, 2]
    starts = descs_np[order, 1]
    gaps = [(int(ends[i]), int(starts[i + 1])) for i in rng.choice(n - 1, 300, replace=False)
            if starts[i + 1] > ends[i]]
    for call in ("first call", "piece count known"):
        if call != "first call":
            dst.fill_(SENTINEL)
        kv.kvm_batch_copy(ctx.handle, dst, w.dst_arena, src, w.src_arena, descs, n)
        torch.cuda.synchronize()
        assert ctx.take_device_errors() == 0
        say(f"  {call}: checking every object and every uncovered granule")
        _check_copies(src, dst, descs_np, sample, gaps)
        _check_all_objects(src, dst, descs_np)
        _check_untouched(dst, descs_np)
    del src, dst, descs
    torch.cuda.empty_cache()


def test_one_object_above_4gib(ctx, gpu):
    """One 5 GiB + 5 byte object at offsets 3 and 19 (equal modulo 16: a byte
    head, 16-byte body, byte tail), so lengths and vector counts need 64 bits.
    Every byte is compared on the device; the bytes around it keep the sentinel."""
    n = (5 << 30) + 5
    size = n + 64
    need_free(2 * size + (1 << 30))
    say(f"  one object of {n} bytes")
    u8 = dict(dtype=torch.uint8, device=gpu)
    src = torch.empty(size, **u8)
    wl.fill_random_bytes_(src, 1006, 1)
    dst = torch.full((size,), SENTINEL, **u8)
    descs_np = np.array([[3, 19, n]], np.uint64)
    descs = torch.from_numpy(descs_np.view(np.uint8).reshape(-1)).to(gpu)
    kv.kvm_batch_copy(ctx.handle, dst, size, src, size, descs, 1)
    torch.cuda.synchronize()
    assert ctx.take_device_errors() == 0
    assert torch.equal(dst[19:19 + n], src[3:3 + n])
    assert bool((dst[:19] == SENTINEL).all().item())
    assert bool((dst[19 + n:] == SENTINEL).all().item())
    del src, dst, descs
    torch.cuda.empty_cache()
