"""Helpers for the GPU parity tests: host <-> device byte buffers and the
generic parity runners that feed the same seeded inputs to the HIP library
(through the C ABI) and to the oracle, then compare every byte."""
from __future__ import annotations

import zlib

import numpy as np
import torch

import oracle
from paged_kv_cache_kvm_amd import kvmove as kv
from paged_kv_cache_kvm_amd import workloads as wl

SENTINEL = 0xA5


def case_seed(case) -> int:
    """A seed fixed by a test case's parameters (Python's own str hash is
    salted per process, so it would change the inputs from run to run)."""
    return zlib.crc32(repr(case).encode()) & 0xFFFF


def say(msg: str) -> None:
    print(msg, flush=True)


def up(a: np.ndarray, dev, pad: int = 0) -> torch.Tensor:
    """Device copy of a host byte array, with `pad` spare bytes in front."""
    a = np.ascontiguousarray(a).view(np.uint8).ravel()
    t = torch.empty(a.size + pad, dtype=torch.uint8, device=dev)
    if pad:
        t[:pad] = 0
    t[pad:].copy_(torch.from_numpy(a))
    return t


def down(t: torch.Tensor, start: int = 0, nbytes: int | None = None) -> np.ndarray:
    flat = t.view(-1).view(torch.uint8)
    end = flat.numel() if nbytes is None else start + nbytes
    return flat[start:end].cpu().numpy()


def layout_geometry(kind: str, L, S, N, B, rb, block_pad=0):
    """(block_stride, side_stride, layer_stride, pool_bytes) of a pool layout."""
    obj = B * rb + block_pad
    if kind == "dense":        # [L][S][N][B][rb]
        return obj, N * obj, S * N * obj, L * S * N * obj
    if kind == "block_major":  # [N][L][S][B][rb]
        return L * S * obj, obj, S * obj, N * L * S * obj
    if kind == "slot":         # [S][N][B][rb], reused by every layer
        return obj, N * obj, 0, S * N * obj
    raise ValueError(kind)


def run_pack_unpack(ctx, dev, L, S, N, B, rb, Ts, kind="dense", block_pad=0, ts_pad=0,
                    offset=0, seed=0, layers=None, check_errors=True):
    """pack_full of every sequence, then unpack_layer of each listed layer into a
    sentinel pool; each result compared byte for byte with the oracle."""
    bs, ss, ls, pool_bytes = layout_geometry(kind, L, S, N, B, rb, block_pad)
    layout = kv.pool_layout(S, B, rb, bs, ss, ls, N)
    ref = oracle.pool_struct(S, B, rb, bs, ss, ls, N)
    rng = np.random.default_rng(seed)
    tables = wl.block_tables(seed, 1, N, [wl.blocks_needed(t, B) for t in Ts])
    ts = L * S * rb + ts_pad
    say(f"  case L={L} S={S} N={N} B={B} rb={rb} T={list(Ts)[:6]}{'...' if len(Ts) > 6 else ''}"
        f" n={len(Ts)} kind={kind} ts_pad={ts_pad} offset={offset} seed={seed}")

    pool_np = rng.integers(0, 256, size=pool_bytes, dtype=np.uint8)
    # the oracle runs first: it bounds-checks every row on the CPU, so a
    # mis-sized case fails here before any kernel touches device memory
    wants = []
    for i, T in enumerate(Ts):
        want = np.full(max(T, 1) * ts, SENTINEL, np.uint8)
        oracle.pack_full(pool_np, ref, L, tables[i], T, want, token_stride=ts)
        wants.append(want)
    pool = up(pool_np, dev, offset)
    pool_ptr = pool.data_ptr() + offset
    bts = [up(t, dev) if len(t) else None for t in tables]
    fulls = [up(np.full(max(T, 1) * ts, SENTINEL, np.uint8), dev, offset) for T in Ts]
    seqs = [kv.seq(bts[i].data_ptr() if bts[i] is not None else 0,
                   fulls[i].data_ptr() + offset if T else 0, T, ts if ts_pad else 0)
            for i, T in enumerate(Ts)]
    kv.kvm_pack_full(ctx.handle, layout, pool_ptr, L, seqs)
    torch.cuda.synchronize()
    for i, T in enumerate(Ts):
        got = down(fulls[i], offset)
        assert np.array_equal(got, wants[i]), f"pack_full differs for sequence {i} (T={T})"

    # unpack from fresh Full Blocks into a sentinel pool
    fb_np = [rng.integers(0, 256, size=max(T, 1) * ts, dtype=np.uint8) for T in Ts]
    fbs = [up(f, dev, offset) for f in fb_np]
    useqs = [kv.seq(bts[i].data_ptr() if bts[i] is not None else 0,
                    fbs[i].data_ptr() + offset if T else 0, T, ts if ts_pad else 0)
             for i, T in enumerate(Ts)]
    pool_b = up(np.full(pool_bytes, SENTINEL, np.uint8), dev, offset)
    want = np.full(pool_bytes, SENTINEL, np.uint8)
    for layer in (range(L) if layers is None else layers):
        for i, T in enumerate(Ts):
            oracle.unpack_layer(want, ref, L, layer, tables[i], T, fb_np[i], token_stride=ts)
        kv.kvm_unpack_layer(ctx.handle, layout, pool_b.data_ptr() + offset, L, layer, useqs)
        torch.cuda.synchronize()
        assert np.array_equal(down(pool_b, offset), want), f"unpack_layer {layer} differs"
    if check_errors:
        assert ctx.take_device_errors() == 0


def run_merge(ctx, dev, C, reqs, L=3, hit_pad=0, miss_pad=0, out_pad=0, offset=0, seed=0):
    """merge_layer for requests [(t_hit, t_miss)], hit taken as layer `l` of a
    Full Block [T_hit][L][C] (row stride L*C + hit_pad)."""
    rng = np.random.default_rng(seed)
    say(f"  merge C={C} reqs={reqs[:4]}{'...' if len(reqs) > 4 else ''} n={len(reqs)} L={L} "
        f"pads=({hit_pad},{miss_pad},{out_pad}) offset={offset} seed={seed}")
    hs, ms, os_ = L * C + hit_pad, C + miss_pad, C + out_pad
    hit_np = [rng.integers(0, 256, size=max(h, 1) * hs, dtype=np.uint8) for h, _ in reqs]
    miss_np = [rng.integers(0, 256, size=max(m, 1) * ms, dtype=np.uint8) for _, m in reqs]
    hits = [up(a, dev, offset) for a in hit_np]
    misses = [up(a, dev, offset) for a in miss_np]
    for layer in sorted({0, L - 1}):
        wants = []
        for i, (h, m) in enumerate(reqs):   # oracle first: CPU bounds checks
            want = np.full(max(h + m, 1) * os_, SENTINEL, np.uint8)
            oracle.merge_layer(C, hit_np[i][layer * C:] if h else None, hs, h,
                               miss_np[i] if m else None, ms, m, want, os_)
            wants.append(want)
        outs = [up(np.full(max(h + m, 1) * os_, SENTINEL, np.uint8), dev, offset) for h, m in reqs]
        ms_list = [kv.merge_seq(hits[i].data_ptr() + offset + layer * C if h else 0, hs, h,
                                misses[i].data_ptr() + offset if m else 0, ms, m,
                                outs[i].data_ptr() + offset if h + m else 0, os_)
                   for i, (h, m) in enumerate(reqs)]
        kv.kvm_merge_layer(ctx.handle, C, ms_list)
        torch.cuda.synchronize()
        for i in range(len(reqs)):
            assert np.array_equal(down(outs[i], offset), wants[i]), f"merge differs for request {i}"


def run_batch_copy(ctx, dev, src_np, dst_np, descs_np, expect_skipped=0, same_buffer=False,
                   label=""):
    say(f"  batch_copy {label} n={len(descs_np)} src={src_np.size} dst={dst_np.size}")
    src = up(src_np, dev)
    dst = src if same_buffer else up(dst_np, dev)
    d = up(descs_np.astype(np.uint64).view(np.uint8), dev)
    kv.kvm_batch_copy(ctx.handle, dst, dst_np.size, src, src_np.size, d, len(descs_np))
    torch.cuda.synchronize()
    want = src_np.copy() if same_buffer else dst_np.copy()
    if expect_skipped:
        lens = descs_np[:, 2]
        ok = ((descs_np[:, 0] <= src_np.size) & (lens <= src_np.size - np.minimum(descs_np[:, 0], src_np.size)) &
              (descs_np[:, 1] <= dst_np.size) & (lens <= dst_np.size - np.minimum(descs_np[:, 1], dst_np.size)))
        descs_ok = descs_np[ok]
    else:
        descs_ok = descs_np
    oracle.batch_copy(want, want if same_buffer else src_np, descs_ok)
    assert np.array_equal(down(dst), want), f"batch_copy differs ({label})"
    assert ctx.take_device_errors() == expect_skipped


def run_unpack_merge(ctx, dev, L, S, N, B, rb, reqs, kind="dense", ts_pad=0, miss_pad=0,
                     out_pad=0, offset=0, seed=0):
    """kvm_unpack_merge_layer against the oracle's unpack_layer followed by
    merge_layer (its definition), for layers 0 and L-1."""
    bs, ss, ls, pool_bytes = layout_geometry(kind, L, S, N, B, rb)
    layout = kv.pool_layout(S, B, rb, bs, ss, ls, N)
    ref = oracle.pool_struct(S, B, rb, bs, ss, ls, N)
    C = S * rb
    ts, ms, os_ = L * C + ts_pad, C + miss_pad, C + out_pad
    say(f"  fused L={L} S={S} N={N} B={B} rb={rb} reqs={reqs[:3]}{'...' if len(reqs) > 3 else ''}"
        f" n={len(reqs)} kind={kind} pads=({ts_pad},{miss_pad},{out_pad}) offset={offset}")
    rng = np.random.default_rng(seed)
    tables = wl.block_tables(seed, 1, N, [wl.blocks_needed(h + m, B) for h, m in reqs])
    fb_np = [rng.integers(0, 256, max(h, 1) * ts, dtype=np.uint8) for h, _ in reqs]
    miss_np = [rng.integers(0, 256, max(m, 1) * ms, dtype=np.uint8) for _, m in reqs]
    pool_np = rng.integers(0, 256, pool_bytes, dtype=np.uint8)
    pool = up(pool_np, dev, offset)
    bts = [up(t, dev) for t in tables]
    fbs = [up(a, dev, offset) for a in fb_np]
    misses = [up(a, dev, offset) for a in miss_np]
    want_pool = pool_np.copy()
    for layer in sorted({0, L - 1}):
        want_out = []
        for i, (h, m) in enumerate(reqs):   # the oracle first: CPU bounds checks
            oracle.unpack_layer(want_pool, ref, L, layer, tables[i], h, fb_np[i], token_stride=ts)
            o = np.full(max(h + m, 1) * os_, SENTINEL, np.uint8)
            oracle.merge_layer(C, fb_np[i][layer * C:] if h else None, ts, h,
                               miss_np[i] if m else None, ms, m, o, os_)
            want_out.append(o)
        outs = [up(np.full(max(h + m, 1) * os_, SENTINEL, np.uint8), dev, offset) for h, m in reqs]
        seqs = [kv.layer_seq(bts[i] if h else 0, fbs[i].data_ptr() + offset if h else 0, h,
                             misses[i].data_ptr() + offset if m else 0, ms, m,
                             outs[i].data_ptr() + offset if h + m else 0, os_,
                             token_stride=ts if ts_pad else 0)
                for i, (h, m) in enumerate(reqs)]
        kv.kvm_unpack_merge_layer(ctx.handle, layout, pool.data_ptr() + offset, L, layer, seqs)
        torch.cuda.synchronize()
        assert np.array_equal(down(pool, offset), want_pool), f"pool after layer {layer}"
        for i in range(len(reqs)):
            assert np.array_equal(down(outs[i], offset), want_out[i]), \
                f"complete_layer {layer} request {i}"
    assert ctx.take_device_errors() == 0
