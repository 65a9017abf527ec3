"""Pins that tie the oracle to what the pages and plain mathematics fix.

Each pin takes a loaded oracle library and raises (AssertionError or
oracle.OracleError) if the oracle disagrees. They are independent of the
oracle's own address arithmetic:

  * labelled payloads: every 4-byte word of the input names its own
    coordinates, so the output can be decoded and compared with the meaning
    of the Full Block (DualPath KV Loading, key-objects table: [T, L, C_KV]
    with the layer slice [T, C_KV]) and of a paged block (Tutti reading notes,
    prerequisites 3, eq. 2: token t sits in block table entry t // B, row t % B);
  * numpy gathers and transposes of the same bytes (a library routine);
  * round trips and the cross-op identity of the layer loop;
  * textbook memcpy for the batched copy, and the counts the pages print.

``ALL_PINS`` lists them so that a mutated oracle can be run through every pin.
"""
from __future__ import annotations

import os

import numpy as np

import oracle
from paged_kv_cache_kvm_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "page_counts.txt")
SENTINEL = 0xA5

# (L, S, N, B, row_bytes, T) shapes: several tiles, ragged last blocks, B = 1,
# a single side, and the tiny workload itself.
SHAPES = [
    (4, 2, 64, 16, 256, 256),
    (4, 2, 64, 16, 256, 240),
    (3, 1, 20, 3, 12, 17),
    (2, 2, 9, 1, 8, 7),
    (5, 2, 40, 7, 20, 100),
    (1, 1, 4, 5, 4, 1),
]


def dense_pool(L, S, N, B, rb):
    return oracle.pool_struct(S, B, rb, B * rb, N * B * rb, S * N * B * rb, N)


def perm_table(seed, N, T, B):
    nb = -(-T // B)
    return np.random.default_rng(seed).permutation(N)[:nb].astype(np.int32)


# word layout of a labelled pool: w 8 bits | r 8 bits | n 10 bits | s 1 bit | l 5 bits
def _pool_labels(L, S, N, B, W):
    l, s, n, r, w = np.indices((L, S, N, B, W), dtype=np.uint32)
    return (l << 27) | (s << 26) | (n << 16) | (r << 8) | w


def _decode_pool_label(x):
    x = x.astype(np.uint32)
    return x >> 27, (x >> 26) & 1, (x >> 16) & 1023, (x >> 8) & 255, x & 255


# word layout of a labelled Full Block: w 8 bits | s 1 bit | l 5 bits | t 18 bits
def _full_labels(T, L, S, W):
    t, l, s, w = np.indices((T, L, S, W), dtype=np.uint32)
    return (t << 14) | (l << 9) | (s << 8) | w


def _decode_full_label(x):
    x = x.astype(np.uint32)
    return x >> 14, (x >> 9) & 31, (x >> 8) & 1, x & 255


def pin_pack_labelled(lib):
    """Full[t, l, side s, word w] holds pool (layer l, side s, block bt[t//B], row t%B, word w)."""
    for i, (L, S, N, B, rb, T) in enumerate(SHAPES):
        W = rb // 4
        pool = _pool_labels(L, S, N, B, W).view(np.uint8).ravel()
        bt = perm_table(10 + i, N, T, B)
        full = np.zeros(T * L * S * rb, np.uint8)
        oracle.pack_full(pool, dense_pool(L, S, N, B, rb), L, bt, T, full, lib=lib)
        l, s, n, r, w = _decode_pool_label(full.view(np.uint32).reshape(T, L, S, W))
        t = np.arange(T)[:, None, None, None]
        assert np.array_equal(l, np.broadcast_to(np.arange(L)[None, :, None, None], l.shape)), "layer"
        assert np.array_equal(s, np.broadcast_to(np.arange(S)[None, None, :, None], s.shape)), "side"
        assert np.array_equal(n, np.broadcast_to(bt[t // B], n.shape)), "block"
        assert np.array_equal(r, np.broadcast_to(t % B, r.shape)), "row"
        assert np.array_equal(w, np.broadcast_to(np.arange(W)[None, None, None, :], w.shape)), "word"


def pin_pack_gather(lib):
    """Dense and block-major pools, dense and padded Full Blocks: numpy gather + transpose."""
    rng = np.random.default_rng(7)
    for i, (L, S, N, B, rb, T) in enumerate(SHAPES):
        bt = perm_table(20 + i, N, T, B)
        nb = len(bt)
        # dense [L][S][N][B][rb]
        pool5 = rng.integers(0, 256, size=(L, S, N, B, rb), dtype=np.uint8)
        want = pool5[:, :, bt].transpose(2, 3, 0, 1, 4).reshape(nb * B, L, S * rb)[:T]
        full = np.zeros(T * L * S * rb, np.uint8)
        oracle.pack_full(pool5.ravel(), dense_pool(L, S, N, B, rb), L, bt, T, full, lib=lib)
        assert np.array_equal(full.reshape(T, L, S * rb), want), "dense pool"
        # block-major [N][L][S][B][rb] described by strides, Full Block padded by 96 bytes per token
        blk = np.ascontiguousarray(pool5.transpose(2, 0, 1, 3, 4))
        p = oracle.pool_struct(S, B, rb, L * S * B * rb, B * rb, S * B * rb, N)
        ts = L * S * rb + 96
        fullp = np.full(T * ts, SENTINEL, np.uint8)
        oracle.pack_full(blk.ravel(), p, L, bt, T, fullp, token_stride=ts, lib=lib)
        fp = fullp.reshape(T, ts)
        assert np.array_equal(fp[:, :L * S * rb].reshape(T, L, S * rb), want), "strided pool"
        assert np.all(fp[:, L * S * rb:] == SENTINEL), "token padding written"


def pin_unpack_labelled(lib):
    """After unpack(layer): slot (side s, bt[b], row r) holds Full[b*B + r, layer, s] for
    b*B + r < T; every other slot and every other layer keeps the sentinel."""
    for i, (L, S, N, B, rb, T) in enumerate(SHAPES):
        W = rb // 4
        full = _full_labels(T, L, S, W).view(np.uint8).ravel()
        bt = perm_table(30 + i, N, T, B)
        inv = np.full(N, -1, np.int64)
        inv[bt] = np.arange(len(bt))
        for layer in sorted({0, L - 1}):
            pool = np.full(L * S * N * B * rb, SENTINEL, np.uint8)
            oracle.unpack_layer(pool, dense_pool(L, S, N, B, rb), L, layer, bt, T, full, lib=lib)
            pw = pool.view(np.uint32).reshape(L, S, N, B, W)
            sent = np.uint32(0xA5A5A5A5)
            others = np.delete(pw, layer, axis=0)
            assert np.all(others == sent), "another layer written"
            lay = pw[layer]                                  # [S, N, B, W]
            tok = inv[:, None] * B + np.arange(B)[None, :]   # [N, B] token held by each slot
            held = (inv[:, None] >= 0) & (tok < T)
            assert np.all(lay[:, ~held] == sent), "slot outside the hit tokens written"
            t, l, s, w = _decode_full_label(lay[:, held])    # [S, count, W]
            assert np.array_equal(t, np.broadcast_to(tok[held][None, :, None], t.shape)), "token"
            assert np.all(l == layer), "layer"
            assert np.array_equal(s, np.broadcast_to(np.arange(S)[:, None, None], s.shape)), "side"
            assert np.array_equal(w, np.broadcast_to(np.arange(W)[None, None, :], w.shape)), "word"


def pin_unpack_scatter(lib):
    """numpy scatter of the layer slice into the block-table slots; slot pool (layer stride 0)."""
    rng = np.random.default_rng(8)
    for i, (L, S, N, B, rb, T) in enumerate(SHAPES):
        bt = perm_table(40 + i, N, T, B)
        full = rng.integers(0, 256, size=(T, L, S, rb), dtype=np.uint8)
        t = np.arange(T)
        for layer in range(L):
            pool = np.full((L, S, N, B, rb), SENTINEL, np.uint8)
            want = pool.copy()
            want[layer][:, bt[t // B], t % B, :] = full[:, layer].transpose(1, 0, 2)
            oracle.unpack_layer(pool.ravel(), dense_pool(L, S, N, B, rb), L, layer, bt, T,
                                full.ravel(), lib=lib)
            assert np.array_equal(pool, want), f"layer {layer}"
        # one-layer slot pool reused by every layer: the last unpack wins
        slot = np.full((S, N, B, rb), SENTINEL, np.uint8)
        p = oracle.pool_struct(S, B, rb, B * rb, N * B * rb, 0, N)
        for layer in range(L):
            oracle.unpack_layer(slot.ravel(), p, L, layer, bt, T, full.ravel(), lib=lib)
            want = np.full((S, N, B, rb), SENTINEL, np.uint8)
            want[:, bt[t // B], t % B, :] = full[:, layer].transpose(1, 0, 2)
            assert np.array_equal(slot, want), f"slot pool layer {layer}"


def pin_roundtrip(lib):
    """pack(unpack_all(FB)) == FB through a second, independent table, and
    unpack(pack(P)) restores P's used slots."""
    rng = np.random.default_rng(9)
    for i, (L, S, N, B, rb, T) in enumerate(SHAPES):
        p = dense_pool(L, S, N, B, rb)
        bta = perm_table(50 + i, N, T, B)
        btb = perm_table(60 + i, N, T, B)
        pool_a = rng.integers(0, 256, size=L * S * N * B * rb, dtype=np.uint8)
        fb = np.zeros(T * L * S * rb, np.uint8)
        oracle.pack_full(pool_a, p, L, bta, T, fb, lib=lib)
        pool_b = np.full_like(pool_a, SENTINEL)
        for layer in range(L):
            oracle.unpack_layer(pool_b, p, L, layer, btb, T, fb, lib=lib)
        fb2 = np.zeros_like(fb)
        oracle.pack_full(pool_b, p, L, btb, T, fb2, lib=lib)
        assert np.array_equal(fb2, fb), "pack(unpack(FB)) != FB"
        # back into pool A's own slots: bytes of the used slots return unchanged
        pool_c = pool_a.copy()
        for layer in range(L):
            oracle.unpack_layer(pool_c, p, L, layer, bta, T, fb, lib=lib)
        assert np.array_equal(pool_c, pool_a), "unpack(pack(P)) != P"
        # only hit slots were written into pool B
        assert int((pool_b != SENTINEL).sum()) <= T * L * S * rb


def pin_merge(lib):
    """complete = hit rows (the strided layer slice of the Full Block) then miss rows."""
    rng = np.random.default_rng(11)
    cases = [(4, 512, 240, 16, 0), (3, 36, 5, 0, 8), (2, 64, 0, 9, 128), (61, 16, 33, 7, 16),
             (1, 4, 1, 1, 0)]
    for L, C, t_hit, t_miss, pad in cases:
        fb = rng.integers(0, 256, size=(max(t_hit, 1), L, C), dtype=np.uint8)
        miss = rng.integers(0, 256, size=(max(t_miss, 1), C + 8), dtype=np.uint8)  # padded rows
        ostride = C + pad
        t_all = t_hit + t_miss
        for layer in sorted({0, L - 1}):
            out = np.full((t_all + 2) * ostride, SENTINEL, np.uint8)
            hit_view = fb.ravel()[layer * C:]
            oracle.merge_layer(C, hit_view if t_hit else None, L * C, t_hit,
                               miss.ravel() if t_miss else None, C + 8, t_miss,
                               out, ostride, lib=lib)
            o = out.reshape(t_all + 2, ostride)
            assert np.array_equal(o[:t_hit, :C], fb[:t_hit, layer]), "hit rows"
            assert np.array_equal(o[t_hit:t_all, :C], miss[:t_miss, :C]), "miss rows"
            assert np.all(o[:, C:] == SENTINEL), "row padding written"
            assert np.all(o[t_all:] == SENTINEL), "rows past T_all written"


def pin_cross_op(lib):
    """Layer loop of one request: unpack each layer of the Full Block (hit rows and
    appended miss rows) into the pool, merge hit||miss into complete[l], then
    pack_full(T_all) equals complete[l] row for row, for every layer."""
    L, S, N, B, rb = 4, 2, 64, 16, 256
    t_hit, t_miss = 240, 16
    t_all = t_hit + t_miss
    C = S * rb
    rng = np.random.default_rng(12)
    p = dense_pool(L, S, N, B, rb)
    bt = perm_table(70, N, t_all, B)
    fb_hit = rng.integers(0, 256, size=(t_hit, L, C), dtype=np.uint8)
    miss = rng.integers(0, 256, size=(L, t_miss, C), dtype=np.uint8)
    fb_all = np.concatenate([fb_hit, miss.transpose(1, 0, 2)], axis=0)  # this round's tokens
    pool = np.full(L * S * N * B * rb, SENTINEL, np.uint8)
    complete = np.zeros((L, t_all, C), np.uint8)
    for layer in range(L):
        oracle.unpack_layer(pool, p, L, layer, bt, t_all, np.ascontiguousarray(fb_all).ravel(),
                            lib=lib)
        out = complete[layer].ravel()
        oracle.merge_layer(C, fb_hit.ravel()[layer * C:], L * C, t_hit, miss[layer].ravel(), C,
                           t_miss, out, C, lib=lib)
        complete[layer] = out.reshape(t_all, C)
    packed = np.zeros(t_all * L * C, np.uint8)
    oracle.pack_full(pool, p, L, bt, t_all, packed, lib=lib)
    assert np.array_equal(packed.reshape(t_all, L, C).transpose(1, 0, 2), complete)


def pin_batch_copy(lib):
    """Textbook memcpy per object; gaps keep their bytes; any alignment and length."""
    rng = np.random.default_rng(13)
    for n, gran, arena in [(300, 1, 1 << 20), (200, 256, 1 << 22), (50, 16, 1 << 16)]:
        if gran == 1:
            lens = rng.integers(0, 3000, size=n)
        else:
            lens = gran * rng.integers(0, 40, size=n)
        src_off = wl.placements(1, 2 + gran, lens, arena, gran)
        dst_off = wl.placements(1, 3 + gran, lens, arena, gran)
        src = rng.integers(0, 256, size=arena, dtype=np.uint8)
        dst = np.full(arena, SENTINEL, np.uint8)
        want = dst.copy()
        for so, do, ln in zip(src_off, dst_off, lens):
            want[do:do + ln] = src[so:so + ln]
        descs = np.stack([src_off, dst_off, lens], axis=1).astype(np.uint64)
        oracle.batch_copy(dst, src, descs, lib=lib)
        assert np.array_equal(dst, want), f"batch copy n={n} granule={gran}"
        assert int((dst != SENTINEL).sum()) <= int(lens.sum())
    # copy inside one buffer with disjoint source and destination ranges
    buf = rng.integers(0, 256, size=4096, dtype=np.uint8)
    want = buf.copy()
    want[2000:2100] = buf[10:110]
    want[3000:3005] = buf[500:505]
    oracle.batch_copy(buf, buf, np.array([[10, 2000, 100], [500, 3000, 5]], np.uint64), lib=lib)
    assert np.array_equal(buf, want), "in-buffer copy"


def pin_batch_copy_rejects(lib):
    """Overlapping destinations, a destination over a source in one buffer, and
    out-of-range objects are refused and nothing is written."""
    src = np.arange(1024, dtype=np.uint32).view(np.uint8)
    dst = np.full(4096, SENTINEL, np.uint8)
    bad = [
        (np.array([[0, 0, 64], [100, 32, 64]], np.uint64), oracle.EPRECOND),
        (np.array([[0, 0, 64], [100, 63, 64]], np.uint64), oracle.EPRECOND),  # one byte
        (np.array([[0, 4000, 200]], np.uint64), oracle.ERANGE),
        (np.array([[4090, 0, 16]], np.uint64), oracle.ERANGE),
    ]
    for descs, rc in bad:
        try:
            oracle.batch_copy(dst, src, descs, lib=lib)
        except oracle.OracleError as e:
            assert e.rc == rc, (e.rc, rc)
        else:
            raise AssertionError("accepted an invalid copy list")
        assert np.all(dst == SENTINEL), "wrote on a refused call"
    buf = np.zeros(512, np.uint8)
    try:
        oracle.batch_copy(buf, buf, np.array([[0, 32, 64]], np.uint64), lib=lib)
    except oracle.OracleError as e:
        assert e.rc == oracle.EPRECOND
    else:
        raise AssertionError("accepted a destination overlapping a source")
    # zero-length objects may sit anywhere in range, even on top of each other
    oracle.batch_copy(dst, src, np.array([[5, 7, 0], [5, 7, 0]], np.uint64), lib=lib)
    assert np.all(dst == SENTINEL)
    # touching (not overlapping) destinations are fine
    oracle.batch_copy(dst, src, np.array([[0, 0, 64], [100, 64, 64]], np.uint64), lib=lib)
    assert np.array_equal(dst[:64], src[:64]) and np.array_equal(dst[64:128], src[100:164])


def pin_block_tables(lib):
    """Block tables used together must be in range and disjoint."""
    oracle.check_block_tables([np.array([3, 1]), np.array([0, 2])], 4, lib=lib)
    for tables, rc in [([np.array([3, 1]), np.array([1])], oracle.EPRECOND),
                       ([np.array([4])], oracle.ERANGE), ([np.array([-1])], oracle.ERANGE)]:
        try:
            oracle.check_block_tables(tables, 4, lib=lib)
        except oracle.OracleError as e:
            assert e.rc == rc
        else:
            raise AssertionError("accepted bad block tables")


def read_golden():
    rows = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, inp, exp, cite = [x.strip() for x in line.split("|")]
            kv = lambda s: {k: int(v) for k, v in (x.split("=") for x in s.split())}
            rows.append((name, kv(inp), kv(exp), cite))
    return rows


def pin_page_counts(lib):
    """Block and object counts printed by the pages for their examples."""
    for name, i, e, _ in read_golden():
        assert oracle.blocks_for_tokens(i["tokens"], i["B"], lib=lib) == e["blocks"], name
        got = oracle.objects_for_tokens(i["tokens"], i["B"], i["L"], i["sides"], lib=lib)
        assert got == e["objects"], name
    # ragged sequences: the fewest blocks of B tokens that hold T tokens
    for T in range(0, 70):
        for B in range(1, 18):
            nb = oracle.blocks_for_tokens(T, B, lib=lib)
            assert nb * B >= T and (nb == 0 or (nb - 1) * B < T), (T, B, nb)
            assert oracle.objects_for_tokens(T, B, 3, 2, lib=lib) == 6 * nb


def pin_kv_bytes(lib):
    """eq. 1 (Tutti reading notes, prerequisites 2): KV bytes = 2*L*T*H*d*e, and a
    packed Full Block holds exactly that many bytes for H = H_kv."""
    assert oracle.kv_bytes(32, 128000, 8, 128, 2, lib=lib) == 16_777_216_000
    assert oracle.kv_bytes(64, 128000, 8, 128, 2, lib=lib) == 2000 * 64 * 2 * 131072
    L, S, N, B, rb, T = SHAPES[0]
    full = np.zeros(T * L * S * rb, np.uint8)
    oracle.pack_full(np.zeros(L * S * N * B * rb, np.uint8), dense_pool(L, S, N, B, rb), L,
                     perm_table(1, N, T, B), T, full, lib=lib)
    assert full.nbytes == oracle.kv_bytes(L, T, 2, 64, 2, lib=lib)


ALL_PINS = [pin_pack_labelled, pin_pack_gather, pin_unpack_labelled, pin_unpack_scatter,
            pin_roundtrip, pin_merge, pin_cross_op, pin_batch_copy, pin_batch_copy_rejects,
            pin_block_tables, pin_page_counts, pin_kv_bytes]
