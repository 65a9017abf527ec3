"""bench.py --verify's checks, on the CPU: on a tiny layer loop and a copy list
whose outputs the oracle computed they pass, and each planted mistake in one
output (a slot row, a complete_layer row, a packed miss-token row, a copied
byte) makes them fail."""
import importlib.util
import os
import types

import numpy as np
import pytest
import torch

import oracle
from paged_kv_cache_kvm_amd import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _layer_loop():
    """Two requests, L=3, S=2, B=4, 64-byte rows, 20 pool blocks: the state the
    bench's loop leaves (every layer unpacked and merged, then pack_full)."""
    L, S, B, rb, N = 3, 2, 4, 64, 20
    C = S * rb
    th, tm = 9, 3
    ta = th + tm
    R = 2
    rng = np.random.default_rng(5)
    tables = wl.block_tables(5, 1, N, [wl.blocks_needed(ta, B)] * R)
    ref = oracle.pool_struct(S, B, rb, B * rb, N * B * rb, S * N * B * rb, N)
    pool = rng.integers(0, 256, L * S * N * B * rb, dtype=np.uint8)
    fbs = [rng.integers(0, 256, th * L * C, dtype=np.uint8) for _ in range(R)]
    misses = [rng.integers(0, 256, tm * L * C, dtype=np.uint8) for _ in range(R)]
    complete = np.zeros(R * L * ta * C, np.uint8)
    packed = [np.zeros(ta * L * C, np.uint8) for _ in range(R)]
    for l in range(L):
        for r in range(R):
            oracle.unpack_layer(pool, ref, L, l, tables[r], th, fbs[r])
            oracle.merge_layer(C, fbs[r][l * C:], L * C, th, misses[r][l * C:], L * C, tm,
                               complete[(r * L + l) * ta * C:], C)
    for r in range(R):
        oracle.pack_full(pool, ref, L, tables[r], ta, packed[r])
    t = torch.from_numpy
    w = types.SimpleNamespace(shape=types.SimpleNamespace(layers=L, sides=S, block_tokens=B,
                                                          row_bytes=rb),
                              pool_blocks=N, t_hit=[th] * R, t_miss=[tm] * R)
    return {"w": w, "C": C, "pool": t(pool),
            "keep": ([t(x.astype(np.int32)) for x in tables], [t(x) for x in fbs],
                     [t(x) for x in misses], t(complete), [t(x) for x in packed])}


def test_layer_loop_checks_pass_on_oracle_outputs():
    b = _bench()
    b.verify_layer_loop(torch, _layer_loop())


@pytest.mark.parametrize("where", ["slot", "complete_hit", "complete_miss", "packed_miss"])
def test_layer_loop_checks_catch_a_planted_mistake(where):
    b = _bench()
    s = _layer_loop()
    bts, fbs, misses, complete, packed = s["keep"]
    L, C, B, rb = 3, s["C"], 4, 64
    th, ta = 9, 12
    if where == "slot":        # the slot row of hit token 5, layer 1, side 0
        blk = int(bts[1][5 // B])
        off = ((1 * 2 + 0) * 20 + blk) * B * rb + (5 % B) * rb
        s["pool"][off] ^= 1
        # pack read the pool after the loop, so its copy of that row must move too
        packed[1].view(ta, L, 2, rb)[5, 1, 0, 0] ^= 1
    elif where == "complete_hit":
        complete.view(2, L, ta, C)[0, 2, 3, 7] ^= 1
    elif where == "complete_miss":
        complete.view(2, L, ta, C)[1, 0, th + 1, 0] ^= 1
    else:                      # a miss token's row in the packed Full Block
        packed[0].view(ta, L, C)[th + 2, 1, 5] ^= 1
    with pytest.raises(b.VerifyError):
        b.verify_layer_loop(torch, s)


def test_copy_checks():
    b = _bench()
    rng = np.random.default_rng(6)
    lens = 256 * rng.integers(1, 5, size=50)
    arena = int(lens.sum()) + 8192
    d = np.stack([wl.placements(6, 1, lens, arena), wl.placements(6, 2, lens, arena), lens],
                 axis=1).astype(np.uint64)
    src = rng.integers(0, 256, arena, dtype=np.uint8)
    dst = np.zeros(arena, np.uint8)
    oracle.batch_copy(dst, src, d)
    b.verify_copies(torch, torch.from_numpy(src), torch.from_numpy(dst), d)
    dst[int(d[17, 1]) + int(d[17, 2]) - 1] ^= 1          # last byte of object 17
    with pytest.raises(b.VerifyError):
        b.verify_copies(torch, torch.from_numpy(src), torch.from_numpy(dst), d)
