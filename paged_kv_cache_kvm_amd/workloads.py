"""Seeded synthetic workloads for the KV-move path.

This module only draws inputs: block tables, token counts, payload bytes and
object placements. It performs none of the moves and computes no address of a
token row; the oracle and the HIP library both take what it draws. Every draw
is seeded: host metadata from ``numpy.random.default_rng([seed, tag])``,
device payload from ``torch.Generator`` seeded with ``seed * 100 + tag``.

Workloads (sizes from the pages' examples, see the class docstrings):
  * ``TINY``          L=4, H_kv=2, d=64, B=16, 64-block pool, T_hit=240, T_miss=16
  * ``LLAMA8B``       L=32, H_kv=8, d=128, B=16, 8 x (32768 + 512) tokens, 24576 blocks
  * ``QWEN32B_OBJS``  L=64, H_kv=8, d=128, B=64, one 128000-token sequence as 256000
                      K/V objects scattered in a 36 GiB staging arena
  * ``MLA_AGENTIC``   L=61, one 576-wide latent, B=64, 64 requests,
                      T_hit ~ U{16384..65536}, T_miss ~ U{128..1024}
  * ``SMALL_OBJS``    200000 copies of 256*U{16..512} bytes between two 16 GiB arenas
"""
from __future__ import annotations

import dataclasses
from typing import List, Sequence

import numpy as np

GiB = 1 << 30
KiB = 1 << 10


@dataclasses.dataclass(frozen=True)
class KVShape:
    """Model geometry of the KV cache.

    sides = 2 keeps K and V as separate objects; sides = 1 is one latent
    (MLA-style). head_elems is H_kv * d elements per side per token."""
    layers: int
    sides: int
    head_elems: int
    elem_bytes: int
    block_tokens: int

    @property
    def row_bytes(self) -> int:  # one token, one side, one layer
        return self.head_elems * self.elem_bytes

    @property
    def c_kv_bytes(self) -> int:  # one token, one layer, all sides
        return self.sides * self.row_bytes


@dataclasses.dataclass(frozen=True)
class PagedWorkload:
    name: str
    seed: int
    shape: KVShape
    pool_blocks: int          # 0: exactly the blocks the requests need
    t_hit: tuple              # per request
    t_miss: tuple             # per request
    slot_pool: bool = False   # one-layer slot pool reused by every layer

    @property
    def t_all(self) -> tuple:
        return tuple(h + m for h, m in zip(self.t_hit, self.t_miss))


@dataclasses.dataclass(frozen=True)
class CopyWorkload:
    name: str
    seed: int
    n_descs: int
    src_arena: int
    dst_arena: int
    granule: int = 256


def _rng(seed: int, tag: int) -> np.random.Generator:
    return np.random.default_rng([seed, tag])


# ---------------------------------------------------------------- configs --

TINY = PagedWorkload(
    name="tiny L=4 Hkv=2 d=64 B=16 pool=64 T_hit=240 T_miss=16",
    seed=1001,
    shape=KVShape(layers=4, sides=2, head_elems=2 * 64, elem_bytes=2, block_tokens=16),
    pool_blocks=64, t_hit=(240,), t_miss=(16,))

LLAMA8B = PagedWorkload(
    name="llama3-8b-like L=32 Hkv=8 d=128 B=16 8x(32768+512) pool=24576",
    seed=1002,
    shape=KVShape(layers=32, sides=2, head_elems=8 * 128, elem_bytes=2, block_tokens=16),
    pool_blocks=24576, t_hit=(32768,) * 8, t_miss=(512,) * 8)


def mla_agentic(seed: int = 1004, n_req: int = 64) -> PagedWorkload:
    """DeepSeek-style MLA agentic turn: 61 layers, one 576-element latent per
    token-layer, block 64; long hits and short appends drawn per request."""
    r = _rng(seed, 1)
    t_hit = tuple(int(x) for x in r.integers(16384, 65536, endpoint=True, size=n_req))
    t_miss = tuple(int(x) for x in r.integers(128, 1024, endpoint=True, size=n_req))
    return PagedWorkload(
        name=f"mla-agentic L=61 C=576 B=64 {n_req} requests",
        seed=seed,
        shape=KVShape(layers=61, sides=1, head_elems=576, elem_bytes=2, block_tokens=64),
        pool_blocks=0, t_hit=t_hit, t_miss=t_miss, slot_pool=True)


QWEN32B_SHAPE = KVShape(layers=64, sides=2, head_elems=8 * 128, elem_bytes=2, block_tokens=64)
QWEN32B_TOKENS = 128000
QWEN32B_STAGING = 36 * GiB

SMALL_OBJS = CopyWorkload(name="small-objects 200000 x 256*U{16..512} B, 16 GiB arenas",
                          seed=1005, n_descs=200000, src_arena=16 * GiB, dst_arena=16 * GiB)


# ------------------------------------------------------------ draws ------

def blocks_needed(tokens: int, block_tokens: int) -> int:
    """Block-table entries a request of `tokens` tokens holds (ceil)."""
    return -(-tokens // block_tokens)


def block_tables(seed: int, tag: int, num_blocks: int, per_request: Sequence[int]) -> List[np.ndarray]:
    """Disjoint random block tables: request r takes the next per_request[r]
    entries of one random permutation of the pool's blocks."""
    need = int(sum(per_request))
    if need > num_blocks:
        raise ValueError(f"pool of {num_blocks} blocks cannot hold {need}")
    perm = _rng(seed, tag).permutation(num_blocks).astype(np.int32)
    out, at = [], 0
    for n in per_request:
        out.append(perm[at:at + n].copy())
        at += n
    return out


def bf16_normal_bits(seed: int, tag: int, count: int) -> np.ndarray:
    """count bf16 values ~ N(0,1) as uint16 bit patterns: float32 draws rounded
    to nearest-even bf16 (the same rounding torch's .to(bfloat16) applies)."""
    x = _rng(seed, tag).standard_normal(count, dtype=np.float32).view(np.uint32)
    bits = (x + np.uint32(0x7FFF) + ((x >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return bits.astype(np.uint16)


def random_bytes(seed: int, tag: int, count: int) -> np.ndarray:
    return _rng(seed, tag).integers(0, 256, size=count, dtype=np.uint8)


def placements(seed: int, tag: int, lengths: np.ndarray, arena_bytes: int,
               granule: int = 256) -> np.ndarray:
    """Random non-overlapping offsets for objects of the given lengths inside an
    arena: the objects go in a random order, and the free granules are split
    into len+1 gaps by sorted uniform cut points (stars and bars)."""
    lengths = np.asarray(lengths, dtype=np.int64)
    if np.any(lengths % granule):
        raise ValueError("lengths must be whole granules")
    units = lengths // granule
    free = arena_bytes // granule - int(units.sum())
    if free < 0:
        raise ValueError("objects do not fit the arena")
    r = _rng(seed, tag)
    order = r.permutation(len(lengths))
    cuts = np.sort(r.integers(0, free + 1, size=len(lengths)))
    gaps = np.diff(cuts, prepend=0)
    # start of the k-th placed object = gaps so far + units of earlier objects
    placed_units = units[order]
    starts = np.cumsum(gaps) + np.concatenate(([0], np.cumsum(placed_units)[:-1]))
    off = np.empty(len(lengths), dtype=np.int64)
    off[order] = starts * granule
    return off


def small_object_lengths(w: CopyWorkload) -> np.ndarray:
    return w.granule * _rng(w.seed, 1).integers(16, 512, endpoint=True, size=w.n_descs).astype(np.int64)


def small_object_descs(w: CopyWorkload) -> np.ndarray:
    """[n, 3] uint64 (src_off, dst_off, nbytes) with independent random
    placements in the source and destination arenas."""
    lens = small_object_lengths(w)
    src = placements(w.seed, 2, lens, w.src_arena, w.granule)
    dst = placements(w.seed, 3, lens, w.dst_arena, w.granule)
    return np.stack([src, dst, lens], axis=1).astype(np.uint64)


def qwen32b_object_descs(seed: int = 1003, tokens: int = QWEN32B_TOKENS,
                         shape: KVShape = QWEN32B_SHAPE, staging: int = QWEN32B_STAGING):
    """Restore list of one long sequence stored as separate K and V objects per
    (layer, block): descriptors in (layer, block, side) order from random
    staging offsets to the object of (layer, side, block_table[block]) in a
    dense [L][S][N][B][H*d] pool of exactly the sequence's blocks.

    Returns (descs [n,3] uint64, block_table, pool_bytes). The destination
    offset is the caller's description of where each object lives, the same
    role as a per-layer I/O context entry; the copy itself is the library's."""
    nb = blocks_needed(tokens, shape.block_tokens)
    bt = block_tables(seed, 1, nb, [nb])[0]
    obj = shape.block_tokens * shape.row_bytes
    block_stride, side_stride = obj, nb * obj
    layer_stride = shape.sides * side_stride
    L, S = shape.layers, shape.sides
    l_idx, b_idx, s_idx = np.meshgrid(np.arange(L), np.arange(nb), np.arange(S), indexing="ij")
    l_idx, b_idx, s_idx = l_idx.ravel(), b_idx.ravel(), s_idx.ravel()
    dst = (l_idx.astype(np.int64) * layer_stride + s_idx * side_stride
           + bt[b_idx].astype(np.int64) * block_stride)
    lens = np.full(dst.shape, obj, dtype=np.int64)
    src = placements(seed, 2, lens, staging, 256)
    descs = np.stack([src, dst, lens], axis=1).astype(np.uint64)
    return descs, bt, L * layer_stride


# ------------------------------------------------------ device payload ----

def fill_bf16_normal_(t, seed: int, tag: int, chunk_elems: int = 1 << 28) -> None:
    """Fill a device byte tensor with bf16 ~ N(0,1) from a seeded generator."""
    import torch
    flat = t.view(-1).view(torch.uint8)
    if flat.numel() % 2:
        raise ValueError("bf16 fill needs an even byte count")
    as16 = flat.view(torch.bfloat16)
    g = torch.Generator(device=t.device).manual_seed(seed * 100 + tag)
    for a in range(0, as16.numel(), chunk_elems):
        b = min(as16.numel(), a + chunk_elems)
        as16[a:b].copy_(torch.randn(b - a, dtype=torch.float32, device=t.device, generator=g))


def fill_random_bytes_(t, seed: int, tag: int, chunk: int = 1 << 30) -> None:
    """Fill a device byte tensor with uniform random bytes from a seeded generator."""
    import torch
    flat = t.view(-1).view(torch.uint8)
    g = torch.Generator(device=t.device).manual_seed(seed * 100 + tag)
    for a in range(0, flat.numel(), chunk):
        b = min(flat.numel(), a + chunk)
        flat[a:b] = torch.randint(0, 256, (b - a,), dtype=torch.uint8, device=t.device, generator=g)
