"""The C-ABI contract on the GPU: status codes for bad arguments, a refused call
writes nothing, degenerate calls are no-ops, and the device-side guards skip
and count bad block ids."""
import ctypes

import numpy as np
import pytest
import torch

from gpu_util import SENTINEL, down, up
from paged_kv_cache_kvm_amd import kvmove as kv

pytestmark = pytest.mark.gpu

L, S, N, B, RB = 3, 2, 16, 4, 32


@pytest.fixture(scope="module")
def ctx(gpu):
    c = kv.Context(0)
    yield c
    c.close()


def _layout(**kw):
    d = dict(num_sides=S, block_tokens=B, row_bytes=RB, block_stride=B * RB,
             side_stride=N * B * RB, layer_stride=S * N * B * RB, num_blocks=N)
    d.update(kw)
    return kv.kvm_pool_layout(**d)


@pytest.fixture()
def bufs(gpu):
    pool = up(np.full(L * S * N * B * RB, SENTINEL, np.uint8), gpu)
    bt = up(np.array([3, 9, 0], np.int32), gpu)
    full = up(np.arange(12 * L * S * RB, dtype=np.uint32).astype(np.uint8), gpu)
    return pool, bt, full


def _status(fn, *args):
    try:
        fn(*args)
    except kv.KvmError as e:
        return e.status
    return kv.KVM_OK


BAD_LAYOUTS = [dict(num_sides=0), dict(block_tokens=0), dict(row_bytes=0), dict(num_blocks=0),
               dict(block_stride=-1), dict(side_stride=-8), dict(layer_stride=-1),
               dict(block_stride=B * RB - 1)]


@pytest.mark.parametrize("bad", BAD_LAYOUTS, ids=[next(iter(b)) for b in BAD_LAYOUTS])
def test_bad_layout_is_refused_and_writes_nothing(ctx, bufs, bad):
    pool, bt, full = bufs
    st = _status(kv.kvm_unpack_layer, ctx.handle, _layout(**bad), pool, L, 0, [kv.seq(bt, full, 12)])
    assert st == kv.KVM_EINVAL
    torch.cuda.synchronize()
    assert np.all(down(pool) == SENTINEL)


def test_bad_arguments(ctx, bufs):
    pool, bt, full = bufs
    lay = _layout()
    one = [kv.seq(bt, full, 12)]
    cases = [
        ((kv.kvm_unpack_layer, ctx.handle, lay, pool, L, L, one), kv.KVM_ERANGE),
        ((kv.kvm_unpack_layer, ctx.handle, lay, pool, L, -1, one), kv.KVM_ERANGE),
        ((kv.kvm_unpack_layer, ctx.handle, lay, 0, L, 0, one), kv.KVM_EINVAL),
        ((kv.kvm_unpack_layer, ctx.handle, lay, pool, 0, 0, one), kv.KVM_EINVAL),
        ((kv.kvm_unpack_layer, ctx.handle, lay, pool, L, 0, [kv.seq(bt, full, -1)]), kv.KVM_EINVAL),
        ((kv.kvm_unpack_layer, ctx.handle, lay, pool, L, 0, [kv.seq(0, full, 3)]), kv.KVM_EINVAL),
        ((kv.kvm_unpack_layer, ctx.handle, lay, pool, L, 0, [kv.seq(bt, 0, 3)]), kv.KVM_EINVAL),
        ((kv.kvm_unpack_layer, ctx.handle, lay, pool, L, 0, [kv.seq(bt, full, 3, 8)]), kv.KVM_EINVAL),
        ((kv.kvm_pack_full, ctx.handle, lay, pool, L, [kv.seq(bt, full, 12, -4)]), kv.KVM_EINVAL),
        ((kv.kvm_merge_layer, ctx.handle, 0, [kv.merge_seq(full, 8, 1, 0, 0, 0, pool, 8)]), kv.KVM_EINVAL),
        ((kv.kvm_merge_layer, ctx.handle, 8, [kv.merge_seq(0, 8, 1, 0, 0, 0, pool, 8)]), kv.KVM_EINVAL),
        ((kv.kvm_merge_layer, ctx.handle, 8, [kv.merge_seq(full, 8, 1, 0, 0, 2, pool, 8)]), kv.KVM_EINVAL),
        ((kv.kvm_merge_layer, ctx.handle, 8, [kv.merge_seq(full, 8, 1, 0, 0, 0, 0, 8)]), kv.KVM_EINVAL),
        ((kv.kvm_merge_layer, ctx.handle, 8, [kv.merge_seq(full, -8, 1, 0, 0, 0, pool, 8)]), kv.KVM_EINVAL),
        ((kv.kvm_merge_layer, ctx.handle, 1 << 31, [kv.merge_seq(full, 8, 1, 0, 0, 0, pool, 8)]), kv.KVM_ERANGE),
        ((kv.kvm_batch_copy, ctx.handle, pool, 64, full, 64, 0, 1), kv.KVM_EINVAL),
        ((kv.kvm_batch_copy, ctx.handle, pool, 64, full, 64, bt, -1), kv.KVM_EINVAL),
        ((kv.kvm_batch_copy, ctx.handle, 0, 64, full, 64, bt, 1), kv.KVM_EINVAL),
    ]
    for args, want in cases:
        assert _status(*args) == want, args[0].__name__
    torch.cuda.synchronize()
    assert np.all(down(pool) == SENTINEL), "a refused call wrote"


def test_unpack_sequence_limit(ctx, bufs):
    pool, bt, full = bufs
    many = [kv.seq(bt, full, 1)] * 2049      # 17 launch batches of sequences with tokens
    assert _status(kv.kvm_unpack_layer, ctx.handle, _layout(), pool, L, 0, many) == kv.KVM_ERANGE
    torch.cuda.synchronize()
    assert np.all(down(pool) == SENTINEL)


def test_size_limits_are_refused(ctx, bufs):
    """The documented maximum sizes: 2^31 work items in one launch (tiles x
    sides for unpack, tiles x layers for pack), a tile of 2^31 bytes or more,
    more than 2^20 sequences, and more than 2^32 copy objects. Each is refused
    before anything is read from the (here too small) buffers."""
    pool, bt, full = bufs
    lay1 = kv.pool_layout(S, 1, RB, RB, N * RB, S * N * RB, N)        # B = 1
    huge = [kv.seq(bt, full, 1 << 31)]                               # 2^31 tiles
    half = [kv.seq(bt, full, (1 << 30) + 1)]                          # x 2 sides > 2^31
    cases = [
        ((kv.kvm_unpack_layer, ctx.handle, lay1, pool, L, 0, huge), kv.KVM_ERANGE),
        ((kv.kvm_unpack_layer, ctx.handle, lay1, pool, L, 0, half), kv.KVM_ERANGE),
        ((kv.kvm_pack_full, ctx.handle, lay1, pool, L, [kv.seq(bt, full, 1 << 30)]), kv.KVM_ERANGE),
        ((kv.kvm_unpack_merge_layer, ctx.handle, lay1, pool, L, 0,
          [kv.layer_seq(bt, full, (1 << 30) + 1, 0, 0, 0, pool, S * RB)]), kv.KVM_ERANGE),
        ((kv.kvm_unpack_layer, ctx.handle,
          kv.pool_layout(S, 1 << 16, 1 << 15, 1 << 31, 1 << 32, 1 << 33, N), pool, L, 0,
          [kv.seq(bt, full, 1)]), kv.KVM_ERANGE),                     # 2^32-byte tile
    ]
    for args, want in cases:
        assert _status(*args) == want, args[0].__name__
    lib = kv.load()
    one = (kv.kvm_seq * 1)(kv.seq(bt, full, 1))
    assert lib.kvm_unpack_layer(ctx.handle, ctypes.byref(_layout()), pool.data_ptr(), L, 0, one,
                                (1 << 20) + 1, None) == kv.KVM_ERANGE
    assert lib.kvm_batch_copy(ctx.handle, pool.data_ptr(), 64, full.data_ptr(), 64, bt.data_ptr(),
                              (1 << 32) + 1, None) == kv.KVM_ERANGE
    torch.cuda.synchronize()
    assert np.all(down(pool) == SENTINEL), "a refused call wrote"


def test_degenerate_calls_are_noops(ctx, bufs):
    pool, bt, full = bufs
    lay = _layout()
    kv.kvm_unpack_layer(ctx.handle, lay, pool, L, 0, [])
    kv.kvm_unpack_layer(ctx.handle, lay, pool, L, 1, [kv.seq(0, 0, 0)])
    kv.kvm_pack_full(ctx.handle, lay, pool, L, [])
    kv.kvm_merge_layer(ctx.handle, 64, [])
    kv.kvm_merge_layer(ctx.handle, 64, [kv.merge_seq(0, 0, 0, 0, 0, 0, 0, 0)])
    kv.kvm_batch_copy(ctx.handle, 0, 0, 0, 0, 0, 0)
    zero = up(np.array([[0, 0, 0], [7, 9, 0]], np.uint64).view(np.uint8), pool.device)
    kv.kvm_batch_copy(ctx.handle, pool, 16, full, 16, zero, 2)
    torch.cuda.synchronize()
    assert np.all(down(pool) == SENTINEL)
    assert ctx.take_device_errors() == 0


def test_bad_block_ids_are_skipped_and_counted(ctx, bufs, gpu):
    pool, _, _ = bufs
    full = up(np.arange(16 * L * S * RB, dtype=np.uint32).astype(np.uint8), gpu)  # 16 tokens
    bt = up(np.array([3, N, -1, 1], np.int32), gpu)    # entries 1 and 2 are out of range
    kv.kvm_unpack_layer(ctx.handle, _layout(), pool, L, 1, [kv.seq(bt, full, 16)])
    assert ctx.take_device_errors() == 2
    p = down(pool).reshape(L, S, N, B * RB)
    touched = {n for n in range(N) if not np.all(p[1, :, n] == SENTINEL)}
    assert touched == {3, 1}
    assert np.all(np.delete(p, 1, axis=0) == SENTINEL)


def test_reserve_and_context_cycle(gpu):
    for _ in range(3):
        c = kv.Context(0)
        c.reserve(5000, 1 << 20)
        with pytest.raises(kv.KvmError):
            c.reserve(-1, 0)
        c.close()
    lib = kv.load()
    out = ctypes.c_void_p()
    assert lib.kvm_create(10 ** 6, ctypes.byref(out)) == kv.KVM_EHIP
