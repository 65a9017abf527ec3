"""Debug mode (kvm_ctx_set_checks): a violated caller precondition returns
KVM_ECHECK, names the offending entries and enqueues nothing; inputs that meet
the preconditions give the same bytes as with checks off (the oracle's); and
entries the kernels skip by design (bad ids, objects outside their buffer) are
not violations."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import SENTINEL, down, say, up
from paged_kv_cache_kvm_amd import kvmove as kv

pytestmark = pytest.mark.gpu

L, S, N, B, RB = 3, 2, 16, 4, 32
C = S * RB


@pytest.fixture(scope="module")
def ctx(gpu):
    c = kv.Context(0)
    c.set_checks(True)
    yield c
    c.close()


def _layout():
    return kv.pool_layout(S, B, RB, B * RB, N * B * RB, S * N * B * RB, N)


def _status(fn, *args):
    try:
        fn(*args)
    except kv.KvmError as e:
        return e.status
    return kv.KVM_OK


def _pool(gpu):
    return up(np.full(L * S * N * B * RB, SENTINEL, np.uint8), gpu)


def _full(gpu, tokens):
    return up((np.arange(tokens * L * C, dtype=np.uint32) % 253).astype(np.uint8), gpu)


def test_repeated_block_in_one_table(ctx, gpu):
    say("  checks: repeated id in one table")
    pool = _pool(gpu)
    bt = up(np.array([3, 9, 3], np.int32), gpu)
    full = _full(gpu, 12)
    st = _status(kv.kvm_unpack_layer, ctx.handle, _layout(), pool, L, 1, [kv.seq(bt, full, 12)])
    assert st == kv.KVM_ECHECK
    assert "block id 3" in kv.kvm_ctx_last_error(ctx.handle)
    torch.cuda.synchronize()
    assert np.all(down(pool) == SENTINEL)


def test_repeated_block_across_sequences_and_fused(ctx, gpu):
    say("  checks: repeated id across two sequences, unpack and fused")
    pool = _pool(gpu)
    bt0 = up(np.array([1, 2], np.int32), gpu)
    bt1 = up(np.array([7, 2], np.int32), gpu)
    f0, f1 = _full(gpu, 8), _full(gpu, 5)
    st = _status(kv.kvm_unpack_layer, ctx.handle, _layout(), pool, L, 0,
                 [kv.seq(bt0, f0, 8), kv.seq(bt1, f1, 5)])
    assert st == kv.KVM_ECHECK
    out = up(np.full(13 * C, SENTINEL, np.uint8), gpu)
    st = _status(kv.kvm_unpack_merge_layer, ctx.handle, _layout(), pool, L, 0,
                 [kv.layer_seq(bt0, f0, 8, None, C, 0, out, C),
                  kv.layer_seq(bt1, f1, 5, None, C, 0, out.data_ptr() + 8 * C, C)])
    assert st == kv.KVM_ECHECK
    torch.cuda.synchronize()
    assert np.all(down(pool) == SENTINEL)
    assert np.all(down(out) == SENTINEL)


def test_valid_tables_match_the_oracle_with_checks_on(ctx, gpu):
    say("  checks: valid tables, pack with a repeated id (reads only), bad ids skipped")
    rng = np.random.default_rng(4)
    pool_np = rng.integers(0, 256, L * S * N * B * RB, dtype=np.uint8)
    pool = up(pool_np, gpu)
    ref = oracle.pool_struct(S, B, RB, B * RB, N * B * RB, S * N * B * RB, N)
    tables = [np.array([5, 0, 12], np.int32), np.array([8], np.int32)]
    fulls_np = [rng.integers(0, 256, 11 * L * C, dtype=np.uint8),
                rng.integers(0, 256, 3 * L * C, dtype=np.uint8)]
    # every buffer stays referenced until the stream has run the call
    bts = [up(t, gpu) for t in tables]
    fulls = [up(f, gpu) for f in fulls_np]
    kv.kvm_unpack_layer(ctx.handle, _layout(), pool, L, 2,
                        [kv.seq(bts[0], fulls[0], 11), kv.seq(bts[1], fulls[1], 3)])
    want = pool_np.copy()
    oracle.unpack_layer(want, ref, L, 2, tables[0], 11, fulls_np[0])
    oracle.unpack_layer(want, ref, L, 2, tables[1], 3, fulls_np[1])
    torch.cuda.synchronize()
    assert np.array_equal(down(pool), want)
    # pack reads: a repeated id is allowed
    rep = up(np.array([4, 4], np.int32), gpu)
    packed = up(np.full(8 * L * C, SENTINEL, np.uint8), gpu)
    kv.kvm_pack_full(ctx.handle, _layout(), pool, L, [kv.seq(rep, packed, 8)])
    torch.cuda.synchronize()
    got = down(packed).reshape(8, L, C)
    assert np.array_equal(got[:4], got[4:])
    # an id outside [0, N) is skipped and counted, not a violation
    bad = up(np.array([2, N + 3], np.int32), gpu)
    full8 = _full(gpu, 8)
    kv.kvm_unpack_layer(ctx.handle, _layout(), pool, L, 0, [kv.seq(bad, full8, 8)])
    assert ctx.take_device_errors() == 1


def test_checks_off_accepts_a_repeated_id(gpu):
    c = kv.Context(0)
    try:
        pool = _pool(gpu)
        bt = up(np.array([3, 3], np.int32), gpu)
        full = _full(gpu, 8)
        kv.kvm_unpack_layer(c.handle, _layout(), pool, L, 1, [kv.seq(bt, full, 8)])
        torch.cuda.synchronize()
    finally:
        c.close()


def _descs(rows):
    return np.array(rows, dtype=np.uint64)


@pytest.mark.parametrize("rows,same,why", [
    ([[0, 0, 64], [100, 63, 10]], False, "overlap in the destination"),
    ([[0, 4096, 4096], [8192, 8191, 2]], False, "overlap in the destination"),
    ([[0, 1000, 100], [1050, 2000, 10]], True, "writes over a source range"),
    ([[500, 0, 600], [5000, 6000, 10]], True, "writes over a source range"),
], ids=["dst-overlap", "dst-touch-by-one", "same-buffer-dst-on-src", "same-buffer-src-on-dst"])
def test_copy_list_violations(ctx, gpu, rows, same, why):
    say(f"  checks: copy list {rows} same_buffer={same}")
    src = up(np.arange(1 << 16, dtype=np.uint32).astype(np.uint8), gpu)
    dst = src if same else up(np.full(1 << 16, SENTINEL, np.uint8), gpu)
    before = down(dst)
    d = up(_descs(rows).view(np.uint8), gpu)
    st = _status(kv.kvm_batch_copy, ctx.handle, dst, 1 << 16, src, 1 << 16, d, len(rows))
    assert st == kv.KVM_ECHECK
    assert why in kv.kvm_ctx_last_error(ctx.handle)
    torch.cuda.synchronize()
    assert np.array_equal(down(dst), before)


def test_valid_copy_lists_pass(ctx, gpu):
    say("  checks: valid copy lists")
    src_np = np.arange(1 << 16, dtype=np.uint32).astype(np.uint8)
    rows = [[0, 100, 50], [4000, 150, 1], [9000, 20000, 0], [70000, 0, 16], [10, 30000, 4096]]
    src = up(src_np, gpu)
    dst = up(np.full(1 << 16, SENTINEL, np.uint8), gpu)
    d = up(_descs(rows).view(np.uint8), gpu)
    kv.kvm_batch_copy(ctx.handle, dst, 1 << 16, src, 1 << 16, d, len(rows))
    assert ctx.take_device_errors() == 1          # the object starting at 70000 is outside src
    want = np.full(1 << 16, SENTINEL, np.uint8)
    oracle.batch_copy(want, src_np, _descs([r for r in rows if r[0] + r[2] <= (1 << 16)]))
    assert np.array_equal(down(dst), want)
    # same buffer, disjoint sources and destinations
    buf_np = np.arange(1 << 16, dtype=np.uint32).astype(np.uint8) ^ 0x5A
    buf = up(buf_np, gpu)
    rows = [[0, 20000, 1000], [1000, 30000, 500], [40000, 5000, 100]]
    d2 = up(_descs(rows).view(np.uint8), gpu)
    kv.kvm_batch_copy(ctx.handle, buf, 1 << 16, buf, 1 << 16, d2, len(rows))
    want = buf_np.copy()
    oracle.batch_copy(want, want, _descs(rows))
    torch.cuda.synchronize()
    assert np.array_equal(down(buf), want)
