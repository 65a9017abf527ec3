"""ctypes binding of libkvmove (include/kvm.h), same names as the C entry points.

Argument marshalling only: every move runs in the library's HIP kernels. Device
buffers are passed as integer device addresses or as torch tensors (their
data_ptr); streams as a torch stream, an integer hipStream_t, or None for the
current torch stream. Record lists (kvm_seq, kvm_merge_seq, kvm_layer_seq) are
passed as a list, or as a ctypes array built once with records() and reused
by later calls (a per-layer loop), which saves building it on every call. Each
call raises KvmError on a non-zero status.

The library must be built (paged_kv_cache_kvm_amd/build.py): the first call
into it raises if libkvmove.so is missing, and there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Iterable, Sequence

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libkvmove.so")

KVM_OK, KVM_EINVAL, KVM_ERANGE, KVM_ENOMEM, KVM_EHIP, KVM_ECHECK = 0, -1, -2, -3, -4, -5


class KvmError(RuntimeError):
    def __init__(self, fn: str, status: int, detail: str = ""):
        msg = f"{fn}: {strerror(status)} ({status})"
        if detail:
            msg += f": {detail}"
        super().__init__(msg)
        self.status = status


class kvm_pool_layout(ctypes.Structure):
    _fields_ = [("num_sides", ctypes.c_int32), ("block_tokens", ctypes.c_int32),
                ("row_bytes", ctypes.c_int64), ("block_stride", ctypes.c_int64),
                ("side_stride", ctypes.c_int64), ("layer_stride", ctypes.c_int64),
                ("num_blocks", ctypes.c_int64)]


class kvm_seq(ctypes.Structure):
    _fields_ = [("block_table", ctypes.c_void_p), ("full", ctypes.c_void_p),
                ("num_tokens", ctypes.c_int64), ("token_stride", ctypes.c_int64)]


class kvm_merge_seq(ctypes.Structure):
    _fields_ = [("hit", ctypes.c_void_p), ("hit_stride", ctypes.c_int64),
                ("t_hit", ctypes.c_int64), ("miss", ctypes.c_void_p),
                ("miss_stride", ctypes.c_int64), ("t_miss", ctypes.c_int64),
                ("out", ctypes.c_void_p), ("out_stride", ctypes.c_int64)]


class kvm_layer_seq(ctypes.Structure):
    _fields_ = [("block_table", ctypes.c_void_p), ("full", ctypes.c_void_p),
                ("t_hit", ctypes.c_int64), ("token_stride", ctypes.c_int64),
                ("miss", ctypes.c_void_p), ("miss_stride", ctypes.c_int64),
                ("t_miss", ctypes.c_int64), ("out", ctypes.c_void_p),
                ("out_stride", ctypes.c_int64)]


class kvm_copy_desc(ctypes.Structure):
    _fields_ = [("src_off", ctypes.c_uint64), ("dst_off", ctypes.c_uint64),
                ("nbytes", ctypes.c_uint64)]


# Exported symbols and their signatures, in include/kvm.h order.
_P = ctypes.c_void_p
_I32, _I64, _U64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64
SIGNATURES = {
    "kvm_version": ([], ctypes.c_int),
    "kvm_strerror": ([ctypes.c_int], ctypes.c_char_p),
    "kvm_create": ([ctypes.c_int, ctypes.POINTER(_P)], ctypes.c_int),
    "kvm_destroy": ([_P], None),
    "kvm_ctx_reserve": ([_P, _I64, _I64], ctypes.c_int),
    "kvm_ctx_reserve_unpack": ([_P, _I64, _I64], ctypes.c_int),
    "kvm_ctx_device_bytes": ([_P, ctypes.POINTER(_I64)], ctypes.c_int),
    "kvm_ctx_set_checks": ([_P, _I32], ctypes.c_int),
    "kvm_ctx_set_max_workgroups": ([_P, _I32], ctypes.c_int),
    "kvm_ctx_last_error": ([_P], ctypes.c_char_p),
    "kvm_take_device_errors": ([_P, ctypes.POINTER(_I64)], ctypes.c_int),
    "kvm_pack_full": ([_P, ctypes.POINTER(kvm_pool_layout), _P, _I32, ctypes.POINTER(kvm_seq),
                       _I32, _P], ctypes.c_int),
    "kvm_unpack_layer": ([_P, ctypes.POINTER(kvm_pool_layout), _P, _I32, _I32,
                          ctypes.POINTER(kvm_seq), _I32, _P], ctypes.c_int),
    "kvm_merge_layer": ([_P, _I64, ctypes.POINTER(kvm_merge_seq), _I32, _P], ctypes.c_int),
    "kvm_unpack_merge_layer": ([_P, ctypes.POINTER(kvm_pool_layout), _P, _I32, _I32,
                                ctypes.POINTER(kvm_layer_seq), _I32, _P], ctypes.c_int),
    "kvm_batch_copy": ([_P, _P, _U64, _P, _U64, _P, _I64, _P], ctypes.c_int),
    "kvm_batch_copy_noalloc": ([_P, _P, _U64, _P, _U64, _P, _I64, _P], ctypes.c_int),
}

KVM_NOALLOC_MAX_DESCS = (1 << 25) - 64

_lib = None


def load(path: str = LIB_PATH):
    """Load libkvmove.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run paged_kv_cache_kvm_amd/build.py "
                           "(or __graft_entry__.build()) first")
    lib = ctypes.CDLL(path)
    for name, (args, res) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def _addr(x) -> int | None:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        return x.data_ptr()
    raise TypeError(f"expected a device address or tensor, got {type(x).__name__}")


_current_raw_stream = None


def _stream(s) -> int | None:
    global _current_raw_stream
    if s is None:
        if _current_raw_stream is None:
            import torch
            raw, dev = (getattr(torch._C, "_cuda_getCurrentRawStream", None),
                        getattr(torch._C, "_cuda_getDevice", None))
            if raw is not None and dev is not None:
                _current_raw_stream = lambda: raw(dev())
            else:
                _current_raw_stream = lambda: torch.cuda.current_stream().cuda_stream
        return _current_raw_stream()
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _check(fn: str, status: int, ctx=None):
    if status != KVM_OK:
        detail = ""
        if ctx is not None and status in (KVM_EHIP, KVM_ECHECK):
            detail = (load().kvm_ctx_last_error(ctx) or b"").decode()
        raise KvmError(fn, status, detail)


def kvm_version() -> int:
    return load().kvm_version()


def strerror(status: int) -> str:
    return load().kvm_strerror(status).decode()


kvm_strerror = strerror


def kvm_create(device: int = 0) -> int:
    out = _P()
    _check("kvm_create", load().kvm_create(device, ctypes.byref(out)))
    return out.value


def kvm_destroy(ctx: int) -> None:
    load().kvm_destroy(ctx)


def kvm_ctx_reserve(ctx: int, max_seqs: int, max_descs: int) -> None:
    _check("kvm_ctx_reserve", load().kvm_ctx_reserve(ctx, max_seqs, max_descs), ctx)


def kvm_ctx_reserve_unpack(ctx: int, max_tiles: int, max_pool_blocks: int) -> None:
    _check("kvm_ctx_reserve_unpack", load().kvm_ctx_reserve_unpack(ctx, max_tiles, max_pool_blocks),
           ctx)


def kvm_ctx_device_bytes(ctx: int) -> int:
    n = _I64()
    _check("kvm_ctx_device_bytes", load().kvm_ctx_device_bytes(ctx, ctypes.byref(n)), ctx)
    return n.value


def kvm_ctx_set_checks(ctx: int, enable: bool) -> None:
    _check("kvm_ctx_set_checks", load().kvm_ctx_set_checks(ctx, 1 if enable else 0), ctx)


def kvm_ctx_set_max_workgroups(ctx: int, max_workgroups: int) -> None:
    _check("kvm_ctx_set_max_workgroups", load().kvm_ctx_set_max_workgroups(ctx, max_workgroups), ctx)


def kvm_ctx_last_error(ctx: int) -> str:
    return (load().kvm_ctx_last_error(ctx) or b"").decode()


def kvm_take_device_errors(ctx: int) -> int:
    n = _I64()
    _check("kvm_take_device_errors", load().kvm_take_device_errors(ctx, ctypes.byref(n)), ctx)
    return n.value


def pool_layout(num_sides, block_tokens, row_bytes, block_stride, side_stride, layer_stride,
                num_blocks) -> kvm_pool_layout:
    return kvm_pool_layout(num_sides, block_tokens, row_bytes, block_stride, side_stride,
                           layer_stride, num_blocks)


def seq(block_table, full, num_tokens: int, token_stride: int = 0) -> kvm_seq:
    return kvm_seq(_addr(block_table), _addr(full), num_tokens, token_stride)


def merge_seq(hit, hit_stride: int, t_hit: int, miss, miss_stride: int, t_miss: int, out,
              out_stride: int) -> kvm_merge_seq:
    return kvm_merge_seq(_addr(hit), hit_stride, t_hit, _addr(miss), miss_stride, t_miss,
                         _addr(out), out_stride)


def layer_seq(block_table, full, t_hit: int, miss, miss_stride: int, t_miss: int, out,
              out_stride: int, token_stride: int = 0) -> kvm_layer_seq:
    return kvm_layer_seq(_addr(block_table), _addr(full), t_hit, token_stride, _addr(miss),
                         miss_stride, t_miss, _addr(out), out_stride)


def records(items: Sequence):
    """A ctypes array of the given records (all of one type: kvm_seq,
    kvm_merge_seq or kvm_layer_seq), for calls that pass the same records
    again and again."""
    items = list(items)
    if not items:
        raise ValueError("records() needs at least one record; pass [] to a call instead")
    return (type(items[0]) * len(items))(*items)


def _array(cls, items):
    if isinstance(items, ctypes.Array):
        if items._type_ is not cls:
            raise TypeError(f"expected an array of {cls.__name__}, got one of "
                            f"{items._type_.__name__}")
        return items, len(items)
    if type(items) in (list, tuple) and len(items) == 1 and type(items[0]) is cls:
        # one record: passed by reference, no array built (about 1.3 us less per call)
        return ctypes.byref(items[0]), 1
    items = list(items)
    arr = (cls * max(1, len(items)))(*items)
    return arr, len(items)


def kvm_pack_full(ctx: int, layout: kvm_pool_layout, pool, num_layers: int,
                  seqs: Iterable[kvm_seq], stream=None) -> None:
    arr, n = _array(kvm_seq, seqs)
    st = load().kvm_pack_full(ctx, ctypes.byref(layout), _addr(pool), num_layers, arr, n,
                              _stream(stream))
    _check("kvm_pack_full", st, ctx)


def kvm_unpack_layer(ctx: int, layout: kvm_pool_layout, pool, num_layers: int, layer: int,
                     seqs: Iterable[kvm_seq], stream=None) -> None:
    arr, n = _array(kvm_seq, seqs)
    st = load().kvm_unpack_layer(ctx, ctypes.byref(layout), _addr(pool), num_layers, layer, arr,
                                 n, _stream(stream))
    _check("kvm_unpack_layer", st, ctx)


def kvm_merge_layer(ctx: int, row_bytes: int, seqs: Iterable[kvm_merge_seq], stream=None) -> None:
    arr, n = _array(kvm_merge_seq, seqs)
    st = load().kvm_merge_layer(ctx, row_bytes, arr, n, _stream(stream))
    _check("kvm_merge_layer", st, ctx)


def kvm_unpack_merge_layer(ctx: int, layout: kvm_pool_layout, pool, num_layers: int, layer: int,
                           seqs: Iterable[kvm_layer_seq], stream=None) -> None:
    arr, n = _array(kvm_layer_seq, seqs)
    st = load().kvm_unpack_merge_layer(ctx, ctypes.byref(layout), _addr(pool), num_layers, layer,
                                       arr, n, _stream(stream))
    _check("kvm_unpack_merge_layer", st, ctx)


def kvm_batch_copy(ctx: int, dst_base, dst_bytes: int, src_base, src_bytes: int, descs,
                   n_descs: int, stream=None) -> None:
    """descs: device address or tensor holding n_descs kvm_copy_desc (24 bytes each)."""
    st = load().kvm_batch_copy(ctx, _addr(dst_base), dst_bytes, _addr(src_base), src_bytes,
                               _addr(descs), n_descs, _stream(stream))
    _check("kvm_batch_copy", st, ctx)


def kvm_batch_copy_noalloc(ctx: int, dst_base, dst_bytes: int, src_base, src_bytes: int, descs,
                           n_descs: int, stream=None) -> None:
    """kvm_batch_copy with its scratch in the device's static array (no allocation)."""
    st = load().kvm_batch_copy_noalloc(ctx, _addr(dst_base), dst_bytes, _addr(src_base), src_bytes,
                                       _addr(descs), n_descs, _stream(stream))
    _check("kvm_batch_copy_noalloc", st, ctx)


class Context:
    """Owns one kvm_ctx on a device; the methods forward to the entry points."""

    def __init__(self, device: int = 0):
        self.handle = kvm_create(device)

    def close(self):
        if self.handle:
            kvm_destroy(self.handle)
            self.handle = 0

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def reserve(self, max_seqs: int, max_descs: int):
        kvm_ctx_reserve(self.handle, max_seqs, max_descs)

    def reserve_unpack(self, max_tiles: int, max_pool_blocks: int):
        kvm_ctx_reserve_unpack(self.handle, max_tiles, max_pool_blocks)

    def device_bytes(self) -> int:
        return kvm_ctx_device_bytes(self.handle)

    def set_checks(self, enable: bool):
        kvm_ctx_set_checks(self.handle, enable)

    def set_max_workgroups(self, max_workgroups: int):
        kvm_ctx_set_max_workgroups(self.handle, max_workgroups)

    def take_device_errors(self) -> int:
        return kvm_take_device_errors(self.handle)

    def pack_full(self, layout, pool, num_layers, seqs, stream=None):
        kvm_pack_full(self.handle, layout, pool, num_layers, seqs, stream)

    def unpack_layer(self, layout, pool, num_layers, layer, seqs, stream=None):
        kvm_unpack_layer(self.handle, layout, pool, num_layers, layer, seqs, stream)

    def merge_layer(self, row_bytes, seqs, stream=None):
        kvm_merge_layer(self.handle, row_bytes, seqs, stream)

    def unpack_merge_layer(self, layout, pool, num_layers, layer, seqs, stream=None):
        kvm_unpack_merge_layer(self.handle, layout, pool, num_layers, layer, seqs, stream)

    def batch_copy(self, dst_base, dst_bytes, src_base, src_bytes, descs, n_descs, stream=None):
        kvm_batch_copy(self.handle, dst_base, dst_bytes, src_base, src_bytes, descs, n_descs,
                       stream)
