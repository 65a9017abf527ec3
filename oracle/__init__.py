"""Oracle for the paged <-> Full Block KV-cache moves (CPU, plain C).

TEST INFRASTRUCTURE. Only the test suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package. The HIP library does
not use it and shares no code with it.

The C source ``kvm_ref.c`` holds the definitions; this module builds it with
gcc and wraps it with ctypes over numpy byte buffers. Each wrapper raises
``OracleError`` when the C function rejects its arguments.

Definitions followed (page title, section):
  * DualPath KV Loading, "Dual-Path Loading" key-objects table and "two read
    paths": Full Block [T, L, C_KV]; layer slice; hit-then-miss concatenation.
  * Tutti reading notes, prerequisites 3 (eq. 2) and 5 (eq. 3-4): paged blocks
    of B_tokens tokens reached through a block table; one K and one V object
    per layer per block.
  * Tutti reading notes, design 1 (eq. 9): one (offset, length) entry per
    contiguous object.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kvm_ref.c")
_LIB = os.path.join(_HERE, "libkvmref.so")

OK, EINVAL, ERANGE, EPRECOND = 0, -1, -2, -5


class OracleError(RuntimeError):
    def __init__(self, fn: str, rc: int):
        super().__init__(f"{fn} rejected its arguments (rc={rc})")
        self.rc = rc


class RefPool(ctypes.Structure):
    _fields_ = [
        ("sides", ctypes.c_int32),
        ("block_tokens", ctypes.c_int32),
        ("row_bytes", ctypes.c_int64),
        ("block_stride", ctypes.c_int64),
        ("side_stride", ctypes.c_int64),
        ("layer_stride", ctypes.c_int64),
        ("num_blocks", ctypes.c_int64),
    ]


def build(out: str = _LIB, src: str = _SRC, extra_flags=()) -> str:
    """Compile the oracle into a shared library with gcc (-O2, no OpenMP)."""
    cmd = ["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-Wall", "-Wextra", *extra_flags,
           "-o", out, src]
    subprocess.run(cmd, check=True)
    return out


_lib = None


def load(path: str | None = None):
    """Load the built oracle (building it first only if nothing is built)."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        _lib = _bind(ctypes.CDLL(_LIB))
    return _lib


def _bind(lib):
    P = ctypes.c_void_p
    I32, I64, U64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64
    pool_p = ctypes.POINTER(RefPool)
    sig = {
        "ref_pack_full": [P, I64, pool_p, I32, P, I64, P, I64, I64],
        "ref_unpack_layer": [P, I64, pool_p, I32, I32, P, I64, P, I64, I64],
        "ref_merge_layer": [I64, P, I64, I64, I64, P, I64, I64, I64, P, I64, I64],
        "ref_batch_copy": [P, U64, P, U64, P, I64],
        "ref_check_block_tables": [P, P, P, I64, I64],
        "ref_blocks_for_tokens": [I64, I64],
        "ref_objects_for_tokens": [I64, I64, I64, I64],
        "ref_kv_bytes": [I64, I64, I64, I64, I64],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = I64 if name.startswith(("ref_blocks", "ref_objects", "ref_kv")) else ctypes.c_int
    return lib


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    if not a.flags["C_CONTIGUOUS"]:
        raise ValueError("oracle buffers must be C-contiguous")
    return a.ctypes.data


def _check(fn: str, rc: int):
    if rc != OK:
        raise OracleError(fn, rc)


def pool_struct(sides, block_tokens, row_bytes, block_stride, side_stride, layer_stride,
                num_blocks) -> RefPool:
    return RefPool(sides, block_tokens, row_bytes, block_stride, side_stride, layer_stride,
                   num_blocks)


def pack_full(pool: np.ndarray, p: RefPool, num_layers: int, block_table: np.ndarray,
              num_tokens: int, full: np.ndarray, token_stride: int = 0, lib=None) -> None:
    lib = lib or load()
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    rc = lib.ref_pack_full(_ptr(pool), pool.nbytes, ctypes.byref(p), num_layers, _ptr(bt),
                           num_tokens, _ptr(full), full.nbytes, token_stride)
    _check("ref_pack_full", rc)


def unpack_layer(pool: np.ndarray, p: RefPool, num_layers: int, layer: int,
                 block_table: np.ndarray, num_tokens: int, full: np.ndarray,
                 token_stride: int = 0, lib=None) -> None:
    lib = lib or load()
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    rc = lib.ref_unpack_layer(_ptr(pool), pool.nbytes, ctypes.byref(p), num_layers, layer,
                              _ptr(bt), num_tokens, _ptr(full), full.nbytes, token_stride)
    _check("ref_unpack_layer", rc)


def merge_layer(row_bytes: int, hit: np.ndarray | None, hit_stride: int, t_hit: int,
                miss: np.ndarray | None, miss_stride: int, t_miss: int, out: np.ndarray,
                out_stride: int, lib=None) -> None:
    lib = lib or load()
    rc = lib.ref_merge_layer(row_bytes,
                             _ptr(hit), 0 if hit is None else hit.nbytes, hit_stride, t_hit,
                             _ptr(miss), 0 if miss is None else miss.nbytes, miss_stride, t_miss,
                             _ptr(out), out.nbytes, out_stride)
    _check("ref_merge_layer", rc)


def batch_copy(dst: np.ndarray, src: np.ndarray, descs: np.ndarray, lib=None) -> None:
    """descs: uint64 array of shape [n, 3] = (src_off, dst_off, nbytes).

    Pass the same array as dst and src for a copy within one buffer."""
    lib = lib or load()
    d = np.ascontiguousarray(descs, dtype=np.uint64).reshape(-1, 3)
    rc = lib.ref_batch_copy(_ptr(dst), dst.nbytes, _ptr(src), src.nbytes, _ptr(d), d.shape[0])
    _check("ref_batch_copy", rc)


def check_block_tables(tables: list[np.ndarray], num_blocks: int, lib=None) -> None:
    lib = lib or load()
    counts = np.array([len(t) for t in tables], dtype=np.int64)
    offsets = np.zeros(len(tables), dtype=np.int64)
    if len(tables) > 1:
        offsets[1:] = np.cumsum(counts)[:-1]
    flat = (np.concatenate([np.asarray(t, dtype=np.int32) for t in tables])
            if tables else np.zeros(1, np.int32))
    flat = np.ascontiguousarray(flat, dtype=np.int32)
    rc = lib.ref_check_block_tables(_ptr(flat), _ptr(offsets), _ptr(counts), len(tables),
                                    num_blocks)
    _check("ref_check_block_tables", rc)


def blocks_for_tokens(tokens: int, block_tokens: int, lib=None) -> int:
    return int((lib or load()).ref_blocks_for_tokens(tokens, block_tokens))


def objects_for_tokens(tokens: int, block_tokens: int, layers: int, sides: int, lib=None) -> int:
    return int((lib or load()).ref_objects_for_tokens(tokens, block_tokens, layers, sides))


def kv_bytes(layers: int, tokens: int, heads: int, head_dim: int, elem_bytes: int,
             lib=None) -> int:
    return int((lib or load()).ref_kv_bytes(layers, tokens, heads, head_dim, elem_bytes))
