"""The C-ABI library loads and exports every symbol include/kvm.h declares (CPU only:
no compute call is made)."""
import ctypes
import os
import re

import pytest

from paged_kv_cache_kvm_amd import kvmove

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvm.h")
PKG = os.path.join(ROOT, "paged_kv_cache_kvm_amd")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^[A-Za-z_][\w \*]*?\b(kvm_\w+)\s*\(", text, flags=re.M)


def test_header_declares_the_four_operations():
    names = declared_functions()
    for op in ("kvm_pack_full", "kvm_unpack_layer", "kvm_merge_layer", "kvm_batch_copy"):
        assert op in names
    assert len(names) == len(set(names))


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(kvmove.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), f"libkvmove.so does not export {name}"


def test_binding_covers_every_declared_symbol():
    assert set(declared_functions()) == set(kvmove.SIGNATURES)


def test_version_and_status_text():
    m = re.search(r"#define KVM_ABI_VERSION (\d+)", open(HEADER).read())
    assert kvmove.kvm_version() == int(m.group(1))
    for code in (0, -1, -2, -3, -4, -5):
        assert kvmove.strerror(code)
    assert kvmove.strerror(12345) == "unknown status"


def test_status_codes_match_header():
    text = open(HEADER).read()
    for name, val in [("KVM_OK", 0), ("KVM_EINVAL", -1), ("KVM_ERANGE", -2), ("KVM_ENOMEM", -3),
                      ("KVM_EHIP", -4), ("KVM_ECHECK", -5)]:
        assert re.search(rf"#define {name} \(?{re.escape(str(val))}\)?", text), name
        assert getattr(kvmove, name) == val


def test_struct_sizes_match_header_layout():
    assert ctypes.sizeof(kvmove.kvm_pool_layout) == 48
    assert ctypes.sizeof(kvmove.kvm_seq) == 32
    assert ctypes.sizeof(kvmove.kvm_merge_seq) == 64
    assert ctypes.sizeof(kvmove.kvm_copy_desc) == 24
    assert ctypes.sizeof(kvmove.kvm_layer_seq) == 72


def test_null_arguments_rejected_without_a_device():
    """Argument checks run before any HIP call."""
    lib = kvmove.load()
    assert lib.kvm_create(0, None) == kvmove.KVM_EINVAL
    assert lib.kvm_create(-1, ctypes.byref(ctypes.c_void_p())) == kvmove.KVM_EINVAL
    assert lib.kvm_pack_full(None, None, None, 1, None, 0, None) == kvmove.KVM_EINVAL
    assert lib.kvm_merge_layer(None, 16, None, 0, None) == kvmove.KVM_EINVAL
    assert lib.kvm_batch_copy(None, None, 0, None, 0, None, 0, None) == kvmove.KVM_EINVAL
    assert lib.kvm_batch_copy_noalloc(None, None, 0, None, 0, None, 0, None) == kvmove.KVM_EINVAL
    assert lib.kvm_ctx_reserve(None, 1, 1) == kvmove.KVM_EINVAL
    assert lib.kvm_unpack_merge_layer(None, None, None, 1, 0, None, 0, None) == kvmove.KVM_EINVAL
    assert lib.kvm_ctx_set_max_workgroups(None, 4) == kvmove.KVM_EINVAL
    assert lib.kvm_ctx_set_checks(None, 1) == kvmove.KVM_EINVAL
    assert lib.kvm_ctx_reserve_unpack(None, 1, 1) == kvmove.KVM_EINVAL
    assert lib.kvm_ctx_device_bytes(None, ctypes.byref(ctypes.c_int64())) == kvmove.KVM_EINVAL
    lib.kvm_destroy(None)


def test_missing_library_fails_loudly(tmp_path, monkeypatch):
    monkeypatch.setattr(kvmove, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        kvmove.load(str(tmp_path / "nope.so"))


def test_product_code_never_touches_the_oracle():
    for dirpath, _, files in os.walk(PKG):
        for f in files:
            if f.endswith((".py", ".cpp", ".hip", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(import|from)\s+oracle\b", text, flags=re.M), f
                assert "kvm_ref" not in text, f
    for f in os.listdir(os.path.join(PKG, "csrc")):
        assert "kvm_ref" not in open(os.path.join(PKG, "csrc", f)).read()


def test_noalloc_limit_matches_header():
    text = open(HEADER).read()
    m = re.search(r"#define KVM_NOALLOC_MAX_DESCS \(\(INT64_C\(1\) << (\d+)\) - (\d+)\)", text)
    assert m, "KVM_NOALLOC_MAX_DESCS not found"
    assert kvmove.KVM_NOALLOC_MAX_DESCS == (1 << int(m.group(1))) - int(m.group(2))
