"""libkvmove for MI355X (gfx950): paged <-> Full Block KV-cache movement.

The compute path is the HIP library libkvmove.so (csrc/, include/kvm.h);
``kvmove`` is its ctypes binding and ``workloads`` the seeded synthetic inputs.
"""
