"""The oracle built with AddressSanitizer and UndefinedBehaviorSanitizer and run
through every pin (CPU only).

The instrumented oracle is loaded into a child Python process that has the
ASan runtime preloaded (ASan must be the first library a process loads), so
numpy's buffers get redzones and every memcpy of the oracle is bounds-checked.
Two planted mistakes, built the same way, show that the build really reports:
a dropped destination range check (a heap overflow, caught by ASan) and a
byte count of eq. 1 kept in int (a signed overflow, caught by UBSan).
"""
import os
import subprocess
import sys

import pytest

import oracle
import oracle_pins

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(os.path.dirname(oracle.__file__), "kvm_ref.c")
FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
         "-g"]

RUN_PINS = """
import sys
sys.path[:0] = [{root!r}, {tests!r}]
import oracle, oracle_pins
lib = oracle.load(path={lib!r})
for pin in oracle_pins.ALL_PINS:
    pin(lib)
print("pins ok", len(oracle_pins.ALL_PINS))
"""


def _asan_runtime():
    r = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        pytest.skip("gcc has no ASan runtime here")
    return path


def _run_pins(lib_path):
    env = dict(os.environ)
    pre = env.get("LD_PRELOAD", "")
    env["LD_PRELOAD"] = _asan_runtime() + (":" + pre if pre else "")
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:exitcode=23"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1:exitcode=24"
    code = RUN_PINS.format(root=ROOT, tests=HERE, lib=lib_path)
    return subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                          timeout=600)


def _build(tmp_path, name, text=None):
    src = SRC
    if text is not None:
        src = str(tmp_path / f"{name}.c")
        with open(src, "w") as f:
            f.write(text)
        # the copy includes kvm_ref.h from the oracle directory
        flags = FLAGS + ["-I", os.path.dirname(SRC)]
    else:
        flags = FLAGS
    return oracle.build(out=str(tmp_path / f"lib{name}.so"), src=src, extra_flags=flags)


def test_pins_pass_under_asan_and_ubsan(tmp_path):
    r = _run_pins(_build(tmp_path, "kvmref_san"))
    assert r.returncode == 0, r.stderr[-4000:]
    assert f"pins ok {len(oracle_pins.ALL_PINS)}" in r.stdout


PLANTED = [
    ("dropped destination range check", "AddressSanitizer",
     "        if (d_o > dst_bytes || len > dst_bytes - d_o) return REF_ERANGE;\n", ""),
    ("eq. 1 byte count kept in int", "runtime error: signed integer overflow",
     "return 2 * layers * tokens * heads * head_dim * elem_bytes;",
     "int l = (int)layers, t = (int)tokens, h = (int)heads, d = (int)head_dim,"
     " e = (int)elem_bytes;\n    return 2 * l * t * h * d * e;"),
]


@pytest.mark.parametrize("label,report,old,new", PLANTED, ids=[p[0] for p in PLANTED])
def test_sanitizers_report_planted_mistakes(tmp_path, label, report, old, new):
    text = open(SRC).read()
    assert text.count(old) == 1, label
    r = _run_pins(_build(tmp_path, "kvmref_planted", text.replace(old, new)))
    assert r.returncode != 0, f"{label}: the sanitized pins passed"
    assert report in r.stderr, r.stderr[-4000:]
