"""bench.py's command line on the CPU: more than one GPU is refused with a
message before anything touches a device, and the helpers that shape the JSON
line (quantiles, the profile-hash check) behave as documented."""
import importlib.util
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    out = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert out.returncode == 2
    assert "one GPU only" in out.stderr
    assert out.stdout == ""


def test_quantile_interpolates():
    b = _bench()
    xs = [4.0, 1.0, 3.0, 2.0]
    assert b.quantile(xs, 0.0) == 1.0
    assert b.quantile(xs, 1.0) == 4.0
    assert abs(b.quantile(xs, 0.5) - 2.5) < 1e-12


def test_traffic_only_for_matching_kernel_sources(tmp_path, monkeypatch):
    """A traffic summary under profiles/ is used only while the kernel sources
    hash to the hash it records; a summary of other sources reports nothing,
    and an op no current summary has reports nothing."""
    import json
    b = _bench()
    h = b.kernel_source_sha256()
    (tmp_path / "current.md").write_text(
        "text\ntraffic-json: " + json.dumps({"kernel_source_sha256": h,
                                            "bytes_per_launch": {"merge_layer": 123}}) + "\n")
    (tmp_path / "stale.md").write_text(
        "traffic-json: " + json.dumps({"kernel_source_sha256": "0" * 64,
                                       "bytes_per_launch": {"unpack_layer": 456}}) + "\n")
    monkeypatch.setattr(b, "PROFILES", str(tmp_path))
    assert b.measured_traffic("merge_layer") == 123
    assert b.measured_traffic("unpack_layer") is None
    assert b.measured_traffic("pack_full") is None
    monkeypatch.setattr(b, "PROFILES", str(tmp_path / "missing"))
    assert b.measured_traffic("merge_layer") is None


def test_committed_traffic_matches_its_sources():
    """Each committed traffic line either matches the sources built now (and
    then gives positive byte counts) or is ignored."""
    import glob
    import json
    b = _bench()
    h = b.kernel_source_sha256()
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        for line in open(path):
            if not line.startswith("traffic-json: "):
                continue
            rec = json.loads(line[len("traffic-json: "):])
            for op, v in rec["bytes_per_launch"].items():
                got = b.measured_traffic(op)
                if rec["kernel_source_sha256"] == h:
                    assert isinstance(got, int) and got > 0, (path, op)


def test_profile_commands_run_committed_files_with_known_flags():
    """Every rocprofv3 command quoted in profiles/ runs the repository's
    bench.py with flags it accepts, and counter runs stay counter-only."""
    import glob
    import shlex
    b = _bench()
    files = sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md")))
    assert files
    seen = 0
    for path in files:
        cmds = [l.strip() for l in open(path) if "rocprofv3 --" in l and " -- " in l]
        assert cmds, f"{os.path.basename(path)} quotes no rocprofv3 command"
        for cmd in cmds:
            tool, _, prog = cmd.partition(" -- ")
            argv = shlex.split(prog)
            assert argv[:3] == ["python", "-u", "<repo>/bench.py"], cmd
            old = sys.argv
            try:
                sys.argv = ["bench.py", *argv[3:]]
                args = b.parse()
            finally:
                sys.argv = old
            assert args.gpus == 1 and args.steps >= 1, cmd
            # counter runs take no API or memory trace domain alongside
            assert "--pmc" not in tool or not any(
                t in tool for t in ("--sys-trace", "--runtime-trace", "--hip-trace", "--hsa-trace",
                                    "--memory-copy-trace", "--scratch-memory-trace",
                                    "--marker-trace", " -s ", " -r ")), cmd
            seen += 1
    assert seen >= 4


def test_config_and_reps_flags():
    """--config picks the workloads run after the layer loop (the --no-* flags
    still apply), --reps sets the repetitions; unknown workloads are refused."""
    b = _bench()
    old = sys.argv
    try:
        sys.argv = ["bench.py"]
        a = b.parse()
        assert (a.no_restore, a.no_mla, a.no_batch_copy, a.reps) == (False, False, False, 0)
        sys.argv = ["bench.py", "--config", "c3, C5", "--reps", "4"]
        a = b.parse()
        assert (a.no_restore, a.no_mla, a.no_batch_copy, a.reps) == (False, True, False, 4)
        sys.argv = ["bench.py", "--config", "none", "--no-restore"]
        a = b.parse()
        assert a.no_restore and a.no_mla and a.no_batch_copy
        for bad in (["--config", "c2"], ["--reps", "-1"]):
            sys.argv = ["bench.py", *bad]
            try:
                b.parse()
            except SystemExit as e:
                assert e.code == 2
            else:
                raise AssertionError(f"{bad} accepted")
    finally:
        sys.argv = old
