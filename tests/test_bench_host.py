"""Host logic of bench.py (CPU): the kernel-source hash that keys the committed
traffic profile changes with the code and not with its comments."""
import importlib.util
import os
import shutil
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_host", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    argv = sys.argv
    try:
        sys.argv = ["bench.py"]
        spec.loader.exec_module(mod)
    finally:
        sys.argv = argv
    return mod


def test_source_hash_ignores_comments_only(tmp_path):
    b = _bench()
    for f in b.KERNEL_SOURCES:
        os.makedirs(tmp_path / os.path.dirname(f), exist_ok=True)
        shutil.copy(os.path.join(ROOT, f), tmp_path / f)
    b.ROOT = str(tmp_path)
    base = b.kernel_sources_sha256()
    target = tmp_path / b.KERNEL_SOURCES[0]
    src = target.read_text()
    target.write_text("// a comment\n/* and a\n   block */\n" + src.replace("\n", "\n\n", 3))
    assert b.kernel_sources_sha256() == base
    assert "constexpr int RB = 12;" in src
    target.write_text(src.replace("constexpr int RB = 12;", "constexpr int RB = 12 + 0;", 1))
    assert b.kernel_sources_sha256() != base



def test_profiled_traffic_sums_a_calls_launches(tmp_path):
    b = _bench()
    os.makedirs(tmp_path / "profiles")
    (tmp_path / "profiles" / os.path.basename(b.TRAFFIC_PROFILE)).write_text(
        f"traffic: kernel_sources_sha256 = {b.kernel_sources_sha256()}\n"
        "traffic: bytes_per_launch.group_down = 700\n"
        "traffic: bytes_per_launch.group_gate_up = 1400\n")
    for f in b.KERNEL_SOURCES:
        os.makedirs(tmp_path / os.path.dirname(f), exist_ok=True)
        shutil.copy(os.path.join(ROOT, f), tmp_path / f)
    b.ROOT = str(tmp_path)
    assert b.profiled_traffic("group_down") == 700
    assert b.profiled_traffic("group_gate_up+group_down") == 2100
    assert b.profiled_traffic("group_gate_up+group_act_v4") is None   # a launch without a count
    target = tmp_path / b.KERNEL_SOURCES[0]
    target.write_text(target.read_text() + "\nint changed_code;\n")
    assert b.profiled_traffic("group_down") is None                  # the code changed since
