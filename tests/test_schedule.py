"""The decode schedules replayed on the CPU (no GPU): a C++ check built from the
host source with the kernel launches stubbed (tests/cpp/schedule_check.cpp) —
the bins form (built in full, and updated in place over decode steps), and the
split form with shared-prefix groups."""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bins_schedule_covers_every_tile_once_and_merges_every_split(tmp_path):
    exe = tmp_path / "schedule_check"
    subprocess.run(["/opt/rocm/bin/hipcc", "-O1", "-std=c++17",
                    "-I", os.path.join(ROOT, "include"),
                    "-I", os.path.join(ROOT, "paged_kv_cache_09_amd", "csrc"),
                    os.path.join(ROOT, "tests", "cpp", "schedule_check.cpp"), "-o", str(exe)],
                   check=True, capture_output=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout[-2000:]
    assert "ALL OK" in r.stdout
    assert r.stdout.count("ok: ") >= 50
    assert r.stdout.count("ok groups: ") >= 40
    # schedules updated in place over decode steps were checked too, and both
    # the update and the full rebuild took place
    import re
    grown = re.findall(r"ok: (\d+) grown steps, (\d+) updates, (\d+) rebuilds", r.stdout)
    assert len(grown) >= 4
    for steps, upd, reb in grown:
        assert int(upd) > 0 and int(reb) > 0 and int(upd) + int(reb) == int(steps)
