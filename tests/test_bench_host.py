"""bench.py's host-side helpers (CPU)."""
import subprocess
import sys

import bench


def test_source_digest_ignores_comments(tmp_path):
    a = tmp_path / "a.hip"
    b = tmp_path / "b.hip"
    c = tmp_path / "c.hip"
    a.write_text("// header\nint f(int x) { return x + 1; }  /* tail */\n")
    b.write_text("// another header\n/* block\n   comment */\nint f(int x) { return x + 1; }\n")
    c.write_text("// header\nint f(int x) { return x + 2; }\n")
    da, db, dc = (bench.source_digest([str(p)]) for p in (a, b, c))
    assert da == db, "comment edits keep the digest"
    assert da != dc, "code edits change it"
    assert len(bench.source_digest()) == 16


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, bench.__file__, "--gpus", "2"], capture_output=True,
                         text=True, timeout=120)
    assert res.returncode == 2 and "one GPU" in res.stderr
