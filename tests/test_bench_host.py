"""Host logic of bench.py (no GPU): the source hash that ties committed counter
data to the kernels, the lookup of that data per plan, and the one-GPU rule."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_code_only_drops_comments_and_spacing_but_keeps_literals():
    src = 'int a = 1;  // one\n/* two\n   lines */ const char* s = "x // y /* z */";\nchar c = \'/\';\n'
    assert bench._code_only(src) == 'int a = 1; const char* s = "x // y /* z */"; char c = \'/\';'
    # a comment edit leaves the code unchanged; a code edit does not
    assert bench._code_only(src.replace("// one", "// uno")) == bench._code_only(src)
    assert bench._code_only(src.replace("= 1", "= 2")) != bench._code_only(src)


def test_kernel_source_sha_is_stable():
    a = bench.kernel_source_sha()
    assert len(a) == 16 and a == bench.kernel_source_sha()


def _table(tmp_path, rows):
    d = tmp_path / "profiles"
    d.mkdir()
    (d / "pmc_traffic.txt").write_text("# header\n" + "".join(" ".join(map(str, r)) + "\n" for r in rows))


def test_measured_traffic_takes_the_rows_of_the_plan(tmp_path, monkeypatch):
    sha = "f" * 16
    monkeypatch.setattr(bench, "kernel_source_sha", lambda: sha)
    _table(tmp_path, [
        ("wl", "kda_index_fixed", sha, 10, 1),
        ("wl", "kda_chunk_kernel_c4<1>", sha, 100, 20),
        ("wl", "kda_chunk_kernel<2>", sha, 30, 4),
        ("other", "kda_chunk_kernel<0>", sha, 7, 7),
        ("wl", "kda_chunk_kernel<0>", "0" * 16, 5, 5),  # other sources: ignored
    ])
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic("wl", (1, 2)) == 154  # either consumer variant, both passes
    assert bench.measured_traffic("wl", (0,)) is None  # the serial plan was not profiled
    assert bench.measured_traffic("other", (0,)) == 14
    assert bench.measured_traffic("missing", (0,)) is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


@pytest.mark.parametrize("flag", ["--preheat-ms", "--steps", "--warmup"])
def test_cli_knobs_exist(flag):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--help"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0 and flag in r.stdout
