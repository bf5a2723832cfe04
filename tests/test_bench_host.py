"""Host-side logic of bench.py (CPU): the source hash that ties stored
HBM-traffic counters to the attention kernels, and the one-GPU guard."""
import os
import shutil
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_code_lines_drop_comments_keep_strings():
    src = ('// header\n'
           '\n'
           'int a = 1;   // trailing\n'
           'const char* s = "a//b";  // comment after a string\n'
           '  x = y; \\\n'
           '    // indented comment\n')
    assert list(bench._code_lines(src)) == ['int a = 1;', 'const char* s = "a//b";', '  x = y; \\']


def _copy_sources(tmp_path):
    d = tmp_path / "head_latent_attention_cache_amd" / "csrc"
    shutil.copytree(os.path.join(ROOT, "head_latent_attention_cache_amd", "csrc"), d)
    return d


def test_source_hash_ignores_comments_not_code(tmp_path, monkeypatch):
    d = _copy_sources(tmp_path)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h0 = bench.source_hash()
    assert h0 == bench.source_hash()
    p = d / "attention_dsplit.hip"
    text = p.read_text()
    p.write_text("// a new comment line\n\n" + text.replace("\n", "  // note\n", 1))
    assert bench.source_hash() == h0
    p.write_text(text.replace("constexpr int DS_PF_AHEAD = 8;", "constexpr int DS_PF_AHEAD = 9;"))
    assert "DS_PF_AHEAD = 9" in p.read_text()
    assert bench.source_hash() != h0
    p.write_text(text)
    # files outside the attention kernels do not enter the hash
    (d / "gemm.hip").write_text((d / "gemm.hip").read_text() + "\nint unrelated_change;\n")
    assert bench.source_hash() == h0


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
