"""Host logic of bench.py that needs no GPU: the code hash that keys the stored
rocprofv3 counters (bench.py reports them only while the kernel code is the one
they were taken on), and the refusal of more than one GPU."""
import os
import shutil
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "dense_descriptor_matching_amd", "csrc")


def test_code_only_drops_comments_and_layout_keeps_literals():
    src = 'int a = 1;  // note\n/* block\n   comment */ const char *s = "x // y /* z */";\nchar c = \'/\';\n'
    assert bench.code_only(src) == 'int a = 1; const char *s = "x // y /* z */"; char c = \'/\';'
    assert bench.code_only("a  \n\t b") == "a b"
    assert bench.code_only('s = "a\\"// b";') == 's = "a\\"// b";'      # escaped quote inside a literal


def _copy(tmp_path):
    d = tmp_path / "csrc"
    shutil.copytree(CSRC, d, ignore=shutil.ignore_patterns("*.so", "*.o"))
    return d


def test_hash_survives_comment_edits_and_sees_code_edits(tmp_path):
    d = _copy(tmp_path)
    ref = bench.kernel_source_hash(str(d))
    assert ref == bench.kernel_source_hash()                           # the copy hashes like the tree
    f = d / "ddm_frm.hpp"
    text = f.read_text()
    f.write_text("// a new comment line\n" + text.replace("\n", "\n\n", 3) + "\n/* trailing */\n")
    assert bench.kernel_source_hash(str(d)) == ref                     # comments and blank lines only
    f.write_text(text.replace("kSpinLimit = 1 << 20", "kSpinLimit = 1 << 21", 1))
    assert "1 << 21" in f.read_text()
    assert bench.kernel_source_hash(str(d)) != ref                     # a code change


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr and r.stdout == ""
