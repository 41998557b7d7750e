"""Host logic of bench.py that decides whether stored HBM counters still
describe the kernels: the source hash ignores comments and layout but not
code, and a counter record is used only under the hash it was taken with."""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


SRC = '''// header comment with "quotes" and 'apostrophes'
#include "x.h"   /* block
comment */
int f(int a) {
  const char* s = "// not a comment";   // trailing
  return a + '/';
}
'''


def test_code_text_drops_comments_and_layout_only():
    t = bench.code_text(SRC)
    assert "header comment" not in t and "block" not in t and "trailing" not in t
    assert '"// not a comment"' in t and "'/'" in t and '"x.h"' in t
    reflowed = SRC.replace("return a + '/';", "return a\n      + '/';   // reflowed")
    assert bench.code_text(reflowed) == t
    assert bench.code_text(SRC.replace("a + '/'", "a - '/'")) != t
    assert bench.code_text(SRC.replace('"// not a comment"', '"// other"')) != t


def test_traffic_record_used_only_under_its_hash(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "traffic.json").write_text(json.dumps({"decode": {"source_hash": "abc", "bytes_per_launch": 123}}))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.load_traffic("decode", "abc") == 123
    assert bench.load_traffic("decode", "abd") is None
    assert bench.load_traffic("prefill", "abc") is None

