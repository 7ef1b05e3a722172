"""Host-side pieces of bench.py: the code digest that decides whether the
committed counter traffic still applies to an entry point's sources."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _digest_of(tmp_path, name, text):
    p = tmp_path / name
    p.write_text(text)
    old = bench.ROOT
    bench.ROOT = str(tmp_path)
    try:
        return bench.source_digest([name])
    finally:
        bench.ROOT = old


def test_digest_ignores_comments_and_blank_lines(tmp_path):
    code = 'int f(int x) {\n    return x + 1;\n}\nconst char* s = "a // b /* c */";\n'
    commented = ('// header\n/* block\n   comment */\nint f(int x) {  // trailing\n\n'
                 '    return x + 1;   \n}\nconst char* s = "a // b /* c */";  /* end */\n')
    assert _digest_of(tmp_path, "a.hip", code) == _digest_of(tmp_path, "a.hip", commented)


def test_digest_sees_code_and_string_changes(tmp_path):
    base = _digest_of(tmp_path, "a.hip", "int f(int x) { return x + 1; }\n")
    assert _digest_of(tmp_path, "a.hip", "int f(int x) { return x + 2; }\n") != base
    s1 = _digest_of(tmp_path, "b.hip", 'const char* s = "// kept";\n')
    s2 = _digest_of(tmp_path, "b.hip", 'const char* s = "// kept!";\n')
    assert s1 != s2


def test_digest_python_comments(tmp_path):
    a = _digest_of(tmp_path, "m.py", "x = 1\n# note\ny = 2\n")
    b = _digest_of(tmp_path, "m.py", "x = 1\n\n    # other note\ny = 2\n")
    c = _digest_of(tmp_path, "m.py", "x = 1\ny = 3\n")
    assert a == b != c

