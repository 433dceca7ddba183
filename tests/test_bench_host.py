"""Host logic of bench.py that runs without a GPU: the source digest that ties
the committed rocprofv3 counters to the kernels they were taken from (bench
reports the counted HBM traffic only while it matches)."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_code_tokens_drop_comments_keep_literals():
    src = ('int a;  // note\n/* block\n comment */ const char* s = "// not a comment";\n'
           "char c = '/'; char q = '\\''; int d; /* tail */")
    assert bench._code_tokens(src) == (
        "int a; const char* s = \"// not a comment\"; char c = '/'; char q = '\\''; int d;")


def test_code_tokens_ignore_comment_reflow_but_not_code():
    a = "// one line\nint f(int x) { return x + 1; }\n"
    b = "// one\n// two lines\n\nint f(int x)   {\n  return x + 1;\n}\n"
    c = "int f(int x) { return x + 2; }"
    assert bench._code_tokens(a) == bench._code_tokens(b)
    assert bench._code_tokens(a) != bench._code_tokens(c)

