"""Host-side pieces of bench.py (no GPU): the code hash that decides whether committed
counter summaries still describe the kernels."""
import bench


def test_code_only_drops_comments_and_keeps_strings():
    src = 'int a;  // note\n/* block\n comment */ const char *s = "// kept /* too */";\nint b;\n'
    assert bench._code_only(src) == 'int a; const char *s = "// kept /* too */"; int b;'


def test_code_only_handles_escaped_quotes():
    src = 'const char *s = "a\\"b // x"; // gone\nint c;'
    assert bench._code_only(src) == 'const char *s = "a\\"b // x"; int c;'


def test_hash_ignores_comments_but_not_code(tmp_path, monkeypatch):
    a, b = tmp_path / "a.hip", tmp_path / "b.h"
    a.write_text("int f() { return 1; }  // one\n")
    b.write_text("#define X 2\n")
    monkeypatch.setattr(bench, "KERNEL_SRCS", [str(a), str(b)])
    h0 = bench.kernel_source_hash()
    a.write_text("// a new comment\nint f() {\n  return 1;   /* still one */\n}\n")
    assert bench.kernel_source_hash() == h0
    a.write_text("int f() { return 2; }\n")
    assert bench.kernel_source_hash() != h0
    a.write_text("int f() { return 1; }\n")
    b.write_text("#define X 3\n")
    assert bench.kernel_source_hash() != h0
