"""Host-side logic of bench.py that needs no GPU: the kernel-source digest
under which measured HBM traffic is stored."""
import bench


def test_code_text_drops_comments_and_whitespace_only():
    a = 'int f(int x) {  // one\n  return x + 1; /* two\n three */ }\n'
    b = 'int f(int x) { return x + 1; }'
    assert bench.code_text(a) == bench.code_text(b)


def test_code_text_keeps_string_and_char_literals():
    src = 'static_assert(N > 0, "a // b /* c */"); char q = \'"\'; // gone'
    out = bench.code_text(src)
    assert '"a // b /* c */"' in out
    assert "'\"'" in out
    assert "gone" not in out


def test_code_text_sees_code_changes():
    assert bench.code_text("x = a + b;") != bench.code_text("x = a - b;")
    assert bench.code_text("f(a, b)") != bench.code_text("f(b, a)")


def test_source_digest_is_stable_and_per_file():
    d1 = bench.source_digest("prefill.hip")
    assert d1 == bench.source_digest("prefill.hip") and len(d1) == 16
    assert d1 != bench.source_digest("decode.hip")
