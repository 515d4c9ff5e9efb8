"""Host logic of bench.py that needs no GPU: the kernel-code hash that decides
whether the stored HBM-traffic counters still describe the current kernel."""
import bench


def test_code_lines_ignore_comments_and_blank_lines():
    a = "int x = 1;  // one\n// a full-line comment\n\nint y;\n"
    b = "int x = 1;\nint y;  // another comment\n"
    assert bench._code_lines(a) == bench._code_lines(b)


def test_code_lines_see_code_changes():
    assert bench._code_lines("int x = 2;") != bench._code_lines("int x = 1;")


def test_code_lines_keep_string_literals_whole():
    s = 'asm volatile("s_nop 0 // not a comment");'
    assert bench._code_lines(s) == s


def test_kernel_source_hash_is_stable():
    h = bench.kernel_source_hash()
    assert len(h) == 16 and h == bench.kernel_source_hash()
