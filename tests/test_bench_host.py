"""bench.py host logic (no GPU): the kernel-source hash that decides whether
the committed HBM counters still describe the kernels ignores comments and
layout, and nothing else."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_code_tokens_drops_comments_and_layout_only():
    src = ('int a = 1;  // trailing\n/* block\n comment */ const char *s = "x // y /* z */";\n'
           "char q = '\"';\n\n    int   b;  /**/int c;")
    assert bench.code_tokens(src) == ('int a = 1; const char *s = "x // y /* z */"; '
                                      "char q = '\"'; int b; int c;")
    # an escaped quote does not end a literal
    assert bench.code_tokens('f("a\\" // b"); // c') == 'f("a\\" // b");'


def test_code_change_changes_tokens_comment_change_does_not():
    base = "x = y + 1; // one\n"
    assert bench.code_tokens(base) == bench.code_tokens("x = y + 1; // two\n")
    assert bench.code_tokens(base) == bench.code_tokens("x  =  y + 1;\n\n/* three */")
    assert bench.code_tokens(base) != bench.code_tokens("x = y + 2; // one\n")


def test_kernel_source_hash_covers_every_kernel_source():
    for f in bench.KERNEL_SOURCES:
        assert os.path.exists(os.path.join(ROOT, "latency_decode_gemm_amd", "csrc", f)), f
    assert len(bench.kernel_source_hash()) == 16
