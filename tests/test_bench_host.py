"""Host logic of the benchmark: the code digest that ties the committed HBM
counter figures to the kernel code they were taken on."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402

SRC = '''#include "a.h"
// a comment
int f(int x) {   /* inline */ return x + 1; }
const char* s = "http://x";  // the // inside the literal is code
'''


def test_digest_ignores_comments_indentation_and_blank_lines():
    edited = '''#include "a.h"

// another comment, longer
int f(int x) { /* changed
   over two lines */ return x + 1; }
    const char*    s = "http://x";
'''
    assert bench.code_digest([SRC]) == bench.code_digest([edited])


def test_digest_changes_with_any_code_edit():
    base = bench.code_digest([SRC])
    assert bench.code_digest([SRC.replace("x + 1", "x + 2")]) != base
    assert bench.code_digest([SRC.replace('"http://x"', '"http://y"')]) != base  # literal content is code
    assert bench.code_digest([SRC.replace("int f", "intf")]) != base            # token boundary
    assert bench.code_digest([SRC, "int g;"]) != base                           # an extra source
    assert bench.code_digest(["int a;", "int b;"]) != bench.code_digest(["int b;", "int a;"])  # order


def test_measured_traffic_unknown_kernel_is_null():
    assert bench.measured_traffic("no_such_kernel", "gqa_1m") is None
