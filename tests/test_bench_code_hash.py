"""bench.py reports the GEMM's measured HBM traffic only while the kernel's
code is the code the counters were taken for; the check hashes gemm.hip
without its comments.  CPU only."""
import hashlib
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

SRC = """// header
#include "x.h"  /* inline
   block */
const char* s = "a // not a comment /* nor this */";
char c = '/';
int f(int a) {   // trailing
  return a  *  2;
}
"""


def _h(text):
    return hashlib.sha256(bench._code_text(text).encode()).hexdigest()


def test_comments_and_whitespace_do_not_count():
    text = bench._code_text(SRC)
    assert "header" not in text and "inline" not in text and "trailing" not in text
    assert '"a // not a comment /* nor this */"' in text
    assert "'/'" in text
    edited = SRC.replace("// trailing", "// another remark").replace("a  *  2", "a * 2") + "\n// end\n"
    assert _h(edited) == _h(SRC)


def test_code_edits_count():
    assert _h(SRC.replace("a  *  2", "a * 3")) != _h(SRC)
    assert _h(SRC.replace('"a // not', '"b // not')) != _h(SRC)


def test_escaped_quote_inside_a_string():
    src = 'const char* s = "say \\"hi\\" // still a string"; // gone\nint x;'
    text = bench._code_text(src)
    assert "// still a string" in text and "gone" not in text and text.endswith("int x;")

