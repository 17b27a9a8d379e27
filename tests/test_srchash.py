"""The code hash that ties the committed counter summaries to the kernel they were
taken on: comments and layout do not change it, code does."""
from gated_deltanet_recurrence_gdn_amd.srchash import code_hash, code_hash_text

SRC = """// header comment
template <int N>
__device__ int f(int x) {   /* block
                               comment */
    return x * N;  // trailing
}
"""


def test_comments_and_whitespace_do_not_count():
    same = SRC.replace("// header comment", "// another header").replace("trailing", "changed")
    same = same.replace("/* block\n                               comment */", "/* one line */")
    same = same.replace("    return", "\n\n        return")
    assert code_hash_text(same) == code_hash_text(SRC)


def test_code_changes_count():
    assert code_hash_text(SRC.replace("x * N", "x + N")) != code_hash_text(SRC)
    assert code_hash_text(SRC.replace("int N", "long N")) != code_hash_text(SRC)


def test_kernel_source_hashes():
    h = code_hash("gdn_chunk.hip")
    assert len(h) == 16 and int(h, 16) >= 0
