"""The counter summaries under profiles/ are tied to the kernel code they
were measured on by a digest of the source and the library headers it
includes, comments and layout left out: a code change marks a summary
stale, a comment or a line break does not (CPU only)."""
import os
import shutil

import bench


def test_code_only_drops_comments_and_keeps_literals():
    src = (b'int a = 1;  // note\n/* block\n   comment */\n\nconst char* s = "x // y /* z */";\n'
           b"char q = '\"'; int b = 2; // trailing\n")
    assert bench.code_only(src) == b'int a = 1; const char* s = "x // y /* z */"; char q = \'"\'; int b = 2;'


def _tree(tmp_path):
    root = tmp_path / "t"
    shutil.copytree(os.path.join(bench.ROOT, "jagged_flashattention_amd", "csrc"),
                    root / "jagged_flashattention_amd" / "csrc")
    shutil.copytree(os.path.join(bench.ROOT, "include"), root / "include")
    return str(root)


def test_digest_follows_code_not_comments(tmp_path):
    root = _tree(tmp_path)
    base = bench.source_digest("bwd.hip", root)
    assert base == bench.source_digest("bwd.hip")
    hdr = os.path.join(root, "jagged_flashattention_amd", "csrc", "qtile.h")
    text = open(hdr).read()
    open(hdr, "w").write("// a new comment line\n" + text.replace("namespace qtile {", "namespace qtile {  // here")
                         .replace("constexpr int kWaves = 8;", "constexpr  int\n    kWaves = 8;"))
    assert bench.source_digest("bwd.hip", root) == base
    # a code change in an included header marks every kernel using it stale
    open(hdr, "w").write(text.replace("constexpr int kWaves = 8;", "constexpr int kWaves = 4;"))
    assert bench.source_digest("bwd.hip", root) != base
    assert bench.source_digest("no_such.hip", root) is None
