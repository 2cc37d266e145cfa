"""Host-side helpers of the measurement tooling (CPU only): the device-code
hash that ties the counter summaries under profiles/ to the code they were
taken on must ignore comments and whitespace and change with the code."""
import os
import shutil

from gated_delta_amd import srchash


def test_code_only_strips_comments_and_whitespace():
    a = "int x = 1; // one\n/* block\n comment */ float y;\n"
    b = "int  x = 1;\nfloat   y;   // other words\n"
    assert srchash._code_only(a) == srchash._code_only(b) == "int x = 1; float y;"


def test_hash_follows_code_not_comments(tmp_path, monkeypatch):
    src = srchash._CSRC
    dst = tmp_path / "csrc"
    shutil.copytree(src, dst)
    monkeypatch.setattr(srchash, "_CSRC", str(dst))
    h0 = srchash.kernel_source_hash()
    f = dst / "rda_walk.hip"
    text = f.read_text()
    f.write_text("// a new comment line\n" + text.replace("\n", "\n\n", 3))
    assert srchash.kernel_source_hash() == h0
    f.write_text(text.replace("kPfAhead = 4", "kPfAhead = 5"))
    assert srchash.kernel_source_hash() != h0
    # the host-side launch code is not part of the device-code hash
    g = dst / "rda_api.hip"
    g.write_text(g.read_text() + "\nint unused_marker;\n")
    f.write_text(text)
    assert srchash.kernel_source_hash() == h0
    assert os.path.exists(src)
