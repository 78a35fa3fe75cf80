"""Host logic of bench.py: the kernel-source digest that keeps the committed
HBM counters tied to the code they were taken on."""
import json
import os
import shutil

import pytest

import bench


def test_code_only_drops_comments_and_keeps_literals():
    src = ('int a = 1; // line comment\n'
           '/* block\n   comment */ const char* s = "a // b /* c */";\n'
           "char q = '\"'; char r = '\\''; int   b =\t2;\n")
    got = bench._code_only(src)
    assert got == ('int a = 1; const char* s = "a // b /* c */"; '
                   "char q = '\"'; char r = '\\''; int b = 2;")


@pytest.fixture()
def csrc_copy(tmp_path, monkeypatch):
    root = tmp_path / "repo"
    src = os.path.join(bench.ROOT, "diffusion_transformer_elementwise_amd", "csrc")
    dst = root / "diffusion_transformer_elementwise_amd" / "csrc"
    shutil.copytree(src, dst, ignore=shutil.ignore_patterns("__pycache__"))
    monkeypatch.setattr(bench, "ROOT", str(root))
    return root, dst


def test_digest_ignores_comment_edits_and_sees_code_edits(csrc_copy):
    root, csrc = csrc_copy
    d0 = bench.kernel_source_digest()
    k = csrc / "gate_add.hip"
    text = k.read_text()
    k.write_text("// a new comment line\n" + text.replace("\n", "\n  /* note */ ", 1))
    assert bench.kernel_source_digest() == d0
    k.write_text(text + "\nstatic int probe_only = 1;\n")
    assert bench.kernel_source_digest() != d0


def test_traffic_is_used_only_for_matching_sources(csrc_copy):
    root, csrc = csrc_copy
    prof = root / "profiles"
    prof.mkdir()
    entry = {"kernels": {"gate_add_bcast_kernel": {"bytes_per_launch": 1234}}}
    (prof / "traffic.json").write_text(
        json.dumps(dict(entry, source_digest=bench.kernel_source_digest())))
    assert bench.load_traffic("gate_add_bcast_kernel") == 1234
    assert bench.load_traffic("no_such_kernel") is None
    (prof / "traffic.json").write_text(json.dumps(dict(entry, source_digest="0" * 16)))
    assert bench.load_traffic("gate_add_bcast_kernel") is None
