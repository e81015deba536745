"""Host-side logic of bench.py: the kernel-source hash that decides whether a
committed counter summary still describes the kernel (no GPU needed)."""
import os
import shutil
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _copy_sources(tmp_path):
    for n in ("ffn_prefill.hip",) + bench.KERNEL_HEADERS:
        shutil.copy(os.path.join(bench.CSRC, n), tmp_path / n)


def test_source_hash_ignores_comments_and_whitespace(tmp_path, monkeypatch):
    _copy_sources(tmp_path)
    monkeypatch.setattr(bench, "CSRC", str(tmp_path))
    h0 = bench.source_hash("ffn_prefill.hip")
    p = tmp_path / "ffn_prefill.hip"
    p.write_text("// a new leading comment\n/* and a block\n   comment */\n" + p.read_text().replace("\n", "\n\n"))
    assert bench.source_hash("ffn_prefill.hip") == h0


def test_source_hash_follows_code_and_headers(tmp_path, monkeypatch):
    _copy_sources(tmp_path)
    monkeypatch.setattr(bench, "CSRC", str(tmp_path))
    h0 = bench.source_hash("ffn_prefill.hip")
    p = tmp_path / "ffn_prefill.hip"
    text = p.read_text()
    p.write_text(text.replace("constexpr int kStages = 4;", "constexpr int kStages = 3;"))
    h1 = bench.source_hash("ffn_prefill.hip")
    assert h1 != h0
    p.write_text(text)
    hdr = tmp_path / "moe_internal.h"
    hdr.write_text(hdr.read_text() + "\nconstexpr int kProbe = 1;\n")
    assert bench.source_hash("ffn_prefill.hip") not in (h0, h1)
