"""Host logic of bench.py that needs no GPU: the source digest that keeps
the recorded HBM-traffic counters tied to the FFN code they were taken on."""
import os
import shutil

import bench


def _digest_of(tmp_path, edit=None):
    srcs = []
    for f in bench.FFN_SOURCES:
        dst = tmp_path / os.path.basename(f)
        shutil.copy(f, dst)
        srcs.append(str(dst))
    if edit is not None:
        p = srcs[2]  # ffn_wide.hip
        with open(p, encoding="utf-8") as fh:
            text = fh.read()
        with open(p, "w", encoding="utf-8") as fh:
            fh.write(edit(text))
    saved = bench.FFN_SOURCES
    bench.FFN_SOURCES = srcs
    try:
        return bench.source_digest()
    finally:
        bench.FFN_SOURCES = saved


def test_digest_ignores_comments_and_blank_lines(tmp_path):
    (tmp_path / "a").mkdir()
    (tmp_path / "b").mkdir()
    base = _digest_of(tmp_path / "a")
    edited = _digest_of(tmp_path / "b", lambda t: "// a new comment line\n\n" +
                        t.replace("constexpr int kWW = 8;", "constexpr int kWW = 8;  /* note */\n"))
    assert edited == base


def test_digest_follows_code(tmp_path):
    (tmp_path / "a").mkdir()
    (tmp_path / "b").mkdir()
    base = _digest_of(tmp_path / "a")
    edited = _digest_of(tmp_path / "b", lambda t: t.replace("constexpr int kWW = 8;",
                                                            "constexpr int kWW = 9;"))
    assert edited != base


def test_recorded_traffic_matches_current_sources():
    # the committed counter summaries were taken on the FFN code as it is
    assert bench.recorded_traffic("dsv2", "fused", "tiled") is not None
    assert bench.recorded_traffic("batch", "fused", "tiled") is not None
