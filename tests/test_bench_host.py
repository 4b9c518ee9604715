"""Host-side logic of bench.py (no GPU): the one-GPU guard, the reader of the
committed rocprofv3 summaries, and the roofline object's arithmetic."""
import glob
import os
import re

import pytest

import bench
import synth


def test_more_than_one_gpu_is_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err


def test_a_multi_rank_launch_is_refused(monkeypatch, capsys):
    monkeypatch.setenv("WORLD_SIZE", "2")
    assert bench.main([]) == 2
    assert "one GPU" in capsys.readouterr().err


def test_counter_summary_is_read_only_for_the_source_it_was_taken_on(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    (tmp_path / "k.md").write_text(
        "# k on some workload\n\n"
        "## first workload\n\n"
        "- hbm_bytes_per_launch: 4.5e+09\n"
        "- traffic_over_algorithmic: 1.07\n\n"
        "## second workload\n\n"
        "- hbm_bytes_per_launch: 8.0e+07\n\n"
        "- kernel_source_sha256: 0123456789abcdef\n")
    # the first line holding the key wins
    assert bench.read_counter_summary("k.md", "0123456789abcdef") == 4.5e9
    assert bench.read_counter_summary("k.md", "0123456789abcdef",
                                      "traffic_over_algorithmic") == 1.07
    # another kernel source, a missing key, a missing file: no figure
    assert bench.read_counter_summary("k.md", "fedcba9876543210") is None
    assert bench.read_counter_summary("k.md", "0123456789abcdef", "mfma_busy_pct") is None
    assert bench.read_counter_summary("absent.md", "0123456789abcdef") is None


def test_committed_summaries_name_their_commands_and_source():
    paths = sorted(glob.glob(os.path.join(bench.PROFILES, "*.md")))
    assert paths
    for p in paths:
        text = open(p).read()
        assert re.search(r"^- kernel_source_sha256: [0-9a-f]{16}$", text, re.M), p
        cmds = [ln.strip() for ln in text.splitlines() if ln.strip().startswith("rocprofv3 --")]
        assert cmds, p
        for c in cmds:
            # every command runs committed files, by paths relative to the repository
            assert "_work" not in c and " /" not in c, (p, c)
            assert " -- python3 bench.py" in c, (p, c)


def test_roofline_object_relates_algorithmic_bytes_to_the_peak():
    cfg = synth.CFG_WKV4_LONG
    r = bench.wkv4_roofline(cfg, 0.75, "wkv4_fwd_tiled_B1_T65536_C5120.md")
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert r["algorithmic_bytes_per_launch"] == 12 * cfg.B * cfg.T * cfg.C
    assert r["achieved"] == pytest.approx(12 * cfg.B * cfg.T * cfg.C / 0.75e-3 / 1e9, rel=1e-6)
    assert r["frac"] == pytest.approx(r["achieved"] / r["peak"], abs=1e-4)
    assert r["kernel_source"] == bench.kernel_source_hash()
    # the counter figure is either absent or HBM bytes of the same order
    assert r["traffic"] is None or 1.0 <= r["traffic"] / r["algorithmic_bytes_per_launch"] < 1.5
