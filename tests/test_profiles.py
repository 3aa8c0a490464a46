"""The committed measurement summaries under profiles/ are self-describing
and point only at committed files.

* every traffic record names the kernel source hash it was taken on and a
  summary file that exists;
* every summary gives the command that produced it, and those commands run
  bench.py (a committed file) and nothing else of the repository;
* every bench line is one JSON object carrying the metric, roofline and
  kernel source hash fields;
* profiles/ holds text only (no raw profiler databases or programs).
"""
import glob
import json
import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROF = os.path.join(ROOT, "profiles")


def test_profiles_hold_text_only():
    for p in os.listdir(PROF):
        assert p.endswith((".md", ".json", ".txt")), p
        assert os.path.getsize(os.path.join(PROF, p)) < 64 * 1024, p


def test_traffic_records_point_at_existing_summaries():
    recs = glob.glob(os.path.join(PROF, "traffic_*.json"))
    assert recs
    for p in recs:
        rec = json.load(open(p))
        assert re.fullmatch(r"[0-9a-f]{16}", rec["kernel_source_hash"]), p
        assert rec["hbm_bytes_per_launch"] > 0, p
        assert os.path.exists(os.path.join(PROF, rec["summary"])), (p, rec["summary"])


def test_summaries_give_their_commands_over_committed_files():
    for p in glob.glob(os.path.join(PROF, "*.md")):
        txt = open(p).read()
        cmds = re.findall(r"`((?:rocprofv3|python3?) [^`]*)`", txt)
        assert cmds, f"{os.path.basename(p)} gives no command"
        for c in cmds:
            assert "bench.py" in c, (p, c)
            for tok in c.split():
                if tok.endswith((".py", ".sh")):
                    assert tok == "bench.py" and os.path.exists(os.path.join(ROOT, tok)), (p, tok)


def test_bench_lines_are_complete():
    for p in glob.glob(os.path.join(PROF, "bench_*.json")):
        d = json.loads(open(p).read().strip().splitlines()[-1])
        for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "dtype", "config",
                    "roofline", "kernel_source_hash"):
            assert key in d, (p, key)
        assert d["n_gpus"] == 1 and d["value"] > 0, p
        r = d["roofline"]
        assert r["bound"] in ("hbm", "mfma") and 0 < r["frac"] <= 1 and r["peak"] > 0, (p, r)
