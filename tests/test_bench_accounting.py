"""bench.py's algorithmic work model against the closed form of the path.

Per layer call the method's products are, per (batch, head): the L logits,
L^T q and L U over b1 key blocks for every query token, once per iteration
except L U (once), and the R logits and R V (or R K) over b2 keys for every
(tile, key) row once per iteration:
  flops = 2 d [(2T + 1) Nq b1 + 2 T t N b2]
(a chunk against cached keys has Nq query tokens; the R side runs over all N).
The per-kernel figures bench.py reports the roofline with must add up to
this, whatever the launch counts of an iteration count.
"""
import pytest

import bench
from structured_attention_video_monarch_amd import inputs as I


def closed_form_flops(wl):
    T = wl.iters
    return wl.B * wl.H * 2.0 * wl.d * ((2 * T + 1) * wl.Nq * wl.b1 + 2 * T * wl.tiles * wl.N * wl.b2)


@pytest.mark.parametrize("name", ["latent720p", "clip480p_spikes_t4_T1", "chunk480p_kv", "clip480p_frames"])
@pytest.mark.parametrize("T", [1, 2, 10])
def test_forward_work_sums_to_closed_form(name, T):
    wl = I.get_workload(name).with_(iters=T)
    launches = {"k_kbar": 1, "k_lse": T, "k_aggregate": T, "k_rstep": T, "k_apply": 1}
    tot = bench.step_work(wl, "fwd", launches)
    flops = sum(tot[k][0] for k in launches)
    assert abs(flops - closed_form_flops(wl)) <= 1e-9 * closed_form_flops(wl)


def test_latent720p_one_iteration_is_2690_gflop():
    # 40 heads of 75600 tokens, d = 128, blocks (945, 80), 4 tiles:
    # 2*128*(3*75600*945 + 2*4*75600*80) per head = 6.726e10; x 40 = 2.690e12
    wl = I.get_workload("latent720p")
    tot = bench.step_work(wl, "fwd", {"k_kbar": 1, "k_lse": 1, "k_aggregate": 1, "k_rstep": 1, "k_apply": 1})
    flops = sum(v[0] for v in tot.values())
    assert abs(flops - 2.690e12) <= 0.001 * 2.690e12


def test_per_kernel_bytes_are_the_layer_tensors_only():
    """Algorithmic bytes are the layer's own tensors each kernel touches
    (Q, K, V, O), never the implementation's intermediates: the first
    L-step's kernels read Q, the R-step reads K and V, the apply reads Q and
    writes O; over the call Q, K, V are read and O is written once each
    (4*B*H*N*d*e, 3097 MB at the 720p latent in bf16)."""
    wl = I.get_workload("latent720p")
    e = 2
    x = wl.B * wl.H * wl.N * wl.d * e
    w = bench.algorithmic_work(wl)
    assert w["k_kbar"][1] == x and w["k_lse"][1] == x and w["k_aggregate"][1] == x
    assert w["k_rstep"][1] == 2 * x and w["k_apply"][1] == 2 * x
    assert abs(4 * x - 3.097e9) <= 0.001 * 3.097e9
    # the aggregated queries and U (t*N*d*e each, written and read) are
    # intermediates, reported apart: 12.4 GB over the call
    inter = bench.intermediate_bytes(wl)
    tnd = wl.B * wl.H * wl.tiles * wl.N * wl.d * e
    assert inter["k_aggregate"] >= tnd and inter["k_rstep"] == 2 * tnd and inter["k_apply"] >= tnd
    assert abs(4 * tnd - 12.39e9) <= 0.01 * 12.39e9


def test_roofline_bounds_follow_the_method_work():
    """The logit kernels and the R-step are MFMA-bound by their algorithmic
    work at the 720p latent (arithmetic intensity above the 312 flop/B
    ridge), the block means HBM-bound; k_aggregate at 2240.7 us per launch is
    0.7316 TFLOP / 2.2407 ms = 326.5 TFLOP/s, 0.131 of 2.5 PFLOP/s."""
    wl = I.get_workload("latent720p")
    w = bench.algorithmic_work(wl)
    fl, by = w["k_aggregate"]
    assert abs(fl - 2 * wl.B * wl.H * wl.Nq * wl.b1 * wl.d) == 0
    r = bench.roofline_entry("k_aggregate", fl, by, 2240.7e-6, "bf16", None)
    assert r["bound"] == "mfma" and abs(r["frac"] - 0.1306) <= 5e-4, r
    r = bench.roofline_entry("k_rstep", *w["k_rstep"], 1614.3e-6, "bf16", None)
    assert r["bound"] == "mfma" and abs(r["frac"] - 0.1228) <= 5e-4, r
    r = bench.roofline_entry("k_kbar", *w["k_kbar"], 145.1e-6, "bf16", None)
    assert r["bound"] == "hbm" and abs(r["frac"] - 0.6669) <= 5e-4, r
    assert bench.roofline_entry("k_objective", *w["k_objective"], 1e-5, "bf16", None)["bound"] == "none"


def test_more_than_one_gpu_is_refused_with_a_message():
    """bench.py measures one GPU; --gpus above 1 exits with status 2 and says
    so, before any GPU work."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2", "--steps", "1"],
                       capture_output=True, text=True, timeout=120, cwd=root)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_traffic_counters_are_used_only_on_the_sources_they_were_taken_on(monkeypatch, tmp_path):
    """A committed HBM-traffic figure is reported only while the kernel
    sources hash to the value recorded with it; any change to a kernel
    source changes the hash, and the figure is then dropped (null)."""
    import json
    import os
    rec = {"kernel": "k_demo", "workload": "demo", "hbm_bytes_per_launch": 12345, "kernel_source_hash": "abc"}
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "traffic_k_demo_demo.json").write_text(json.dumps(rec))
    src = tmp_path / "k.h"
    src.write_text("// kernel v1\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "KERNEL_SOURCES", ["k.h"])
    h1 = bench.kernel_source_hash()
    assert bench.read_traffic("k_demo", "demo") is None          # recorded on other sources
    rec["kernel_source_hash"] = h1
    (prof / "traffic_k_demo_demo.json").write_text(json.dumps(rec))
    assert bench.read_traffic("k_demo", "demo") == 12345
    src.write_text("// kernel v2\n")
    assert bench.kernel_source_hash() != h1
    assert bench.read_traffic("k_demo", "demo") is None
    assert bench.read_traffic("k_other", "demo") is None          # never measured
    assert os.path.exists(prof / "traffic_k_demo_demo.json")
