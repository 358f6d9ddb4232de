"""Host-side checks of bench.py: the one-GPU guard, the algorithmic work model
and the lookup of recorded HBM traffic (no GPU needed)."""
import hashlib
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from workloads import get  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_algorithmic_work_of_decode_32k():
    wl = get("decode_32k")
    a = bench.algorithmic(wl)
    # every key of every sequence is scored once: 64 x 32768 keys x 128 dims x 2 bytes
    assert a["indexer"]["bytes"] >= 64 * 32768 * 128 * 2
    assert a["indexer"]["flops"] == 2.0 * 64 * 32768 * 64 * 128
    # 2048 selected rows per query, 128 heads, QK over 576 and PV over 512
    assert a["mla"]["flops"] == 2.0 * 64 * 2048 * 128 * (576 + 512)
    assert a["mla"]["bytes"] >= 64 * 2048 * 576 * 2


def test_algorithmic_counts_only_causal_pairs():
    wl = get("tiny_f32")  # 256 queries over 256 keys: 256 * 257 / 2 causal pairs
    a = bench.algorithmic(wl)
    assert a["indexer"]["flops"] == 2.0 * (256 * 257 // 2) * wl.idx_heads * wl.idx_dim


def test_recorded_traffic_follows_the_kernel_source(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_text("kernel v1\n")
    bld = tmp_path / "build.py"
    bld.write_text("flags v1\n")
    prof = tmp_path / "profiles"
    prof.mkdir()
    sha = hashlib.sha256(src.read_bytes() + bld.read_bytes()).hexdigest()
    (prof / "x.md").write_text(
        "# summary\n"
        f"bench-traffic: workload=decode_32k stage=indexer fetch_bytes=1000 write_bytes=24 source=k.hip,build.py "
        f"sha256={sha}\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    wl = get("decode_32k")
    assert bench.recorded_traffic(wl, "indexer") == 1024
    assert bench.recorded_traffic(wl, "mla") is None
    assert bench.recorded_traffic(get("decode_128k_fp8"), "indexer") is None
    bld.write_text("flags v2\n")  # other compile flags: counters no longer describe this kernel
    assert bench.recorded_traffic(wl, "indexer") is None
    bld.write_text("flags v1\n")
    assert bench.recorded_traffic(wl, "indexer") == 1024
    src.write_text("kernel v2\n")  # other source: the same
    assert bench.recorded_traffic(wl, "indexer") is None


def test_backward_algorithmic_work():
    """Five contractions per selected (query, key) pair and head; decode pairs are
    B * K, prefill pairs follow the causal ramp (short rows keep every key)."""
    import bench
    from workloads import get
    d = bench.bwd_algorithmic(get("decode_32k"))
    assert d["pairs"] == 64 * 2048
    assert d["flops"] == 2.0 * 64 * 2048 * 128 * (3 * 576 + 2 * 512)
    p = bench.bwd_algorithmic(get("prefill_4k"))
    assert p["pairs"] == sum(min(2048, t + 1) for t in range(4096))
    assert p["flops"] / p["pairs"] == d["flops"] / d["pairs"]


def test_default_run_covers_the_metric_points():
    import bench
    from workloads import get
    assert set(bench.POINTS) == {"decode_32k", "prefill_32k", "decode_128k_fp8"}
    ctx = {get(n).kv_len for n in bench.POINTS}
    assert ctx == {32768, 131072}
    assert bench.SWEEP_CONTEXTS[0] <= 4096 and bench.SWEEP_CONTEXTS[-1] >= 131072


def test_stage_fractions_against_the_box_ceilings():
    box = {"hbm_read": {"achieved": 5000.0}, "row_gather": {"achieved": 4000.0}, "bf16_mfma": {"achieved": 1250.0}}
    # decode: the sparse MLA is held to the random-row gather ceiling, the others to the streaming read
    fr = {"indexer": {"bound": "hbm", "frac": 0.5}, "topk": {"bound": "hbm", "frac": 0.05},
          "mla": {"bound": "hbm", "frac": 0.25}}
    bench.add_stage_box_fractions("decode_32k", fr, box)
    assert fr["indexer"]["frac_of_box"] == pytest.approx(0.5 * 8000 / 5000)
    assert fr["topk"]["frac_of_box"] == pytest.approx(0.05 * 8000 / 5000)
    assert fr["mla"]["frac_of_box"] == pytest.approx(0.25 * 8000 / 4000)
    assert fr["mla"]["box_ceiling"] == "row_gather"
    # prefill: MFMA-bound stages against the sustained bf16 MFMA rate
    fr = {"indexer": {"bound": "mfma", "frac": 0.5}, "mla": {"bound": "mfma", "frac": 0.4}}
    bench.add_stage_box_fractions("prefill_32k", fr, box)
    assert fr["indexer"]["frac_of_box"] == pytest.approx(0.5 * 2500 / 1250)
    assert fr["mla"]["frac_of_box"] == pytest.approx(0.4 * 2500 / 1250)
    assert "box_ceiling" not in fr["mla"]
