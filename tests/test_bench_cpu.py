"""Host-side checks of the measurement harness: the byte accounting per call, the
one-GPU contract of bench.py, and the staleness guard on committed counter summaries."""

import os
import subprocess
import sys

import pytest

import bench
from residual_add_rmsnorm_fp32_amd import workloads as wk

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bytes(name, T=None, **kw):
    wl = wk.WORKLOADS[name]
    T = wl.T if T is None else T
    return wk.algorithmic_bytes(wl.P, T, wl.H, 2, kw.get("quant", wl.quant),
                                kw.get("with_norm", wl.quant == "none"))


def test_algorithmic_bytes_of_the_workloads():
    # hand count per call: T*H*(P*e + e residual + e new residual [+ e norm_out] [+ 1 code])
    # + H*e gamma [+ 4 static scale] [+ 4*T per-token scales], e = 2
    assert _bytes("c1") == 16 * 2048 * (2 * 2 + 2 + 2 + 2) + 2048 * 2 == 331_776
    assert _bytes("c2") == 80 * 4096 * (8 * 2 + 6) + 4096 * 2 == 7_217_152
    assert _bytes("c2", T=1) == 98_304
    assert _bytes("c2", T=8) == 729_088
    assert _bytes("c2", T=32) == 2_891_776
    assert _bytes("c3") == 64 * 8192 * (4 * 2 + 4 + 1) + 8192 * 2 + 4 == 6_832_132
    assert _bytes("c3", with_norm=True) == 7_880_708
    assert _bytes("c4") == 2048 * 5120 * (2 * 2 + 4 + 1) + 5120 * 2 + 4 * 2048 == 94_390_272
    assert _bytes("c4", with_norm=True) == 115_361_792
    assert _bytes("c5") == 16384 * 3584 * (8 * 2 + 6) + 3584 * 2 == 1_291_852_800


def test_algorithmic_bytes_of_the_other_forms():
    T, H = 2048, 5120
    base = wk.algorithmic_bytes(2, T, H, 2, "dynamic", False)
    assert wk.algorithmic_bytes(2, T, H, 2, "group", False) == base - 4 * T + 4 * T * (H // 128)
    assert wk.algorithmic_bytes(2, T, H, 2, "tensor", False) == base - 4 * T + 4
    assert wk.algorithmic_bytes(2, T, H, 2, "dynamic", False, with_residual=False) == base - 2 * T * H
    assert wk.algorithmic_bytes(2, T, H, 2, "dynamic", False, with_residual_out=False) == base - 2 * T * H
    # a ragged last group still gets a scale
    assert wk.algorithmic_bytes(1, 1, 130, 2, "group", False) == 130 * (2 + 2 + 2 + 1) + 130 * 2 + 8


def test_bench_refuses_more_than_one_gpu():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
    assert res.stdout == ""


def test_traffic_summary_is_ignored_when_kernels_changed(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "far_vec_kernel_cx_traffic.md").write_text(
        "traffic_bytes_per_launch: 1234\nkernel_sources_sha256_16: 0000000000000000\n")
    (prof / "far_vec_kernel_cy_traffic.md").write_text(
        f"traffic_bytes_per_launch: 1234\nkernel_sources_sha256_16: {bench.kernel_sources_sha()}\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_sources_sha", lambda: open(prof / "far_vec_kernel_cy_traffic.md").read().split()[-1])
    assert bench.read_traffic("cx") is None
    assert bench.read_traffic("cy") == 1234.0
    assert bench.read_traffic("missing") is None


@pytest.mark.parametrize("name", ["c2", "c4", "c5"])
def test_committed_traffic_summaries_parse(name):
    path = os.path.join(ROOT, "profiles", f"far_vec_kernel_{name}_traffic.md")
    text = open(path).read()
    assert "traffic_bytes_per_launch:" in text and "kernel_sources_sha256_16:" in text
    assert "rocprofv3 --pmc FETCH_SIZE" in text and "rocprofv3 --pmc WRITE_SIZE" in text


@pytest.mark.parametrize("K,W,chunks", [(20, 5, 5), (10000, 200, 5), (7, 0, 5), (3, 1, 5), (1030, 3, 4)])
def test_region_plan_times_exactly_k_steps(K, W, chunks):
    """The timed region holds exactly K steps in (at most) the requested number of
    near-equal chunks, in rotation order after the warm-up, with a stamp before the
    first chunk and after every chunk, in graph pieces of at most 512 steps."""
    lens, pieces = bench.plan_region(K, W, chunks)
    assert sum(lens) == K and len(lens) == min(chunks, K) and max(lens) - min(lens) <= 1
    nodes = [nd for p in pieces for nd in p]
    steps = [v for kind, v in nodes if kind == "step"]
    assert steps == list(range(W, W + K))
    stamps = [i for i, (kind, _) in enumerate(nodes) if kind == "stamp"]
    assert [nodes[i][1] for i in stamps] == list(range(len(lens) + 1))
    assert stamps[0] == 0 and stamps[-1] == len(nodes) - 1
    between = [stamps[i + 1] - stamps[i] - 1 for i in range(len(lens))]
    assert between == lens
    assert all(sum(kind == "step" for kind, _ in p) <= bench.MAX_GRAPH_NODES for p in pieces)


def test_median():
    assert bench.median([3.0, 1.0, 2.0]) == 2.0
    assert bench.median([4.0, 1.0, 2.0, 3.0]) == 2.5


def test_workload_with_another_hidden_size():
    """'c4h5124' is c4's recipe at H = 5124 (the partial-last-pack form); names that are
    not a workload, or a workload with a bad suffix, are refused."""
    wl = bench.workload_of("c4h5124")
    c4 = wk.WORKLOADS["c4"]
    assert wl.H == 5124 and wl.name == "c4h5124"
    assert (wl.P, wl.T, wl.dtype, wl.quant, wl.seed, wl.eps) == (c4.P, c4.T, c4.dtype, c4.quant, c4.seed, c4.eps)
    assert "[2048,5124]" in wl.description
    assert bench.workload_of("c2") is wk.WORKLOADS["c2"]
    assert wk.algorithmic_bytes(wl.P, wl.T, wl.H, 2, wl.quant, False) == \
        2048 * 5124 * (2 * 2 + 4 + 1) + 5124 * 2 + 4 * 2048
    for bad in ("c9", "c4h", "c4x5124", "h5124", ""):
        with pytest.raises(SystemExit):
            bench.workload_of(bad)


def test_default_line_measures_the_partial_pack_form():
    assert "c4h5124" in bench.PREFILL_EXTRA and {"c4", "c5"} <= set(bench.PREFILL_EXTRA)
