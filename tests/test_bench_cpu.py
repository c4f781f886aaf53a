"""bench.py's host-side pieces, without a GPU: the one-GPU guard, the kernel-source
hash that keys the committed HBM counters, and the consistency of those counters."""

import json
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode != 0
    assert "one GPU" in r.stderr and not r.stdout.strip()


def test_source_hash_ignores_comments_and_whitespace(tmp_path):
    src = os.path.join(ROOT, "mxfp8_block_scaled_amd", "csrc")
    for f in bench.HASHED_SOURCES:
        shutil.copy(os.path.join(src, f), tmp_path / f)
    h0 = bench.src_hash(str(tmp_path))
    assert h0 == bench.src_hash()
    g = tmp_path / "gemm.hip"
    text = g.read_text()
    g.write_text("// a new comment\n/* and a\n   block one */\n" + text.replace("\n", "\n\n", 5) + "\n   \n")
    assert bench.src_hash(str(tmp_path)) == h0
    g.write_text(text.replace("constexpr int64_t GM = 4;", "constexpr int64_t GM = 8;", 1))
    assert "constexpr int64_t GM = 4;" in text
    assert bench.src_hash(str(tmp_path)) != h0


def test_source_hash_ignores_the_instrumented_blocks(tmp_path):
    # the blocks only the cycle-stamp build compiles do not change the product kernels
    src = os.path.join(ROOT, "mxfp8_block_scaled_amd", "csrc")
    for f in bench.HASHED_SOURCES:
        shutil.copy(os.path.join(src, f), tmp_path / f)
    g = tmp_path / "gemm.hip"
    text = g.read_text()
    assert text.count("#ifdef MX_CYCLE_STAMPS") >= 5
    h0 = bench.src_hash(str(tmp_path))
    out, rest = [], text
    while "#ifdef MX_CYCLE_STAMPS\n" in rest:
        pre, post = rest.split("#ifdef MX_CYCLE_STAMPS\n", 1)
        out.append(pre)
        rest = post.split("#endif\n", 1)[1]
    g.write_text("".join(out) + rest)
    assert "MX_CYCLE_STAMPS" not in g.read_text()
    assert bench.src_hash(str(tmp_path)) == h0
    # code outside such a block still counts
    g.write_text(text.replace("#ifdef MX_CYCLE_STAMPS\n", "#if 1\n", 1))
    assert bench.src_hash(str(tmp_path)) != h0


def test_stamp_summary():
    import numpy as np

    # two compute units of XCC 3, two blocks each: start, loop start, loop end, end
    def row(t0, t1, t2, t3, cu, n_iter):
        return [t0, t1, t2, t3, 0, (3 << 32) | (cu << 8), n_iter, 1]

    rec = np.array([row(0, 100, 1100, 1300, 1, 10), row(1400, 1500, 2500, 2700, 1, 10),
                    row(0, 200, 1200, 1400, 2, 10), row(1500, 1600, 2600, 2800, 2, 10),
                    [0] * 8], dtype=np.uint64)
    s = bench.stamp_summary(rec)
    assert s["blocks"] == 4 and s["compute_units"] == 2
    assert s["setup_cycles"] == 125 and s["loop_cycles"] == 1000 and s["loop_cycles_per_k_step"] == 100
    assert s["epilogue_cycles"] == 200 and s["gap_between_blocks_cycles"] == 100
    assert s["cu_span_cycles"] == {"mean": 2750, "min": 2700, "max": 2800}
    assert s["busy_frac"] == round((1300 + 1300 + 1400 + 1300) / (2700 + 2800), 3)
    assert s["per_xcd_span_mean_max"] == {"3": [2750, 2800]}
    assert not s["blocks_overlap_on_a_cu"]
    assert bench.stamp_summary(np.zeros((4, 8), dtype=np.uint64)) is None
    # two blocks at once on one compute unit: no gap, no busy fraction
    o = bench.stamp_summary(np.array([row(0, 100, 1100, 1300, 1, 10), row(50, 150, 1150, 1350, 1, 10)],
                                     dtype=np.uint64))
    assert o["blocks_overlap_on_a_cu"] and o["gap_between_blocks_cycles"] is None and o["busy_frac"] is None


def test_traffic_table_is_consistent():
    with open(os.path.join(ROOT, "profiles", "traffic.json")) as fh:
        d = json.load(fh)
    ff, fw = d["_factors"]["fetch"], d["_factors"]["write"]
    assert 1.9 < ff < 2.1 and 0.9 < fw < 1.1  # a 1 GiB copy reads as 0.5 GiB of FETCH_SIZE, 1 GiB of WRITE_SIZE
    ops = {k: v for k, v in d.items() if not k.startswith("_")}
    assert {"gemm_fwd grouped", "gemm_dgrad grouped", "gemm_wgrad grouped"} <= set(ops)
    for name, e in ops.items():
        want = e["fetch_kib"] * 1024 * ff + e["write_kib"] * 1024 * fw
        assert abs(e["hbm_bytes_per_launch"] - want) <= 1e-4 * want, name  # the factors are stored rounded
    # the grouped GEMMs' writes are their bf16 outputs (16384 x 4096, and 8 x 4096 x 4096 for wgrad)
    assert abs(ops["gemm_fwd grouped"]["write_kib"] * 1024 - 16384 * 4096 * 2) < 0.01 * 16384 * 4096 * 2
    assert abs(ops["gemm_wgrad grouped"]["write_kib"] * 1024 - 8 * 4096 * 4096 * 2) < 0.01 * 8 * 4096 * 4096 * 2
    hashes = {e["source_hash"] for e in ops.values()}
    if hashes != {bench.src_hash()}:
        pytest.skip("the counters were taken on other kernel sources; bench.py reports traffic as null")
