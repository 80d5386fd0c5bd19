"""Host-side pieces of bench.py that run without a GPU: the one-GPU guard,
the source digest that gates counter-derived traffic figures, and workload
name parsing."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_digest_is_stable_and_per_variant():
    d = bench.kernel_source_digest("decode_32x64")
    assert d == bench.kernel_source_digest("decode_32x64")
    assert len(d) == 16
    # same header, different rows of the variant table (ring kind, depth, K split)
    assert d != bench.kernel_source_digest("decode_32x64_k2")
    assert d != bench.kernel_source_digest("decode_16x64")
    # kernels from other headers
    assert bench.kernel_source_digest("tile_256x256") != bench.kernel_source_digest("stream_1x1_k4")


def test_digest_unknown_kernel():
    with pytest.raises(ValueError):
        bench.kernel_source_digest("no_such_kernel")


def test_traffic_only_for_the_kernel_it_was_taken_on():
    # a record is never reported for another variant of the same workload
    assert bench.recorded_traffic("c2_fp4_32x14336x4096", "decode_32x64_k2") is None
    assert bench.recorded_traffic("no_such_workload", "decode_32x64") is None


@pytest.mark.parametrize("name", ["quant_fp4", "quant_fp16_8x64", "quant_fp4_8x33", "xquant_fp4_8x64"])
def test_bad_quant_workload_names(name):
    with pytest.raises(SystemExit):
        bench.parse_quant_workload(name)


def test_quant_workload_name():
    assert bench.parse_quant_workload("quant_fp8_8192x8192") == ("fp8", 8192, 8192)


def test_digest_separates_stream_variants():
    # the stream families carry no quoted name in the variant table: their
    # rows are found from the parameters the name spells out
    d = {n: bench.kernel_source_digest(n) for n in ("stream_2x2_k4", "gstream_1x2_k4", "stream_4x2_k8",
                                                    "stream_2x4_k8", "fstream_2x4_k8")}
    assert len(set(d.values())) == len(d)


def test_roofline_reading():
    # c2's bytes at 4.023 us are exactly the HBM roofline; c5's FLOPs at the
    # dense MXFP4 peak are the MFMA roofline
    r = bench.roofline_for("fp4", 2.0 * 32 * 14336 * 4096, 32182272.0, 32182272.0 / 8e12 * 1e3)
    assert r["bound"] == "hbm" and abs(r["frac"] - 1.0) < 1e-3
    fl = 2.0 * 8192 ** 3
    r = bench.roofline_for("fp4", fl, 205.5e6, fl / 10066e12 * 1e3 * 2)
    assert r["bound"] == "mfma" and abs(r["frac"] - 0.5) < 1e-3
