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
