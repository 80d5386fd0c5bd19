"""GPU: the default path's environment overrides, end to end.

MXG_CONFIG makes mx_scaled_mm_fp4/fp8 run the named configuration (output
bit-identical to the same configuration forced through
mx_scaled_mm_config), and MXG_LOG=1 prints each call's configuration.  The
variables are read once per process, so the overridden calls run in a
child process that writes its output to a file.
"""
from __future__ import annotations

import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import mxgen

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

_CHILD = r"""
import sys
import numpy as np, torch
sys.path.insert(0, sys.argv[1])
import mxgen
import block_scaled_precision_mm_amd as mx
fmt, M, N, K, path = sys.argv[2], int(sys.argv[3]), int(sys.argv[4]), int(sys.argv[5]), sys.argv[6]
a, sa = mxgen.quantize(mxgen.normal_bf16(41, (M, K)), fmt)
b, sb = mxgen.quantize(mxgen.normal_bf16(42, (N, K)), fmt)
d = [torch.from_numpy(np.ascontiguousarray(x)).cuda() for x in (a, b, sa, sb)]
c = torch.empty((M, N), dtype=torch.float32, device="cuda")
fn = mx.mx_scaled_mm_fp4 if fmt == "fp4" else mx.mx_scaled_mm_fp8
fn(*d, c, M, N, K)
torch.cuda.synchronize()
np.save(path, c.cpu().numpy())
"""


@pytest.mark.parametrize("fmt,shape,config", [
    ("fp4", (100, 130, 1152), "tile_128x128"),
    ("fp8", (70, 300, 2688), "tile_64x64_r4:2"),
    ("fp4", (33, 200, 8192), "stream_2x1_k4:4"),
])
def test_env_config_and_log(tmp_path, fmt, shape, config):
    import block_scaled_precision_mm_amd as mx
    M, N, K = shape
    name, _, parts = config.partition(":")
    parts = int(parts or 1)
    out = str(tmp_path / "c.npy")
    env = {k: v for k, v in os.environ.items() if not k.startswith("MXG_")}
    env.update(MXG_CONFIG=config, MXG_LOG="1")
    print("case", fmt, shape, config, flush=True)
    r = subprocess.run([sys.executable, "-c", _CHILD, ROOT, fmt, str(M), str(N), str(K), out],
                       env=env, capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, r.stderr[-2000:]
    line = "mxgemm: mx%s M=%d N=%d K=%d -> %s, %d K part%s (MXG_CONFIG)" % (
        fmt, M, N, K, name, parts, "" if parts == 1 else "s")
    assert line in r.stderr, r.stderr[-2000:]
    got = np.load(out)
    # the same configuration forced in this process
    a, sa = mxgen.quantize(mxgen.normal_bf16(41, (M, K)), fmt)
    b, sb = mxgen.quantize(mxgen.normal_bf16(42, (N, K)), fmt)
    d = [torch.from_numpy(np.ascontiguousarray(x)).cuda() for x in (a, b, sa, sb)]
    c = torch.empty((M, N), dtype=torch.float32, device="cuda")
    v = next(i for i in range(mx.mx_num_variants()) if mx.mx_variant_name(i) == name)
    mx.mx_scaled_mm_config(fmt == "fp4", *d, c, M, N, K, v, splits=parts)
    torch.cuda.synchronize()
    assert np.array_equal(got, c.cpu().numpy())
