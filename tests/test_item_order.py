"""Index maps of the kernels, checked on the host (CPU only).

Out-axis work-item order:

The out-axis kernels map each workgroup id to a (channel, slot tile, row
pair, batch entry) item through ``out_tile`` (XCD-blocked ids; row pairs or
slot tiles fastest depending on the tile width).  tests/host/item_order.cpp
builds that host/device function for the host and checks, for 2-D and 3-D
geometries of every padded out-axis length from 8 to 2048 and inner extents
from 2 to 256, that every item is visited exactly once with the right mirror
row, for the forward, spectrum and backward tile widths.  A permutation that
dropped or repeated an item would leave part of y unwritten on the GPU.
"""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not found")
def test_out_axis_items_are_a_permutation(tmp_path):
    exe = str(tmp_path / "item_order")
    r = subprocess.run([HIPCC, "-std=c++20", "-O1", "-x", "hip", "--offload-host-only",
                        "-I", os.path.join(ROOT, "include"),
                        os.path.join(ROOT, "tests", "host", "item_order.cpp"), "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip().endswith("all ok"), r.stdout[-4000:]


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not found")
def test_row_tile_layouts_are_exact(tmp_path):
    """tests/host/row_layout.cpp: every row length's tile layout places each
    element at a distinct index inside the tile, and the split index the LDS
    passes use equals the plain index for every access of the radix plan."""
    exe = str(tmp_path / "row_layout")
    r = subprocess.run([HIPCC, "-std=c++20", "-O1", "-x", "hip", "--offload-host-only",
                        "-I", os.path.join(ROOT, "include"),
                        os.path.join(ROOT, "tests", "host", "row_layout.cpp"), "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip().endswith("all ok"), r.stdout[-4000:]
