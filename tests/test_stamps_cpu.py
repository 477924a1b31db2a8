"""The kernels' clock stamps (csrc/stamps.h): compiled out of the product library, and every stamp point in the
sources labelled by the timeline tool (long_context_sparse_ds_amd/stamps.py) and the other way round."""
import os
import re
import subprocess

import long_context_sparse_ds_amd as L
from long_context_sparse_ds_amd import build as B
from long_context_sparse_ds_amd.stamps import PHASES


def _exported(path):
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True, check=True).stdout
    return {line.split()[-1] for line in out.splitlines() if line.strip()}


def test_product_library_has_no_stamps():
    L.lib()   # built
    assert not [s for s in _exported(B.LIB) if s.startswith("ds_stamps_")]


def test_every_stamp_point_is_labelled():
    points = {}
    for f in os.listdir(B.CSRC):
        if not f.endswith(".hip"):
            continue
        text = open(os.path.join(B.CSRC, f)).read()
        for name, slot in re.findall(r"\bDS_STAMP\((\w+),\s*(\d+)\)", text):
            points.setdefault(name, set()).add(int(slot))
        for name in re.findall(r"^DS_STAMP_BUFFER\((\w+)\)", text, flags=re.M):
            points.setdefault(name, set())
    assert set(points) == set(PHASES)
    for name, slots in points.items():
        assert slots == set(PHASES[name]), name
        assert all(2 <= s < 31 for s in slots), name   # 0, 1 and 31 belong to the start and end stamps


def test_stamped_library_exports_its_buffers_when_built():
    if not os.path.exists(B.LIB_STAMPS):
        import pytest
        pytest.skip("stamped library not built (python -m long_context_sparse_ds_amd.build --stamps)")
    syms = _exported(B.LIB_STAMPS)
    for name in PHASES:
        assert f"ds_stamps_dump_{name}" in syms and f"ds_stamps_clear_{name}" in syms
