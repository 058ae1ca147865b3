"""The peak-rate microbenchmarks (peak_probe.py) run and give rates inside
physical bounds: every matrix-core rate is positive and at most its
data-sheet peak (plus measurement slack), the device copy lies below the HBM
figure, and the global-to-LDS DMA moves data."""
from __future__ import annotations

import os
import sys

import pytest

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import peak_probe  # noqa: E402

pytestmark = pytest.mark.gpu


def test_peak_probe_rates_are_physical():
    res = peak_probe.run(quick=True)
    assert len(res["mfma"]) == 4
    for m in res["mfma"]:
        for k in ("tflops_256_groups", "tflops_512_groups"):
            assert 0.05 * m["spec_tflops"] < m[k] < 1.1 * m["spec_tflops"], m
    assert 100.0 < res["copy"]["gbps"] < 1.1 * 8000.0
    d = res["lds_dma"]
    assert d["gbps_per_workgroup_alone"] > 1.0 and d["gbps_per_workgroup_256"] > 1.0
    assert res["lds_read"]["gbps_per_workgroup_256"] > 1.0
