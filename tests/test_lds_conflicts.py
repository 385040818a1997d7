"""The LDS layout on the hardware: zero bank conflicts in the product kernel.

The pages ask for the bank-conflict counter to be read on the kernel itself,
not only reasoned about ("Memory-bank mechanism and accelerated compute",
section on turning derivations into measurements).  Each case runs a short
bench.py as a child process under ``rocprofv3 --pmc SQ_LDS_BANK_CONFLICT``
(bench_profile.lds_conflicts) and requires the counter to read 0 on every
dispatch of the product kernel, for each workload's tile: the 16-row-block A
layout and the XOR-8 swizzled B layout of the direct-to-LDS kernel, and the
zeroing of A words past K (ragged: K = 777 ends inside a 16-byte group), must
stay conflict-free.
"""
from __future__ import annotations

import os
import shutil
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


@pytest.mark.parametrize("workload,plan", [("4096cube", "mfma_lds_256x256x32_vavb"),
                                           ("8192cube", "mfma_lds_256x256x32_vavb"),
                                           ("ragged", "mfma_lds_32x64x32_ks2_savb"),
                                           ("skinny", "mfma_lds_128x128x32_vavb"),
                                           ("256cube", "mfma_lds_32x64x64_ks4_vavb")])
def test_product_kernel_has_no_lds_bank_conflicts(workload, plan, tmp_path):
    if shutil.which("rocprofv3") is None:
        pytest.skip("rocprofv3 is not installed")
    import bench_profile
    print(f"[gpu] rocprofv3 --pmc SQ_LDS_BANK_CONFLICT over bench.py --workload {workload}",
          flush=True)
    got_plan, values = bench_profile.lds_conflicts(workload, str(tmp_path))
    assert got_plan == plan
    assert values, "no dispatch of the product kernel was counted"
    assert all(v == 0 for v in values), values
