"""Resources of the compiled gfx950 kernels (CPU only: hipcc cross-compiles).

The GEMM kernels run one workgroup of four full-register waves per CU, so a
register spill puts scratch traffic next to the MFMA loop (measured at 5-15 %
of a kernel) and more than 160 KB of LDS would not launch at all.  This test
compiles kernels.hip with the library's flags and reads the code object's
metadata: the bf16 instances of the four hot kernels must not spill, and no
kernel may ask for more LDS than a CU has."""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest
import yaml

from grpo_policy_loss_amd import build as libbuild

LDS_PER_CU = 160 * 1024
# mangled-name fragments of the bf16 (DF16b) instances that must not spill
HOT = ("k_lse_partialsIDF16bLb0E", "k_lse_partialsIDF16bLb1E", "k_dzIDF16bLb0E", "k_dzIDF16bLb1E",
       "k_dh_gemmIDF16bE", "k_dw_gemmIDF16bE")


def _readelf():
    for cand in ("/opt/rocm/llvm/bin/llvm-readelf", shutil.which("llvm-readelf")):
        if cand and os.path.exists(cand):
            return cand
    return None


@pytest.fixture(scope="module")
def kernels(tmp_path_factory):
    try:
        hipcc = libbuild.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    readelf = _readelf()
    if readelf is None:
        pytest.skip("llvm-readelf not available")
    out = tmp_path_factory.mktemp("co") / "kernels.co"
    cmd = [hipcc, *libbuild.HIPCC_FLAGS, "--cuda-device-only", "--no-gpu-bundle-output", "-c",
           os.path.join(libbuild.CSRC, "kernels.hip"), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    notes = subprocess.run([readelf, "--notes", str(out)], capture_output=True, text=True,
                           timeout=120).stdout
    start = notes.index("---")
    end = notes.index("\n...", start)
    meta = yaml.safe_load(notes[start:end])
    assert meta["amdhsa.target"].endswith("gfx950")
    return {k[".name"]: k for k in meta["amdhsa.kernels"]}


def test_hot_bf16_kernels_do_not_spill(kernels):
    for frag in HOT:
        names = [n for n in kernels if frag in n]
        assert len(names) == 1, (frag, names)
        k = kernels[names[0]]
        assert k[".private_segment_fixed_size"] == 0, (frag, k[".private_segment_fixed_size"])
        assert k[".vgpr_spill_count"] == 0 and k[".sgpr_spill_count"] == 0, frag


def test_every_kernel_fits_the_lds_of_one_cu(kernels):
    for name, k in kernels.items():
        assert k[".group_segment_fixed_size"] <= LDS_PER_CU, (name, k[".group_segment_fixed_size"])


def test_gemm_kernels_run_four_waves(kernels):
    for frag in HOT:
        name = next(n for n in kernels if frag in n)
        assert kernels[name][".max_flat_workgroup_size"] == 256, name
