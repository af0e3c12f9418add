"""The built library's kernels, from the metadata of its gfx950 code objects (no GPU needed):
every kernel instance keeps its data in registers and LDS (no scratch, no VGPR spills), and
the kernel families of every path are present."""

import os

import pytest

from row_wise_normalization_fp32_amd import kernel_resources as kr

pytestmark = pytest.mark.skipif(not os.path.exists(os.path.join(kr.LLVM_BIN, "llvm-readelf")),
                                reason="ROCm llvm tools not found")


@pytest.fixture(scope="module")
def kernels():
    return kr.kernels()


def test_every_kernel_runs_without_scratch(kernels):
    assert len(kernels) > 100
    bad = [(k["name"], k.get("private_segment_fixed_size"), k.get("vgpr_spill_count")) for k in kernels
           if k.get("private_segment_fixed_size", 0) != 0 or k.get("vgpr_spill_count", 0) != 0]
    assert not bad, bad


def test_every_path_is_built(kernels):
    names = {k["name"] for k in kernels}
    for fam in ("rownorm_vec_kernel", "rownorm_elem_kernel", "rownorm_pair_kernel", "rownorm_general_kernel",
                "rownorm_wide_stats_kernel", "rownorm_wide_norm_kernel", "rownorm_wide_elem_stats_kernel",
                "rownorm_wide_elem_norm_kernel", "rownorm_bwd_vec_kernel", "rownorm_bwd_elem_kernel",
                "rownorm_bwd_cols_kernel", "rownorm_bwd_wide_stats_kernel", "rownorm_bwd_wide_dx_kernel"):
        assert any(fam in n for n in names), fam


def test_workgroup_sizes_fit_the_register_file(kernels):
    # 1024-lane workgroups get at most 128 VGPRs per lane (16 waves on 4 SIMDs of 512)
    for k in kernels:
        if k.get("max_flat_workgroup_size", 0) >= 1024:
            assert k["vgpr_count"] + k.get("agpr_count", 0) <= 128, k
