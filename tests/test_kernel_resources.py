"""Register budgets of the hot kernels, from the compiler's resource remarks.

Scalar-register spills land in vector-register lanes (v_writelane /
v_readlane pairs with their wait states) and scratch spills in memory; in the
attention kernels either cost several percent of the kernel's time, so the
kernels that carry the block and its backward must compile without them.
Compile-only (device code for gfx950); no GPU needed."""
import importlib.util
import os
import shutil

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _build_module():
    spec = importlib.util.spec_from_file_location(
        "_dit_build_res", os.path.join(ROOT, "joint_audio_video_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


# (source, kernel name as the report prints it, largest scratch B/lane allowed)
HOT = [
    ("attn.hip", "dit::attn_bf16_kernel", 0),
    ("attn_fp8.hip", "dit::attn_fp8_kernel", 0),
    ("attn_bwd.hip", "dit::attn_bwd_dkdv_kernel", 0),
    ("attn_bwd.hip", "dit::attn_bwd_dq_kernel", 0),
    ("gemm.hip", "dit::gemm_bf16_kernel<0>", 0),
    ("gemm.hip", "dit::gemm_bf16_kernel<1>", 0),
    ("gemm.hip", "dit::gemm_bf16_kernel<2>", 0),
    ("gemm.hip", "dit::gemm_bf16_kernel<3>", 0),
    ("gemm.hip", "dit::gemm_fp8_kernel<0>", 0),
    ("gemm.hip", "dit::gemm_fp8_kernel<1>", 0),
    ("gemm.hip", "dit::gemm_fp8_kernel<2>", 0),
    ("adaln.hip", "dit::adaln_bwd_kernel<10>", 0),
    ("adaln.hip", "dit::adaln_kernel<unsigned short, 10, 2, false>", 0),
    ("rope.hip", "dit::rope_row_kernel<unsigned short, 128>", 0),
]


@pytest.fixture(scope="module")
def rows():
    mod = _build_module()
    if not os.path.exists(mod.HIPCC) and shutil.which("hipcc") is None:
        pytest.skip("hipcc not available")
    got = mod.resource_rows(sorted({src for src, _, _ in HOT}))
    return {(r["src"], r["name"]): r for r in got}


@pytest.mark.parametrize("src,name,scratch", HOT)
def test_hot_kernel_has_no_register_spills(rows, src, name, scratch):
    r = rows.get((src, name))
    assert r is not None, f"{name} not found in the compiler's remarks for {src}"
    assert int(r.get("SGPRs Spill", 0)) == 0, r
    assert int(r.get("ScratchSize [bytes/lane]", 0)) <= scratch, r
    # two waves per SIMD (attention) or one (the GEMMs) must still fit
    assert int(r.get("Occupancy [waves/SIMD]", 0)) >= 1, r
