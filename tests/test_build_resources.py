"""Build check (no GPU): the compiler's kernel-resource report, recorded by the build,
shows no kernel spilling registers or using scratch memory. Spills turn the hot kernels'
register-resident tiles into memory traffic (a prefill attention kernel at 28 spilled
VGPRs ran twice as slow), so they are caught here rather than in a timing."""
import json
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
RES = os.path.join(ROOT, "looped_ngpt_transformer_amd", "_build", "kernel_resources.json")


def resources():
    with open(RES) as f:
        return json.load(f)


def test_every_kernel_reported():
    r = resources()
    names = " ".join(r)
    for k in ("k_gemm_pp", "k_gemm_pipe", "k_gemm_mx32", "k_attn_prefill", "k_attn_decode",
              "k_decode_merge", "k_update", "k_rope_tile", "k_rope_kv", "k_swiglu"):
        assert k in names, k


def test_no_register_spills():
    for name, v in resources().items():
        assert v.get("vgpr_spill", 0) == 0 and v.get("sgpr_spill", 0) == 0, (name, v)
        assert v.get("scratch", 0) == 0, (name, v)


def test_hot_kernels_occupancy():
    """Two waves per SIMD for the 8-wave prefill kernels (their schedules pair the waves
    of a SIMD), and at least two for the update."""
    for name, v in resources().items():
        if "k_gemm_pp" in name or "k_attn_prefill" in name or "k_update" in name:
            assert v.get("occupancy", 0) >= 2, (name, v)
