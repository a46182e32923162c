"""Compiler-reported resources of every kernel in the HIP library: no kernel
spills registers to scratch memory (a spill inside a GEMM loop or epilogue
costs far more than the arithmetic around it)."""
import json
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
RES = os.path.join(ROOT, "bit_quantized_matmul_col_amd", "libllmint8.kernels.json")



@pytest.fixture(autouse=True)
def _library(built_library):
    return built_library


def test_every_kernel_reported():
    res = json.load(open(RES))
    names = " ".join(res)
    for k in ("k_gemm_prefill", "k_gemm_pair", "k_gemm_split", "k_decode_gemm", "k_decode_fused",
              "k_detect_partial", "k_layer_prep", "k_colquant", "k_quant_tensor"):
        assert k in names, k


def test_no_kernel_spills():
    res = json.load(open(RES))
    bad = {k: v for k, v in res.items()
           if v.get("ScratchSize", 0) or v.get("VGPRs Spill", 0) or v.get("SGPRs Spill", 0)}
    assert not bad, bad
