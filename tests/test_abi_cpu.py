"""CPU-side checks of the C-ABI library (no GPU needed): the built library loads, exports every
entry point include/amk.h declares, its host quantizer is bit-exact against the oracle's, and
argument validation rejects bad calls before any HIP call is made."""
import ctypes
import json
import os
import re

import numpy as np
import pytest
import torch

import decode_megakernel_cooperative_amd as D
from decode_megakernel_cooperative_amd import amk as A
from oracle.quant import quantize_rows_int8
import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_library_exports_every_declared_symbol():
    header = open(os.path.join(ROOT, "include", "amk.h")).read()
    declared = sorted(set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+(amk_\w+)\s*\(", header, re.M)))
    assert len(declared) >= 10
    lib = ctypes.CDLL(A.LIB_PATH)
    for name in declared:
        assert hasattr(lib, name), name
    assert set(declared) == set(A.EXPORTED)


def _bits(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("rows,cols,std", [(96, 576, 0.02), (33, 4096, 0.02), (7, 1536, 0.5), (64, 2048, 3.0)])
def test_host_quantizer_bit_exact_vs_oracle(rows, cols, std):
    w = _bits(np.random.default_rng(rows * cols).standard_normal((rows, cols)) * std)
    c1, s1 = D.amk_quantize_int8(w)
    c2, s2 = quantize_rows_int8(w)
    assert np.array_equal(c1, c2)
    assert np.array_equal(s1.view(np.uint32), s2.view(np.uint32))


def test_host_quantizer_worked_rows():
    d = json.load(open(os.path.join(ROOT, "tests", "golden", "quant_tie_row.json")))
    for row in d["rows"]:
        c, s = D.amk_quantize_int8(_bits(np.array([row["w_float"]], np.float32)))
        assert c[0].tolist() == row["codes"], row["why"]
        assert s[0] == np.float32(row["scale"])


def test_host_quantizer_bf16_shapes_of_real_models():
    # every (rows, cols) shape a W8A16 model of the measured workloads quantizes, on a few rows
    for shape in (W.SMOLLM2_135M, W.LLAMA32_1B, W.LLAMA3_8B):
        for name, dims, kind in W.tensor_specs(shape)[:11]:
            if kind != "matrix":
                continue
            w = _bits(np.random.default_rng(dims[1]).standard_normal((8, dims[1])) * 0.02)
            c1, s1 = D.amk_quantize_int8(w)
            c2, s2 = quantize_rows_int8(w)
            assert np.array_equal(c1, c2) and np.array_equal(s1, s2), (shape.name, name)


def test_argument_validation_without_gpu():
    lib = A.lib()
    cfg = D.make_config(W.SMOLLM2_135M, 32, D.AMK_W8A16)
    h = ctypes.c_void_p()
    # wrong tensor count -> INVALID_ARG before any device work
    ptrs = (ctypes.c_void_p * 3)()
    assert lib.amk_load_weights(ctypes.byref(cfg), ptrs, 3, ctypes.byref(h)) == A.AMK_ERR_INVALID_ARG
    assert lib.amk_load_weights(None, ptrs, 3, ctypes.byref(h)) == A.AMK_ERR_INVALID_ARG
    # unsupported shapes -> UNSUPPORTED
    for field, value in (("head_dim", 96), ("n_kv_heads", 4), ("hidden", 580), ("weight_format", 7), ("vocab", 49153)):
        bad = D.make_config(W.SMOLLM2_135M, 32, D.AMK_W8A16)
        setattr(bad, field, value)
        st = lib.amk_load_weights(ctypes.byref(bad), ptrs, 3, ctypes.byref(h))
        assert st == A.AMK_ERR_UNSUPPORTED, (field, st, D.amk_status_string(st))
    # calls on a null handle
    assert lib.amk_decode_step(None, 0, 0, None, None, None) == A.AMK_ERR_INVALID_ARG
    assert lib.amk_sync(None, None) == A.AMK_ERR_INVALID_ARG
    assert lib.amk_kv_cache_bytes(None) == 0
    assert lib.amk_free(None) == A.AMK_OK
    assert lib.amk_set_spin_limit(None, 5) == A.AMK_ERR_INVALID_ARG
    assert lib.amk_set_trace(None, None, 0) == A.AMK_ERR_INVALID_ARG
    assert lib.amk_export_quantized(None, 1, None, None) == A.AMK_ERR_INVALID_ARG
    assert lib.amk_get_info(None, None) == A.AMK_ERR_INVALID_ARG
    fs = ctypes.c_float()
    assert lib.amk_bench_barrier(0, ctypes.byref(fs)) == A.AMK_ERR_INVALID_ARG
    assert lib.amk_quantize_int8(None, 1, 1, None, None) == A.AMK_ERR_INVALID_ARG
    assert "invalid argument" in D.amk_status_string(A.AMK_ERR_INVALID_ARG)


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(A, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(A, "_lib", None)
    with pytest.raises(FileNotFoundError):
        A.lib()
