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
from oracle.quant import quantize_rows_int4, quantize_rows_int4_g128, quantize_rows_int8
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


@pytest.mark.parametrize("rows,cols,std", [(96, 576, 0.02), (33, 4096, 0.02), (7, 1536, 0.5), (64, 2048, 3.0)])
def test_host_int4_quantizer_bit_exact_vs_oracle(rows, cols, std):
    w = _bits(np.random.default_rng(rows * cols + 4).standard_normal((rows, cols)) * std)
    c1, s1 = D.amk_quantize_int4(w)
    c2, s2 = quantize_rows_int4(w)
    assert np.array_equal(c1, c2)
    assert np.array_equal(s1.view(np.uint32), s2.view(np.uint32))


def test_host_int4_quantizer_worked_rows():
    d = json.load(open(os.path.join(ROOT, "tests", "golden", "quant4_tie_row.json")))
    for row in d["rows"]:
        c, s = D.amk_quantize_int4(_bits(np.array([row["w_float"]], np.float32)))
        assert c[0].tolist() == row["codes"], row["why"]
        assert s[0] == np.float32(row["scale"])


@pytest.mark.parametrize("rows,cols,std", [(96, 576, 0.02), (33, 4096, 0.02), (7, 1536, 0.5), (64, 2080, 3.0),
                                           (5, 200, 1e-4), (3, 128, 2e5)])
def test_host_int4_g128_quantizer_bit_exact_vs_oracle(rows, cols, std):
    # includes a ragged last group (576, 2080, 200 columns), half-precision subnormal scales
    # (std 1e-4: amax / 7 below 2^-14) and saturated ones (std 2e5: amax / 7 above 65504)
    rng = np.random.default_rng(rows * cols + 5)
    w = rng.standard_normal((rows, cols)) * std
    w[0, :128] = 0.0  # an all-zero group
    w = _bits(w)
    c1, s1 = D.amk_quantize_int4_g128(w)
    c2, s2 = quantize_rows_int4_g128(w)
    assert s1.shape == (rows, (cols + 127) // 128)
    assert np.array_equal(c1, c2)
    assert np.array_equal(s1.view(np.uint32), s2.view(np.uint32))
    assert np.all(s1[0, 0] == 0) and np.all(c1[0, :128] == 0)
    if std == 1e-4:
        assert np.any((s1 > 0) & (s1 < 2.0 ** -14))
    if std == 2e5:
        assert np.any(s1 == np.float32(65504.0))


def test_host_int4_g128_quantizer_worked_rows():
    d = json.load(open(os.path.join(ROOT, "tests", "golden", "quant4g_tie_rows.json")))
    for row in d["rows"]:
        w = np.zeros(d["cols"], np.float32)
        for k, v in row["nonzero_float"].items():
            w[int(k)] = v
        c, s = D.amk_quantize_int4_g128(_bits(w[None]))
        want = np.zeros(d["cols"], np.int8)
        for k, v in row["codes_nonzero"].items():
            want[int(k)] = v
        assert np.array_equal(c[0], want), row["why"]
        assert np.array_equal(s[0], np.array(row["scales"], np.float32)), row["why"]


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
    # inconsistent Llama-3 RoPE scaling -> UNSUPPORTED
    bad = D.make_config(W.SMOLLM2_135M, 32, D.AMK_W8A16)
    bad.rope_scale_factor, bad.rope_low_freq_factor, bad.rope_high_freq_factor, bad.rope_original_ctx = 8.0, 4.0, 1.0, 8192
    assert lib.amk_load_weights(ctypes.byref(bad), ptrs, 3, ctypes.byref(h)) == A.AMK_ERR_UNSUPPORTED
    # calls on a null handle
    assert lib.amk_decode_step(None, 0, 0, None, None, None) == A.AMK_ERR_INVALID_ARG
    assert lib.amk_decode_step_greedy(None, None, 0, None, None, None, None) == A.AMK_ERR_INVALID_ARG
    assert lib.amk_sync(None, None) == A.AMK_ERR_INVALID_ARG
    assert lib.amk_kv_cache_bytes(None) == 0
    assert lib.amk_free(None) == A.AMK_OK
    assert lib.amk_set_spin_limit(None, 5) == A.AMK_ERR_INVALID_ARG
    assert lib.amk_set_trace(None, None, 0) == A.AMK_ERR_INVALID_ARG
    assert lib.amk_export_quantized(None, 1, None, None) == A.AMK_ERR_INVALID_ARG
    assert lib.amk_get_info(None, None) == A.AMK_ERR_INVALID_ARG
    assert lib.amk_set_dump(None, None, 0) == A.AMK_ERR_INVALID_ARG
    assert lib.amk_validate_config(None, 256) == A.AMK_ERR_INVALID_ARG
    assert lib.amk_validate_config(ctypes.byref(cfg), 0) == A.AMK_ERR_INVALID_ARG
    assert lib.amk_quantize_int8(None, 1, 1, None, None) == A.AMK_ERR_INVALID_ARG
    assert lib.amk_quantize_int4(None, 1, 1, None, None) == A.AMK_ERR_INVALID_ARG
    assert lib.amk_quantize_int4_g128(None, 1, 1, None, None) == A.AMK_ERR_INVALID_ARG
    # W4A16 rows must hold whole 16-byte lane loads: 32-column multiples
    for fmt in (D.AMK_W4A16, D.AMK_W4A16_G128):
        bad = D.make_config(W.SMOLLM2_135M, 32, fmt)
        bad.ffn = 1552
        assert lib.amk_load_weights(ctypes.byref(bad), ptrs, 3, ctypes.byref(h)) == A.AMK_ERR_UNSUPPORTED
    assert "invalid argument" in D.amk_status_string(A.AMK_ERR_INVALID_ARG)


def _cfg(shape, fmt=D.AMK_W8A16, max_ctx=64):
    return D.make_config(shape, max_ctx, fmt)


def _rejected(cfg, cus=256):
    st = A.lib().amk_validate_config(ctypes.byref(cfg), cus)
    return st == A.AMK_ERR_UNSUPPORTED, D.amk_status_string(st) if st else "ok"


def test_validate_config_measured_shapes_pass():
    """Every measured workload's model loads on a 256-CU device (MI355X) in its format."""
    for wl in W.WORKLOADS.values():
        D.amk_validate_config(_cfg(wl.shape, wl.weight_format, wl.max_ctx + 1), 256)


def test_validate_config_handoff_conditions():
    """The grid conditions the tagged hand-offs need (one row pair of the QKV and gate/up stages
    per block, one attention unit per kv head), checked on the host for a given CU count."""
    # two layers whose QKV stage has 128 row pairs: blocks 128..255 would own none
    small = W.ModelShape("l2-small-qkv", 256, 2, 2, 1, 64, 512, 512, True, 10000.0)
    bad, why = _rejected(_cfg(small))
    assert bad and "compute units" in why, why
    # the same stage is fine on a 128-CU device, and with one layer (no later stage rewrites x)
    D.amk_validate_config(_cfg(small), 128)
    D.amk_validate_config(_cfg(W.ModelShape("l1-small-qkv", 256, 1, 2, 1, 64, 512, 512, True, 10000.0)), 256)
    # gate/up with fewer row pairs than blocks
    bad, why = _rejected(_cfg(W.ModelShape("small-ffn", 512, 2, 8, 2, 64, 240, 512, True, 10000.0)))
    assert bad and "ffn" in why, why
    # more kv heads than blocks (one attention unit per block)
    assert _rejected(_cfg(W.ModelShape("kv-heavy", 4096, 1, 64, 64, 64, 4096, 512, True, 10000.0)), 32)[0]


def test_validate_config_rejects_matrices_of_2gib():
    """The kernel addresses each matrix, the embedding and each KV block with 32-bit offsets."""
    big = W.ModelShape("wide-vocab", 8192, 2, 64, 8, 128, 28672, 131072, False, 500000.0)
    for fmt in (D.AMK_BF16, D.AMK_W8A16_BF16_HEAD, D.AMK_W8A16):  # bf16 head / bf16 embedding: 2^31 bytes
        bad, why = _rejected(_cfg(big, fmt))
        assert bad and "2^31" in why, (fmt, why)
    ok = W.ModelShape("wide-ok", 8192, 2, 64, 8, 128, 28672, 131070, False, 500000.0)
    D.amk_validate_config(_cfg(ok, D.AMK_W8A16), 256)
    # a (layer, K/V, kv head) cache block of 2^31 bytes
    bad, why = _rejected(_cfg(W.LLAMA3_8B, D.AMK_W8A16, max_ctx=1 << 23))
    assert bad and "2^31" in why, why
    D.amk_validate_config(_cfg(W.LLAMA3_8B, D.AMK_W8A16, max_ctx=(1 << 23) - 1), 256)


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(A, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(A, "_lib", None)
    with pytest.raises(FileNotFoundError):
        A.lib()


def test_trace_summary_layout():
    """The trace summary reads the kernel's event layout: entry, 11 events per layer, final
    RMSNorm, lm_head end. A synthetic trace with known per-stage durations comes back exact."""
    from decode_megakernel_cooperative_amd import trace as T
    L, nb = 3, 4
    dur_ticks = np.arange(1, 12) * 10  # stage k takes 10 (k + 1) ticks in every block and layer
    t = np.zeros((nb, T.events_per_block(L)), dtype=np.int64)
    for b in range(nb):
        now = 1000 * b
        t[b, 0] = now
        for l in range(L):
            for k in range(11):
                now += int(dur_ticks[k]) + b  # block b is b ticks slower per stage
                t[b, 1 + 11 * l + k] = now
        t[b, 1 + 11 * L] = now + 5
        t[b, 2 + 11 * L] = now + 5 + 700
    s = T.summarize(t, L)
    for k, name in enumerate(T.STAGES):
        assert s[name]["mean_us"] == pytest.approx((dur_ticks[k] + 1.5) * 0.01)
        assert s[name]["max_over_blocks_us"] == pytest.approx((dur_ticks[k] + 3) * 0.01)
    assert s["lm_head_us"] == pytest.approx(7.0)
    assert s["layer_us"] == pytest.approx(sum(dur_ticks + 1.5) * 0.01)


def test_bench_traffic_record_tracks_kernel_sources(tmp_path):
    """bench.py reports counter-measured HBM traffic only while the kernel sources are the ones the
    counters were taken on."""
    import bench
    rec = {"workload": "w", "bytes_per_launch": 123456, "kernel_sha256": bench.kernel_source_hash()}
    (tmp_path / "decode_w_hbm_traffic.md").write_text("notes\ntraffic-record: " + json.dumps(rec) + "\n")
    assert bench.counter_traffic("w", profiles=str(tmp_path)) == 123456
    rec["kernel_sha256"] = "0" * 64
    (tmp_path / "decode_w_hbm_traffic.md").write_text("traffic-record: " + json.dumps(rec) + "\n")
    assert bench.counter_traffic("w", profiles=str(tmp_path)) is None
    assert bench.counter_traffic("missing", profiles=str(tmp_path)) is None
