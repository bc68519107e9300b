"""Pins for the CPU oracle: each test ties one part of the oracle to something other than
itself — a closed form, an invariant, brute force, a library routine, or a hand-derived case
stored under tests/golden/. Chosen so a dropped term, a wrong sign or index, or a transposed
operand anywhere in the oracle fails at least one of them.

Whole-model logits at the real shapes have no external pin (no checkpoint or printed logits
exist on the pages): they are pinned only through these parts ("parity unpinned" for the
composed model at full size).
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import llama as L
from oracle.numerics import bf16_bits_to_f32, f32_to_bf16_bits, round_bf16
from oracle.quant import (dequantize_groups, quantize_rows_int4_g128, quantize_rows_int4_g128_f32)
from oracle.quant import (dequantize_rows, quantize_rows_int4, quantize_rows_int4_f32, quantize_rows_int8,
                          quantize_rows_int8_f32)
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
F32 = np.float32


def to_bits(a) -> np.ndarray:
    """float array -> bf16 patterns via torch's own conversion (independent of the oracle)."""
    t = torch.as_tensor(np.asarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def rng_bf16(shape, std, seed):
    g = np.random.default_rng(seed)
    return to_bits(g.standard_normal(shape).astype(np.float32) * std)


# ------------------------------------------------------------------------------------------
# bf16 conversions: against torch's conversion (library routine), incl. ties, inf, nan
# ------------------------------------------------------------------------------------------
def test_bf16_round_matches_torch():
    g = np.random.default_rng(0)
    x = np.concatenate([
        g.standard_normal(100000).astype(np.float32) * np.float32(10.0) ** g.integers(-30, 30, 100000),
        np.array([0.0, -0.0, np.inf, -np.inf, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 3.0e38, -3.4e38], np.float32),
    ]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(f32_to_bf16_bits(x), ref)
    # ties to even: 1 + 2^-8 lies halfway between 1 and 1 + 2^-7 -> 1 (even); 1 + 3*2^-8 -> 1 + 2^-6
    assert round_bf16(np.float32(1 + 2 ** -8)) == 1.0
    assert round_bf16(np.float32(1 + 3 * 2 ** -8)) == np.float32(1 + 2 ** -6)
    assert np.isnan(round_bf16(np.array([np.nan], np.float32)))[0]
    # widening is exact
    b = g.integers(0, 0x7F80, 1000).astype(np.uint16)
    assert np.array_equal(f32_to_bf16_bits(bf16_bits_to_f32(b)), b)


# ------------------------------------------------------------------------------------------
# C1 GEMV: brute force in float64 double loops on tiny non-square shapes
# ------------------------------------------------------------------------------------------
@pytest.mark.parametrize("rows,cols", [(5, 300), (3, 128)])
def test_gemv_brute_force_groups(rows, cols):
    """Group-wise int4: y_n = sum_k q_nk s_n,g(k) x_k, by float64 double loops over the codes and
    the fp16 group scales (groups of 128 columns; 300 columns end with a 44-column group)."""
    wb = rng_bf16((rows, cols), 0.5, rows * cols + 9)
    x = round_bf16(np.random.default_rng(2).standard_normal(cols).astype(np.float32))
    lin = L.Linear(wb, L.FMT_W4A16_G128, widen_once=False)
    y = lin.apply(x)
    assert lin.gscales.shape == (rows, (cols + 127) // 128)
    for r in range(rows):
        terms = [float(lin.codes[r, c]) * float(lin.gscales[r, c // 128]) * float(x[c]) for c in range(cols)]
        exact, absum = sum(terms), sum(abs(t) for t in terms)
        assert abs(float(y[r]) - exact) <= cols * 2.0 ** -24 * absum + 1e-30, r


@pytest.mark.parametrize("rows,cols", [(7, 13), (5, 64), (16, 33)])
@pytest.mark.parametrize("fmt", [L.FMT_BF16, L.FMT_W8A16, L.FMT_W4A16])
def test_gemv_brute_force(rows, cols, fmt):
    wb = rng_bf16((rows, cols), 0.5, rows * cols + fmt)
    x = round_bf16(np.random.default_rng(1).standard_normal(cols).astype(np.float32))
    lin = L.Linear(wb, fmt, widen_once=False)
    y = lin.apply(x)
    assert y.shape == (rows,)
    w = bf16_bits_to_f32(wb).astype(np.float64)
    if fmt != L.FMT_BF16:
        codes, scales = lin.codes.astype(np.float64), lin.scales.astype(np.float64)
        assert np.max(np.abs(codes)) == (127 if fmt == L.FMT_W8A16 else 7)
    for r in range(rows):
        terms = [(codes[r, c] if fmt else w[r, c]) * float(x[c]) for c in range(cols)]
        exact = sum(terms)
        absum = sum(abs(t) for t in terms)
        if fmt != L.FMT_BF16:
            exact *= scales[r]
            absum *= scales[r]
        bound = (cols + 1) * 2.0 ** -24 * absum + 1e-30
        assert abs(float(y[r]) - exact) <= bound, (r, float(y[r]), exact, bound)
    # batched application (used by the full-sequence forward) agrees row by row
    X = np.stack([x, -x, 2 * x]).astype(np.float32)
    Y = lin.apply(X)
    assert np.allclose(Y[0], y, rtol=1e-6, atol=1e-6) and np.allclose(Y[2], 2 * y, rtol=1e-6, atol=1e-6)


# ------------------------------------------------------------------------------------------
# C2 RMSNorm: closed forms and scale invariance
# ------------------------------------------------------------------------------------------
def test_rmsnorm_closed_form():
    x = np.array([3.0, 4.0], np.float32)
    y = L.rmsnorm(x, np.ones(2, np.float32), 0.0)
    assert np.allclose(y, [3 / math.sqrt(12.5), 4 / math.sqrt(12.5)], rtol=2e-7)
    g = np.random.default_rng(3)
    for H in (4, 576, 4096):
        x = g.standard_normal(H).astype(np.float32) * 0.3
        eps = 1e-5
        y = L.rmsnorm(x, np.ones(H, np.float32), eps)
        ms = float(np.mean(x.astype(np.float64) ** 2))
        assert abs(math.sqrt(np.mean(y.astype(np.float64) ** 2)) - math.sqrt(ms / (ms + eps))) < 1e-5
        y4 = L.rmsnorm(np.float32(4.0) * x, np.ones(H, np.float32), eps)
        assert np.allclose(y, y4, rtol=1e-4, atol=1e-6)
        w = g.standard_normal(H).astype(np.float32)
        assert np.allclose(L.rmsnorm(x, w, eps), y * w, rtol=1e-6, atol=1e-7)


# ------------------------------------------------------------------------------------------
# C3 RoPE: identity at 0, norm preservation, relative position, composition, hand value
# ------------------------------------------------------------------------------------------
def test_rope_properties():
    g = np.random.default_rng(4)
    for hd, theta in ((64, 1e4), (128, 5e5)):
        v = g.standard_normal(hd).astype(np.float32)
        c0, s0 = L.rope_tables([0], hd, theta)
        assert np.array_equal(L.apply_rope(v, c0[0], s0[0]), v)  # bit-exact identity at position 0
        for p in (1, 7, 4096, 32800):
            c, s = L.rope_tables([p], hd, theta)
            r = L.apply_rope(v, c[0], s[0])
            assert abs(np.linalg.norm(r.astype(np.float64)) / np.linalg.norm(v.astype(np.float64)) - 1) < 2e-6
        q = g.standard_normal(hd).astype(np.float32)
        k = g.standard_normal(hd).astype(np.float32)
        def rot(x, p):
            c, s = L.rope_tables([p], hd, theta)
            return L.apply_rope(x, c[0], s[0]).astype(np.float64)
        for (p1, p2, d) in ((5, 2, 11), (100, 37, 1000)):
            a = rot(q, p1) @ rot(k, p2)
            b = rot(q, p1 + d) @ rot(k, p2 + d)
            assert abs(a - b) < 1e-4 * (1 + abs(a))
        assert np.allclose(rot(rot(q, 3).astype(np.float32), 9), rot(q, 12), atol=1e-5)


def test_rope_hand_values():
    # hd = 4: pairs (0, 2) and (1, 3); inv_freq = (1, theta^-1/2); rotate-half convention
    theta = 1e4
    c, s = L.rope_tables([1], 4, theta)
    e = np.eye(4, dtype=np.float32)
    r0 = L.apply_rope(e[0], c[0], s[0])
    assert np.allclose(r0, [math.cos(1), 0, math.sin(1), 0], atol=1e-7)
    r2 = L.apply_rope(e[2], c[0], s[0])
    assert np.allclose(r2, [-math.sin(1), 0, math.cos(1), 0], atol=1e-7)
    r1 = L.apply_rope(e[1], c[0], s[0])
    f = theta ** -0.5
    assert np.allclose(r1, [0, math.cos(f), 0, math.sin(f)], atol=1e-7)


# ------------------------------------------------------------------------------------------
# C4 softmax / attention head
# ------------------------------------------------------------------------------------------
def test_attention_softmax_properties():
    g = np.random.default_rng(5)
    hd = 16
    sc = np.float32(1 / 4)
    v = round_bf16(g.standard_normal((1, hd)).astype(np.float32))
    k = round_bf16(g.standard_normal((1, hd)).astype(np.float32))
    q = g.standard_normal(hd).astype(np.float32)
    assert np.array_equal(L.attention_head(q, k, v, sc), v[0])  # one key: weight exactly 1
    # weights sum to 1: with V = I the output is the weight vector
    T = hd
    K = g.standard_normal((T, hd)).astype(np.float32)
    a = L.attention_head(q, K, np.eye(T, dtype=np.float32), sc)
    assert abs(float(np.sum(a, dtype=np.float64)) - 1) < 1e-6 and np.all(a > 0)
    # ordering follows the scores
    s = (K.astype(np.float64) @ q) * 0.25
    assert np.array_equal(np.argsort(a), np.argsort(s))
    # identical keys -> mean of V
    V = g.standard_normal((T, hd)).astype(np.float32)
    o = L.attention_head(q, np.repeat(K[:1], T, axis=0), V, sc)
    assert np.allclose(o, V.astype(np.float64).mean(0), atol=1e-6)
    # two keys with scores s0, 0 -> sigmoid weights (closed form)
    K2 = np.zeros((2, hd), np.float32); K2[0, 0] = 1.0
    q2 = np.zeros(hd, np.float32); q2[0] = 3.0
    o2 = L.attention_head(q2, K2, np.eye(2, hd, dtype=np.float32), np.float32(0.5))
    w0 = 1 / (1 + math.exp(-1.5))
    assert np.allclose(o2[:2], [w0, 1 - w0], atol=1e-7)


def test_silu_values():
    assert L.silu(np.float32(0.0)) == 0.0
    assert abs(float(L.silu(np.float32(2.0))) - 2 / (1 + math.exp(-2))) < 1e-6
    assert abs(float(L.silu(np.float32(-3.0))) - (-3 / (1 + math.exp(3)))) < 1e-7
    assert float(L.silu(np.float32(30.0))) == pytest.approx(30.0, rel=1e-7)


# ------------------------------------------------------------------------------------------
# C6 quantizer
# ------------------------------------------------------------------------------------------
def test_quantizer_worked_rows():
    d = json.load(open(os.path.join(GOLDEN, "quant_tie_row.json")))
    for row in d["rows"]:
        wb = to_bits(np.array([row["w_float"]], np.float32))
        assert np.array_equal(bf16_bits_to_f32(wb)[0], np.array(row["w_float"], np.float32))  # exact in bf16
        codes, scales = quantize_rows_int8(wb)
        assert codes[0].tolist() == row["codes"], row["why"]
        assert scales[0] == np.float32(row["scale"])


def test_quantizer_invariants_and_round_trip():
    g = np.random.default_rng(6)
    for cols in (576, 2048, 4096):
        wb = rng_bf16((256, cols), 0.02, cols)
        codes, s = quantize_rows_int8(wb)
        w = bf16_bits_to_f32(wb)
        assert np.all(np.max(np.abs(codes.astype(np.int32)), axis=1) == 127)
        assert codes.min() >= -127
        err = np.abs(w - dequantize_rows(codes, s))
        assert np.all(err <= s[:, None] * (0.5 + 1e-5))
        # round trip: quantizing the dequantized fp32 weights returns the same codes and scales
        wd = dequantize_rows(codes, s)
        c2, s2 = quantize_rows_int8_f32(wd)
        assert np.array_equal(c2, codes) and np.array_equal(s2, s)
    # block boundaries do not matter
    wb = rng_bf16((37, 64), 0.02, 9)
    a = quantize_rows_int8(wb, block_rows=5)
    b = quantize_rows_int8(wb, block_rows=4096)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_int4_quantizer_worked_rows():
    d = json.load(open(os.path.join(GOLDEN, "quant4_tie_row.json")))
    for row in d["rows"]:
        wb = to_bits(np.array([row["w_float"]], np.float32))
        assert np.array_equal(bf16_bits_to_f32(wb)[0], np.array(row["w_float"], np.float32))  # exact in bf16
        codes, scales = quantize_rows_int4(wb)
        assert codes[0].tolist() == row["codes"], row["why"]
        assert scales[0] == np.float32(row["scale"])


def test_int4_quantizer_invariants_and_round_trip():
    for cols in (576, 2048, 4096):
        wb = rng_bf16((256, cols), 0.02, cols + 1)
        codes, s = quantize_rows_int4(wb)
        w = bf16_bits_to_f32(wb)
        assert np.all(np.max(np.abs(codes.astype(np.int32)), axis=1) == 7)
        assert codes.min() >= -7 and codes.max() <= 7
        assert np.all(np.abs(w - dequantize_rows(codes, s)) <= s[:, None] * (0.5 + 1e-5))
        c2, s2 = quantize_rows_int4_f32(dequantize_rows(codes, s))
        assert np.array_equal(c2, codes) and np.array_equal(s2, s)
        # the int8 and int4 rules differ only in the code range: 127 / 7 of the int4 scale is
        # the int8 scale up to one rounding
        c8, s8 = quantize_rows_int8(wb)
        assert np.allclose(s8 * np.float32(127 / 7), s, rtol=3e-7)


def test_int4_g128_quantizer_worked_rows():
    d = json.load(open(os.path.join(GOLDEN, "quant4g_tie_rows.json")))
    for row in d["rows"]:
        w = np.zeros(d["cols"], np.float32)
        for k, v in row["nonzero_float"].items():
            w[int(k)] = v
        wb = to_bits(w[None])
        assert np.array_equal(bf16_bits_to_f32(wb)[0], w)  # exact in bf16
        codes, scales = quantize_rows_int4_g128(wb)
        want = np.zeros(d["cols"], np.int8)
        for k, v in row["codes_nonzero"].items():
            want[int(k)] = v
        assert np.array_equal(codes[0], want), row["why"]
        assert np.array_equal(scales[0], np.array(row["scales"], np.float32)), row["why"]


def test_int4_g128_invariants_and_round_trip():
    for cols in (576, 2048, 4160):
        wb = rng_bf16((96, cols), 0.02, cols + 3)
        codes, s = quantize_rows_int4_g128(wb)
        w = bf16_bits_to_f32(wb)
        ng = (cols + 127) // 128
        assert s.shape == (96, ng)
        assert np.array_equal(s.astype(np.float16).astype(np.float32), s)  # fp16 values
        assert codes.min() >= -7 and codes.max() <= 7
        for g in range(ng):  # every nonzero group uses the full code range
            assert np.all(np.max(np.abs(codes[:, g * 128:(g + 1) * 128].astype(np.int32)), axis=1) == 7)
        sf = np.repeat(s, 128, axis=1)[:, :cols]
        assert np.all(np.abs(w - dequantize_groups(codes, s)) <= sf * (0.5 + 1e-5))
        c2, s2 = quantize_rows_int4_g128_f32(dequantize_groups(codes, s))
        assert np.array_equal(c2, codes) and np.array_equal(s2, s)
        # group scales track the local magnitude: a row whose first group is 64x larger keeps its
        # other groups' codes, while a per-row scale flattens them
        big = w.copy()
        big[:, :128] *= 64
        cb, sb = quantize_rows_int4_g128(to_bits(big))
        assert np.array_equal(cb[:, 128:], codes[:, 128:])
        cr, _ = quantize_rows_int4(to_bits(big))
        assert np.mean(cr[:, 128:] == 0) > 0.9


# ------------------------------------------------------------------------------------------
# small-model helpers
# ------------------------------------------------------------------------------------------
def random_model_tensors(shape, seed=0, std=0.02):
    out = []
    for i, (name, dims, kind) in enumerate(W.tensor_specs(shape)):
        if kind == "norm":
            out.append(to_bits(np.ones(dims, np.float32)))
        else:
            out.append(rng_bf16(dims, std, seed * 1000 + i))
    return out


def fresh_kv(shape, max_ctx):
    return np.zeros(W.kv_cache_shape(shape, max_ctx), dtype=np.uint16)


# ------------------------------------------------------------------------------------------
# C5 GQA == MHA on repeat_kv-expanded K/V
# ------------------------------------------------------------------------------------------
def test_gqa_equals_expanded_mha():
    gqa = W.small_shape(hidden=64, n_layers=2, n_q_heads=4, n_kv_heads=2, head_dim=16, ffn=96, vocab=128)
    mha = W.small_shape(hidden=64, n_layers=2, n_q_heads=4, n_kv_heads=4, head_dim=16, ffn=96, vocab=128)
    t = random_model_tensors(gqa, seed=11, std=0.2)
    te = list(t)
    G = 2
    for l in range(gqa.n_layers):
        for off in (2, 3):  # k_proj, v_proj
            idx = 1 + 9 * l + off
            w = t[idx].reshape(gqa.n_kv_heads, gqa.head_dim, gqa.hidden)
            te[idx] = np.repeat(w, G, axis=0).reshape(mha.kv_dim, mha.hidden)  # kv head g -> q heads gG..gG+G-1
    a = L.OracleModel(gqa, t, L.FMT_BF16)
    b = L.OracleModel(mha, te, L.FMT_BF16)
    kva, kvb = fresh_kv(gqa, 8), fresh_kv(mha, 8)
    for pos, tok in enumerate([3, 70, 5, 127, 0]):
        la = a.decode_step(tok, pos, kva)
        lb = b.decode_step(tok, pos, kvb)
        assert np.allclose(la, lb, rtol=1e-5, atol=1e-6)
    # and a wrong head mapping (h % n_kv) is distinguishable: swap the two kv heads' K rows
    tw = list(t)
    for l in range(gqa.n_layers):
        idx = 1 + 9 * l + 2
        w = t[idx].reshape(2, gqa.head_dim, gqa.hidden)
        tw[idx] = w[::-1].reshape(gqa.kv_dim, gqa.hidden).copy()
    c = L.OracleModel(gqa, tw, L.FMT_BF16)
    kvc, kva = fresh_kv(gqa, 8), fresh_kv(gqa, 8)
    for pos, tok in enumerate([3, 70, 5]):
        la = a.decode_step(tok, pos, kva)
        lc = c.decode_step(tok, pos, kvc)
    assert not np.allclose(la, lc, atol=1e-4)


# ------------------------------------------------------------------------------------------
# C7 cross-format: k * 2^-m weights with max |k| = 127 quantize exactly
# ------------------------------------------------------------------------------------------
def test_cross_format_exact_codes():
    shape = W.small_shape(hidden=64, n_layers=2, n_q_heads=2, n_kv_heads=1, head_dim=32, ffn=128, vocab=96)
    g = np.random.default_rng(7)
    tensors = []
    for name, dims, kind in W.tensor_specs(shape):
        if kind == "norm":
            tensors.append(to_bits(np.ones(dims, np.float32)))
            continue
        k = g.integers(-127, 128, dims)
        k[:, 0] = np.where(g.random(dims[0]) < 0.5, 127, -127)
        tensors.append(to_bits(k.astype(np.float32) * np.float32(2.0 ** -9)))
    a = L.OracleModel(shape, tensors, L.FMT_BF16)
    b = L.OracleModel(shape, tensors, L.FMT_W8A16)
    lin = b.layers[0]["q"]
    assert np.all(lin.scales == np.float32(2.0 ** -9))
    assert np.array_equal(lin.codes.astype(np.float32) * np.float32(2.0 ** -9), bf16_bits_to_f32(tensors[2]))
    kva, kvb = fresh_kv(shape, 4), fresh_kv(shape, 4)
    for pos, tok in enumerate([1, 50, 95]):
        la = a.decode_step(tok, pos, kva)
        lb = b.decode_step(tok, pos, kvb)
        assert np.allclose(la, lb, rtol=1e-5, atol=1e-5)


def test_int4_exact_codes_match_bf16_model():
    """Projections of k * 2^-9 with |k| <= 7 and one |k| = 7 per row are exact int4 codes with
    s = 2^-9, so the W4A16 model equals the bf16 model on the same tensors to rounding. The
    lm_head stays bf16 under W4A16 (its rows here are ordinary random values)."""
    shape = W.small_shape(hidden=64, n_layers=2, n_q_heads=2, n_kv_heads=1, head_dim=32, ffn=128, vocab=96,
                          tied=False)
    g = np.random.default_rng(17)
    tensors = []
    for i, (name, dims, kind) in enumerate(W.tensor_specs(shape)):
        if kind == "norm":
            tensors.append(to_bits(np.ones(dims, np.float32)))
        elif i == len(W.tensor_specs(shape)) - 1 or i == 0:  # lm_head, embedding: plain bf16
            tensors.append(rng_bf16(dims, 0.05, 170 + i))
        else:
            k = g.integers(-7, 8, dims)
            k[:, 0] = np.where(g.random(dims[0]) < 0.5, 7, -7)
            tensors.append(to_bits(k.astype(np.float32) * np.float32(2.0 ** -9)))
    a = L.OracleModel(shape, tensors, L.FMT_BF16)
    b = L.OracleModel(shape, tensors, L.FMT_W4A16)
    lin = b.layers[1]["gate"]
    assert lin.fmt == L.FMT_W4A16 and b.lm_head.fmt == L.FMT_BF16
    assert np.all(lin.scales == np.float32(2.0 ** -9))
    assert np.array_equal(lin.codes.astype(np.float32) * np.float32(2.0 ** -9), bf16_bits_to_f32(tensors[1 + 9 + 6]))
    kva, kvb = fresh_kv(shape, 4), fresh_kv(shape, 4)
    for pos, tok in enumerate([1, 50, 95]):
        la = a.decode_step(tok, pos, kva)
        lb = b.decode_step(tok, pos, kvb)
        assert np.allclose(la, lb, rtol=1e-5, atol=1e-5)
    # on ordinary random weights int4 is lossy: the logits move well beyond rounding
    t = random_model_tensors(shape, seed=18, std=0.05)
    a, b = L.OracleModel(shape, t, L.FMT_BF16), L.OracleModel(shape, t, L.FMT_W4A16)
    kva, kvb = fresh_kv(shape, 4), fresh_kv(shape, 4)
    assert np.max(np.abs(a.decode_step(3, 0, kva) - b.decode_step(3, 0, kvb))) > 1e-2


def test_int4_g128_exact_codes_match_bf16_model():
    """Projections whose every group of 128 columns is k * 2^-m (|k| <= 7, one |k| = 7 in the
    group, m varying by group) are exact group-wise int4 codes with s = 2^-m per group, so the
    W4A16-G128 model equals the bf16 model on the same tensors to rounding; a per-row int4 scale
    cannot represent them."""
    shape = W.small_shape(hidden=256, n_layers=2, n_q_heads=2, n_kv_heads=1, head_dim=64, ffn=384, vocab=96,
                          tied=False)
    g = np.random.default_rng(19)
    tensors = []
    for i, (name, dims, kind) in enumerate(W.tensor_specs(shape)):
        if kind == "norm":
            tensors.append(to_bits(np.ones(dims, np.float32)))
        elif i == len(W.tensor_specs(shape)) - 1 or i == 0:
            tensors.append(rng_bf16(dims, 0.05, 190 + i))
        else:
            k = g.integers(-7, 8, dims).astype(np.float32)
            e = np.repeat(-(7 + g.integers(0, 5, (dims[0], (dims[1] + 127) // 128))), 128, axis=1)[:, :dims[1]]
            k[:, ::128] = np.where(g.random(k[:, ::128].shape) < 0.5, 7, -7)
            tensors.append(to_bits(k * np.exp2(e).astype(np.float32)))
    a = L.OracleModel(shape, tensors, L.FMT_BF16)
    b = L.OracleModel(shape, tensors, L.FMT_W4A16_G128)
    c = L.OracleModel(shape, tensors, L.FMT_W4A16)
    lin = b.layers[1]["gate"]
    assert lin.fmt == L.FMT_W4A16_G128 and b.lm_head.fmt == L.FMT_BF16
    assert np.array_equal(dequantize_groups(lin.codes, lin.gscales), bf16_bits_to_f32(tensors[1 + 9 + 6]))
    kva, kvb, kvc = fresh_kv(shape, 4), fresh_kv(shape, 4), fresh_kv(shape, 4)
    worst_rowwise = 0.0
    for pos, tok in enumerate([1, 50, 95]):
        la, lb, lc = a.decode_step(tok, pos, kva), b.decode_step(tok, pos, kvb), c.decode_step(tok, pos, kvc)
        assert np.allclose(la, lb, rtol=1e-5, atol=1e-5)
        worst_rowwise = max(worst_rowwise, float(np.max(np.abs(la - lc))))
    assert worst_rowwise > 1e-3


def test_bf16_head_format_differs_only_in_the_head():
    """W8A16 with a bf16 lm_head: random (not exactly quantizable) projections, an lm_head of
    k * 2^-9 rows that int8 represents exactly. Only the head differs between the two formats and
    it computes the same products, so the logits agree to rounding; a bf16-projection model
    (which keeps the projections unquantized) does not."""
    shape = W.small_shape(hidden=64, n_layers=2, n_q_heads=2, n_kv_heads=1, head_dim=32, ffn=128, vocab=96,
                          tied=False)
    t = random_model_tensors(shape, seed=61, std=0.05)
    g = np.random.default_rng(61)
    k = g.integers(-127, 128, (shape.vocab, shape.hidden))
    k[:, 0] = np.where(g.random(shape.vocab) < 0.5, 127, -127)
    t[-1] = to_bits(k.astype(np.float32) * np.float32(2.0 ** -9))
    a = L.OracleModel(shape, t, L.FMT_W8A16)
    b = L.OracleModel(shape, t, L.FMT_W8A16_BF16_HEAD)
    c = L.OracleModel(shape, t, L.FMT_BF16)
    assert b.lm_head.fmt == L.FMT_BF16 and b.layers[1]["down"].fmt == L.FMT_W8A16
    kva, kvb, kvc = fresh_kv(shape, 4), fresh_kv(shape, 4), fresh_kv(shape, 4)
    for pos, tok in enumerate([3, 70, 11]):
        la, lb, lc = a.decode_step(tok, pos, kva), b.decode_step(tok, pos, kvb), c.decode_step(tok, pos, kvc)
        assert np.allclose(la, lb, rtol=1e-5, atol=1e-5)
        assert np.max(np.abs(lb - lc)) > 1e-3  # the projections really are quantized


# ------------------------------------------------------------------------------------------
# Llama-3 RoPE frequency scaling: bands, a worked midpoint, continuity, monotonicity
# ------------------------------------------------------------------------------------------
LLAMA31_SCALING = (8.0, 1.0, 4.0, 8192)


def test_rope_scaling_bands_and_worked_midpoint():
    hd, theta = 128, 500000.0
    i = np.arange(hd // 2, dtype=np.float64)
    f = np.power(theta, -(2.0 * i) / hd)
    g = L.scaled_inv_freq(f, LLAMA31_SCALING)
    wl = 2 * np.pi / f
    keep, div = wl < 8192 / 4.0, wl > 8192 / 1.0
    mid = ~keep & ~div
    assert keep.sum() > 0 and div.sum() > 0 and mid.sum() > 0  # all three bands occur at hd 128
    assert np.array_equal(g[keep], f[keep])
    assert np.array_equal(g[div], f[div] / 8.0)
    assert np.all(g[mid] > f[mid] / 8.0) and np.all(g[mid] < f[mid])
    assert np.all(np.diff(g) <= 0)  # longer wavelengths never get a higher frequency
    # worked value: original_ctx / wavelength halfway between the factors (2.5) gives
    # t = 1/2, so the frequency is (1/8 + 1) / 2 = 9/16 of the unscaled one
    fm = np.array([2 * np.pi * 2.5 / 8192])
    assert np.isclose(L.scaled_inv_freq(fm, LLAMA31_SCALING)[0], fm[0] * 9.0 / 16.0, rtol=1e-14)
    # continuity at both band edges
    for edge in (8192 / 4.0, 8192 / 1.0):
        fe = 2 * np.pi / (edge * np.array([1 - 1e-9, 1 + 1e-9]))
        ge = L.scaled_inv_freq(fe, LLAMA31_SCALING)
        assert np.isclose(ge[0] / fe[0], ge[1] / fe[1], rtol=1e-6)


def test_rope_scaling_factor_one_is_plain_rope():
    f = np.power(500000.0, -np.arange(64) / 64.0)
    assert np.allclose(L.scaled_inv_freq(f, (1.0, 1.0, 4.0, 8192)), f, rtol=1e-15, atol=0)
    c0, s0 = L.rope_tables([37, 900], 128, 500000.0)
    c1, s1 = L.rope_tables([37, 900], 128, 500000.0, (1.0, 1.0, 4.0, 8192))
    assert np.allclose(c0, c1, atol=1e-6) and np.allclose(s0, s1, atol=1e-6)


# ------------------------------------------------------------------------------------------
# C8 decode step-by-step == independently written full-sequence causal forward
# ------------------------------------------------------------------------------------------
@pytest.mark.parametrize("fmt", [L.FMT_BF16, L.FMT_W8A16, L.FMT_W4A16, L.FMT_W4A16_G128])
def test_decode_equals_prefill(fmt):
    shape = W.small_shape(hidden=64, n_layers=3, n_q_heads=4, n_kv_heads=2, head_dim=16, ffn=96, vocab=200)
    t = random_model_tensors(shape, seed=21, std=0.1)
    m = L.OracleModel(shape, t, fmt)
    toks = [5, 199, 0, 42, 42, 7]
    ref = m.prefill_logits(toks)
    kv = fresh_kv(shape, 8)
    for p, tok in enumerate(toks):
        lg = m.decode_step(tok, p, kv)
        assert np.max(np.abs(lg - ref[p])) < 2e-3, p
    # an exclusive key range or an off-by-one slot would break agreement at p >= 1
    assert np.max(np.abs(ref[1] - ref[0])) > 1e-2


# ------------------------------------------------------------------------------------------
# C9 hand-computable cases (tests/golden)
# ------------------------------------------------------------------------------------------
def _mat(spec, n):
    if spec == "zeros":
        return np.zeros((n, n), np.float32)
    if spec == "identity":
        return np.eye(n, dtype=np.float32)
    return np.array(spec, np.float32)


def _golden_shape(d):
    s = d["shape"]
    return W.ModelShape("hand", s["hidden"], s["n_layers"], s["n_q_heads"], s["n_kv_heads"], s["head_dim"],
                        s["ffn"], s["vocab"], s["tied"], s["rope_theta"], s["rms_eps"])


def test_hand_two_layer_case():
    d = json.load(open(os.path.join(GOLDEN, "hand_two_layer.json")))
    shape = _golden_shape(d)
    wts = d["weights"]
    one = to_bits(np.ones(4, np.float32))
    tensors = [to_bits(np.array(wts["embed_tokens"], np.float32))]
    for lw in wts["layers"]:
        tensors += [one] + [to_bits(_mat(lw[k], 4)) for k in ("q_proj", "k_proj", "v_proj", "o_proj")] + [one] + \
                   [to_bits(_mat(lw[k], 4)) for k in ("gate_proj", "up_proj", "down_proj")]
    tensors.append(one)
    e = d["expected"]
    for fmt in (L.FMT_BF16, L.FMT_W8A16):
        m = L.OracleModel(shape, tensors, fmt)
        kv = fresh_kv(shape, 2)
        tr = {}
        lg = m.decode_step(0, 0, kv, trace=tr)
        if fmt == L.FMT_BF16:
            assert np.array_equal(tr["h"][0], np.array(e["h_layer0"], np.float32))
            assert np.array_equal(tr["m"][0], np.array(e["m_layer0"], np.float32))
            assert np.array_equal(tr["x"][0], np.array(e["x_layer0"], np.float32))
            assert np.array_equal(tr["m"][1], np.array(e["m_layer1"], np.float32))
            assert np.array_equal(tr["x"][1], np.array(e["x_layer1"], np.float32))
            assert np.array_equal(tr["hf"], np.array(e["hf"], np.float32))
            assert np.array_equal(bf16_bits_to_f32(kv[0, 1, 0, 0]), np.array(e["v_cache_layer0_pos0"], np.float32))
            assert np.array_equal(bf16_bits_to_f32(kv[1, 1, 0, 0]), np.array(e["v_cache_layer1_pos0"], np.float32))
        # identity / power-of-two weights quantize exactly, so both formats give the hand logits
        assert np.allclose(lg, e["logits"], atol=1e-6), (fmt, lg)


def test_hand_pos1_attention_case():
    d = json.load(open(os.path.join(GOLDEN, "hand_pos1_attention.json")))
    shape = _golden_shape(d)
    w = d["weights"]
    one = to_bits(np.ones(4, np.float32))
    tensors = [to_bits(np.array(w["embed_tokens"], np.float32)), one] + \
              [to_bits(_mat(w[k], 4)) for k in ("q_proj", "k_proj", "v_proj", "o_proj")] + [one] + \
              [to_bits(_mat(w[k], 4)) for k in ("gate_proj", "up_proj", "down_proj")] + [one]
    e = d["expected"]
    m = L.OracleModel(shape, tensors, L.FMT_BF16)
    kv = fresh_kv(shape, 2)
    m.decode_step(d["tokens"][0], 0, kv)
    tr = {}
    lg = m.decode_step(d["tokens"][1], 1, kv, trace=tr)
    assert np.array_equal(bf16_bits_to_f32(kv[0, 0, 0, 0]), np.array(e["k_cache_pos0"], np.float32))
    assert np.array_equal(bf16_bits_to_f32(kv[0, 0, 0, 1]), np.array(e["k_cache_pos1"], np.float32))
    assert np.array_equal(tr["o"][0], np.array(e["o_pos1"], np.float32))
    assert np.array_equal(lg, np.array(e["logits_pos1"], np.float32))


# ------------------------------------------------------------------------------------------
# C10 logits scale at random init; C11 idempotence
# ------------------------------------------------------------------------------------------
def test_logits_scale_statistics():
    shape = W.small_shape(hidden=256, n_layers=2, n_q_heads=4, n_kv_heads=2, head_dim=64, ffn=512, vocab=4096)
    t = random_model_tensors(shape, seed=31)
    m = L.OracleModel(shape, t, L.FMT_W8A16)
    kv = fresh_kv(shape, 4)
    lg = m.decode_step(17, 0, kv)
    assert abs(float(np.std(lg)) / (0.02 * math.sqrt(shape.hidden)) - 1) < 0.1


def test_sensitivity_probe_is_small_on_shallow_models():
    """float32 and float64 summation of the same definition agree closely on a shallow model
    (the probe measures conditioning, it is not a second definition)."""
    shape = W.small_shape(hidden=128, n_layers=2, n_q_heads=4, n_kv_heads=2, head_dim=32, ffn=256, vocab=512)
    m = L.OracleModel(shape, random_model_tensors(shape, seed=51), L.FMT_W8A16)
    kv = fresh_kv(shape, 4)
    before = kv.copy()
    assert m.sensitivity(3, 0, kv) < 1e-4
    assert np.array_equal(kv, before) and m.accum == np.float32


def test_step_idempotent():
    shape = W.small_shape(hidden=64, n_layers=2, n_q_heads=4, n_kv_heads=2, head_dim=16, ffn=96, vocab=100)
    m = L.OracleModel(shape, random_model_tensors(shape, seed=41, std=0.1), L.FMT_W8A16)
    kv = fresh_kv(shape, 6)
    for p, tok in enumerate([1, 2, 3]):
        m.decode_step(tok, p, kv)
    snap = kv.copy()
    a = m.decode_step(9, 3, kv)
    kv_a = kv.copy()
    b = m.decode_step(9, 3, kv)
    assert np.array_equal(a, b) and np.array_equal(kv, kv_a)
    assert np.array_equal(kv[:, :, :, :3], snap[:, :, :, :3])


def test_generator_is_deterministic_and_shaped():
    s = W.small_shape()
    a = W.gen_weights(s, seed0=3)
    b = W.gen_weights(s, seed0=3)
    c = W.gen_weights(s, seed0=4)
    assert all(torch.equal(x, y) for x, y in zip(a, b))
    assert not torch.equal(a[0], c[0])
    assert [tuple(x.shape) for x in a] == [d for _, d, _ in W.tensor_specs(s)]
    kv = W.gen_kv_cache(s, 10, 6, seed0=0)
    assert kv.shape == W.kv_cache_shape(s, 10) and kv[:, :, :, 6:].abs().sum() == 0
    assert abs(float(kv[:, :, :, :6].float().std()) - 1.0) < 0.1


# ------------------------------------------------------------------------------------------
# the pins catch planted mistakes (mistakes are planted in the oracle, on the CPU)
# ------------------------------------------------------------------------------------------
def _rope_sign_flipped(v, cos, sin):
    v = np.asarray(v, dtype=F32)
    half = v.shape[-1] // 2
    a, b = v[..., :half], v[..., half:]
    out = np.empty_like(v)
    out[..., :half] = a * cos + b * sin
    out[..., half:] = b * cos - a * sin
    return out


def _rope_interleaved(v, cos, sin):
    v = np.asarray(v, dtype=F32)
    a, b = v[..., 0::2], v[..., 1::2]
    out = np.empty_like(v)
    out[..., 0::2] = a * cos - b * sin
    out[..., 1::2] = b * cos + a * sin
    return out


def _silu_wrong(z):
    z = np.asarray(z, dtype=F32)
    return z / (F32(1.0) + np.exp(z, dtype=F32))


def _rmsnorm_eps_outside(x, w, eps):
    x = np.asarray(x, dtype=F32)
    return (x / (np.sqrt(np.mean(x * x, dtype=F32)) + F32(eps))) * np.asarray(w, dtype=F32)


def _attention_no_scale(q, K, V, scale, accum=F32):
    return _ORIG_ATT(q, K, V, F32(1.0), accum)


_ORIG_ATT = L.attention_head


@pytest.mark.parametrize("name,mutant,pins", [
    ("rope sign", _rope_sign_flipped, [test_rope_hand_values]),
    ("rope pairing", _rope_interleaved, [test_rope_hand_values]),
    ("silu", _silu_wrong, [test_silu_values, test_hand_two_layer_case]),
    ("rmsnorm eps", _rmsnorm_eps_outside, [test_rmsnorm_closed_form]),
    ("attention scale", _attention_no_scale, [test_hand_pos1_attention_case]),
])
def test_pins_catch_planted_mistakes(monkeypatch, name, mutant, pins):
    target = {"rope sign": "apply_rope", "rope pairing": "apply_rope", "silu": "silu",
              "rmsnorm eps": "rmsnorm", "attention scale": "attention_head"}[name]
    monkeypatch.setattr(L, target, mutant)
    for pin in pins:
        with pytest.raises(AssertionError):
            pin()
