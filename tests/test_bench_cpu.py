"""CPU checks of the benchmark's own arithmetic: the algorithmic bytes per token that the
roofline figure divides by, against figures derived independently from the model shapes
(bytes per token at each workload's mean position, the parameter counts the model names
imply, the K/V bytes per attended position)."""
import numpy as np
import pytest

import bench
import workloads as W


def _mean_bytes(key):
    wl = W.WORKLOADS[key]
    pos = range(wl.first_pos, wl.first_pos + wl.n_steps)
    return float(np.mean([bench.algorithmic_bytes(wl.shape, wl.weight_format, p) for p in pos]))


@pytest.mark.parametrize("key,expected", [
    ("smollm2-135m-bf16", 269.5e6),          # positions 0-23
    ("smollm2-135m-w8a16", 137.8e6),         # positions 0-191
    ("llama3.2-1b-w8a16-ctx1024", 1.274e9),  # positions 1024-1151
    ("llama3-8b-bf16-ctx4096", 15.556e9),    # positions 4096-4223
    ("llama3-8b-w8a16-ctx4096", 8.057e9),
    ("llama3-8b-w8a16-ctx32768", 11.811e9),  # positions 32768-32831
])
def test_algorithmic_bytes_per_token(key, expected):
    assert abs(_mean_bytes(key) - expected) <= 5e-4 * expected


@pytest.mark.parametrize("shape,params", [
    (W.SMOLLM2_135M, 134_515_008),
    (W.LLAMA32_1B, 1_235_814_400),
])
def test_parameter_counts(shape, params):
    assert sum(int(np.prod(dims)) for _, dims, _ in W.tensor_specs(shape)) == params


def test_llama3_8b_shape_terms():
    shape = W.WORKLOADS["llama3-8b-w8a16-ctx4096"].shape
    assert sum(int(np.prod(dims)) for _, dims, _ in W.tensor_specs(shape)) == 8_030_261_248
    # one more attended position adds its K and V in every layer: 2 * L * nkv * hd * 2 bytes
    a = bench.algorithmic_bytes(shape, W.FMT_W8A16, 4096)
    b = bench.algorithmic_bytes(shape, W.FMT_W8A16, 4097)
    assert b - a == 131072
    # position 0, term by term: int8 projections and lm_head, fp32 row scales, K/V read (one
    # position) and write, the 2L + 1 norm vectors, the embedding row, the fp32 logits
    L, H, F, V = 32, 4096, 14336, 128256
    proj = L * (6144 * H + H * H + 2 * F * H + H * F)
    weights = proj + V * H + 4 * (L * (6144 + H + 2 * F + H) + V)
    assert weights == 7_510_676_480
    assert a - 131072 * 4096 == weights + 131072 + 131072 + 2 * H * (2 * L + 1) + 2 * H + 4 * V
