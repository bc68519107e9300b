"""Seeded synthetic inputs shared by the CPU oracle and the HIP decode path.

This module holds model shapes, the decode workloads measured on them, and the
seeded random generators for weights, prompt tokens and KV-cache prefill. It
holds none of the decode arithmetic: it only draws numbers and stores them as
bfloat16 bit patterns, so both sides receive identical bytes.

Source of the workloads: the decode-megakernel pages describe batch-1 decode of
HuggingFace Llama-family models (AutoMegaKernel paper index, Abstract; gist.science
explainer, Technical Summary > Problem Statement). Their real checkpoints are not
available, so each workload is a random-init model of a named architecture:
Linear and embedding weights ~ N(0, 0.02) (HF ``initializer_range``), RMSNorm
weights 1.0 (HF init), bf16 storage.

Generator definition (reproducible from this text alone):
  * every tensor is produced in row-major chunks of ``CHUNK`` elements; chunk c of
    tensor i draws ``torch.randn`` from ``torch.Generator().manual_seed(s)`` with the
    32-bit seed s = stream * 2**30 + seed0 * 2**26 + i * 2**16 + c (the CPU generator
    keeps 32 seed bits), then multiplies by the tensor's std in fp32 and converts to
    bfloat16 with ``Tensor.to``;
  * stream 0 = weights (i = canonical tensor index), stream 1 = tokens
    (``torch.randint(0, vocab)`` with i = c = 0), stream 2 = KV prefill with
    i = layer * 2 + (0 for K, 1 for V) and c = kv_head * 2**12 + chunk.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
from typing import List, Optional, Tuple

import numpy as np
import torch

CHUNK = 1 << 22
WEIGHT_STD = 0.02
FMT_BF16 = 0
FMT_W8A16 = 1
FMT_W8A16_BF16_HEAD = 2  # W8A16 projections, bf16 lm_head
FMT_W4A16 = 3            # int4 per-row projections, bf16 lm_head
FMT_W4A16_G128 = 4       # int4 projections with an fp16 scale per group of 128 columns, bf16 lm_head


@dataclass(frozen=True)
class ModelShape:
    name: str
    hidden: int
    n_layers: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    vocab: int
    tied: bool
    rope_theta: float
    rms_eps: float = 1e-5
    # Llama-3 frequency scaling (factor, low_freq_factor, high_freq_factor, original context), or
    # None for plain RoPE
    rope_scaling: Optional[Tuple[float, float, float, int]] = None

    @property
    def q_dim(self) -> int:
        return self.n_q_heads * self.head_dim

    @property
    def kv_dim(self) -> int:
        return self.n_kv_heads * self.head_dim

    @property
    def n_tensors(self) -> int:
        return 2 + 9 * self.n_layers + (0 if self.tied else 1)


SMOLLM2_135M = ModelShape("SmolLM2-135M", 576, 30, 9, 3, 64, 1536, 49152, True, 10000.0)
LLAMA32_1B = ModelShape("Llama-3.2-1B", 2048, 16, 32, 8, 64, 8192, 128256, True, 500000.0)
LLAMA3_8B = ModelShape("Llama-3-8B", 4096, 32, 32, 8, 128, 14336, 128256, False, 500000.0)


@dataclass(frozen=True)
class Workload:
    """One decode run: prompt tokens fed one per step (or a prefilled cache), then greedy steps."""
    key: str
    shape: ModelShape
    weight_format: int
    prompt_len: int      # tokens fed one per decode step starting at pos 0 (fresh cache)
    prefill_len: int     # cache slots [0, prefill_len) hold N(0,1) bf16; first step at pos = prefill_len
    greedy_steps: int    # steps after the prompt / prefill, each feeding the previous argmax

    @property
    def first_pos(self) -> int:
        return self.prefill_len

    @property
    def n_steps(self) -> int:
        return self.prompt_len + self.greedy_steps

    @property
    def max_ctx(self) -> int:
        return self.prefill_len + self.prompt_len + self.greedy_steps

    @property
    def fmt_name(self) -> str:
        return {FMT_BF16: "bf16", FMT_W8A16: "w8a16", FMT_W8A16_BF16_HEAD: "w8a16-bf16head",
                FMT_W4A16: "w4a16", FMT_W4A16_G128: "w4a16-g128"}[self.weight_format]


WORKLOADS = {
    "smollm2-135m-bf16": Workload("smollm2-135m-bf16", SMOLLM2_135M, FMT_BF16, 8, 0, 16),
    "smollm2-135m-w8a16": Workload("smollm2-135m-w8a16", SMOLLM2_135M, FMT_W8A16, 64, 0, 128),
    "llama3.2-1b-w8a16-ctx1024": Workload("llama3.2-1b-w8a16-ctx1024", LLAMA32_1B, FMT_W8A16, 0, 1024, 128),
    "llama3-8b-bf16-ctx4096": Workload("llama3-8b-bf16-ctx4096", LLAMA3_8B, FMT_BF16, 0, 4096, 128),
    "llama3-8b-w8a16-ctx4096": Workload("llama3-8b-w8a16-ctx4096", LLAMA3_8B, FMT_W8A16, 0, 4096, 128),
    # the pages' "0.61x the bytes" reading: the same W8A16 model with the lm_head kept in bf16
    "llama3-8b-w8a16hb-ctx4096": Workload("llama3-8b-w8a16hb-ctx4096", LLAMA3_8B, FMT_W8A16_BF16_HEAD, 0, 4096, 128),
    "llama3-8b-w8a16-ctx32768": Workload("llama3-8b-w8a16-ctx32768", LLAMA3_8B, FMT_W8A16, 0, 32768, 64),
    # the pages' int4 weight-only variant (lossy, 2.42x less weight traffic than bf16)
    "smollm2-135m-w4a16": Workload("smollm2-135m-w4a16", SMOLLM2_135M, FMT_W4A16, 64, 0, 128),
    "llama3-8b-w4a16-ctx4096": Workload("llama3-8b-w4a16-ctx4096", LLAMA3_8B, FMT_W4A16, 0, 4096, 128),
    # the same variant with group-wise scales (one fp16 scale per 128 columns of a row)
    "smollm2-135m-w4a16g": Workload("smollm2-135m-w4a16g", SMOLLM2_135M, FMT_W4A16_G128, 64, 0, 128),
    "llama3-8b-w4a16g-ctx4096": Workload("llama3-8b-w4a16g-ctx4096", LLAMA3_8B, FMT_W4A16_G128, 0, 4096, 128),
}


# ----------------------------------------------------------------------------------------------
# canonical tensor order (HF LlamaForCausalLM state-dict order, each Linear stored [out, in])
# ----------------------------------------------------------------------------------------------
LAYER_TENSORS = ("input_layernorm", "q_proj", "k_proj", "v_proj", "o_proj",
                 "post_attention_layernorm", "gate_proj", "up_proj", "down_proj")


def tensor_specs(shape: ModelShape) -> List[Tuple[str, Tuple[int, ...], str]]:
    """(name, dims, kind) per tensor in canonical order; kind is 'matrix' or 'norm'."""
    H, F = shape.hidden, shape.ffn
    specs = [("embed_tokens", (shape.vocab, H), "matrix")]
    for l in range(shape.n_layers):
        dims = {
            "input_layernorm": (H,), "q_proj": (shape.q_dim, H), "k_proj": (shape.kv_dim, H),
            "v_proj": (shape.kv_dim, H), "o_proj": (H, shape.q_dim),
            "post_attention_layernorm": (H,), "gate_proj": (F, H), "up_proj": (F, H),
            "down_proj": (H, F),
        }
        for n in LAYER_TENSORS:
            specs.append((f"layers.{l}.{n}", dims[n], "norm" if n.endswith("layernorm") else "matrix"))
    specs.append(("norm", (H,), "norm"))
    if not shape.tied:
        specs.append(("lm_head", (shape.vocab, H), "matrix"))
    return specs


def tensor_index(shape: ModelShape, name: str) -> int:
    for i, (n, _, _) in enumerate(tensor_specs(shape)):
        if n == name:
            return i
    raise KeyError(name)


def _seed(seed0: int, stream: int, i: int, c: int) -> int:
    assert 0 <= seed0 < 16 and 0 <= stream < 4 and 0 <= i < 1024 and 0 <= c < 65536
    return (stream << 30) | (seed0 << 26) | (i << 16) | c


def _n_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def normal_bf16(n: int, std: float, seed0: int, stream: int, i: int, c_base: int = 0,
                pool: Optional[ThreadPoolExecutor] = None) -> torch.Tensor:
    """n draws of N(0, std^2) as a flat bf16 CPU tensor (chunked, seeded as in the module doc)."""
    out = torch.empty(n, dtype=torch.bfloat16)
    n_chunks = (n + CHUNK - 1) // CHUNK

    def fill(c: int) -> None:
        lo, hi = c * CHUNK, min(n, (c + 1) * CHUNK)
        g = torch.Generator().manual_seed(_seed(seed0, stream, i, c_base + c))
        x = torch.randn(hi - lo, generator=g, dtype=torch.float32)
        if std != 1.0:
            x.mul_(std)
        out[lo:hi] = x.to(torch.bfloat16)

    if n_chunks <= 1 or pool is None:
        for c in range(n_chunks):
            fill(c)
    else:
        list(pool.map(fill, range(n_chunks)))
    return out


def gen_tensor(shape: ModelShape, index: int, seed0: int = 0,
               pool: Optional[ThreadPoolExecutor] = None) -> torch.Tensor:
    """Tensor `index` (canonical order) as a bf16 CPU tensor of its dims."""
    name, dims, kind = tensor_specs(shape)[index]
    n = int(np.prod(dims))
    if kind == "norm":
        return torch.ones(dims, dtype=torch.bfloat16)
    return normal_bf16(n, WEIGHT_STD, seed0, 0, index, 0, pool).view(dims)


def gen_weights(shape: ModelShape, seed0: int = 0) -> List[torch.Tensor]:
    """All tensors in canonical order (bf16 CPU tensors)."""
    with ThreadPoolExecutor(_n_threads()) as pool:
        return [gen_tensor(shape, i, seed0, pool) for i in range(shape.n_tensors)]


def gen_tokens(shape: ModelShape, n: int, seed0: int = 0) -> List[int]:
    g = torch.Generator().manual_seed(_seed(seed0, 1, 0, 0))
    return [int(t) for t in torch.randint(0, shape.vocab, (n,), generator=g)]


def kv_cache_shape(shape: ModelShape, max_ctx: int) -> Tuple[int, ...]:
    """KV cache layout [L][2 (K,V)][n_kv][max_ctx][head_dim], bf16."""
    return (shape.n_layers, 2, shape.n_kv_heads, max_ctx, shape.head_dim)


def gen_kv_cache(shape: ModelShape, max_ctx: int, prefill_len: int, seed0: int = 0) -> torch.Tensor:
    """bf16 CPU KV cache; slots [0, prefill_len) hold N(0,1), the rest zero."""
    kv = torch.zeros(kv_cache_shape(shape, max_ctx), dtype=torch.bfloat16)
    if prefill_len == 0:
        return kv
    n = prefill_len * shape.head_dim
    jobs = [(l, s, g) for l in range(shape.n_layers) for s in range(2) for g in range(shape.n_kv_heads)]

    def fill(job) -> None:
        l, s, g = job
        kv[l, s, g, :prefill_len, :] = normal_bf16(n, 1.0, seed0, 2, l * 2 + s, g << 12).view(
            prefill_len, shape.head_dim)

    with ThreadPoolExecutor(_n_threads()) as pool:
        list(pool.map(fill, jobs))
    return kv


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """The uint16 bit patterns of a bf16 CPU tensor, as a numpy array (shares memory)."""
    assert t.dtype == torch.bfloat16
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def small_shape(name: str = "tiny", hidden: int = 128, n_layers: int = 2, n_q_heads: int = 4,
                n_kv_heads: int = 2, head_dim: int = 32, ffn: int = 256, vocab: int = 512,
                tied: bool = True, rope_theta: float = 10000.0, rms_eps: float = 1e-5) -> ModelShape:
    return ModelShape(name, hidden, n_layers, n_q_heads, n_kv_heads, head_dim, ffn, vocab, tied,
                      rope_theta, rms_eps)
