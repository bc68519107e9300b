"""Reading a HuggingFace Llama checkpoint directory for the decode library.

The decode pages run HuggingFace Llama models (AutoMegaKernel paper index, Abstract; gist.science
explainer, Technical Summary > Problem Statement). A checkpoint directory in that format holds
``config.json`` and either ``model.safetensors`` or ``model.safetensors.index.json`` plus the
shards it names. This module turns one into what ``amk_load_weights`` takes: a shape record
and the bf16 host tensors in canonical order (embed_tokens; per layer input_layernorm, q_proj,
k_proj, v_proj, o_proj, post_attention_layernorm, gate_proj, up_proj, down_proj; norm; lm_head
unless the embeddings are tied).

Only the safetensors format is read, through its own loader, which executes nothing from the
file. Tensors stored in float16 or float32 are rounded to bfloat16 (round to nearest even).
What the decode kernel does not compute raises ``CheckpointError`` instead of loading a model
that would decode differently: attention or MLP biases, an activation other than SiLU, and RoPE
scaling other than none or the Llama-3 rule.

HF Llama checkpoints already store q_proj and k_proj rows in the rotate-half RoPE order the
kernel uses (pairs i and i + head_dim/2), so no row permutation is applied.
"""
from __future__ import annotations

import json
import os
from dataclasses import dataclass
from typing import Dict, List, Optional, Tuple

LAYER_NAMES = (("input_layernorm", "input_layernorm"), ("q_proj", "self_attn.q_proj"),
               ("k_proj", "self_attn.k_proj"), ("v_proj", "self_attn.v_proj"),
               ("o_proj", "self_attn.o_proj"), ("post_attention_layernorm", "post_attention_layernorm"),
               ("gate_proj", "mlp.gate_proj"), ("up_proj", "mlp.up_proj"), ("down_proj", "mlp.down_proj"))


class CheckpointError(ValueError):
    pass


@dataclass(frozen=True)
class LlamaShape:
    """The model dimensions the decode library needs; field names match ``make_config``."""
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
    rms_eps: float = 1e-6
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


def shape_from_config(cfg: Dict, name: str = "checkpoint") -> LlamaShape:
    """A LlamaShape from the parsed ``config.json`` of a HF Llama model.

    Defaults follow the HF Llama configuration class where a key is absent: key/value heads =
    attention heads, head_dim = hidden / heads, rope_theta 10000, rms_norm_eps 1e-6, untied
    embeddings."""
    def need(key):
        if key not in cfg:
            raise CheckpointError(f"config.json lacks {key!r}")
        return cfg[key]

    mt = cfg.get("model_type", "llama")
    if mt != "llama":
        raise CheckpointError(f"model_type {mt!r} is not a Llama model")
    act = cfg.get("hidden_act", "silu")
    if act != "silu":
        raise CheckpointError(f"hidden_act {act!r}: the decode kernel computes SiLU only")
    for key in ("attention_bias", "mlp_bias"):
        if cfg.get(key, False):
            raise CheckpointError(f"{key} is set: the decode kernel has no bias terms")
    hidden = int(need("hidden_size"))
    nq = int(need("num_attention_heads"))
    nkv = int(cfg.get("num_key_value_heads") or nq)
    hd = cfg.get("head_dim")
    hd = int(hd) if hd else hidden // nq
    scaling = None
    rs = cfg.get("rope_scaling")
    if rs:
        kind = rs.get("rope_type", rs.get("type"))
        if kind == "llama3":
            scaling = (float(rs["factor"]), float(rs["low_freq_factor"]), float(rs["high_freq_factor"]),
                       int(rs["original_max_position_embeddings"]))
        elif kind != "default":
            raise CheckpointError(f"rope_scaling type {kind!r}: only the Llama-3 rule is computed")
    return LlamaShape(name=name, hidden=hidden, n_layers=int(need("num_hidden_layers")), n_q_heads=nq,
                      n_kv_heads=nkv, head_dim=hd, ffn=int(need("intermediate_size")),
                      vocab=int(need("vocab_size")), tied=bool(cfg.get("tie_word_embeddings", False)),
                      rope_theta=float(cfg.get("rope_theta", 10000.0)),
                      rms_eps=float(cfg.get("rms_norm_eps", 1e-6)), rope_scaling=scaling)


def canonical_names(shape: LlamaShape) -> List[Tuple[str, Tuple[int, ...]]]:
    """(HF tensor name, dims) per tensor, in the order ``amk_load_weights`` takes them."""
    H, F = shape.hidden, shape.ffn
    dims = {"input_layernorm": (H,), "q_proj": (shape.q_dim, H), "k_proj": (shape.kv_dim, H),
            "v_proj": (shape.kv_dim, H), "o_proj": (H, shape.q_dim), "post_attention_layernorm": (H,),
            "gate_proj": (F, H), "up_proj": (F, H), "down_proj": (H, F)}
    out = [("model.embed_tokens.weight", (shape.vocab, H))]
    for l in range(shape.n_layers):
        for key, hf in LAYER_NAMES:
            out.append((f"model.layers.{l}.{hf}.weight", dims[key]))
    out.append(("model.norm.weight", (H,)))
    if not shape.tied:
        out.append(("lm_head.weight", (shape.vocab, H)))
    return out


def _weight_files(path: str) -> Dict[str, str]:
    """Tensor name -> safetensors file holding it."""
    index = os.path.join(path, "model.safetensors.index.json")
    if os.path.exists(index):
        with open(index) as f:
            wm = json.load(f)["weight_map"]
        return {k: os.path.join(path, v) for k, v in wm.items()}
    single = os.path.join(path, "model.safetensors")
    if not os.path.exists(single):
        raise CheckpointError(f"{path}: neither model.safetensors nor model.safetensors.index.json")
    from safetensors import safe_open
    with safe_open(single, framework="pt") as f:
        return {k: single for k in f.keys()}


def load_checkpoint(path: str, name: Optional[str] = None):
    """(LlamaShape, list of contiguous bf16 CPU tensors in canonical order) for a HF Llama
    checkpoint directory. Raises CheckpointError for a missing tensor, a tensor of the wrong
    dims or dtype, or a model the kernel does not compute."""
    import torch
    from safetensors import safe_open

    with open(os.path.join(path, "config.json")) as f:
        cfg = json.load(f)
    shape = shape_from_config(cfg, name or os.path.basename(os.path.normpath(path)))
    where = _weight_files(path)
    wanted = canonical_names(shape)
    missing = [n for n, _ in wanted if n not in where]
    if missing:
        raise CheckpointError(f"checkpoint lacks {len(missing)} tensors, first {missing[0]!r}")
    by_file: Dict[str, List[int]] = {}
    for i, (n, _) in enumerate(wanted):
        by_file.setdefault(where[n], []).append(i)
    out: List[Optional[object]] = [None] * len(wanted)
    for fname, idx in by_file.items():
        with safe_open(fname, framework="pt") as f:
            for i in idx:
                n, dims = wanted[i]
                t = f.get_tensor(n)
                if tuple(t.shape) != dims:
                    raise CheckpointError(f"{n}: dims {tuple(t.shape)}, expected {dims}")
                if t.dtype not in (torch.bfloat16, torch.float16, torch.float32):
                    raise CheckpointError(f"{n}: dtype {t.dtype} is not a floating weight")
                out[i] = t.to(torch.bfloat16).contiguous()
    return shape, out
