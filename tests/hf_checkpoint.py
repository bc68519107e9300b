"""Writes a seeded synthetic model as a HuggingFace Llama checkpoint directory (config.json plus
safetensors files), the layout the checkpoint reader takes. Test infrastructure only."""
from __future__ import annotations

import json
import os
from typing import Dict, List, Optional

import torch

import workloads as W

HF_LAYER = ("input_layernorm", "self_attn.q_proj", "self_attn.k_proj", "self_attn.v_proj", "self_attn.o_proj",
            "post_attention_layernorm", "mlp.gate_proj", "mlp.up_proj", "mlp.down_proj")


def hf_config(shape: W.ModelShape) -> Dict:
    cfg = {"architectures": ["LlamaForCausalLM"], "model_type": "llama", "hidden_act": "silu",
           "hidden_size": shape.hidden, "intermediate_size": shape.ffn, "num_hidden_layers": shape.n_layers,
           "num_attention_heads": shape.n_q_heads, "num_key_value_heads": shape.n_kv_heads,
           "head_dim": shape.head_dim, "vocab_size": shape.vocab, "tie_word_embeddings": shape.tied,
           "rope_theta": shape.rope_theta, "rms_norm_eps": shape.rms_eps, "attention_bias": False,
           "mlp_bias": False, "torch_dtype": "bfloat16"}
    if shape.rope_scaling is not None:
        f, lo, hi, orig = shape.rope_scaling
        cfg["rope_scaling"] = {"rope_type": "llama3", "factor": f, "low_freq_factor": lo,
                               "high_freq_factor": hi, "original_max_position_embeddings": orig}
    return cfg


def hf_names(shape: W.ModelShape) -> List[str]:
    names = ["model.embed_tokens.weight"]
    for l in range(shape.n_layers):
        names += [f"model.layers.{l}.{n}.weight" for n in HF_LAYER]
    names.append("model.norm.weight")
    if not shape.tied:
        names.append("lm_head.weight")
    return names


def write_checkpoint(path: str, shape: W.ModelShape, tensors: List[torch.Tensor], shards: int = 1,
                     as_float32: Optional[List[str]] = None, extra: Optional[Dict[str, torch.Tensor]] = None,
                     config: Optional[Dict] = None) -> None:
    """tensors in canonical order. Tensors named in `as_float32` are stored as float32 (exactly
    the bf16 values); `extra` adds tensors the reader must ignore. The names are spread round-robin
    over `shards` files, with an index when shards > 1. The file order is reversed against the
    canonical order, so the reader has to look names up."""
    from safetensors.torch import save_file
    os.makedirs(path, exist_ok=True)
    named = dict(zip(hf_names(shape), tensors))
    for n in as_float32 or []:
        named[n] = named[n].float()
    named.update(extra or {})
    items = list(named.items())[::-1]
    with open(os.path.join(path, "config.json"), "w") as f:
        json.dump(config if config is not None else hf_config(shape), f, indent=1)
    if shards == 1:
        save_file({k: v.contiguous() for k, v in items}, os.path.join(path, "model.safetensors"))
        return
    weight_map = {}
    for s in range(shards):
        fname = f"model-{s + 1:05d}-of-{shards:05d}.safetensors"
        part = {k: v.contiguous() for k, v in items[s::shards]}
        save_file(part, os.path.join(path, fname))
        weight_map.update({k: fname for k in part})
    with open(os.path.join(path, "model.safetensors.index.json"), "w") as f:
        json.dump({"metadata": {}, "weight_map": weight_map}, f, indent=1)
