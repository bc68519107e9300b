"""The HuggingFace checkpoint reader on synthetic checkpoints written to a temporary directory:
dims from config.json, canonical tensor order, shards, dtype rounding, and the models it must
refuse. CPU only."""
from __future__ import annotations

import json
import os

import pytest
import torch

import workloads as W
from decode_megakernel_cooperative_amd.checkpoint import CheckpointError, load_checkpoint, shape_from_config
from hf_checkpoint import hf_config, write_checkpoint

FIELDS = ("hidden", "n_layers", "n_q_heads", "n_kv_heads", "head_dim", "ffn", "vocab", "tied", "rope_theta",
          "rms_eps", "rope_scaling")

SCALED = W.ModelShape("tiny-scaled", 128, 2, 4, 2, 32, 256, 512, False, 500000.0, 1e-5,
                      rope_scaling=(8.0, 1.0, 4.0, 8192))
TIED = W.small_shape("tiny-tied")


def same_fields(a, b):
    return all(getattr(a, f) == getattr(b, f) for f in FIELDS)


def test_llama31_8b_config_gives_the_8b_shape():
    """The published Llama-3.1-8B config.json values give the 8B dims, untied, with the Llama-3
    RoPE rule (factor 8, low 1, high 4, original context 8192)."""
    cfg = {"model_type": "llama", "hidden_act": "silu", "hidden_size": 4096, "intermediate_size": 14336,
           "num_hidden_layers": 32, "num_attention_heads": 32, "num_key_value_heads": 8,
           "vocab_size": 128256, "rms_norm_eps": 1e-5, "rope_theta": 500000.0, "tie_word_embeddings": False,
           "rope_scaling": {"factor": 8.0, "low_freq_factor": 1.0, "high_freq_factor": 4.0,
                            "original_max_position_embeddings": 8192, "rope_type": "llama3"}}
    s = shape_from_config(cfg)
    assert same_fields(s, W.ModelShape("x", 4096, 32, 32, 8, 128, 14336, 128256, False, 500000.0, 1e-5,
                                       rope_scaling=(8.0, 1.0, 4.0, 8192)))
    assert s.n_tensors == W.LLAMA3_8B.n_tensors


def test_config_defaults():
    """Absent keys take the HF Llama defaults: kv heads = heads, head_dim = hidden / heads,
    theta 10000, eps 1e-6, untied; an old-style {"type": "default"} scaling is plain RoPE."""
    s = shape_from_config({"hidden_size": 256, "intermediate_size": 512, "num_hidden_layers": 1,
                           "num_attention_heads": 4, "vocab_size": 100, "rope_scaling": {"type": "default"}})
    assert (s.n_kv_heads, s.head_dim, s.rope_theta, s.rms_eps, s.tied, s.rope_scaling) == \
        (4, 64, 10000.0, 1e-6, False, None)


@pytest.mark.parametrize("shape,shards", [(SCALED, 1), (SCALED, 3), (TIED, 2)], ids=["untied", "sharded", "tied"])
def test_round_trip(tmp_path, shape, shards):
    ws = W.gen_weights(shape, seed0=3)
    write_checkpoint(str(tmp_path), shape, ws, shards=shards)
    s, ts = load_checkpoint(str(tmp_path))
    assert same_fields(s, shape) and s.name == os.path.basename(str(tmp_path))
    assert len(ts) == shape.n_tensors
    for a, b in zip(ts, ws):
        assert a.dtype == torch.bfloat16 and a.is_contiguous() and torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_float_tensors_round_to_bf16(tmp_path):
    """A float32 tensor holding bf16 values loads to the same bits; a float32 value between two
    bf16 values rounds to the nearer (1 + 2^-8 + 2^-10 -> 1 + 2^-7), a tie to even
    (1 + 2^-8 -> 1, 1 + 3*2^-8 -> 1 + 2^-6)."""
    ws = W.gen_weights(TIED, seed0=4)
    ws[1] = torch.tensor([1 + 2 ** -8 + 2 ** -10, 1 + 2 ** -8, 1 + 3 * 2 ** -8] + [1.0] * 125,
                         dtype=torch.float32)
    write_checkpoint(str(tmp_path), TIED, ws, as_float32=["model.embed_tokens.weight"])
    _, ts = load_checkpoint(str(tmp_path))
    assert torch.equal(ts[0].view(torch.int16), ws[0].view(torch.int16))
    assert ts[1][:3].float().tolist() == [1 + 2 ** -7, 1.0, 1 + 2 ** -6]


def test_tied_checkpoint_with_lm_head_ignores_it(tmp_path):
    ws = W.gen_weights(TIED, seed0=5)
    write_checkpoint(str(tmp_path), TIED, ws, extra={"lm_head.weight": torch.zeros(TIED.vocab, TIED.hidden,
                                                                                   dtype=torch.bfloat16)})
    s, ts = load_checkpoint(str(tmp_path))
    assert len(ts) == TIED.n_tensors and torch.equal(ts[0], ws[0])


@pytest.mark.parametrize("change,match", [
    ({"attention_bias": True}, "bias"), ({"mlp_bias": True}, "bias"), ({"hidden_act": "gelu"}, "SiLU"),
    ({"model_type": "mistral"}, "Llama"), ({"rope_scaling": {"rope_type": "yarn", "factor": 4.0}}, "Llama-3"),
])
def test_refused_configs(tmp_path, change, match):
    cfg = hf_config(TIED)
    cfg.update(change)
    write_checkpoint(str(tmp_path), TIED, W.gen_weights(TIED), config=cfg)
    with pytest.raises(CheckpointError, match=match):
        load_checkpoint(str(tmp_path))


def test_missing_and_misshapen_tensors(tmp_path):
    ws = W.gen_weights(SCALED)
    write_checkpoint(str(tmp_path / "a"), SCALED, ws[:-1] + [ws[-1][:10]])
    with pytest.raises(CheckpointError, match="lm_head.weight: dims"):
        load_checkpoint(str(tmp_path / "a"))
    # a tied model's tensors under a config that declares untied embeddings: no lm_head.weight
    write_checkpoint(str(tmp_path / "b"), TIED, W.gen_weights(TIED),
                     config=dict(hf_config(TIED), tie_word_embeddings=False))
    with pytest.raises(CheckpointError, match="lacks 1 tensors"):
        load_checkpoint(str(tmp_path / "b"))
    os.makedirs(tmp_path / "c")
    with open(tmp_path / "c" / "config.json", "w") as f:
        json.dump(hf_config(TIED), f)
    with pytest.raises(CheckpointError, match="neither"):
        load_checkpoint(str(tmp_path / "c"))
