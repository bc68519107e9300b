"""A model read from a HuggingFace checkpoint directory decodes like the oracle run on the
weights that were written into it. The checkpoint is synthetic (seeded weights in the HF Llama
layout, sharded, Llama-3 RoPE scaling, untied head), written to a temporary directory."""
import numpy as np
import pytest

import decode_megakernel_cooperative_amd as D
import workloads as W
from decode_megakernel_cooperative_amd.checkpoint import load_checkpoint
from gpu_harness import LOGIT_TOL, log, run_teacher_forced
from hf_checkpoint import write_checkpoint
from oracle.llama import OracleModel

pytestmark = pytest.mark.gpu

SHAPE = W.ModelShape("hf-hd128-gqa4-scaled", 512, 3, 8, 2, 128, 1376, 1000, False, 500000.0,
                     rope_scaling=(8.0, 1.0, 4.0, 8192))


@pytest.mark.parametrize("fmt", [D.AMK_BF16, D.AMK_W8A16, D.AMK_W4A16, D.AMK_W4A16_G128],
                         ids=["bf16", "w8a16", "w4a16", "w4a16-g128"])
def test_checkpoint_decode_matches_oracle(tmp_path, fmt):
    ws = W.gen_weights(SHAPE, seed0=12)
    write_checkpoint(str(tmp_path), SHAPE, ws, shards=2)
    shape, tensors = load_checkpoint(str(tmp_path))
    log(f"  checkpoint {shape.name}: {len(tensors)} tensors, fmt {fmt}")
    dec = D.Decoder(shape, tensors, fmt, 48)
    orc = OracleModel(SHAPE, [W.bf16_bits(t) for t in ws], fmt)
    kv = np.zeros(W.kv_cache_shape(SHAPE, 48), dtype=np.uint16)
    prompt = W.gen_tokens(SHAPE, 8, seed0=12)
    res = run_teacher_forced(dec, orc, kv, SHAPE, 0, prompt, 24, check_kv=True)
    worst = max(res.max_abs)
    log(f"  worst max|dlogit| {worst:.3e}; greedy checked {res.greedy_checked}, mismatches {res.greedy_mismatch}")
    assert worst <= LOGIT_TOL and res.greedy_mismatch == 0
    dec.close()
