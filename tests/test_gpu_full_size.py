"""GPU parity at the full sizes of the measured workloads, in the launch configuration bench.py
times (one persistent 256-block launch per token at the workload's positions).

At these widths the bf16 rounding of activations makes the max-abs over 128256 logits sensitive
to summation order: two equally valid orders of the oracle itself (float32 vs float64 sums) land
~1-2e-2 apart after 2 layers and ~6-11e-2 apart after 32 layers of the 8B shape. Every step's
gate is therefore conditioned on that spread, measured by the oracle alone
(gpu_harness.conditioned_tolerance: max(2e-2, 2 x spread)); order-insensitive checks pin the
arithmetic more tightly: the layer-0 K/V written at each position must match the oracle within
1 bf16 ulp, and a 2-layer prefix of the same full-width weights is run at the same positions.
"""
import gc

import numpy as np
import pytest

import decode_megakernel_cooperative_amd as D
import workloads as W
from gpu_harness import build, log, run_teacher_forced

pytestmark = pytest.mark.gpu


def _prefix_shape(shape, n_layers):
    return W.ModelShape(shape.name + f"-prefix{n_layers}", shape.hidden, n_layers, shape.n_q_heads,
                        shape.n_kv_heads, shape.head_dim, shape.ffn, shape.vocab, shape.tied, shape.rope_theta,
                        shape.rms_eps)


def _run(key, steps, prefix_layers=2, conditioned_steps=2):
    wl = W.WORKLOADS[key]
    # strict gate on a shallow prefix of the same weights (tensor seeds are per canonical index,
    # so the prefix model's embedding / layers / KV prefill equal the full model's; its final norm
    # and lm_head are drawn at the prefix model's own indices)
    ps = _prefix_shape(wl.shape, prefix_layers)
    max_ctx = wl.first_pos + steps + 1
    dec, orc, kv = build(ps, wl.weight_format, max_ctx, wl.prefill_len, oracle_threads=16)
    tok = W.gen_tokens(ps, 1)[0]
    res = run_teacher_forced(dec, orc, kv, ps, wl.first_pos, [], steps, first_token=tok, conditioned=True,
                             kv_layer0_ulp=True)
    log(f"  {key} prefix{prefix_layers}: worst {max(res.max_abs):.2e}, greedy {res.greedy_checked} checked / "
        f"{res.greedy_mismatch} mismatched")
    assert res.greedy_mismatch == 0
    dec.close()
    del dec, orc, kv
    gc.collect()
    # full depth, conditioned gate
    dec, orc, kv = build(wl.shape, wl.weight_format, wl.first_pos + conditioned_steps + 1, wl.prefill_len,
                         oracle_threads=16)
    res = run_teacher_forced(dec, orc, kv, wl.shape, wl.first_pos, [], conditioned_steps, first_token=tok,
                             conditioned=True, kv_layer0_ulp=True)
    log(f"  {key} full: worst {max(res.max_abs):.2e} (tols {[f'{t:.2e}' for t in res.tols]}), greedy "
        f"{res.greedy_checked} checked / {res.greedy_mismatch} mismatched")
    assert res.greedy_mismatch == 0
    dec.close()


def test_llama32_1b_w8a16_ctx1024():
    _run("llama3.2-1b-w8a16-ctx1024", steps=8)


def test_llama3_8b_w8a16_ctx4096():
    _run("llama3-8b-w8a16-ctx4096", steps=4)


def test_llama3_8b_bf16_ctx4096():
    _run("llama3-8b-bf16-ctx4096", steps=2, conditioned_steps=1)


def test_llama3_8b_w8a16_ctx32768():
    _run("llama3-8b-w8a16-ctx32768", steps=2, conditioned_steps=1)


def test_llama3_8b_w4a16_ctx4096():
    _run("llama3-8b-w4a16-ctx4096", steps=2, conditioned_steps=1)
