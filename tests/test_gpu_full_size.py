"""GPU parity at the full sizes of the measured workloads, in the launch configuration bench.py
times (one persistent launch of one block per compute unit per token, at the workload's
positions, on the workload's prefilled cache).

Two kinds of gate run on every workload:

1. Per stage, depth-independent and tight. The first, middle and last steps run with the
   kernel's stage dump on, and every stage of every layer is checked against the oracle's operation applied to the
   kernel's own input for that stage (stage_checks.py): each GEMV (sampled rows) within the
   float32 summation bound of the exact product, RMSNorm / SwiGLU / attention outputs within one
   bf16 ulp, RoPE and the residual adds to the same fp32 operations, the K/V written at the
   position within one bf16 ulp.
2. End to end, teacher forced, over 32 steps (Llama-3.2-1B and Llama-3-8B W8A16) or 8 steps
   (8B bf16, 8B W8A16 at 32k, 8B W8A16 with a bf16 lm_head, 8B W4A16 with row and with group
   scales): logits within tol of the oracle at every step, and
   identical greedy tokens wherever the oracle's top-2 margin exceeds `margin`. At these widths the
   max-abs over 128256 logits is sensitive to summation order: two valid orders of the oracle
   itself (float32 vs float64 sums) land 2-5e-2 apart on the 1B model and ~6-11e-2 apart on the
   8B model, more than the 2e-2 the workload states, and that distance varies by a factor ~2.5
   from one step to the next. So the gate is conditioned on the workload's spread, the largest
   such distance over the run, measured by the oracle alone: tol = max(2e-2, 2 x spread) and
   margin = max(5e-2, 2 x tol) (gpu_harness.conditioned_tolerance). Where the spread is below
   1e-2 this is the stated 2e-2 / 5e-2 rule.
3. The stated greedy rule itself, asserted as well: at every teacher-forced step where the
   oracle's top-2 margin exceeds 5e-2 (27 of 32 steps on the 1B and 8B W8A16 runs), the GPU's
   argmax is the oracle's. The kernel is deterministic, so this is a fixed property of these
   seeded inputs; a flip at a margin below 2 x tol would be a near-tie that both results, each
   within tol of the oracle, may legitimately resolve either way, and the float64-sum distance
   logged beside it (GPU and float32 oracle, each against the oracle with float64 sums) is what
   tells such a flip from a defect.
4. Distance to the oracle run with float64 sums: the GPU's worst max-abs distance to it is at
   most 1.5 x the float32 oracle's own (measured 0.94-1.24 x on these workloads). Both are
   float32 evaluations of the same definition in different summation orders, so the exact-sum
   result is a common reference and neither should sit much farther from it than the other.
"""
import gc

import numpy as np
import pytest

import workloads as W
from gpu_harness import build, log, run_teacher_forced

pytestmark = pytest.mark.gpu

CASES = [
    ("llama3.2-1b-w8a16-ctx1024", 32),
    ("llama3-8b-w8a16-ctx4096", 32),
    ("llama3-8b-bf16-ctx4096", 8),
    ("llama3-8b-w8a16-ctx32768", 8),
    ("llama3-8b-w8a16hb-ctx4096", 8),
    ("llama3-8b-w4a16-ctx4096", 8),
    ("llama3-8b-w4a16g-ctx4096", 8),
]


@pytest.mark.parametrize("key,steps", CASES)
def test_full_size(key, steps):
    wl = W.WORKLOADS[key]
    dec, orc, kv = build(wl.shape, wl.weight_format, wl.first_pos + steps + 1, wl.prefill_len,
                         oracle_threads=16, oracle_f64=True)
    tok = W.gen_tokens(wl.shape, 1)[0]
    res = run_teacher_forced(dec, orc, kv, wl.shape, wl.first_pos, [], steps, first_token=tok,
                             conditioned=True, stage_steps=(0, steps // 2, steps - 1))
    log(f"  {key}: {steps} steps, worst max|dlogit| {max(res.max_abs):.2e} (largest tol {max(res.tols):.2e}), "
        f"greedy {res.greedy_checked} checked / {res.greedy_mismatch} mismatched, "
        f"stage GEMV error / bound {max(res.stage_worst):.3f}")
    log(f"  {key}: stated 5e-2 rule {res.literal_checked} checked / {res.literal_mismatch} mismatched; "
        f"distance to the float64-sum oracle: GPU {res.gpu_vs_f64:.2e}, float32 oracle {res.f32_vs_f64:.2e}")
    assert res.greedy_mismatch == 0
    assert res.literal_mismatch == 0
    assert res.gpu_vs_f64 <= max(2e-2, 1.5 * res.f32_vs_f64), (res.gpu_vs_f64, res.f32_vs_f64)
    if steps >= 32:  # the expected top-2 gap of 128256 logits is ~0.1-0.3, so 32 steps always reach the rule
        assert res.greedy_checked >= 1
        assert res.literal_checked >= 16
    dec.close()
    del dec, orc, kv
    gc.collect()
