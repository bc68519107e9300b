"""GPU parity of the HIP decode library against the CPU oracle (through the C ABI).

Bars: quantized weights bit-exact; logits within 2e-2 max-abs at every step; identical greedy
tokens wherever the oracle's top-2 margin exceeds 5e-2 (teacher forced). Inputs are the seeded
synthetic workloads (random N(0, 0.02) weights in the named architectures' shapes).
"""
import numpy as np
import pytest
import torch

import decode_megakernel_cooperative_amd as D
import workloads as W
from oracle.quant import quantize_rows_int4, quantize_rows_int4_g128, quantize_rows_int8
from gpu_harness import LOGIT_TOL, build, log, run_teacher_forced

pytestmark = pytest.mark.gpu


def _assert_gates(res, name):
    worst = max(res.max_abs)
    log(f"  {name}: worst max|dlogit| {worst:.3e}; greedy checked {res.greedy_checked}, mismatches {res.greedy_mismatch}")
    assert worst <= LOGIT_TOL, f"{name}: logits differ by {worst}"
    assert res.greedy_mismatch == 0, f"{name}: {res.greedy_mismatch} greedy mismatches"


def test_smollm2_bf16_full_run():
    """SmolLM2-135M shape, bf16 weights: 8 prompt tokens one per step, then 16 greedy steps."""
    wl = W.WORKLOADS["smollm2-135m-bf16"]
    dec, orc, kv = build(wl.shape, wl.weight_format, wl.max_ctx, wl.prefill_len)
    prompt = W.gen_tokens(wl.shape, wl.prompt_len)
    res = run_teacher_forced(dec, orc, kv, wl.shape, 0, prompt, wl.greedy_steps, check_kv=True, stage_steps=(0, 7, 20))
    _assert_gates(res, wl.key)
    dec.close()


def test_smollm2_w8a16_full_run_and_quantized_bytes():
    """SmolLM2-135M shape, W8A16: codes/scales bit-exact; 64 prompt + 128 greedy steps (first 32
    greedy steps under the greedy rule)."""
    wl = W.WORKLOADS["smollm2-135m-w8a16"]
    dec, orc, kv = build(wl.shape, wl.weight_format, wl.max_ctx, wl.prefill_len)
    # bit-exact quantized weights for every projection and the (tied) lm_head
    ws = W.gen_weights(wl.shape)
    specs = W.tensor_specs(wl.shape)
    checked = 0
    for i, (name, dims, kind) in enumerate(specs):
        if kind != "matrix":
            continue
        codes, scales = D.amk_export_quantized(dec.model, i, dims[0], dims[1])
        c_ref, s_ref = quantize_rows_int8(W.bf16_bits(ws[i]))
        assert np.array_equal(codes, c_ref), name
        assert np.array_equal(scales.view(np.uint32), s_ref.view(np.uint32)), name
        checked += 1
    assert checked == 1 + 7 * wl.shape.n_layers
    prompt = W.gen_tokens(wl.shape, wl.prompt_len)
    res = run_teacher_forced(dec, orc, kv, wl.shape, 0, prompt, wl.greedy_steps, greedy_window=32,
                             stage_steps=(0, 63, 191))
    _assert_gates(res, wl.key)
    dec.close()


@pytest.mark.parametrize("fmt", [D.AMK_BF16, D.AMK_W8A16, D.AMK_W4A16, D.AMK_W4A16_G128])
def test_hd128_gqa4_prefilled_multi_split(fmt):
    """A small head_dim-128, 4-queries-per-kv-head model with a 300-position prefilled cache, so
    attention runs several KV splits with a ragged last split, and ragged GEMV rows (ffn 1376
    int8 bytes = 1.34 chunks)."""
    shape = W.ModelShape("hd128-gqa4", 512, 3, 8, 2, 128, 1376, 1000, False, 500000.0)
    dec, orc, kv = build(shape, fmt, 340, 300, seed0=3)
    tok = W.gen_tokens(shape, 1, seed0=3)[0]
    res = run_teacher_forced(dec, orc, kv, shape, 300, [], 24, first_token=tok, check_kv=True, stage_steps=(0, 23))
    _assert_gates(res, f"hd128-gqa4 fmt{fmt}")
    dec.close()


@pytest.mark.parametrize("fmt", [D.AMK_BF16, D.AMK_W8A16, D.AMK_W8A16_BF16_HEAD, D.AMK_W4A16, D.AMK_W4A16_G128])
def test_two_slot_items_wide_ragged(fmt):
    """The kernel variant with two 1 KB chunk slots per GEMV item, which the library picks above
    hidden 2048 (one slot at and below): a 2560-wide model with 4416-wide SwiGLU rows, so rows
    span several chunks with a ragged last one and odd item counts, with a prefilled cache (several
    KV splits). Checks the variant choice on both sides of the boundary, then the stage checks and
    the logit and greedy gates."""
    shape = W.ModelShape("wide-ragged", 2560, 2, 20, 5, 128, 4416, 1000, False, 500000.0)
    dec, orc, kv = build(shape, fmt, 140, 100, seed0=11)
    assert dec.info().gemv_item_slots == 2
    narrow_shape = W.ModelShape("hd64-2048", 2048, 1, 32, 8, 64, 2048, 512, True, 500000.0)
    narrow = D.Decoder(narrow_shape, W.gen_weights(narrow_shape, 11), fmt, 16)
    assert narrow.info().gemv_item_slots == 1
    narrow.close()
    tok = W.gen_tokens(shape, 1, seed0=11)[0]
    res = run_teacher_forced(dec, orc, kv, shape, 100, [], 12, first_token=tok, check_kv=True, stage_steps=(0, 11))
    _assert_gates(res, f"wide-ragged fmt{fmt}")
    dec.close()


def test_g3_hd64_long_prefill_w8a16():
    """G = 3 (SmolLM2-like grouping), head_dim 64, prefill 1500: many splits per kv head."""
    shape = W.ModelShape("g3-hd64", 384, 2, 6, 2, 64, 1024, 2048, True, 10000.0)
    dec, orc, kv = build(shape, D.AMK_W8A16, 1520, 1500, seed0=5)
    tok = W.gen_tokens(shape, 1, seed0=5)[0]
    res = run_teacher_forced(dec, orc, kv, shape, 1500, [], 16, first_token=tok)
    _assert_gates(res, "g3-hd64")
    dec.close()


@pytest.mark.parametrize("fmt", [D.AMK_BF16, D.AMK_W8A16])
def test_long_split_current_position_late_in_unit(fmt):
    """8 kv heads and a 12000-position prefilled cache: with one split per block each KV split
    spans hundreds of positions, so the current position (written by this step's QKV stage on
    another block) lies far past the positions a block loads before its q arrives. Its K/V must
    come from the hand-off, not from the cache slot being written concurrently."""
    shape = W.ModelShape("hd128-kv8-long", 512, 2, 16, 8, 128, 1024, 1000, False, 500000.0)
    dec, orc, kv = build(shape, fmt, 12010, 12000, seed0=9)
    info = dec.info()
    log(f"  grid {info.grid_blocks}, max splits {info.max_splits}")
    tok = W.gen_tokens(shape, 1, seed0=9)[0]
    res = run_teacher_forced(dec, orc, kv, shape, 12000, [], 6, first_token=tok, check_kv=True)
    _assert_gates(res, f"hd128-kv8-long fmt{fmt}")
    dec.close()


@pytest.mark.parametrize("fmt", [D.AMK_BF16, D.AMK_W8A16, D.AMK_W4A16, D.AMK_W4A16_G128])
@pytest.mark.parametrize("which", ["hd128-g8", "hd64-g6"])
def test_large_query_groups(which, fmt):
    """More than 4 query heads per kv head (the kernel variant that holds 8 heads per K/V load):
    prompt steps from an empty cache (one split per kv head), then steps on a prefilled cache
    with many splits."""
    if which == "hd128-g8":
        shape = W.ModelShape("hd128-g8", 512, 2, 16, 2, 128, 1024, 1000, False, 500000.0)
    else:
        shape = W.ModelShape("hd64-g6", 384, 2, 12, 2, 64, 1024, 2000, True, 10000.0)
    dec, orc, kv = build(shape, fmt, 16, 0, seed0=4)
    toks = W.gen_tokens(shape, 6, seed0=4)
    res = run_teacher_forced(dec, orc, kv, shape, 0, toks, 4, check_kv=True)
    _assert_gates(res, f"{which} fmt{fmt} fresh")
    dec.close()
    dec, orc, kv = build(shape, fmt, 420, 400, seed0=6)
    tok = W.gen_tokens(shape, 1, seed0=6)[0]
    res = run_teacher_forced(dec, orc, kv, shape, 400, [], 6, first_token=tok, check_kv=True)
    _assert_gates(res, f"{which} fmt{fmt} prefilled")
    dec.close()


@pytest.mark.parametrize("fmt", [D.AMK_BF16, D.AMK_W8A16])
@pytest.mark.parametrize("which", ["mha-hd128", "mha-hd64"])
def test_one_query_head_per_kv_head(which, fmt):
    """Plain multi-head attention (as many kv heads as query heads): in the attention tiles only
    one of the 16 head columns of the score and value products is a real head. Prompt steps from
    an empty cache (one split per kv head), then steps on a prefilled cache with many splits."""
    if which == "mha-hd128":
        shape = W.ModelShape("mha-hd128", 512, 2, 4, 4, 128, 1024, 1000, False, 500000.0)
    else:
        shape = W.ModelShape("mha-hd64", 512, 2, 8, 8, 64, 1024, 1000, True, 10000.0)
    dec, orc, kv = build(shape, fmt, 16, 0, seed0=13)
    toks = W.gen_tokens(shape, 6, seed0=13)
    res = run_teacher_forced(dec, orc, kv, shape, 0, toks, 4, check_kv=True)
    _assert_gates(res, f"{which} fmt{fmt} fresh")
    dec.close()
    dec, orc, kv = build(shape, fmt, 420, 400, seed0=14)
    tok = W.gen_tokens(shape, 1, seed0=14)[0]
    res = run_teacher_forced(dec, orc, kv, shape, 400, [], 6, first_token=tok, check_kv=True)
    _assert_gates(res, f"{which} fmt{fmt} prefilled")
    dec.close()


@pytest.mark.parametrize("fmt", [D.AMK_BF16, D.AMK_W8A16, D.AMK_W4A16, D.AMK_W4A16_G128])
def test_lm_head_in_two_segments(fmt):
    """A vocabulary of 135168 gives every wave 33 lm_head row pairs: more than one 32-pair segment
    (operand window) per wave, so the GEMV starts a second segment mid-stage (with its own window
    and first two items)."""
    shape = W.ModelShape("big-vocab", 512, 1, 4, 2, 128, 768, 135168, True, 500000.0)
    assert shape.vocab // 2 > 32 * 2048
    dec, orc, kv = build(shape, fmt, 24, 0, seed0=9)
    toks = W.gen_tokens(shape, 4, seed0=9)
    res = run_teacher_forced(dec, orc, kv, shape, 0, toks, 3, check_kv=True)
    _assert_gates(res, f"big-vocab fmt{fmt}")
    dec.close()


@pytest.mark.parametrize("which", ["hd128", "hd64"])
def test_single_split_boundary(which):
    """A context of at most 128 positions at head_dim 128 (256 at head_dim 64: one or two
    16-position tiles per wave of one block) runs one split per kv head,
    which writes the attention output without the split merge; one position more switches to
    many splits. Steps on both sides of the switch, and the current position at the last slot of
    the single split."""
    if which == "hd128":
        shape, tstep = W.ModelShape("hd128-gqa4", 512, 3, 8, 2, 128, 1376, 1000, False, 500000.0), 128
    else:
        shape, tstep = W.ModelShape("hd64-gqa3", 576, 3, 9, 3, 64, 1536, 1000, True, 10000.0), 256
    pre = tstep - 2
    dec, orc, kv = build(shape, D.AMK_W8A16, tstep + 3, pre, seed0=11)
    tok = W.gen_tokens(shape, 1, seed0=11)[0]
    # positions tstep-2, tstep-1 (contexts tstep-1, tstep: one split), tstep, tstep+1 (many)
    res = run_teacher_forced(dec, orc, kv, shape, pre, [], 4, first_token=tok, check_kv=True)
    _assert_gates(res, f"single-split boundary {which}")
    dec.close()


@pytest.mark.parametrize("which", ["smollm2-tied", "hd128-untied"])
def test_w8a16_with_bf16_head(which):
    """Int8 projections with the lm_head kept bf16 (for a tied model the head reads the bf16
    embedding table, so the model needs no quantized copy of it)."""
    if which == "smollm2-tied":
        shape, ctx, pre = W.SMOLLM2_135M, 40, 0
    else:
        shape, ctx, pre = W.ModelShape("hd128-gqa4", 512, 3, 8, 2, 128, 1376, 1000, False, 500000.0), 340, 300
    dec, orc, kv = build(shape, W.FMT_W8A16_BF16_HEAD, ctx, pre, seed0=12)
    ref = D.Decoder(shape, W.gen_weights(shape, 12), D.AMK_W8A16, ctx)
    assert dec.info().weight_bytes < ref.info().weight_bytes if shape.tied else \
        dec.info().weight_bytes > ref.info().weight_bytes
    ref.close()
    lm_idx = 0 if shape.tied else 2 + 9 * shape.n_layers
    with pytest.raises(D.AmkError):
        D.amk_export_quantized(dec.model, lm_idx, shape.vocab, shape.hidden)
    codes, scales = D.amk_export_quantized(dec.model, 2, shape.q_dim, shape.hidden)  # q_proj of layer 0
    c_ref, s_ref = quantize_rows_int8(W.bf16_bits(W.gen_weights(shape, 12)[2]))
    assert np.array_equal(codes, c_ref) and np.array_equal(scales.view(np.uint32), s_ref.view(np.uint32))
    toks = W.gen_tokens(shape, 8, seed0=12)
    res = run_teacher_forced(dec, orc, kv, shape, pre, toks[:4], 12)
    _assert_gates(res, f"w8a16 bf16 head {which}")
    dec.close()


@pytest.mark.parametrize("fmt", [D.AMK_W4A16, D.AMK_W4A16_G128])
@pytest.mark.parametrize("which", ["smollm2-tied", "hd128-untied", "wide-ragged"])
def test_w4a16_parity(which, fmt):
    """Int4 projections (four bits per code; one scale per row, or an fp16 scale per row and 128
    columns) with the lm_head kept bf16: every projection's codes and scales bit-exact against
    the oracle's quantizer, then the per-stage checks and the logit and greedy gates over prompt
    and greedy steps (multi-split attention for the prefilled shapes). The wide shape has rows of
    2560 and 4416 columns: several 2048-column chunks per row, ragged last chunks and a ragged
    last group (4416 = 34.5 groups)."""
    if which == "smollm2-tied":
        shape, ctx, pre, n_prompt, n_greedy = W.SMOLLM2_135M, 48, 0, 16, 24
    elif which == "hd128-untied":
        shape, ctx, pre, n_prompt, n_greedy = (W.ModelShape("hd128-gqa4", 512, 3, 8, 2, 128, 1376, 1000, False,
                                                            500000.0), 340, 300, 4, 12)
    else:
        shape, ctx, pre, n_prompt, n_greedy = (W.ModelShape("wide-ragged", 2560, 2, 20, 5, 128, 4416, 1000, False,
                                                            500000.0), 140, 100, 4, 8)
    grouped = fmt == D.AMK_W4A16_G128
    dec, orc, kv = build(shape, fmt, ctx, pre, seed0=13)
    ws = W.gen_weights(shape, 13)
    checked = 0
    for i, (name, dims, kind) in enumerate(W.tensor_specs(shape)):
        if kind != "matrix" or i == 0 or (not shape.tied and i == 2 + 9 * shape.n_layers):
            continue
        codes, scales = D.amk_export_quantized(dec.model, i, dims[0], dims[1], grouped=grouped)
        c_ref, s_ref = (quantize_rows_int4_g128 if grouped else quantize_rows_int4)(W.bf16_bits(ws[i]))
        assert np.array_equal(codes, c_ref), name
        assert np.array_equal(scales.view(np.uint32), s_ref.view(np.uint32)), name
        checked += 1
    assert checked == 7 * shape.n_layers
    lm_idx = 0 if shape.tied else 2 + 9 * shape.n_layers
    with pytest.raises(D.AmkError):
        D.amk_export_quantized(dec.model, lm_idx, shape.vocab, shape.hidden)
    del ws
    toks = W.gen_tokens(shape, n_prompt, seed0=13)
    res = run_teacher_forced(dec, orc, kv, shape, pre, toks, n_greedy, check_kv=True,
                             stage_steps=(0, n_prompt + n_greedy - 1))
    _assert_gates(res, f"{'w4a16-g128' if grouped else 'w4a16'} {which}")
    dec.close()


@pytest.mark.parametrize("fmt", [D.AMK_BF16, D.AMK_W8A16])
def test_llama3_rope_scaling(fmt):
    """Llama-3.1 frequency scaling (factor 8, low 1, high 4, original context 8192) on a
    head_dim-128 model whose frequencies fall in all three bands of the rule."""
    shape = W.ModelShape("hd128-gqa4-scaled", 512, 3, 8, 2, 128, 1376, 1000, False, 500000.0,
                         rope_scaling=(8.0, 1.0, 4.0, 8192))
    dec, orc, kv = build(shape, fmt, 340, 300, seed0=10)
    tok = W.gen_tokens(shape, 1, seed0=10)[0]
    res = run_teacher_forced(dec, orc, kv, shape, 300, [], 12, first_token=tok, check_kv=True)
    _assert_gates(res, f"rope scaling fmt{fmt}")
    dec.close()


def test_determinism_and_idempotence():
    """No float atomics: repeated identical steps give bitwise-identical logits and KV entries."""
    wl = W.WORKLOADS["smollm2-135m-w8a16"]
    shape = wl.shape
    dec = D.Decoder(shape, W.gen_weights(shape), wl.weight_format, 16)
    toks = W.gen_tokens(shape, 6)
    for p, t in enumerate(toks[:5]):
        dec.step(t, p)
    outs, kvs = [], []
    for _ in range(3):
        lg = dec.step(toks[5], 5).clone()
        torch.cuda.synchronize()
        outs.append(lg.cpu())
        kvs.append(dec.kv[:, :, :, 5].clone().cpu())
    dec.sync()
    assert all(torch.equal(outs[0], o) for o in outs[1:])
    assert all(torch.equal(kvs[0], k) for k in kvs[1:])
    dec.close()


def test_invalid_arguments_rejected():
    shape = W.small_shape(hidden=128, n_layers=1, n_q_heads=2, n_kv_heads=1, head_dim=64, ffn=256, vocab=256)
    dec = D.Decoder(shape, W.gen_weights(shape), D.AMK_W8A16, 8)
    with pytest.raises(D.AmkError) as e:
        dec.step(256, 0)
    assert e.value.status == D.amk.AMK_ERR_INVALID_ARG
    with pytest.raises(D.AmkError):
        dec.step(-1, 0)
    with pytest.raises(D.AmkError):
        dec.step(0, 8)
    with pytest.raises(D.AmkError):
        D.amk_decode_step(dec.model, 0, 0, None, dec.logits)
    dec.step(0, 0)  # still usable
    torch.cuda.synchronize()
    dec.sync()
    info = dec.info()
    assert info.grid_blocks >= 1 and info.handoffs_per_step == 6 * shape.n_layers + 1
    assert D.amk_kv_cache_bytes(dec.model) == dec.kv.numel() * 2
    dec.close()
