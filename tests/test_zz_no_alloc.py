"""GPU test of amk_decode_step_noalloc (the step whose exchange words live in the library's
static device array): through the C ABI, its logits and KV writes equal amk_decode_step's bit
for bit, on calls in a row, each with a smaller model and a shorter context than the one before
(so it reuses a smaller part of the array that the earlier calls left written). The first model
is wide enough for the kernel variant with two-slot GEMV items, the others use one-slot items."""
import pytest
import torch

import decode_megakernel_cooperative_amd as D
import workloads as W
from gpu_harness import log

pytestmark = pytest.mark.gpu


def _pair(shape, fmt, max_ctx, prefill, seed0):
    ws = W.gen_weights(shape, seed0)
    kv = W.gen_kv_cache(shape, max_ctx, prefill, seed0).cuda()
    a = D.Decoder(shape, ws, fmt, max_ctx, kv_cache=kv.clone())
    b = D.Decoder(shape, ws, fmt, max_ctx, kv_cache=kv.clone())
    return a, b


def _compare(a, b, tok, pos):
    la = torch.full((a.shape.vocab,), float("nan"), device="cuda")
    lb = torch.full((b.shape.vocab,), float("nan"), device="cuda")
    D.amk_decode_step(a.model, tok, pos, a.kv, la)
    D.amk_decode_step_noalloc(b.model, tok, pos, b.kv, lb)
    torch.cuda.synchronize()
    a.sync()
    b.sync()
    assert torch.equal(la.view(torch.int32), lb.view(torch.int32)), f"logits differ at pos {pos}"
    assert torch.equal(a.kv, b.kv), f"KV caches differ after pos {pos}"
    return float(la.abs().max())


def test_noalloc_step_matches_the_allocating_step():
    wide = W.ModelShape("wide-ragged", 2560, 2, 20, 5, 128, 4416, 1000, False, 500000.0)
    big = W.ModelShape("hd128-gqa4", 512, 3, 8, 2, 128, 1376, 1000, False, 500000.0)
    small = W.ModelShape("hd64-gqa3", 576, 2, 9, 3, 64, 1536, 800, True, 10000.0)
    a, b = _pair(wide, D.AMK_W8A16, 210, 200, 10)
    assert a.info().gemv_item_slots == 2
    wide_bytes = a.info().scratch_bytes
    for i, t in enumerate(W.gen_tokens(wide, 2, seed0=10)):  # several splits per kv head
        _compare(a, b, t, 200 + i)
    a.close()
    b.close()
    a, b = _pair(big, D.AMK_W8A16, 340, 300, 11)
    assert a.info().gemv_item_slots == 1
    big_bytes = a.info().scratch_bytes
    assert big_bytes < wide_bytes
    toks = W.gen_tokens(big, 3, seed0=11)
    for i, t in enumerate(toks):  # several splits per kv head: partials and merge words in use
        _compare(a, b, t, 300 + i)
    a.close()
    b.close()
    a, b = _pair(small, D.AMK_W8A16, 40, 5, 12)
    assert a.info().scratch_bytes < big_bytes
    toks = W.gen_tokens(small, 2, seed0=12)
    for i, t in enumerate(toks):  # one split: a smaller context in the same array
        _compare(a, b, t, 5 + i)
    # the no-alloc step still rejects bad arguments on the host
    with pytest.raises(D.AmkError) as e:
        D.amk_decode_step_noalloc(b.model, small.vocab, 7, b.kv, b.logits)
    assert e.value.status == D.amk.AMK_ERR_INVALID_ARG
    a.close()
    b.close()
    log("  no-alloc step: bit-identical to amk_decode_step on all three models")
