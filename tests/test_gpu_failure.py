"""GPU tests of the failure path and of boundary positions.

The timeout path is forced from the host: a spin limit of one wall-clock tick makes the first
hand-off poll that has to wait give up (every wait in the kernel is bounded, so no launch can
hang). The step is abandoned, later launches do nothing until the failure is reported (by the
next step call once the failed kernel has finished, or by amk_sync), and the model then decodes
exactly as if the failure had not happened.
"""
import numpy as np
import pytest
import torch

import decode_megakernel_cooperative_amd as D
import workloads as W
from gpu_harness import LOGIT_TOL, build

pytestmark = pytest.mark.gpu


def _good_steps(dec, orc, kv, toks, positions):
    for pos in positions:
        g = dec.step(toks[pos], pos).cpu().numpy()
        dec.sync()
        o = orc.decode_step(toks[pos], pos, kv)
        assert float(np.max(np.abs(g - o))) <= LOGIT_TOL, pos


def test_forced_timeout_is_reported_and_recovered():
    """A step that times out; a step launched right after it, before any synchronisation, does
    nothing. The failure is reported exactly once: by that second call if the failed kernel had
    already finished (the call then launches nothing), else by amk_sync."""
    wl = W.WORKLOADS["smollm2-135m-w8a16"]
    shape = wl.shape
    dec, orc, kv = build(shape, wl.weight_format, 32, 0, seed0=2)
    toks = W.gen_tokens(shape, 8, seed0=2)
    _good_steps(dec, orc, kv, toks, range(5))
    # one tick: the first poll that has to wait times out
    D.amk_set_spin_limit(dec.model, 1)
    dec.step(toks[5], 5)
    sentinel = torch.full((shape.vocab,), float("nan"), dtype=torch.float32, device="cuda")
    kv6 = dec.kv[:, :, :, 6].clone()
    reported = 0
    try:
        dec.step(toks[6], 6, logits_out=sentinel)
    except D.AmkError as e:
        assert e.status == D.amk.AMK_ERR_SYNC_TIMEOUT
        reported += 1
    torch.cuda.synchronize()
    try:
        dec.sync()
    except D.AmkError as e:
        assert e.status == D.amk.AMK_ERR_SYNC_TIMEOUT
        reported += 1
    assert reported == 1
    assert torch.isnan(sentinel).all()
    assert torch.equal(dec.kv[:, :, :, 6], kv6)
    # default bound again: the same steps now succeed and match the oracle
    D.amk_set_spin_limit(dec.model, 0)
    dec.sync()
    _good_steps(dec, orc, kv, toks, (5, 6))
    dec.close()


def test_failed_step_is_reported_by_the_next_step_call():
    """The error contract of a step call: a failure of an earlier step that has completed on the
    device is returned by the next amk_decode_step without any amk_sync (the kernel writes the
    code to pinned host memory). That call launches nothing, resets the model's device state on
    the stream, and the model then decodes as if the failure had not happened."""
    wl = W.WORKLOADS["smollm2-135m-w8a16"]
    shape = wl.shape
    dec, orc, kv = build(shape, wl.weight_format, 32, 0, seed0=4)
    toks = W.gen_tokens(shape, 10, seed0=4)
    _good_steps(dec, orc, kv, toks, range(4))
    D.amk_set_spin_limit(dec.model, 1)
    dec.step(toks[4], 4)
    torch.cuda.synchronize()  # the failed kernel has finished; no amk_sync
    D.amk_set_spin_limit(dec.model, 0)
    sentinel = torch.full((shape.vocab,), float("nan"), dtype=torch.float32, device="cuda")
    with pytest.raises(D.AmkError) as e:
        dec.step(toks[4], 4, logits_out=sentinel)
    assert e.value.status == D.amk.AMK_ERR_SYNC_TIMEOUT
    torch.cuda.synchronize()
    assert torch.isnan(sentinel).all()
    dec.sync()  # reported once: nothing left
    _good_steps(dec, orc, kv, toks, (4, 5, 6))
    dec.close()


@pytest.mark.parametrize("fmt", [D.AMK_BF16, D.AMK_W8A16, D.AMK_W4A16])
def test_last_cache_slot(fmt):
    """A step at pos = max_ctx - 1 (the cache's last slot) on a prefilled cache."""
    shape = W.ModelShape("hd128-gqa4", 512, 3, 8, 2, 128, 1376, 1000, False, 500000.0)
    max_ctx = 203
    dec, orc, kv = build(shape, fmt, max_ctx, max_ctx - 3, seed0=6)
    toks = W.gen_tokens(shape, 3, seed0=6)
    for i, pos in enumerate(range(max_ctx - 3, max_ctx)):
        g = dec.step(toks[i], pos).cpu().numpy()
        dec.sync()
        o = orc.decode_step(toks[i], pos, kv)
        assert float(np.max(np.abs(g - o))) <= LOGIT_TOL, pos
    with pytest.raises(D.AmkError):
        dec.step(toks[0], max_ctx)
    dec.close()
