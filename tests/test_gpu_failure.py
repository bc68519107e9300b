"""GPU tests of the failure path and of boundary positions.

The timeout path is forced from the host: a spin limit of one wall-clock tick makes the first
hand-off poll that has to wait give up (every wait in the kernel is bounded, so no launch can
hang). The step is abandoned, later launches do nothing until amk_sync reports it, and the model
then decodes exactly as if the failure had not happened.
"""
import numpy as np
import pytest
import torch

import decode_megakernel_cooperative_amd as D
import workloads as W
from gpu_harness import LOGIT_TOL, build

pytestmark = pytest.mark.gpu


def test_forced_timeout_is_reported_and_recovered():
    wl = W.WORKLOADS["smollm2-135m-w8a16"]
    shape = wl.shape
    dec, orc, kv = build(shape, wl.weight_format, 32, 0, seed0=2)
    toks = W.gen_tokens(shape, 8, seed0=2)
    for pos in range(5):
        g = dec.step(toks[pos], pos).cpu().numpy()
        dec.sync()
        o = orc.decode_step(toks[pos], pos, kv)
        assert float(np.max(np.abs(g - o))) <= LOGIT_TOL
    # one tick: the first poll that has to wait times out
    D.amk_set_spin_limit(dec.model, 1)
    dec.step(toks[5], 5)
    # launched after the failure and before amk_sync: must do nothing
    sentinel = torch.full((shape.vocab,), float("nan"), dtype=torch.float32, device="cuda")
    kv6 = dec.kv[:, :, :, 6].clone()
    dec.step(toks[6], 6, logits_out=sentinel)
    torch.cuda.synchronize()
    with pytest.raises(D.AmkError) as e:
        dec.sync()
    assert e.value.status == D.amk.AMK_ERR_SYNC_TIMEOUT
    assert torch.isnan(sentinel).all()
    assert torch.equal(dec.kv[:, :, :, 6], kv6)
    # default bound again: the same step now succeeds and matches the oracle
    D.amk_set_spin_limit(dec.model, 0)
    dec.sync()
    for pos in (5, 6):
        g = dec.step(toks[pos], pos).cpu().numpy()
        dec.sync()
        o = orc.decode_step(toks[pos], pos, kv)
        assert float(np.max(np.abs(g - o))) <= LOGIT_TOL, pos
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
