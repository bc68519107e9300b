"""GPU tests of the device-resident greedy step (amk_decode_step_greedy): the input token comes
from device memory and the step writes argmax(logits), ties to the lowest index, to device memory.

Gates: the written token equals numpy.argmax of the logits the same launch wrote (exact, also on
an lm_head built to produce exact ties); a chain of launches fed only by each other's tokens
follows the oracle's free-running greedy sequence wherever the oracle's top-2 margin exceeds
5e-2, with logits within 2e-2; graph-captured chains replay the eager chain exactly; an
out-of-range device token is reported by amk_sync and leaves the model usable.
"""
import numpy as np
import pytest
import torch

import decode_megakernel_cooperative_amd as D
import workloads as W
from gpu_harness import LOGIT_TOL, MARGIN, build, log, top2_margin

pytestmark = pytest.mark.gpu

SHAPE = W.ModelShape("hd128-gqa4-greedy", 512, 3, 8, 2, 128, 1376, 1000, False, 500000.0)


def _tok(v):
    return torch.tensor([v], dtype=torch.int32, device="cuda")


def test_greedy_token_is_argmax_of_its_logits():
    """Teacher-forced steps through token tensors: the written token is exactly the lowest index of
    the maximum of the logits written by the same launch; the logits match the host-token path."""
    dec, orc, kv = build(SHAPE, D.AMK_W8A16, 64, 20, seed0=11)
    toks = W.gen_tokens(SHAPE, 8, seed0=11)
    lg = torch.empty(SHAPE.vocab, dtype=torch.float32, device="cuda")
    nxt = _tok(-1)
    for i, t in enumerate(toks):
        kv_snap = dec.kv.clone()
        dec.step_greedy(_tok(t), 20 + i, next_token_out=nxt, logits_out=lg)
        torch.cuda.synchronize()
        dec.sync()
        g = lg.cpu().numpy()
        assert int(nxt.item()) == int(np.argmax(g)), i
        # same step through the host-token entry point: identical logits
        dec.kv.copy_(kv_snap)
        ref = dec.step(t, 20 + i).cpu().numpy()
        dec.sync()
        assert np.array_equal(g.view(np.uint32), ref.view(np.uint32)), i
        o = orc.decode_step(t, 20 + i, kv)
        assert float(np.max(np.abs(g - o))) <= LOGIT_TOL
    dec.close()


@pytest.mark.parametrize("fmt", [D.AMK_BF16, D.AMK_W8A16, D.AMK_W8A16_BF16_HEAD, D.AMK_W4A16])
def test_greedy_ties_go_to_lowest_index(fmt):
    """An lm_head whose rows repeat two row patterns (+r and -r) gives logits with only two
    distinct values, each shared by hundreds of indices spread over all blocks: the token must be
    the lowest index of the larger value, and without logits (logits_out NULL) it is the same."""
    ws = W.gen_weights(SHAPE, 13)
    lm = ws[-1]
    r = lm[7].clone()
    sign = torch.where(torch.arange(SHAPE.vocab) % 3 == 1, 1.0, -1.0).to(lm.dtype)
    ws[-1] = (sign[:, None] * r[None, :]).contiguous()
    dec = D.Decoder(SHAPE, ws, fmt, 32)
    lg = torch.empty(SHAPE.vocab, dtype=torch.float32, device="cuda")
    for i, t in enumerate([3, 500, 999]):
        nxt = _tok(-1)
        dec.step_greedy(_tok(t), i, next_token_out=nxt, logits_out=lg)
        torch.cuda.synchronize()
        dec.sync()
        g = lg.cpu().numpy()
        assert len(np.unique(g)) == 2, np.unique(g)
        assert int(nxt.item()) == int(np.argmax(g)) and int(nxt.item()) in (0, 1), (i, int(nxt.item()))
    # logits_out NULL: the token alone
    nxt2 = _tok(-1)
    dec.step_greedy(_tok(999), 2, next_token_out=nxt2)
    torch.cuda.synchronize()
    dec.sync()
    assert int(nxt2.item()) == int(nxt.item())
    dec.close()


def _chain(dec, tok0, pos0, n, stream=None):
    """n greedy steps chained on the device: token i + 1 is written by step i."""
    toks = torch.empty(n + 1, dtype=torch.int32, device="cuda")
    toks[0] = tok0
    lgs = torch.empty((n, SHAPE.vocab), dtype=torch.float32, device="cuda")
    for i in range(n):
        dec.step_greedy(toks[i:i + 1], pos0 + i, next_token_out=toks[i + 1:i + 2], logits_out=lgs[i], stream=stream)
    return toks, lgs


@pytest.mark.parametrize("fmt", [D.AMK_W4A16, D.AMK_W4A16_G128], ids=["w4a16", "w4a16-g128"])
def test_greedy_w4a16_chain_follows_the_oracle(fmt):
    """A device chain on the int4 formats (int4 projections with row or group scales, bf16
    lm_head): every written token is the argmax of its own logits, and the chain is valid
    against the oracle replaying it."""
    dec, orc, kv = build(SHAPE, fmt, 40, 16, seed0=8)
    tok0 = W.gen_tokens(SHAPE, 1, seed0=8)[0]
    toks, lgs = _chain(dec, tok0, 16, 12)
    torch.cuda.synchronize()
    dec.sync()
    toks, lgs = toks.cpu().numpy(), lgs.cpu().numpy()
    checked = 0
    for i in range(12):
        assert int(toks[i + 1]) == int(np.argmax(lgs[i])), i
        o = orc.decode_step(int(toks[i]), 16 + i, kv)
        assert float(np.max(np.abs(lgs[i] - o))) <= LOGIT_TOL, i
        if top2_margin(o) > MARGIN:
            assert int(toks[i + 1]) == int(np.argmax(o)), i
            checked += 1
    log(f"  fmt {fmt} chain: {checked} of 12 steps above the margin")
    dec.close()


def test_greedy_chain_follows_the_oracle():
    """24 steps with no host involvement between launches. The oracle then replays the chain the
    GPU chose: every step's logits within 2e-2; each GPU token is the oracle's argmax where the
    oracle's top-2 margin exceeds 5e-2, and otherwise a token whose oracle logit is within twice
    the tolerance of the oracle's maximum (near-ties admit either choice)."""
    dec, orc, kv = build(SHAPE, D.AMK_W8A16, 80, 40, seed0=7)
    tok0 = W.gen_tokens(SHAPE, 1, seed0=7)[0]
    n = 24
    toks, lgs = _chain(dec, tok0, 40, n)
    torch.cuda.synchronize()
    dec.sync()
    toks, lgs = toks.cpu().numpy(), lgs.cpu().numpy()
    assert int(toks[0]) == tok0
    exact = 0
    for i in range(n):
        o = orc.decode_step(int(toks[i]), 40 + i, kv)
        assert float(np.max(np.abs(lgs[i] - o))) <= LOGIT_TOL, i
        nt = int(toks[i + 1])
        assert nt == int(np.argmax(lgs[i])), i  # the written token is the argmax of its own logits
        if top2_margin(o) > MARGIN:
            assert nt == int(np.argmax(o)), (i, nt, int(np.argmax(o)))
            exact += 1
        else:
            assert o[nt] >= o.max() - 2 * LOGIT_TOL, (i, nt, float(o[nt]), float(o.max()))
    log(f"  steps whose token the oracle fixes uniquely: {exact} of {n}")
    dec.close()


def test_greedy_chain_graph_replay():
    """The chained launches captured in a HIP graph: three replays, each after restoring the KV
    cache and the first token with eager copies, give the eager chain's tokens and logits."""
    dec, orc, kv = build(SHAPE, D.AMK_W8A16, 48, 16, seed0=14)
    tok0 = W.gen_tokens(SHAPE, 1, seed0=14)[0]
    n = 8
    kv0 = dec.kv.clone()
    ref_t, ref_l = _chain(dec, tok0, 16, n)
    torch.cuda.synchronize()
    dec.sync()
    ref_t, ref_l = ref_t.clone(), ref_l.clone()
    s = torch.cuda.Stream()
    toks = torch.empty(n + 1, dtype=torch.int32, device="cuda")
    lgs = torch.empty((n, SHAPE.vocab), dtype=torch.float32, device="cuda")
    g = torch.cuda.CUDAGraph()
    dec.kv.copy_(kv0)
    toks[0] = tok0
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=s):
        for i in range(n):
            dec.step_greedy(toks[i:i + 1], 16 + i, next_token_out=toks[i + 1:i + 2], logits_out=lgs[i])
    torch.cuda.synchronize()
    dec.sync()
    for rep in range(3):
        dec.kv.copy_(kv0)
        toks.fill_(-1)
        toks[0] = tok0
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        dec.sync()
        assert torch.equal(toks, ref_t), (rep, toks.tolist(), ref_t.tolist())
        assert torch.equal(lgs.view(torch.int32), ref_l.view(torch.int32)), rep
    del g
    dec.close()


def test_greedy_bad_device_token_is_reported():
    """Reported by amk_sync, or, once the failed step has completed, by the next step call (which
    then launches nothing); either way the model is usable afterwards."""
    dec = D.Decoder(SHAPE, W.gen_weights(SHAPE, 15), D.AMK_W8A16, 16)
    nxt = _tok(-7)
    dec.step_greedy(_tok(SHAPE.vocab), 0, next_token_out=nxt)
    torch.cuda.synchronize()
    with pytest.raises(D.AmkError) as e:
        dec.sync()
    assert e.value.status == D.amk.AMK_ERR_INVALID_ARG
    dec.step_greedy(_tok(5), 0, next_token_out=nxt)
    torch.cuda.synchronize()
    dec.sync()
    assert 0 <= int(nxt.item()) < SHAPE.vocab
    # the next step call reports a completed failure without amk_sync, and launches nothing
    dec.step_greedy(_tok(-1), 1, next_token_out=nxt)
    torch.cuda.synchronize()
    nxt.fill_(-7)
    with pytest.raises(D.AmkError) as e:
        dec.step_greedy(_tok(5), 1, next_token_out=nxt)
    assert e.value.status == D.amk.AMK_ERR_INVALID_ARG
    torch.cuda.synchronize()
    assert int(nxt.item()) == -7
    dec.sync()  # nothing left to report
    dec.step_greedy(_tok(5), 1, next_token_out=nxt)
    torch.cuda.synchronize()
    dec.sync()
    assert 0 <= int(nxt.item()) < SHAPE.vocab
    dec.close()
