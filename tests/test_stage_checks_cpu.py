"""CPU pins of the per-stage checker (tests/stage_checks.py) that the GPU tests run on the kernel's
stage dumps: a dump assembled from the oracle's own traced step passes, and a dump with one
planted mistake (each a plausible kernel bug) fails the stage it belongs to."""
import numpy as np
import pytest

import workloads as W
from oracle.llama import OracleModel
from stage_checks import check_step

SHAPE = W.small_shape(hidden=128, n_layers=2, n_q_heads=4, n_kv_heads=2, head_dim=32, ffn=256, vocab=512)


def _traced_step(fmt, pos=5):
    ws = W.gen_weights(SHAPE, seed0=7)
    orc = OracleModel(SHAPE, [W.bf16_bits(t) for t in ws], fmt)
    kv = W.bf16_bits(W.gen_kv_cache(SHAPE, 16, pos, seed0=7)).copy()
    tok = W.gen_tokens(SHAPE, 1, seed0=7)[0]
    tr = {}
    logits = orc.decode_step(tok, pos, kv, trace=tr)
    return orc, tok, pos, tr, kv, logits


def _dump(tr):
    parts = []
    for l in range(SHAPE.n_layers):
        parts += [tr["h"][l], tr["qkv"][l], tr["q"][l], tr["o"][l], tr["wo"][l], tr["xo"][l], tr["h2"][l],
                  tr["gu"][l], tr["m"][l], tr["wd"][l], tr["x"][l]]
    parts.append(tr["hf"])
    return np.concatenate([np.asarray(p, np.float32).reshape(-1) for p in parts])


@pytest.mark.parametrize("fmt", [W.FMT_BF16, W.FMT_W8A16, W.FMT_W4A16, W.FMT_W4A16_G128])
def test_oracle_dump_passes(fmt):
    orc, tok, pos, tr, kv, logits = _traced_step(fmt)
    r = check_step(orc, SHAPE, tok, pos, _dump(tr), kv, logits, log=lambda *a: None)
    assert r["gemv"] < 0.2  # float32 BLAS sums sit far inside the summation bound


def _offsets():
    H, F, QD, QKV = SHAPE.hidden, SHAPE.ffn, SHAPE.q_dim, SHAPE.q_dim + 2 * SHAPE.kv_dim
    sizes = dict(h=H, qkv=QKV, q=QD, o=QD, wo=H, xo=H, h2=H, gu=2 * F, m=F, wd=H, xd=H)
    off, o = {}, 0
    for k, n in sizes.items():
        off[k] = o
        o += n
    return off, o


def test_planted_mistakes_fail():
    orc, tok, pos, tr, kv, logits = _traced_step(W.FMT_W8A16)
    base = _dump(tr)
    off, S = _offsets()
    H, hd = SHAPE.hidden, SHAPE.head_dim
    l1 = S  # layer 1 starts here

    def fails(d, kv_=kv, lg=logits):
        with pytest.raises(AssertionError):
            check_step(orc, SHAPE, tok, pos, d, kv_, lg, log=lambda *a: None)

    # two output rows of the O projection swapped (wrong row index)
    d = base.copy()
    d[off["wo"] + 3], d[off["wo"] + 4] = d[off["wo"] + 4], d[off["wo"] + 3]
    fails(d)
    # one product dropped from a q row
    d = base.copy()
    Wq = orc.layers[0]["q"]
    j = int(np.argmax(np.abs(Wq.codes[0].astype(np.float64) * tr["h"][0])))
    d[off["qkv"]] -= np.float32(Wq.scales[0] * Wq.codes[0, j] * tr["h"][0][j])
    fails(d)
    # RoPE at the wrong position: q rotated by pos + 1
    from oracle.llama import apply_rope, rope_tables
    c, s = rope_tables([pos + 1], hd, SHAPE.rope_theta)
    d = base.copy()
    d[off["q"]:off["q"] + SHAPE.q_dim] = apply_rope(tr["qkv"][0][:SHAPE.q_dim].reshape(-1, hd), c[0], s[0]).reshape(-1)
    fails(d)
    # K of the position stored without RoPE
    kv2 = kv.copy()
    from oracle.numerics import f32_to_bf16_bits
    kv2[0, 0, :, pos, :] = f32_to_bf16_bits(tr["qkv"][0][SHAPE.q_dim:SHAPE.q_dim + SHAPE.kv_dim].reshape(-1, hd))
    fails(d=base, kv_=kv2)
    # attention that leaves out the current position (exclusive key range)
    from oracle.llama import attention_head
    from oracle.numerics import bf16_bits_to_f32, round_bf16
    o = np.empty((SHAPE.n_q_heads, hd), np.float32)
    G = SHAPE.n_q_heads // SHAPE.n_kv_heads
    for hq in range(SHAPE.n_q_heads):
        g = hq // G
        o[hq] = attention_head(tr["q"][1][hq * hd:(hq + 1) * hd], bf16_bits_to_f32(kv[1, 0, g, :pos]),
                               bf16_bits_to_f32(kv[1, 1, g, :pos]), orc.scale)
    d = base.copy()
    d[l1 + off["o"]:l1 + off["o"] + SHAPE.q_dim] = round_bf16(o.reshape(-1))
    fails(d)
    # SwiGLU with the gate and up roles exchanged
    from oracle.llama import silu
    F = SHAPE.ffn
    gu = tr["gu"][1]
    d = base.copy()
    d[l1 + off["m"]:l1 + off["m"] + F] = round_bf16(silu(gu[F:]) * gu[:F])
    fails(d)
    # residual that drops the O projection
    d = base.copy()
    d[off["xo"]:off["xo"] + H] = base[off["xo"]:off["xo"] + H] - base[off["wo"]:off["wo"] + H]
    fails(d)
    # a logit row of the wrong vocabulary entry
    lg = logits.copy()
    lg[[10, 11]] = lg[[11, 10]]
    fails(base, lg=lg)
