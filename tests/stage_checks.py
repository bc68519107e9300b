"""Per-stage checks of one decode step: every stage of every layer, as dumped by the kernel
(amk_set_dump), against the oracle's operation applied to the kernel's OWN input for that stage.

Errors therefore do not compound over layers, and each gate can be tight:

  * GEMV (QKV, O, gate/up, down, lm_head): the exact value sum_k w_k x_k (float64 sums of
    products that are exact in float64: bf16 or integer codes times bf16 activations), times the
    row scale, is compared with the kernel's fp32 result under the bound of a floating-point sum
    of depth n (recursive summation, error <= n * 2^-24 * sum_k |w_k x_k|). The kernel's depth is
    K/64 per lane plus a 6-level wave reduction; the gate uses n = K/32 + 16 and adds one
    rounding of the scale multiply. A wrong row, a dropped term or a wrong column order exceeds it.
  * RMSNorm and SwiGLU outputs (bf16 values): within one bf16 ulp of the oracle op (the mean of
    squares and exp may differ in the last fp32 bits, which can move a bf16 rounding).
  * RoPE and the residual adds: the same fp32 operations in the same order, so equal up to the
    cos/sin table (at most 2 fp32 ulps).
  * K/V written to the cache at the step's position: within one bf16 ulp of bf16(RoPE(k)), bf16(v).
  * attention output (bf16 values): within one bf16 ulp of the oracle's two-pass softmax over
    the kernel's q and the cache the kernel read, plus 64 fp32 roundings of sum_j a_j |v_j| (an
    output near zero is a sum with cancellation).

Large matrices are checked on a seeded sample of rows (the first and last 64 plus up to 1024
random rows); everything else on every element.
"""
from __future__ import annotations

from typing import Dict, Optional, Sequence

import numpy as np

from oracle.llama import apply_rope, attention_head, rmsnorm, rope_tables, silu
from oracle.numerics import bf16_bits_to_f32, round_bf16
from oracle.quant import dequantize_groups

SLOTS = ("h", "qkv", "q", "o", "wo", "xo", "h2", "gu", "m", "wd", "xd")


def split_dump(dump: np.ndarray, shape) -> Dict[str, list]:
    """Splits a dump (fp32, amk_set_dump layout) into per-layer arrays, plus the final norm."""
    H, F = shape.hidden, shape.ffn
    QD, QKV = shape.q_dim, shape.q_dim + 2 * shape.kv_dim
    sizes = (H, QKV, QD, QD, H, H, H, 2 * F, F, H, H)
    S = sum(sizes)
    out = {k: [] for k in SLOTS}
    for l in range(shape.n_layers):
        o = l * S
        for k, n in zip(SLOTS, sizes):
            out[k].append(dump[o:o + n])
            o += n
    out["hf"] = dump[shape.n_layers * S:shape.n_layers * S + H]
    return out


def sample_rows(n: int, seed: int, cap: int = 1024) -> np.ndarray:
    if n <= cap + 128:
        return np.arange(n)
    rng = np.random.default_rng(seed)
    mid = rng.choice(np.arange(64, n - 64), size=cap, replace=False)
    return np.unique(np.concatenate([np.arange(64), mid, np.arange(n - 64, n)]))


def _rows_f64(lin, rows):
    if getattr(lin, "gscales", None) is not None:  # group-wise int4: the exact products q * s
        return dequantize_groups(lin.codes[rows], lin.gscales[rows]).astype(np.float64), None
    if lin.codes is not None:
        return lin.codes[rows].astype(np.float64), lin.scales[rows].astype(np.float64)
    return bf16_bits_to_f32(lin.bits[rows]).astype(np.float64), None


def check_gemv(lin, x: np.ndarray, y: np.ndarray, name: str, seed: int = 0) -> float:
    """y (kernel, fp32 [lin.rows]) against the exact product of the oracle's weights with the
    kernel's input x. Returns the worst |error| / bound."""
    rows = sample_rows(lin.rows, seed)
    Wr, s = _rows_f64(lin, rows)
    x64 = np.asarray(x, np.float64)
    exact = Wr @ x64
    mag = np.abs(Wr) @ np.abs(x64)
    if s is not None:
        exact = exact * s
        mag = mag * s
    depth = lin.cols / 32 + 16
    bound = depth * 2.0 ** -24 * mag + 2.0 ** -24 * np.abs(exact) + 1e-30
    err = np.abs(np.asarray(y, np.float64)[rows] - exact)
    worst = float(np.max(err / bound))
    assert worst <= 1.0, f"{name}: GEMV error {float(np.max(err)):.3e} exceeds its summation bound " \
                         f"(worst ratio {worst:.2f}, row {int(rows[np.argmax(err / bound)])})"
    return worst


def _bf16_ulp(v: np.ndarray) -> np.ndarray:
    a = np.abs(np.asarray(v, np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return 2.0 ** (e - 7)


def check_bf16_close(got: np.ndarray, ref_f32: np.ndarray, name: str, floor=None) -> int:
    """got holds bf16 values; ref_f32 is the oracle op's fp32 result before its bf16 rounding.
    got must be the nearest or the next bf16 value, give or take `floor` (an absolute allowance
    for results that are sums with cancellation). Returns how many differ from the rounding."""
    ref_b = round_bf16(np.asarray(ref_f32, np.float32))
    got = np.asarray(got, np.float32)
    assert np.array_equal(round_bf16(got), got), f"{name}: values are not bf16"
    d = np.abs(got.astype(np.float64) - ref_b.astype(np.float64))
    lim = _bf16_ulp(ref_b) * 1.0001 + 1e-37 + (0.0 if floor is None else np.asarray(floor, np.float64))
    bad = d > lim
    assert not np.any(bad), f"{name}: {int(np.sum(bad))} values more than one bf16 ulp off " \
                            f"(worst {float(np.max(d)):.3e} at {int(np.argmax(d))})"
    return int(np.sum(d > 0))


def check_f32_close(got: np.ndarray, ref: np.ndarray, name: str, ulps: int = 2) -> None:
    got = np.asarray(got, np.float32)
    ref = np.asarray(ref, np.float32)
    lim = ulps * np.spacing(np.abs(ref)) + 1e-37
    d = np.abs(got.astype(np.float64) - ref.astype(np.float64))
    assert np.all(d <= lim), f"{name}: fp32 values differ by more than {ulps} ulps " \
                             f"(worst {float(np.max(d)):.3e} at {int(np.argmax(d))})"


def check_step(orc, shape, token: int, pos: int, dump: np.ndarray, kv_gpu: np.ndarray,
               logits: np.ndarray, layers: Optional[Sequence[int]] = None, log=print) -> Dict[str, float]:
    """Checks one step. kv_gpu: the kernel's KV cache after the step (uint16 bf16 patterns,
    [L][2][nkv][max_ctx][hd]); logits: the kernel's logits of the step."""
    d = split_dump(dump, shape)
    L, hd, nq, nkv = shape.n_layers, shape.head_dim, shape.n_q_heads, shape.n_kv_heads
    G, QD, KD, F = nq // nkv, shape.q_dim, shape.kv_dim, shape.ffn
    eps = shape.rms_eps
    cos, sin = rope_tables([pos], hd, shape.rope_theta, shape.rope_scaling)
    worst = {"gemv": 0.0}
    flips = 0
    for l in (range(L) if layers is None else layers):
        W = orc.layers[l]
        x_in = bf16_bits_to_f32(orc.embed_bits[token]) if l == 0 else d["xd"][l - 1]
        # RMSNorm -> h
        flips += check_bf16_close(d["h"][l], rmsnorm(x_in, W["w_in"], eps), f"L{l} h")
        h = d["h"][l]
        # QKV projection on the kernel's h
        qkv = d["qkv"][l]
        worst["gemv"] = max(worst["gemv"], check_gemv(W["q"], h, qkv[:QD], f"L{l} q_proj", l),
                            check_gemv(W["k"], h, qkv[QD:QD + KD], f"L{l} k_proj", l),
                            check_gemv(W["v"], h, qkv[QD + KD:], f"L{l} v_proj", l))
        # RoPE of the kernel's q; K/V of this position in the cache
        q_rot = apply_rope(qkv[:QD].reshape(nq, hd), cos[0], sin[0])
        check_f32_close(d["q"][l].reshape(nq, hd), q_rot, f"L{l} q RoPE")
        k_rot = apply_rope(qkv[QD:QD + KD].reshape(nkv, hd), cos[0], sin[0])
        kc = bf16_bits_to_f32(kv_gpu[l, 0, :, pos, :])
        vc = bf16_bits_to_f32(kv_gpu[l, 1, :, pos, :])
        flips += check_bf16_close(kc, k_rot, f"L{l} K[pos]")
        flips += check_bf16_close(vc, qkv[QD + KD:].reshape(nkv, hd), f"L{l} V[pos]")
        # attention over the cache the kernel read, with the kernel's q. An output is a weighted
        # sum of values with cancellation; besides one bf16 ulp, it may carry 64 fp32 roundings of
        # the sum of |weight * value| (that sum is the same softmax applied to |V|)
        o_ref = np.empty((nq, hd), np.float32)
        o_mag = np.empty((nq, hd), np.float32)
        for g in range(nkv):
            Kc = bf16_bits_to_f32(kv_gpu[l, 0, g, :pos + 1, :])
            Vc = bf16_bits_to_f32(kv_gpu[l, 1, g, :pos + 1, :])
            for hq in range(g * G, (g + 1) * G):
                qh = d["q"][l][hq * hd:(hq + 1) * hd]
                o_ref[hq] = attention_head(qh, Kc, Vc, orc.scale)
                o_mag[hq] = attention_head(qh, Kc, np.abs(Vc), orc.scale)
        flips += check_bf16_close(d["o"][l], o_ref.reshape(-1), f"L{l} attention",
                                  floor=64 * 2.0 ** -24 * o_mag.reshape(-1))
        # O projection and residual
        worst["gemv"] = max(worst["gemv"], check_gemv(W["o"], d["o"][l], d["wo"][l], f"L{l} o_proj", l))
        check_f32_close(d["xo"][l], x_in + d["wo"][l], f"L{l} residual after O", ulps=0)
        # RMSNorm 2, gate/up, SwiGLU
        flips += check_bf16_close(d["h2"][l], rmsnorm(d["xo"][l], W["w_post"], eps), f"L{l} h2")
        gu = d["gu"][l]
        worst["gemv"] = max(worst["gemv"], check_gemv(W["gate"], d["h2"][l], gu[:F], f"L{l} gate_proj", l),
                            check_gemv(W["up"], d["h2"][l], gu[F:], f"L{l} up_proj", l))
        flips += check_bf16_close(d["m"][l], silu(gu[:F]) * gu[F:], f"L{l} SwiGLU")
        # down projection and residual
        worst["gemv"] = max(worst["gemv"], check_gemv(W["down"], d["m"][l], d["wd"][l], f"L{l} down_proj", l))
        check_f32_close(d["xd"][l], d["xo"][l] + d["wd"][l], f"L{l} residual after down", ulps=0)
    if layers is None or (L - 1) in layers:
        flips += check_bf16_close(d["hf"], rmsnorm(d["xd"][L - 1], orc.w_norm, eps), "final norm")
        worst["gemv"] = max(worst["gemv"], check_gemv(orc.lm_head, d["hf"], logits, "lm_head", L))
    worst["bf16_flips"] = flips
    log(f"    stages at pos {pos}: worst GEMV error / bound {worst['gemv']:.3f}, "
        f"one-ulp bf16 differences {flips}")
    return worst
