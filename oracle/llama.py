"""Plain NumPy float32 Llama decode step — oracle, test infrastructure only.

Definition followed. The pages say the megakernel runs the whole forward pass of a
HuggingFace Llama-family model for one decoded token in one launch and reproduces eager
HuggingFace greedy decode (AutoMegaKernel paper index, Abstract; gist.science explainer,
Technical Summary > Problem Statement, Methodology, Experimental Results). The op list of
that step (RMSNorm, GEMV, attention "etc.", Methodology > Layer 1) is the HF
``LlamaForCausalLM`` decode step, written out here one operation at a time:

    x   = fp32(E[token])                                   residual stream, fp32 throughout
    per layer l:
      h   = bf16((x * rsqrt(mean(x^2) + eps)) * w_in)
      q,k,v = W_q h, W_k h, W_v h                          fp32 results
      q,k = RoPE(q, pos), RoPE(k, pos)                     rotate-half pairs (i, i + hd/2)
      K[l,g,pos], V[l,g,pos] = bf16(k_g), bf16(v_g)
      o_h = softmax((q_h . K[l,g]) / sqrt(hd)) . V[l,g]   g = h // (n_q / n_kv), keys [0, pos]
      x   = x + W_o bf16(o)
      h2  = bf16((x * rsqrt(mean(x^2) + eps)) * w_post)
      x   = x + W_d bf16(silu(W_g h2) * (W_u h2))
    logits = W_lm bf16((x * rsqrt(mean(x^2) + eps)) * w_norm)  fp32

Readings where the pages are silent (each listed with its reason in the design notes):
activations are rounded to bf16 exactly at GEMV inputs and at KV-cache storage, q, scores,
softmax, gate/up and logits stay fp32; the W8A16 GEMV is s_n * sum_k q_nk x_k with the row
scale applied once after the fp32 sum; RoPE angles are computed in float64 and rounded to
fp32 cos/sin, with no frequency scaling; all seven per-layer projections and the lm_head are
int8 under W8A16 while the embedding gather reads the bf16 table. W4A16 quantizes the seven
projections to int4 codes with the same per-row rule (scale max|row| / 7) and keeps the lm_head
bf16; its GEMV is the same s_n * sum_k q_nk x_k. W4A16-G128 quantizes them with one fp16 scale per
group of 128 columns (oracle.quant) and keeps the lm_head bf16; its GEMV is the plain product
with the dequantized weights, sum_k (q_nk * s_n,g(k)) x_k (each q * s is exact in fp32).
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence

import numpy as np

from .numerics import bf16_bits_to_f32, f32_to_bf16_bits, round_bf16
from .quant import dequantize_groups, quantize_rows_int4, quantize_rows_int4_g128, quantize_rows_int8

F32 = np.float32
FMT_BF16 = 0
FMT_W8A16 = 1
FMT_W8A16_BF16_HEAD = 2  # W8A16 projections, lm_head kept in bf16
FMT_W4A16 = 3            # int4 projections (per-row scale), lm_head kept in bf16
FMT_W4A16_G128 = 4       # int4 projections (fp16 scale per group of 128 columns), lm_head kept in bf16


# ------------------------------------------------------------------------------------------
# primitive operations
# ------------------------------------------------------------------------------------------
def rmsnorm(x: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """(x * 1/sqrt(mean(x^2) + eps)) * w in float32 (before the bf16 rounding of the caller)."""
    x = np.asarray(x, dtype=F32)
    ms = np.mean(x * x, dtype=F32)
    r = F32(1.0) / np.sqrt(ms + F32(eps), dtype=F32)
    return (x * r) * np.asarray(w, dtype=F32)


def scaled_inv_freq(inv_freq: np.ndarray, scaling) -> np.ndarray:
    """Llama-3 RoPE frequency scaling (the rule Llama 3.1 / 3.2 checkpoints declare; the pages
    do not describe it). scaling = (factor, low_freq_factor, high_freq_factor, original_ctx).
    A frequency whose wavelength 2 pi / f is shorter than original_ctx / high_freq_factor is
    kept; one longer than original_ctx / low_freq_factor is divided by factor; in between, the
    result moves linearly in original_ctx / wavelength from f / factor (at low_freq_factor) to
    f (at high_freq_factor). Float64 throughout."""
    factor, low, high, orig = (float(v) for v in scaling)
    out = np.empty_like(inv_freq)
    for i, f in enumerate(inv_freq):
        wavelen = 2.0 * np.pi / f
        if wavelen < orig / high:
            out[i] = f
        elif wavelen > orig / low:
            out[i] = f / factor
        else:
            t = (orig / wavelen - low) / (high - low)
            out[i] = (1.0 - t) * f / factor + t * f
    return out


def rope_tables(positions: Sequence[int] | np.ndarray, head_dim: int, theta: float, scaling=None):
    """cos, sin tables [len(positions), head_dim/2] as float32.

    inv_freq_i = theta^(-2i/hd) (then the Llama-3 scaling if `scaling` is given) and
    angle = pos * inv_freq_i are evaluated in float64, then cos/sin are rounded once to float32.
    """
    half = head_dim // 2
    i = np.arange(half, dtype=np.float64)
    inv_freq = np.power(np.float64(theta), -(2.0 * i) / head_dim)
    if scaling is not None:
        inv_freq = scaled_inv_freq(inv_freq, scaling)
    ang = np.asarray(positions, dtype=np.float64)[:, None] * inv_freq[None, :]
    return np.cos(ang).astype(F32), np.sin(ang).astype(F32)


def apply_rope(v: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Rotate-half RoPE of one head vector: pairs (i, i + hd/2) rotated by the angle of i."""
    v = np.asarray(v, dtype=F32)
    half = v.shape[-1] // 2
    a, b = v[..., :half], v[..., half:]
    out = np.empty_like(v)
    out[..., :half] = a * cos - b * sin
    out[..., half:] = b * cos + a * sin
    return out


def silu(z: np.ndarray) -> np.ndarray:
    z = np.asarray(z, dtype=F32)
    return z / (F32(1.0) + np.exp(-z, dtype=F32))


def attention_head(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: np.float32, accum=F32) -> np.ndarray:
    """One query head over keys/values [T, hd]: softmax((K q) * scale) V, two-pass.

    accum = float32 (the oracle) or float64 (the same definition with float64 sums, used only
    to measure how sensitive a workload is to summation order); the result is float32."""
    s = (np.asarray(K, dtype=accum) @ np.asarray(q, dtype=accum)) * accum(scale)
    m = np.max(s)
    e = np.exp(s - m, dtype=accum)
    a = e / np.sum(e, dtype=accum)
    return (a @ np.asarray(V, dtype=accum)).astype(F32)


def gemv(W: "Linear", x: np.ndarray) -> np.ndarray:
    return W.apply(x)


# ------------------------------------------------------------------------------------------
# weights
# ------------------------------------------------------------------------------------------
class Linear:
    """A [rows, cols] projection applied as y = W x (bf16 weights) or y = s * (Q x) (int8 or int4
    codes, one fp32 scale per row)."""

    BLOCK = 8192

    def __init__(self, bits: np.ndarray, fmt: int, widen_once: bool, widen64: bool = False):
        """widen_once keeps the weights (codes or bf16 values) widened to float32 for the life of
        the object instead of widening one row block per call; widen64 also keeps a float64 copy
        for the float64-accumulation variant. Both only trade memory for time: the values are the
        same exact integers or bf16 values either way."""
        bits = np.asarray(bits, dtype=np.uint16)
        self.rows, self.cols = bits.shape
        self.fmt = fmt
        self.codes = self.scales = self.bits = None
        self._f32 = self._f64 = None
        if fmt == FMT_W4A16_G128:
            self.codes, self.gscales = quantize_rows_int4_g128(bits)
            self._f32 = dequantize_groups(self.codes, self.gscales)  # exact values, kept (rows x cols fp32)
        elif fmt in (FMT_W8A16, FMT_W4A16):
            quantize = quantize_rows_int8 if fmt == FMT_W8A16 else quantize_rows_int4
            self.codes, self.scales = quantize(bits)
            if widen_once:
                self._f32 = self.codes.astype(F32)
        else:
            self.bits = bits
            if widen_once:
                self._f32 = bf16_bits_to_f32(bits)
        if widen_once and widen64:
            self._f64 = self._f32.astype(np.float64)

    def _block(self, r0: int, r1: int, accum=F32) -> np.ndarray:
        if accum is np.float64 and self._f64 is not None:
            return self._f64[r0:r1]
        if self._f32 is not None:
            return self._f32[r0:r1]
        if self.codes is not None:
            return self.codes[r0:r1].astype(F32)
        return bf16_bits_to_f32(self.bits[r0:r1])

    def apply(self, x: np.ndarray, accum=F32) -> np.ndarray:
        """x: [cols] or [n, cols] float32 -> [rows] or [n, rows] float32. accum = float32 (the
        oracle) or float64 (sums in float64, rounded to float32 at the end)."""
        x = np.asarray(x, dtype=F32)
        y = np.empty(x.shape[:-1] + (self.rows,), dtype=F32)
        xa = x.astype(accum)
        for r0 in range(0, self.rows, self.BLOCK):
            r1 = min(self.rows, r0 + self.BLOCK)
            W = self._block(r0, r1, accum).astype(accum, copy=False)
            acc = xa @ W.T
            if self.codes is not None and self.fmt != FMT_W4A16_G128:  # per-row scale after the sum
                acc = acc * self.scales[r0:r1].astype(accum)
            y[..., r0:r1] = acc
        return y


class OracleModel:
    """A random- or caller-initialised Llama model evaluated by the plain definition above.

    tensors: bf16 bit patterns (uint16 arrays) in canonical HF order: embed_tokens; per layer
    input_layernorm, q_proj, k_proj, v_proj, o_proj, post_attention_layernorm, gate_proj,
    up_proj, down_proj; norm; lm_head (absent when tied).
    """

    def __init__(self, shape, tensors: List[np.ndarray], weight_format: int,
                 widen_once: Optional[bool] = None, threads: int = 1, widen64: bool = False):
        self.shape = shape
        self.fmt = weight_format
        self.accum = F32  # float64 only to measure a workload's sensitivity to summation order
        L = shape.n_layers
        assert len(tensors) == 2 + 9 * L + (0 if shape.tied else 1)
        n_params = sum(int(np.asarray(t).size) for t in tensors)
        if widen_once is None:
            widen_once = n_params <= 2_000_000_000
        self.embed_bits = np.asarray(tensors[0], dtype=np.uint16)
        lm_bits = self.embed_bits if shape.tied else tensors[2 + 9 * L]
        # the projections are independent; `threads` only spreads their construction
        # (quantization / widening) over a thread pool, the arithmetic is the same
        mats = [tensors[1 + 9 * l + o] for l in range(L) for o in (1, 2, 3, 4, 6, 7, 8)] + [lm_bits]
        proj_fmt = {FMT_BF16: FMT_BF16, FMT_W8A16: FMT_W8A16, FMT_W8A16_BF16_HEAD: FMT_W8A16,
                    FMT_W4A16: FMT_W4A16, FMT_W4A16_G128: FMT_W4A16_G128}[weight_format]
        lm_fmt = FMT_W8A16 if weight_format == FMT_W8A16 else FMT_BF16
        fmts = [proj_fmt] * (len(mats) - 1) + [lm_fmt]
        if threads > 1:
            from concurrent.futures import ThreadPoolExecutor
            with ThreadPoolExecutor(threads) as ex:
                lins = list(ex.map(lambda bf: Linear(bf[0], bf[1], widen_once, widen64), zip(mats, fmts)))
        else:
            lins = [Linear(b, f, widen_once, widen64) for b, f in zip(mats, fmts)]
        self.layers: List[Dict[str, object]] = []
        for l in range(L):
            t = tensors[1 + 9 * l: 1 + 9 * (l + 1)]
            q, k, v, o, gate, up, down = lins[7 * l: 7 * (l + 1)]
            self.layers.append({"w_in": bf16_bits_to_f32(t[0]), "q": q, "k": k, "v": v, "o": o,
                                "w_post": bf16_bits_to_f32(t[5]), "gate": gate, "up": up, "down": down})
        self.w_norm = bf16_bits_to_f32(tensors[1 + 9 * L])
        self.lm_head = lins[-1]
        self.scale = F32(1.0) / np.sqrt(F32(shape.head_dim), dtype=F32)

    # --------------------------------------------------------------------------------------
    def decode_step(self, token: int, pos: int, kv: np.ndarray,
                    trace: Optional[dict] = None, layers: Optional[Sequence[int]] = None) -> np.ndarray:
        """Feed `token` at position `pos`; writes K/V slot `pos` of every layer into `kv`
        (uint16 bf16 patterns, [L][2][n_kv][max_ctx][hd]) and returns fp32 logits [vocab].

        `layers` restricts the pass to a subset of layers (a timing sample only)."""
        s = self.shape
        hd, nq, nkv = s.head_dim, s.n_q_heads, s.n_kv_heads
        G = nq // nkv
        assert 0 <= token < s.vocab and 0 <= pos < kv.shape[3]
        cos, sin = rope_tables([pos], hd, s.rope_theta, s.rope_scaling)
        cos, sin = cos[0], sin[0]
        x = bf16_bits_to_f32(self.embed_bits[token]).copy()
        for l in (range(s.n_layers) if layers is None else layers):
            W = self.layers[l]
            h = round_bf16(rmsnorm(x, W["w_in"], s.rms_eps))
            A = self.accum
            q = W["q"].apply(h, A).reshape(nq, hd)
            k = W["k"].apply(h, A).reshape(nkv, hd)
            v = W["v"].apply(h, A).reshape(nkv, hd)
            if trace is not None:
                trace.setdefault("qkv", []).append(np.concatenate([q.reshape(-1), k.reshape(-1), v.reshape(-1)]))
            q = apply_rope(q, cos, sin)
            k = apply_rope(k, cos, sin)
            kv[l, 0, :, pos, :] = f32_to_bf16_bits(k)
            kv[l, 1, :, pos, :] = f32_to_bf16_bits(v)
            o = np.empty((nq, hd), dtype=F32)
            for g in range(nkv):  # q heads g*G .. g*G + G - 1 read kv head g
                Kc = bf16_bits_to_f32(kv[l, 0, g, :pos + 1, :])
                Vc = bf16_bits_to_f32(kv[l, 1, g, :pos + 1, :])
                for hq in range(g * G, (g + 1) * G):
                    o[hq] = attention_head(q[hq], Kc, Vc, self.scale, A)
            wo = W["o"].apply(round_bf16(o.reshape(-1)), A)
            x = x + wo
            xo = x
            h2 = round_bf16(rmsnorm(x, W["w_post"], s.rms_eps))
            g, u = W["gate"].apply(h2, A), W["up"].apply(h2, A)
            m = round_bf16(silu(g) * u)
            wd = W["down"].apply(m, A)
            x = x + wd
            if trace is not None:
                trace.setdefault("h", []).append(h)
                trace.setdefault("q", []).append(q.reshape(-1))
                trace.setdefault("o", []).append(round_bf16(o.reshape(-1)))
                trace.setdefault("wo", []).append(wo)
                trace.setdefault("xo", []).append(xo.copy())
                trace.setdefault("h2", []).append(h2)
                trace.setdefault("gu", []).append(np.concatenate([g, u]))
                trace.setdefault("m", []).append(m)
                trace.setdefault("wd", []).append(wd)
                trace.setdefault("x", []).append(x.copy())
        hf = round_bf16(rmsnorm(x, self.w_norm, s.rms_eps))
        if trace is not None:
            trace["hf"] = hf
        return self.lm_head.apply(hf, self.accum)

    # --------------------------------------------------------------------------------------
    def sensitivity(self, token: int, pos: int, kv: np.ndarray, reference: Optional[np.ndarray] = None,
                    return_alt: bool = False):
        """max |logits(float32 sums) - logits(float64 sums)| for this step: how far two valid
        summation orders of the same definition land apart. Leaves `kv` unchanged. With
        return_alt, returns (that distance, the float64-sum logits)."""
        ref = reference if reference is not None else self.decode_step(token, pos, kv.copy())
        self.accum = np.float64
        try:
            alt = self.decode_step(token, pos, kv.copy())
        finally:
            self.accum = F32
        d = float(np.max(np.abs(ref - alt)))
        return (d, alt) if return_alt else d

    def prefill_logits(self, tokens: Sequence[int]) -> np.ndarray:
        """Independent full-sequence causal forward over `tokens` at positions 0..P-1 with a
        fresh cache, in matrix form: returns fp32 logits [P, vocab] (one row per position).

        Written separately from `decode_step` (causal mask instead of a growing cache) so the
        two can cross-check the cache indexing and the inclusive key range."""
        s = self.shape
        hd, nq, nkv = s.head_dim, s.n_q_heads, s.n_kv_heads
        G = nq // nkv
        P = len(tokens)
        cos, sin = rope_tables(np.arange(P), hd, s.rope_theta, s.rope_scaling)           # [P, hd/2]
        X = bf16_bits_to_f32(self.embed_bits[np.asarray(tokens)])         # [P, H]
        mask = np.triu(np.ones((P, P), dtype=bool), k=1)                  # True above diagonal
        for W in self.layers:
            Hn = np.stack([round_bf16(rmsnorm(X[p], W["w_in"], s.rms_eps)) for p in range(P)])
            Q = W["q"].apply(Hn).reshape(P, nq, hd)
            Kp = W["k"].apply(Hn).reshape(P, nkv, hd)
            Vp = W["v"].apply(Hn).reshape(P, nkv, hd)
            Q = apply_rope(Q, cos[:, None, :], sin[:, None, :])
            Kp = round_bf16(apply_rope(Kp, cos[:, None, :], sin[:, None, :]))
            Vp = round_bf16(Vp)
            O = np.empty((P, nq, hd), dtype=F32)
            for hq in range(nq):
                g = hq // G
                S = (Q[:, hq, :] @ Kp[:, g, :].T) * self.scale           # [P, P]
                S = np.where(mask, F32(-np.inf), S)
                S = S - S.max(axis=1, keepdims=True)
                E = np.exp(S, dtype=F32)
                A = E / E.sum(axis=1, keepdims=True, dtype=F32)
                O[:, hq, :] = A @ Vp[:, g, :]
            X = X + W["o"].apply(round_bf16(O.reshape(P, nq * hd)))
            H2 = np.stack([round_bf16(rmsnorm(X[p], W["w_post"], s.rms_eps)) for p in range(P)])
            M = round_bf16(silu(W["gate"].apply(H2)) * W["up"].apply(H2))
            X = X + W["down"].apply(M)
        Hf = np.stack([round_bf16(rmsnorm(X[p], self.w_norm, s.rms_eps)) for p in range(P)])
        return self.lm_head.apply(Hf)
