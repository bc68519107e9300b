"""Symmetric per-output-row int8 (W8A16) and int4 (W4A16) weight quantizers — oracle, test
infrastructure only.

The pages report a search-found int8 weight-only (W8A16) megakernel that is greedy-lossless
(AutoMegaKernel paper index, Abstract; gist.science explainer, Technical Summary > Key
Contributions) but do not state the granularity, scale format or rounding. The reading used
here is the one the W8A16 workload states: symmetric int8 per output channel with an fp32
scale equal to max|row| / 127. Every remaining choice is fixed as follows, because exact ties
are common enough at these shapes that the choice changes bytes:

    amax_n = max_k |w_nk|                       (bf16 -> fp32 is exact)
    s_n    = fp32(amax_n / 127)                 IEEE fp32 division, round to nearest even
    q_nk   = clamp(round_half_even(fp32(w_nk / s_n)), -127, 127)   fp32 *division*
    amax_n == 0  ->  s_n = 0, q_n = 0

Dequantized weight: w'_nk = q_nk * s_n; a W8A16 GEMV row is s_n * sum_k q_nk * x_k.

int4 (W4A16). The pages list an int4 weight-only variant as lossy with 2.42x less weight traffic
than bf16 (gist.science explainer, Technical Summary > Key Contributions) and give no format.
The reading used here is the same rule at four bits: symmetric per output row, s_n =
fp32(amax_n / 7) by IEEE division, q_nk = clamp(round_half_even(fp32(w_nk / s_n)), -7, 7), a
zero row gives s_n = 0 and q_n = 0. With the lm_head (and a tied embedding) kept in bf16 this
streams 1 / 2.44 of the bf16 weight bytes for SmolLM2-135M and for Llama-3.2-1B, which matches
the pages' figure to its precision. Codes take four bits each on the GPU side; here they are
kept one per int8.

int4 with group-wise scales (W4A16-G128). The same rule applied per group of 128 consecutive
columns of a row instead of per row, with the scale stored in IEEE half precision, the format
int4 weight-only schemes usually keep group scales in. A row whose length is not a multiple of 128
ends with one shorter group. Per group g of row n:

    amax   = max |w| over the group
    s      = fp16(amax / 7)                     IEEE fp32 division, then round to nearest even
                                                to fp16 (magnitudes past the fp16 range saturate
                                                to 65504)
    q      = clamp(round_half_even(fp32(w / fp32(s))), -7, 7)    s == 0 -> q = 0
    w'     = q * s                              (exact in fp32: at most 3 + 11 significant bits)

With the lm_head kept in bf16 this streams 1 / 2.415 of the bf16 weight bytes on the
SmolLM2-135M and Llama-3.2-1B shapes, the reading closest to the pages' 2.42x.
"""
import numpy as np

from .numerics import bf16_bits_to_f32


def quantize_rows_int8(w_bits: np.ndarray, block_rows: int = 4096):
    """bf16 matrix (uint16 patterns, [rows, cols]) -> (int8 codes [rows, cols], fp32 scales [rows])."""
    w_bits = np.asarray(w_bits, dtype=np.uint16)
    assert w_bits.ndim == 2
    return _quantize(w_bits, bf16_bits_to_f32, block_rows, 127)


def quantize_rows_int8_f32(w: np.ndarray, block_rows: int = 4096):
    """The same quantizer applied to fp32 rows (used to re-quantize dequantized weights)."""
    w = np.asarray(w, dtype=np.float32)
    assert w.ndim == 2
    return _quantize(w, lambda a: a, block_rows, 127)


def quantize_rows_int4(w_bits: np.ndarray, block_rows: int = 4096):
    """bf16 matrix (uint16 patterns) -> (codes in [-7, 7] as int8 [rows, cols], fp32 scales [rows])."""
    w_bits = np.asarray(w_bits, dtype=np.uint16)
    assert w_bits.ndim == 2
    return _quantize(w_bits, bf16_bits_to_f32, block_rows, 7)


def quantize_rows_int4_f32(w: np.ndarray, block_rows: int = 4096):
    """The int4 quantizer applied to fp32 rows (used to re-quantize dequantized weights)."""
    w = np.asarray(w, dtype=np.float32)
    assert w.ndim == 2
    return _quantize(w, lambda a: a, block_rows, 7)


def _quantize(src: np.ndarray, widen, block_rows: int, qmax: int):
    rows, cols = src.shape
    codes = np.empty((rows, cols), dtype=np.int8)
    scales = np.empty(rows, dtype=np.float32)
    for r0 in range(0, rows, block_rows):
        r1 = min(rows, r0 + block_rows)
        w = widen(src[r0:r1])
        amax = np.max(np.abs(w), axis=1)
        s = (amax / np.float32(qmax)).astype(np.float32)
        zero = s == 0
        s_safe = np.where(zero, np.float32(1.0), s).astype(np.float32)
        q = np.rint(w / s_safe[:, None])  # float32 / float32 stays float32; rint = half-even
        q = np.clip(q, -qmax, qmax)
        q[zero] = 0
        codes[r0:r1] = q.astype(np.int8)
        scales[r0:r1] = np.where(zero, np.float32(0.0), s)
    return codes, scales


GROUP = 128
FP16_MAX = 65504.0


def quantize_rows_int4_g128(w_bits: np.ndarray, block_rows: int = 2048):
    """bf16 matrix (uint16 patterns, [rows, cols]) -> (codes in [-7, 7] as int8 [rows, cols],
    fp16 group scales as float32 [rows, ceil(cols / 128)])."""
    w_bits = np.asarray(w_bits, dtype=np.uint16)
    assert w_bits.ndim == 2
    return _quantize_groups(w_bits, bf16_bits_to_f32, block_rows)


def quantize_rows_int4_g128_f32(w: np.ndarray, block_rows: int = 2048):
    """The group-wise int4 quantizer applied to fp32 rows (used to re-quantize dequantized weights)."""
    w = np.asarray(w, dtype=np.float32)
    assert w.ndim == 2
    return _quantize_groups(w, lambda a: a, block_rows)


def _quantize_groups(src: np.ndarray, widen, block_rows: int):
    rows, cols = src.shape
    ng = (cols + GROUP - 1) // GROUP
    codes = np.empty((rows, cols), dtype=np.int8)
    scales = np.empty((rows, ng), dtype=np.float32)
    for r0 in range(0, rows, block_rows):
        r1 = min(rows, r0 + block_rows)
        w = widen(src[r0:r1])
        for g in range(ng):
            c0, c1 = g * GROUP, min(cols, (g + 1) * GROUP)
            wg = w[:, c0:c1]
            amax = np.max(np.abs(wg), axis=1)
            s32 = (amax / np.float32(7)).astype(np.float32)
            s = np.minimum(s32, np.float32(FP16_MAX)).astype(np.float16).astype(np.float32)  # RNE to fp16
            zero = s == 0
            s_safe = np.where(zero, np.float32(1.0), s).astype(np.float32)
            q = np.clip(np.rint(wg / s_safe[:, None]), -7, 7)
            q[zero] = 0
            codes[r0:r1, c0:c1] = q.astype(np.int8)
            scales[r0:r1, g] = s
    return codes, scales


def dequantize_groups(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """int4 codes and per-group scales [rows, ceil(cols / 128)] -> fp32 weights q * s (exact)."""
    rows, cols = codes.shape
    s = np.repeat(np.asarray(scales, np.float32), GROUP, axis=1)[:, :cols]
    return codes.astype(np.float32) * s


def dequantize_rows(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """int8 codes and fp32 row scales -> fp32 weights q * s."""
    return codes.astype(np.float32) * np.asarray(scales, dtype=np.float32)[:, None]
