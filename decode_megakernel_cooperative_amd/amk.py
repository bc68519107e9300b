"""ctypes binding of libamk.so — argument marshalling only.

Every function mirrors one C entry point of include/amk.h under the same name. Torch is used
for device memory and streams: callers pass CUDA/HIP tensors, the binding passes their
data_ptr() and the current stream handle. Nothing here computes any part of the decode step;
if the library is missing, loading fails loudly (there is no fallback path).
"""
from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence

import numpy as np

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libamk.so")

AMK_OK = 0
AMK_ERR_INVALID_ARG = -1
AMK_ERR_UNSUPPORTED = -2
AMK_ERR_HIP = -3
AMK_ERR_COOPERATIVE = -4
AMK_ERR_SYNC_TIMEOUT = -5
AMK_ERR_OOM = -6
AMK_BF16 = 0
AMK_W8A16 = 1
AMK_W8A16_BF16_HEAD = 2
AMK_W4A16 = 3
AMK_W4A16_G128 = 4
GROUP = 128  # columns per group scale of AMK_W4A16_G128

EXPORTED = ("amk_validate_config", "amk_load_weights", "amk_decode_step", "amk_decode_step_noalloc",
            "amk_decode_step_greedy", "amk_sync",
            "amk_kv_cache_bytes", "amk_get_info", "amk_export_quantized", "amk_quantize_int8", "amk_quantize_int4",
            "amk_quantize_int4_g128",
            "amk_set_spin_limit", "amk_set_trace", "amk_set_dump", "amk_free", "amk_status_string")


class AmkError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{msg} (status {status})")
        self.status = status


class amk_config(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("n_layers", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("ffn", ctypes.c_int32),
                ("vocab", ctypes.c_int32), ("max_ctx", ctypes.c_int32), ("rms_eps", ctypes.c_float),
                ("rope_theta", ctypes.c_float), ("tied_embeddings", ctypes.c_int32),
                ("weight_format", ctypes.c_int32), ("rope_scale_factor", ctypes.c_float),
                ("rope_low_freq_factor", ctypes.c_float), ("rope_high_freq_factor", ctypes.c_float),
                ("rope_original_ctx", ctypes.c_int32)]


class amk_info(ctypes.Structure):
    _fields_ = [("grid_blocks", ctypes.c_int32), ("block_threads", ctypes.c_int32), ("lds_bytes", ctypes.c_int32),
                ("handoffs_per_step", ctypes.c_int32), ("weight_bytes", ctypes.c_int64),
                ("scratch_bytes", ctypes.c_int64), ("max_splits", ctypes.c_int32), ("device", ctypes.c_int32),
                ("dump_layer_floats", ctypes.c_int64), ("dump_floats", ctypes.c_int64),
                ("gemv_item_slots", ctypes.c_int32)]


_lib: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    """Loads libamk.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise FileNotFoundError(f"{LIB_PATH} is missing: build it with "
                                    "`python -m decode_megakernel_cooperative_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        L.amk_validate_config.argtypes = [ctypes.POINTER(amk_config), i32]
        L.amk_load_weights.argtypes = [ctypes.POINTER(amk_config), ctypes.POINTER(vp), i32, ctypes.POINTER(vp)]
        L.amk_decode_step.argtypes = [vp, i32, i32, vp, vp, vp]
        L.amk_decode_step_noalloc.argtypes = [vp, i32, i32, vp, vp, vp]
        L.amk_decode_step_greedy.argtypes = [vp, vp, i32, vp, vp, vp, vp]
        L.amk_sync.argtypes = [vp, vp]
        L.amk_kv_cache_bytes.argtypes = [vp]
        L.amk_kv_cache_bytes.restype = ctypes.c_size_t
        L.amk_get_info.argtypes = [vp, ctypes.POINTER(amk_info)]
        L.amk_export_quantized.argtypes = [vp, i32, vp, vp]
        L.amk_quantize_int8.argtypes = [vp, i64, i64, vp, vp]
        L.amk_quantize_int4.argtypes = [vp, i64, i64, vp, vp]
        L.amk_quantize_int4_g128.argtypes = [vp, i64, i64, vp, vp]
        L.amk_set_spin_limit.argtypes = [vp, ctypes.c_uint64]
        L.amk_set_trace.argtypes = [vp, vp, i32]
        L.amk_set_dump.argtypes = [vp, vp, i64]
        L.amk_free.argtypes = [vp]
        L.amk_status_string.argtypes = [ctypes.c_int]
        L.amk_status_string.restype = ctypes.c_char_p
        for name in EXPORTED:
            if name not in ("amk_kv_cache_bytes", "amk_status_string"):
                getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def _check(status: int) -> None:
    if status != AMK_OK:
        raise AmkError(status, amk_status_string(status))


def amk_status_string(status: int) -> str:
    return lib().amk_status_string(status).decode()


def make_config(shape, max_ctx: int, weight_format: int) -> amk_config:
    sc = getattr(shape, "rope_scaling", None) or (0.0, 0.0, 0.0, 0)
    return amk_config(shape.hidden, shape.n_layers, shape.n_q_heads, shape.n_kv_heads, shape.head_dim, shape.ffn,
                      shape.vocab, max_ctx, shape.rms_eps, shape.rope_theta, int(shape.tied), weight_format,
                      float(sc[0]), float(sc[1]), float(sc[2]), int(sc[3]))


def amk_load_weights(cfg: amk_config, host_tensors: Sequence) -> int:
    """host_tensors: contiguous bf16 CPU torch tensors or uint16 numpy arrays, canonical order.
    Returns the model handle (an integer address)."""
    ptrs = (ctypes.c_void_p * len(host_tensors))()
    keep = []
    for i, t in enumerate(host_tensors):
        if isinstance(t, np.ndarray):
            a = np.ascontiguousarray(t, dtype=np.uint16)
            keep.append(a)
            ptrs[i] = a.ctypes.data
        else:
            assert str(t.dtype) == "torch.bfloat16" and t.device.type == "cpu" and t.is_contiguous()
            keep.append(t)
            ptrs[i] = t.data_ptr()
    h = ctypes.c_void_p()
    _check(lib().amk_load_weights(ctypes.byref(cfg), ptrs, len(host_tensors), ctypes.byref(h)))
    return h.value


def _stream_handle(stream) -> int:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return int(getattr(stream, "cuda_stream", stream))


def amk_decode_step(model: int, token: int, pos: int, kv_cache, logits_out, stream=None) -> None:
    """kv_cache: device bf16 tensor [L][2][nkv][max_ctx][hd]; logits_out: device fp32 [V]."""
    kv = kv_cache.data_ptr() if hasattr(kv_cache, "data_ptr") else int(kv_cache or 0)
    lg = logits_out.data_ptr() if hasattr(logits_out, "data_ptr") else int(logits_out or 0)
    _check(lib().amk_decode_step(model, int(token), int(pos), kv, lg, _stream_handle(stream)))


def amk_decode_step_noalloc(model: int, token: int, pos: int, kv_cache, logits_out, stream=None) -> None:
    """As amk_decode_step, with the step's exchange words in the library's static device array."""
    _check(lib().amk_decode_step_noalloc(model, int(token), int(pos), _ptr(kv_cache), _ptr(logits_out),
                                         _stream_handle(stream)))


def _ptr(x) -> int:
    return x.data_ptr() if hasattr(x, "data_ptr") else int(x or 0)


def amk_decode_step_greedy(model: int, token_in, pos: int, kv_cache, logits_out, next_token_out,
                           stream=None) -> None:
    """token_in / next_token_out: device int32 tensors of one element (may be the same tensor);
    logits_out: device fp32 [V] or None."""
    _check(lib().amk_decode_step_greedy(model, _ptr(token_in), int(pos), _ptr(kv_cache), _ptr(logits_out),
                                        _ptr(next_token_out), _stream_handle(stream)))


def amk_sync(model: int, stream=None) -> None:
    _check(lib().amk_sync(model, _stream_handle(stream)))


def amk_kv_cache_bytes(model: int) -> int:
    return int(lib().amk_kv_cache_bytes(model))


def amk_get_info(model: int) -> amk_info:
    info = amk_info()
    _check(lib().amk_get_info(model, ctypes.byref(info)))
    return info


def amk_export_quantized(model: int, tensor_index: int, rows: int, cols: int, grouped: bool = False):
    """codes int8 [rows, cols] and scales: fp32 [rows], or [rows, ceil(cols / 128)] when grouped
    (a projection of an AMK_W4A16_G128 model)."""
    codes = np.empty((rows, cols), dtype=np.int8)
    scales = np.empty((rows, (cols + GROUP - 1) // GROUP) if grouped else rows, dtype=np.float32)
    _check(lib().amk_export_quantized(model, tensor_index, codes.ctypes.data, scales.ctypes.data))
    return codes, scales


def amk_quantize_int8(w_bits: np.ndarray):
    w = np.ascontiguousarray(w_bits, dtype=np.uint16)
    rows, cols = w.shape
    codes = np.empty((rows, cols), dtype=np.int8)
    scales = np.empty(rows, dtype=np.float32)
    _check(lib().amk_quantize_int8(w.ctypes.data, rows, cols, codes.ctypes.data, scales.ctypes.data))
    return codes, scales


def amk_quantize_int4(w_bits: np.ndarray):
    w = np.ascontiguousarray(w_bits, dtype=np.uint16)
    rows, cols = w.shape
    codes = np.empty((rows, cols), dtype=np.int8)
    scales = np.empty(rows, dtype=np.float32)
    _check(lib().amk_quantize_int4(w.ctypes.data, rows, cols, codes.ctypes.data, scales.ctypes.data))
    return codes, scales


def amk_quantize_int4_g128(w_bits: np.ndarray):
    w = np.ascontiguousarray(w_bits, dtype=np.uint16)
    rows, cols = w.shape
    codes = np.empty((rows, cols), dtype=np.int8)
    scales = np.empty((rows, (cols + GROUP - 1) // GROUP), dtype=np.float32)
    _check(lib().amk_quantize_int4_g128(w.ctypes.data, rows, cols, codes.ctypes.data, scales.ctypes.data))
    return codes, scales


def amk_set_spin_limit(model: int, ticks: int) -> None:
    _check(lib().amk_set_spin_limit(model, int(ticks)))


def amk_set_trace(model: int, trace, events_per_block: int) -> None:
    """trace: device uint64/int64 tensor [grid_blocks][events_per_block], or None to stop tracing."""
    ptr = trace.data_ptr() if trace is not None else None
    _check(lib().amk_set_trace(model, ptr, int(events_per_block)))


def amk_set_dump(model: int, dump) -> None:
    """dump: device fp32 tensor of at least amk_get_info(model).dump_floats elements, or None."""
    ptr = dump.data_ptr() if dump is not None else None
    n = dump.numel() if dump is not None else 0
    _check(lib().amk_set_dump(model, ptr, int(n)))


def amk_validate_config(cfg: amk_config, compute_units: int) -> None:
    """Raises AmkError if the library would refuse this model on a device with that many CUs."""
    _check(lib().amk_validate_config(ctypes.byref(cfg), int(compute_units)))


def amk_free(model: int) -> None:
    _check(lib().amk_free(model))


class Decoder:
    """Holds one loaded model plus its caller-owned KV cache and logits buffer (device tensors)."""

    def __init__(self, shape, host_tensors: Sequence, weight_format: int, max_ctx: int, device: str = "cuda:0",
                 kv_cache=None):
        import torch
        self.shape = shape
        self.max_ctx = max_ctx
        self.device = torch.device(device)
        with torch.cuda.device(self.device):
            self.model = amk_load_weights(make_config(shape, max_ctx, weight_format), host_tensors)
            nbytes = amk_kv_cache_bytes(self.model)
            if kv_cache is None:
                kv_cache = torch.zeros((shape.n_layers, 2, shape.n_kv_heads, max_ctx, shape.head_dim),
                                       dtype=torch.bfloat16, device=self.device)
            assert kv_cache.dtype == torch.bfloat16 and kv_cache.is_contiguous()
            assert kv_cache.numel() * 2 == nbytes, (kv_cache.shape, nbytes)
            self.kv = kv_cache
            self.logits = torch.empty(shape.vocab, dtype=torch.float32, device=self.device)

    def step(self, token: int, pos: int, logits_out=None, stream=None):
        out = self.logits if logits_out is None else logits_out
        amk_decode_step(self.model, token, pos, self.kv, out, stream)
        return out

    def step_greedy(self, token_in, pos: int, next_token_out=None, logits_out=None, stream=None):
        """Device-resident greedy step: reads the input token from the int32 device tensor
        token_in, writes the argmax token into next_token_out (default: token_in, in place) and,
        if logits_out is given, the logits."""
        nxt = token_in if next_token_out is None else next_token_out
        amk_decode_step_greedy(self.model, token_in, pos, self.kv, logits_out, nxt, stream)
        return nxt

    def sync(self, stream=None):
        amk_sync(self.model, stream)

    def info(self) -> amk_info:
        return amk_get_info(self.model)

    def close(self):
        if getattr(self, "model", None):
            amk_free(self.model)
            self.model = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
