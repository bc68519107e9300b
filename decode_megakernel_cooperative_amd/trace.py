"""Summaries of the per-block stage trace written by the decode kernel (amk_set_trace).

Each block records the 100 MHz wall clock at kernel entry, at the arrival at and exit from every
grid barrier, and at the end. Per stage s (the work between barrier s-1 and barrier s) this gives
  busy   = arrival_s - exit_{s-1}       (per block)
  wait   = exit_s - arrival_s           (per block)
  skew   = last arrival_s - first arrival_s
  latency= first exit_s - last arrival_s (propagation of the last arrival to the first waiter)
"""
from __future__ import annotations

import numpy as np

TICK_US = 0.01  # 100 MHz wall clock
STAGES = ("qkv", "attn", "o_proj", "gate_up", "down")


def events_per_block(n_layers: int) -> int:
    return 2 + 2 * 5 * n_layers


def summarize(trace: np.ndarray, n_layers: int) -> dict:
    """trace: uint64 [grid][events_per_block] from one step. Returns per-stage-kind mean times in us."""
    t = trace.astype(np.int64)
    nb = 5 * n_layers
    t0 = t[:, 0]
    arr = t[:, 1:1 + 2 * nb:2]
    ext = t[:, 2:2 + 2 * nb:2]
    end = t[:, 1 + 2 * nb]
    prev_exit = np.concatenate([t0[:, None], ext[:, :-1]], axis=1)
    busy = (arr - prev_exit) * TICK_US
    wait = (ext - arr) * TICK_US
    skew = (arr.max(0) - arr.min(0)) * TICK_US
    lat = (ext.min(0) - arr.max(0)) * TICK_US
    out = {"total_us": float((end.max() - t0.min()) * TICK_US),
           "final_stage_us": float((end.max() - ext[:, -1].min()) * TICK_US)}
    for k, name in enumerate(STAGES):
        idx = np.arange(k, nb, 5)
        out[name] = {
            "busy_max_us": float(busy[:, idx].max(0).mean()),
            "busy_mean_us": float(busy[:, idx].mean()),
            "wait_mean_us": float(wait[:, idx].mean()),
            "skew_us": float(skew[idx].mean()),
            "latency_us": float(lat[idx].mean()),
            "span_us": float(((ext.max(0) - np.concatenate([[t0.min()], ext.max(0)[:-1]]))[idx]).mean() * TICK_US),
        }
    return out
