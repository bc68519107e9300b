"""Summaries of the per-block stage trace written by the decode kernel (amk_set_trace).

Each block records the 100 MHz wall clock at kernel entry (event 0), then 11 events per layer
(event 1 + 11 l + k, k indexing STAGES: the end of that stage in this block), then the final
RMSNorm (1 + 11 L) and the end of the lm_head (2 + 11 L). A stage's per-block duration is its
event minus the block's previous event. Stages whose name ends in "wait" (and the two RMSNorm
stages, which poll the residual first) are mostly the block waiting for its producers; the others
are the block's own work plus the prefetch of the next stage.
"""
from __future__ import annotations

import numpy as np

TICK_US = 0.01  # 100 MHz wall clock
STAGES = ("norm", "qkv", "q_wait", "attn", "merge", "o_wait", "o_proj", "norm2", "gate_up", "m_wait", "down")


def events_per_block(n_layers: int) -> int:
    return 3 + len(STAGES) * n_layers


def stage_durations(trace: np.ndarray, n_layers: int) -> np.ndarray:
    """trace: [grid][>= events_per_block] stamps of one step -> [grid][n_layers][11] durations in us."""
    t = np.asarray(trace, dtype=np.int64)
    ns = len(STAGES)
    ev = t[:, 1:1 + ns * n_layers].reshape(t.shape[0], n_layers, ns)
    prev = np.concatenate([t[:, 0:1], ev[:, :-1, -1]], axis=1)
    starts = np.concatenate([prev[:, :, None], ev[:, :, :-1]], axis=2)
    return (ev - starts) * TICK_US


def summarize(trace: np.ndarray, n_layers: int, skip_first_layer: bool = True) -> dict:
    """Mean over layers of each stage's block-mean and block-max duration (us), plus totals."""
    t = np.asarray(trace, dtype=np.int64)
    d = stage_durations(t, n_layers)
    if skip_first_layer and n_layers > 1:
        d = d[:, 1:]
    e_end = 2 + len(STAGES) * n_layers
    out = {
        "total_us": float((t[:, e_end].max() - t[:, 0].min()) * TICK_US),
        "lm_head_us": float(((t[:, e_end] - t[:, e_end - 1]) * TICK_US).mean()),
        "layer_us": float(d.mean(axis=0).sum(axis=-1).mean()),
    }
    for k, name in enumerate(STAGES):
        out[name] = {"mean_us": float(d[:, :, k].mean()), "max_over_blocks_us": float(d[:, :, k].max(axis=0).mean())}
    return out
