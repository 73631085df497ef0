"""Run the fp64 oracle over a seeded decode workload.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import this module.

Inputs come from the shared seeded generator (bf16 bits widened exactly to
fp32, then to fp64); nothing here depends on the GPU path.
"""
from __future__ import annotations

from typing import Iterable, Optional, Sequence

import numpy as np

from inputs import bf16_bits_to_f32

from .deferred import DeferredTile
from .recurrences import eager_step, kaczmarz_beta


def step_arrays(inp, t: int, sel: Optional[Sequence] = None) -> dict:
    """Step t's inputs as float64 arrays, optionally restricted to tiles `sel`.

    sel: None for all tiles (arrays [B][H][...]) or a list of (b, h) pairs
    (arrays [n][...]).
    """
    x = inp.step(t)
    out = {}
    for name in ("q", "k", "v"):
        a = bf16_bits_to_f32(x[name]).astype(np.float64)
        out[name] = a if sel is None else np.stack([a[b, h] for b, h in sel])
    d = x["decay"].astype(np.float64)
    out["decay"] = d if sel is None else np.stack([d[b, h] for b, h in sel])
    if getattr(inp, "eta", None) is not None:
        # Kaczmarz step size from eta and the (bf16) key actually used
        et = inp.eta[inp.slot(t)].astype(np.float64)
        et = et if sel is None else np.array([et[b, h] for b, h in sel])
        out["beta"] = kaczmarz_beta(et, out["k"], inp.eps)
    elif x["beta"] is None:
        out["beta"] = None
    else:
        bt = x["beta"].astype(np.float64)
        out["beta"] = bt if sel is None else np.array([bt[b, h] for b, h in sel])
    if inp.bonus is None:
        out["bonus"] = None
    else:
        bo = inp.bonus.astype(np.float64)
        out["bonus"] = (np.broadcast_to(bo[None], (inp.batch,) + bo.shape) if sel is None
                        else np.stack([bo[h] for _, h in sel]))
    return out


def run_eager(inp, steps: int, sel: Optional[Sequence] = None, keep_outputs: bool = True,
              check_every: Optional[Iterable[int]] = None, s0: Optional[np.ndarray] = None):
    """Eager fp64 recurrence over `steps` steps.

    Returns (S_final, outputs) where outputs is float64 [steps][tiles...][dv]
    (or None if keep_outputs is False).  With check_every = a set of step
    indices, also returns the dict {t: S after step t}.
    """
    if s0 is None:
        s0 = inp.s0 if sel is None else np.stack([inp.s0[b, h] for b, h in sel])
    S = np.array(s0, dtype=np.float64)
    outs = [] if keep_outputs else None
    snaps = {}
    marks = set(check_every or ())
    for t in range(steps):
        a = step_arrays(inp, t, sel)
        S, o = eager_step(inp.variant, S, a["q"], a["k"], a["v"], a["decay"], a["beta"], a["bonus"])
        if keep_outputs:
            outs.append(o)
        if t in marks:
            snaps[t] = S.copy()
    res = (S, None if outs is None else np.stack(outs))
    return res + (snaps,) if check_every is not None else res


def deferred_tiles(inp, sel: Sequence, log_len: Optional[int] = None, low_bit_base: bool = False):
    """Build one DeferredTile per (b, h) in `sel`, started at the workload's fills."""
    L = inp.log_len if log_len is None else log_len
    tiles = []
    for b, h in sel:
        bonus = None if inp.bonus is None else inp.bonus[h]
        tiles.append(DeferredTile(inp.variant, inp.s0[b, h], L, int(inp.fill0[b]), bonus, low_bit_base))
    return tiles


def run_deferred(inp, steps: int, sel: Sequence, log_len: Optional[int] = None, low_bit_base: bool = False):
    """Deferred fp64 model over `steps` steps for tiles `sel`.

    Returns (tiles, outputs [steps][len(sel)][dv], fills [steps][len(sel)],
    slots [steps][len(sel)]) where fills are the log fills after each step and
    slots the slot each step appended to.
    """
    tiles = deferred_tiles(inp, sel, log_len, low_bit_base)
    outs, fills, slots = [], [], []
    for t in range(steps):
        a = step_arrays(inp, t, sel)
        row_o, row_f, row_s = [], [], []
        for i, tile in enumerate(tiles):
            beta = None if a["beta"] is None else a["beta"][i]
            row_o.append(tile.step(a["q"][i], a["k"][i], a["v"][i], a["decay"][i], beta))
            row_f.append(tile.fill)
            row_s.append(tile.last_slot)
        outs.append(np.stack(row_o))
        fills.append(row_f)
        slots.append(row_s)
    return tiles, np.stack(outs), np.array(fills), np.array(slots)


def rel_err(got: np.ndarray, ref: np.ndarray, axes=None) -> float:
    """Largest per-tensor relative error max|got - ref| / max|ref|.

    axes: the trailing axes that form one tensor (e.g. (-2, -1) for a state,
    (-1,) for an output vector); the worst tensor is returned.  A tensor whose
    reference is all zeros is measured in absolute terms.
    """
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    if axes is None:
        axes = tuple(range(ref.ndim))
    num = np.max(np.abs(got - ref), axis=axes)
    den = np.max(np.abs(ref), axis=axes)
    den = np.where(den == 0, 1.0, den)
    return float(np.max(num / den))


def elem_rel_err(got: np.ndarray, ref: np.ndarray, axes=None, floor: float = 1e-6) -> float:
    """Largest element-wise relative error |got - ref| / max(|ref|, floor * max|ref|).

    The floor is taken per tensor (the same trailing `axes` as rel_err), so an
    element whose reference is near zero is measured against a millionth of its
    tensor's largest magnitude instead of against itself.  A tensor whose
    reference is all zeros is measured in absolute terms.  This is the
    element-wise companion of rel_err, reported beside it; the parity bar is
    rel_err's.
    """
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    if axes is None:
        axes = tuple(range(ref.ndim))
    scale = np.max(np.abs(ref), axis=axes, keepdims=True)
    scale = np.where(scale == 0, 1.0 / floor, scale)
    den = np.maximum(np.abs(ref), floor * scale)
    return float(np.max(np.abs(got - ref) / den))
