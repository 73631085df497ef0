"""How far a run with a bf16 base may drift from the exact (unquantised) run, derived
from the rounding alone.  Test infrastructure: it drives the fp64 oracle only.

The low-bit base (LeapQuant abstract, on the card page titled "A Persistent-State
Dataflow Accelerator for Memory-Bound Linear Attention Decode on FPGA": outputs
come from a state stored in few bits plus pending updates kept at full precision) is rounded to
bf16 where it is written: once at the start and once per fold.  Write S_t for the
exact state and S_t + E_t for the state a bf16-base run stands for.

* Rounding.  bf16 keeps 8 significant bits, so rounding x to nearest moves it by
  at most half a unit in its 8th bit: |Q(x) - x| <= 2^-9 2^e <= 2^-8 |x| for
  x = m 2^e, m in [1/2, 1).  A fold or the start therefore adds to each column
  j of E a vector R with ||R||_2 <= 2^-8 ||X[:, j]||_2, X the value rounded.
* Carried by the recurrence.  Between roundings both runs apply the same
  update to the state, and E follows its linear part.  GDN and KDA:
  E_t = (I - b_t k_t k_t^T) D_t E_{t-1}; with 0 <= b_t ||k_t||^2 <= 2 the
  projection factor has 2-norm <= 1, so ||E_t[:, j]|| <= max_i d_t[i] ||E_{t-1}[:, j]||.
  RWKV6: E_t = diag(w_t) E_{t-1}, the same with w for d.
* Into the outputs.  GDN/KDA read the state after the step, RWKV6 the state
  before it, so |o_t[j] - o^_t[j]| <= ||E[:, j]||_2 ||q_t||_2 with E taken at the
  step the readout sees.  A folding step computes its output before it rounds.

So with eb_j = the bound on ||E[:, j]||_2, starting at 2^-8 ||S_0[:, j]||:
each step multiplies eb by max_i d_t[i]; each fold adds 2^-8 (||X_f[:, j]|| + 2 eb_j),
where X_f is the value this oracle rounds at that fold: the run under test rounds
a value within eb_j of the exact state, and the exact state is within eb_j of
X_f, by the same bound applied to both runs.  The bound sums every rounding at
full size with no cancellation, so it is a worst case.
"""
from __future__ import annotations

import numpy as np

import oracle

UNIT = 2.0 ** -8  # |Q(x) - x| <= UNIT |x| for bf16 round to nearest


class _FoldRecorder(oracle.DeferredTile):
    """A bf16-base oracle tile that keeps the unrounded value of its last fold."""

    def merge(self):
        self.fold_value = self.materialize()
        super().merge()


def drift_bound(inp, steps: int, sel):
    """Run the bf16-base oracle (from the workload's start state, not restarted) over
    `steps` steps for tiles `sel` and return

      outs      fp64 [steps][n][dv]  its outputs
      tiles     its tiles after the run (base + log)
      out_bound fp64 [steps][n][dv]  per output element, the bound on |o - o_exact|
      col_bound fp64 [n][dv]         per state column at the end, the bound on the
                                     2-norm of (state - exact state), before any
                                     final fold
      fold_cols fp64 [n][dv]         2-norms of the columns of the tiles' dense
                                     state at the end (for a final fold's rounding)
    """
    n = len(sel)
    L = inp.log_len
    tiles = []
    for b, h in sel:
        bonus = None if inp.bonus is None else inp.bonus[h]
        tiles.append(_FoldRecorder(inp.variant, inp.s0[b, h], L, int(inp.fill0[b]), bonus, low_bit_base=True))
    s0 = np.stack([inp.s0[b, h] for b, h in sel]).astype(np.float64)
    eb = UNIT * np.linalg.norm(s0, axis=-2)        # [n][dv]: the start is rounded
    outs = np.empty((steps, n, inp.dv))
    out_bound = np.empty((steps, n, inp.dv))
    for t in range(steps):
        a = oracle.step_arrays(inp, t, sel)
        d = np.asarray(a["decay"], np.float64).reshape(n, -1).max(axis=1)  # 2-norm of the decay factor
        qn = np.linalg.norm(a["q"], axis=-1)
        if inp.variant == 2:
            out_bound[t] = eb * qn[:, None]          # the readout sees the state before the step
            eb = eb * d[:, None]
        else:
            kk = np.sum(a["k"] ** 2, axis=-1)
            assert np.all(a["beta"] >= 0) and np.all(a["beta"] * kk <= 2), "projection factor not contractive"
            eb = eb * d[:, None]
            out_bound[t] = eb * qn[:, None]
        for i, tile in enumerate(tiles):
            merges = tile.merges
            beta = None if a["beta"] is None else a["beta"][i]
            outs[t, i] = tile.step(a["q"][i], a["k"][i], a["v"][i], a["decay"][i], beta)
            if tile.merges != merges:               # this step folded: its rounding joins E
                eb[i] += UNIT * (np.linalg.norm(tile.fold_value, axis=0) + 2 * eb[i])
    fold_cols = np.stack([np.linalg.norm(t.materialize(), axis=0) for t in tiles])
    return outs, tiles, out_bound, eb, fold_cols
