"""Deferred-materialization model of one recurrent state in fp64 (base + bounded log).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import this module.

This is DeltaLog's representation as the DeltaLog page ("DeltaLog: Deferred
Materialization of Recurrent States for Linear Attention Decoding", Abstract)
describes it: the recurrent state is held as two parts, a dense base plus a
bounded-length log holding the latest low-rank updates; a typical decode step only
adds an update's factors to the log, and now and then a merge folds the logged
updates into the base, so the dense state the model sees is the eager one.
The page's AI Summary says the same of appends taking the place of full
write-backs.

Representation used here (written for clarity, not speed, and independent of
the GPU code, which keeps cumulative log2-decays instead).  With a low-bit base
the base is rounded to bf16 wherever it is written (start and merges):

* base: float64 [dk, dv], the state as of the last merge.
* log entry j: (k_j, u_j, d_j) where u_j is the rank-1 write of its step
  (GDN/KDA: the delta-rule factor; RWKV6: v_j) and d_j is that step's own
  decay (a scalar for GDN, a dk-vector for KDA and RWKV6).
* the state it stands for, after the newest entry:
      S = diag(prod_m d_m) base + sum_j diag(prod_{m > j} d_m) k_j u_j^T
  because each entry is decayed by every step that came after it and the
  base by every step since the merge.

Schedule (a reading; the pages give neither L's role nor the merge trigger):
the log holds at most L entries; a step that appends the L-th entry merges in
the same step and leaves the log empty, so between steps the fill n is in
[0, L).  A ragged start with fill n0 is n0 phantom entries (k = 0, u = 0,
d = 1) that contribute nothing and only shift the merge phase.  Hence before
step t (1-based) a state started at n0 holds (n0 + t - 1) mod L entries, the
new entry goes to slot (n0 + t - 1) mod L, and the base changes only on steps
with (n0 + t) mod L == 0.
"""
from __future__ import annotations

import numpy as np


def round_to_bf16(x) -> np.ndarray:
    """Round to the nearest bfloat16 value (8 significant bits, ties to even), in float64.

    For the low-bit base (LeapQuant abstract, on the card page titled "A
    Persistent-State Dataflow Accelerator for Memory-Bound Linear Attention
    Decode on FPGA": outputs read a state stored in few bits together with pending
    updates held at full precision, and the state is re-quantised once per window).  Written from
    the format's definition: x = m 2^e with m in [0.5, 1); keep m to 2^-8.
    Exact for the normal range (bf16 shares float32's exponent range); values
    below 2^-126 keep 8 significant bits here, where bf16 would flush them
    towards subnormals.
    """
    x = np.asarray(x, np.float64)
    m, e = np.frexp(x)
    return np.ldexp(np.rint(m * 256.0) / 256.0, e)  # np.rint rounds half to even


class DeferredTile:
    """One (sequence, head) state in base + log form, float64."""

    def __init__(self, variant: int, s0: np.ndarray, log_len: int, fill0: int = 0,
                 bonus: np.ndarray | None = None, low_bit_base: bool = False):
        if log_len < 1 or not (0 <= fill0 < log_len):
            raise ValueError("need log_len >= 1 and 0 <= fill0 < log_len")
        self.variant = variant
        self.low_bit_base = low_bit_base  # base kept in bf16: rounded wherever it is written
        self.base = np.array(s0, dtype=np.float64)
        if low_bit_base:
            self.base = round_to_bf16(self.base)
        self.log_len = log_len
        dk, dv = self.base.shape
        g = 1 if variant == 0 else dk
        self.ks = [np.zeros(dk) for _ in range(fill0)]
        self.us = [np.zeros(dv) for _ in range(fill0)]
        self.ds = [np.ones(g) for _ in range(fill0)]
        self.bonus = None if bonus is None else np.asarray(bonus, np.float64)
        self.merges = 0            # number of merges performed (for schedule checks)
        self.last_slot = None      # slot the last step appended to

    @property
    def fill(self) -> int:
        return len(self.ks)

    def _weights(self, extra):
        """Decay multipliers of the base and of each entry, with `extra` more decay applied.

        Returns (w_base, [w_0, ..., w_{n-1}]), each a scalar-or-dk vector:
        w_base = extra * prod_m d_m and w_j = extra * prod_{m > j} d_m.
        """
        w_entries = []
        acc = np.array(extra, dtype=np.float64)
        for d in reversed(self.ds):
            w_entries.append(acc.copy())
            acc = acc * d
        w_entries.reverse()
        return acc, w_entries

    def materialize(self) -> np.ndarray:
        """The dense state this base + log stands for (nothing is changed)."""
        w_base, w = self._weights(np.ones(1))
        S = w_base.reshape(-1, 1) * self.base
        for wj, kj, uj in zip(w, self.ks, self.us):
            S = S + np.outer(wj * kj, uj)
        return S

    def merge(self) -> None:
        """Fold every log entry into the base and empty the log."""
        self.base = self.materialize()
        if self.low_bit_base:
            self.base = round_to_bf16(self.base)
        self.ks, self.us, self.ds = [], [], []
        self.merges += 1

    def _coef(self, w, x):
        """Per-entry read coefficients sigma_j = (w_j * k_j) . x."""
        return [float(np.dot(wj * kj, x)) for wj, kj in zip(w, self.ks)]

    def _append(self, k, u, d) -> None:
        self.last_slot = self.fill
        self.ks.append(np.array(k, np.float64))
        self.us.append(np.array(u, np.float64))
        self.ds.append(np.array(d, np.float64).reshape(-1))
        if self.fill == self.log_len:
            self.merge()

    def step(self, q, k, v, decay, beta=None) -> np.ndarray:
        """One decode step: read base + log, append one entry, merge if the log is full.

        Returns the step's output (float64 [dv]).
        """
        q, k, v = (np.asarray(x, np.float64) for x in (q, k, v))
        d = np.asarray(decay, np.float64).reshape(-1)
        if self.variant == 2:
            # RWKV6: read the state before this step's write, then write k v^T.
            w_base, w = self._weights(np.ones(1))
            sig = self._coef(w, q)
            o = self.base.T @ (w_base * q)
            for s, uj in zip(sig, self.us):
                o = o + s * uj
            o = o + float(np.sum(q * self.bonus * k)) * v
            self._append(k, v, d)
            return o
        # GDN / KDA: all reads see the state decayed by this step.
        w_base, w = self._weights(d)
        read = self.base.T @ (w_base * k)
        for s, uj in zip(self._coef(w, k), self.us):
            read = read + s * uj
        u = float(beta) * (v - read)
        o = self.base.T @ (w_base * q)
        for s, uj in zip(self._coef(w, q), self.us):
            o = o + s * uj
        o = o + float(np.dot(k, q)) * u
        self._append(k, u, d)
        return o
