"""Eager fp64 decode recurrences: the ground truth the GPU path is checked against.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import this module.

Each function takes one decode step on every (sequence, head) state at once.
States are float64 arrays [..., dk, dv] whose rows are key channels and whose
columns are value channels; vectors are float64 [..., dk] or [..., dv].  The
arithmetic is the plain dense (eager) recurrence, the one the DeltaLog page's
Abstract describes as the usual decoder, which rewrites the whole recurrent
state after each token.  The same passage says DeltaLog leaves what the model
computes unchanged, so the deferred state equals this one exactly, and this is
the definition the deferred GPU path must reproduce up to rounding.

Readings (the pages name the models but print no equations for them):

* Gated DeltaNet: gated state decay followed by a delta-rule residual write
  (Kaczmarz Linear Attention abstract, on the DeltaLog card page; the Gated
  DeltaNet-2 abstract on the Q-Delta card page describes a delta rule as
  taking away what the state already returns for the key before writing).  The read uses the decayed state, the write is the
  rank-1 outer product k u^T, and the output is read from the updated state:
      D   = alpha * S
      u   = beta * (v - D^T k)
      S'  = D + k u^T
      o   = S'^T q
  No 1/sqrt(dk) query scale.
* KDA: the same with channel-wise decay on the key rows, D = diag(a) S (per
  channel forgetting, Gated DeltaNet-2 abstract).  With a = alpha * 1 it is
  Gated DeltaNet (the same abstract: KDA becomes Gated DeltaNet once its decay
  is one scalar).
* RWKV6: diagonal per-channel decay, an additive outer-product write and a
  bonus readout through the pre-update state:
      o   = S^T r + (sum_i r_i bonus_i k_i) v
      S'  = diag(w) S + k v^T
"""
from __future__ import annotations

import numpy as np


def _read(S: np.ndarray, x: np.ndarray) -> np.ndarray:
    """S^T x for a batch of states: out[..., j] = sum_i S[..., i, j] * x[..., i]."""
    return np.einsum("...ij,...i->...j", S, x)


def _outer(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    return a[..., :, None] * b[..., None, :]


def gdn_step(S, q, k, v, alpha, beta):
    """One Gated DeltaNet decode step.  alpha, beta: [...] scalars per state.

    Returns (S', o).  Follows the gated delta rule as read above.
    """
    D = alpha[..., None, None] * S
    u = beta[..., None] * (v - _read(D, k))
    S_new = D + _outer(k, u)
    return S_new, _read(S_new, q)


def kda_step(S, q, k, v, a, beta):
    """One KDA decode step.  a: [..., dk] channel-wise decay on key rows; beta: [...]."""
    D = a[..., :, None] * S
    u = beta[..., None] * (v - _read(D, k))
    S_new = D + _outer(k, u)
    return S_new, _read(S_new, q)


def rwkv6_step(S, r, k, v, w, bonus):
    """One RWKV6 decode step.  w: [..., dk] decay; bonus: [..., dk] (per head).

    The output reads the state before this step's write, plus the bonus term.
    """
    o = _read(S, r) + np.sum(r * bonus * k, axis=-1)[..., None] * v
    S_new = w[..., :, None] * S + _outer(k, v)
    return S_new, o


def kaczmarz_beta(eta, k, eps):
    """Kaczmarz step size beta = eta / (||k||^2 + eps) (Kaczmarz Linear Attention abstract).

    eta: [...] per state; k: [..., dk]; eps >= 0.  With eta = 1 and eps = 0 the
    delta-rule write projects the state so that S'^T k = v exactly.
    """
    return np.asarray(eta, np.float64) / (np.sum(np.asarray(k, np.float64) ** 2, axis=-1) + eps)


def eager_step(variant: int, S, q, k, v, decay, beta=None, bonus=None):
    """Dispatch on the variant code (0 = GDN, 1 = KDA, 2 = RWKV6)."""
    if variant == 0:
        return gdn_step(S, q, k, v, decay, beta)
    if variant == 1:
        return kda_step(S, q, k, v, decay, beta)
    if variant == 2:
        return rwkv6_step(S, q, k, v, decay, bonus)
    raise ValueError(f"unknown variant {variant}")
