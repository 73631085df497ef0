"""Plausible mistakes planted in copies of the oracle must each fail a pin (CPU only).

This shows the pins are strong enough: a dropped term, a wrong sign, a
transposed operand or a wrong decay placement anywhere in the oracle's
arithmetic is caught.  The mistakes live only in this file; the oracle itself
is untouched.
"""
import numpy as np
import pytest

import oracle
import oracle_pins as P


def _read(S, x):
    return np.einsum("...ij,...i->...j", S, x)


def _outer(a, b):
    return a[..., :, None] * b[..., None, :]


def make_delta_mutant(kind):
    """GDN/KDA step with one planted mistake; RWKV6 delegates to the oracle."""
    def step(variant, S, q, k, v, decay, beta, bonus):
        if variant == 2:
            return oracle.eager_step(variant, S, q, k, v, decay, beta, bonus)
        d = np.asarray(decay)
        if variant == 0:
            D = d[..., None, None] * S
        elif kind == "kda_decay_on_columns":
            D = S * np.resize(d, S.shape[-1])[None, :]
        else:
            D = d[..., :, None] * S
        if kind == "read_undecayed":
            rd = _read(S, k)
        elif kind == "read_transposed":
            rd = np.einsum("...ij,...j->...i", D, np.resize(k, D.shape[-1]))[..., :D.shape[-1]]
        else:
            rd = _read(D, k)
        b = np.asarray(beta)
        if kind == "residual_sign":
            u = b[..., None] * (v + rd)
        elif kind == "drop_beta":
            u = v - rd
        else:
            u = b[..., None] * (v - rd)
        if kind == "write_undecayed":
            S_new = S + _outer(k, u)
        elif kind == "write_v_not_u":
            S_new = D + b[..., None, None] * _outer(k, v)
        else:
            S_new = D + _outer(k, u)
        if kind == "output_pre_update":
            o = _read(D, q)
        elif kind == "output_reads_k":
            o = _read(S_new, k)
        else:
            o = _read(S_new, q)
        return S_new, o
    return step


def make_rwkv_mutant(kind):
    def step(variant, S, q, k, v, decay, beta, bonus):
        if variant != 2:
            return oracle.eager_step(variant, S, q, k, v, decay, beta, bonus)
        w = np.asarray(decay)
        S_new = w[..., :, None] * S + _outer(k, v)
        if kind == "decay_after_write":
            S_new = w[..., :, None] * (S + _outer(k, v))
        if kind == "output_post_update":
            o = _read(S_new, q) + np.sum(q * bonus * k) * v
        elif kind == "drop_bonus":
            o = _read(S, q)
        elif kind == "bonus_without_k":
            o = _read(S, q) + np.sum(q * bonus) * v
        elif kind == "bonus_uses_decay":
            o = _read(S, q) + np.sum(q * w * k) * v
        else:
            o = _read(S, q) + np.sum(q * bonus * k) * v
        return S_new, o
    return step


EAGER_PINS = [P.pin_golden_eager, P.pin_transition_form, P.pin_rwkv6_unrolled,
              P.pin_closed_forms, P.pin_projection, P.pin_kda_reduces_to_gdn]


def _fails_some_pin(step):
    failed = []
    for pin in EAGER_PINS:
        try:
            pin(step)
        except Exception:  # an assertion, or a shape error from a transposed operand
            failed.append(pin.__name__)
    return failed


@pytest.mark.parametrize("kind", ["read_undecayed", "read_transposed", "residual_sign", "drop_beta",
                                  "write_undecayed", "write_v_not_u", "output_pre_update",
                                  "output_reads_k", "kda_decay_on_columns"])
def test_delta_rule_mutant_is_caught(kind):
    assert _fails_some_pin(make_delta_mutant(kind)), kind


@pytest.mark.parametrize("kind", ["decay_after_write", "output_post_update", "drop_bonus",
                                  "bonus_without_k", "bonus_uses_decay"])
def test_rwkv6_mutant_is_caught(kind):
    assert _fails_some_pin(make_rwkv_mutant(kind)), kind


def test_unmutated_passes_every_pin():
    assert _fails_some_pin(oracle.eager_step) == []


# ------------------------------------------------------------ deferred model --
class SkipCurrentDecay(oracle.DeferredTile):
    """Reads see the base and entries without this step's decay."""
    def _weights(self, extra):
        return super()._weights(np.ones_like(np.asarray(extra, float)))


class OffByOneEntryDecay(oracle.DeferredTile):
    """Each entry is also decayed by its own step's decay."""
    def _weights(self, extra):
        wb, we = super()._weights(extra)
        return wb, [w * d for w, d in zip(we, self.ds)]


class MergeOneLate(oracle.DeferredTile):
    """Merges when the log would exceed L instead of when it reaches L."""
    def _append(self, k, u, d):
        self.last_slot = self.fill
        self.ks.append(np.array(k, np.float64))
        self.us.append(np.array(u, np.float64))
        self.ds.append(np.array(d, np.float64).reshape(-1))
        if self.fill > self.log_len:
            self.merge()


class DropsOldestOnMerge(oracle.DeferredTile):
    """Folds all but the oldest entry at a merge."""
    def merge(self):
        if self.ks:
            self.ks, self.us, self.ds = self.ks[1:], self.us[1:], self.ds[1:]
        super().merge()


@pytest.mark.parametrize("cls", [SkipCurrentDecay, OffByOneEntryDecay, MergeOneLate, DropsOldestOnMerge])
def test_deferred_mutant_is_caught(cls):
    failed = False
    for pin in (lambda: P.pin_golden_deferred(cls),
                lambda: P.pin_deferred_equals_eager(cls, oracle.eager_step, log_lens=(1, 2, 3, 8), T=40)):
        try:
            pin()
        except Exception:
            failed = True
    assert failed, cls.__name__


@pytest.mark.parametrize("kbeta", [
    lambda eta, k, eps: np.asarray(eta) / (np.sqrt(np.sum(k * k, axis=-1)) + eps),   # norm, not its square
    lambda eta, k, eps: np.asarray(eta) / np.sum(k * k, axis=-1),                     # eps dropped
    lambda eta, k, eps: np.asarray(eta) * np.sum(k * k, axis=-1) / (1.0 + eps),       # inverted
])
def test_kaczmarz_mutant_is_caught(kbeta):
    with pytest.raises(AssertionError):
        P.pin_kaczmarz_step_size(oracle.eager_step, kbeta)
