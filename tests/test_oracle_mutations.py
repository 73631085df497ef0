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


# ------------------------------------------------------ the seeded driver ----
def _rel_err_mutant(kind):
    def rel_err(got, ref, axes=None):
        got = np.asarray(got, np.float64)
        ref = np.asarray(ref, np.float64)
        if axes is None:
            axes = tuple(range(ref.ndim))
        d = np.abs(got - ref)
        num = np.mean(d, axis=axes) if kind == "mean_of_errors" else np.max(d, axis=axes)
        if kind == "global_scale":
            den = np.max(np.abs(ref)) + 0 * num
        elif kind == "scale_from_got":
            den = np.max(np.abs(got), axis=axes)
        elif kind == "signed_scale":
            den = np.max(ref, axis=axes)
        else:
            den = np.max(np.abs(ref), axis=axes)
        if kind != "zero_reference_unhandled":
            den = np.where(den == 0, 1.0, den)
        with np.errstate(divide="ignore", invalid="ignore"):
            r = num / den
        return float(np.mean(r) if kind == "mean_over_tensors" else np.max(r))
    return rel_err


@pytest.mark.parametrize("kind", ["global_scale", "mean_of_errors", "scale_from_got", "signed_scale",
                                  "mean_over_tensors", "zero_reference_unhandled"])
def test_rel_err_mutant_is_caught(kind):
    with pytest.raises(AssertionError):
        P.pin_rel_err(_rel_err_mutant(kind))


def _elem_rel_err_mutant(kind):
    def elem_rel_err(got, ref, axes=None, floor=1e-6):
        got = np.asarray(got, np.float64)
        ref = np.asarray(ref, np.float64)
        if axes is None:
            axes = tuple(range(ref.ndim))
        if kind == "global_floor":
            scale = np.max(np.abs(ref)) + np.zeros(np.max(np.abs(ref), axis=axes, keepdims=True).shape)
        else:
            scale = np.max(np.abs(ref), axis=axes, keepdims=True)
        scale = np.where(scale == 0, 1.0 / floor, scale)
        if kind == "no_floor":
            den = np.abs(ref)
        elif kind == "floor_added":
            den = np.abs(ref) + floor * scale
        else:
            den = np.maximum(np.abs(ref), floor * scale)
        with np.errstate(divide="ignore", invalid="ignore"):
            return float(np.max(np.abs(got - ref) / den))
    return elem_rel_err


@pytest.mark.parametrize("kind", ["global_floor", "no_floor", "floor_added"])
def test_elem_rel_err_mutant_is_caught(kind):
    with pytest.raises(AssertionError):
        P.pin_elem_rel_err(_elem_rel_err_mutant(kind))


def _step_arrays_mutant(kind):
    import oracle.drive as D

    def step_arrays(inp, t, sel=None):
        if kind == "bits_as_integers":
            saved = D.bf16_bits_to_f32
            D.bf16_bits_to_f32 = lambda b: np.asarray(b, np.uint16).astype(np.float32)
            try:
                return oracle.step_arrays(inp, t, sel)
            finally:
                D.bf16_bits_to_f32 = saved
        if kind == "bits_as_half":
            saved = D.bf16_bits_to_f32
            D.bf16_bits_to_f32 = lambda b: np.asarray(b, np.uint16).view(np.float16).astype(np.float32)
            try:
                with np.errstate(all="ignore"):
                    return oracle.step_arrays(inp, t, sel)
            finally:
                D.bf16_bits_to_f32 = saved
        if kind == "sel_swapped":
            return oracle.step_arrays(inp, t, None if sel is None else [(h, b) for b, h in sel])
        out = oracle.step_arrays(inp, t, sel)
        if kind == "bonus_per_sequence" and out["bonus"] is not None:
            bo = inp.bonus.astype(np.float64)
            out["bonus"] = (np.stack([bo[b] for b in range(inp.batch)])[:, None].repeat(inp.heads, 1)
                            if sel is None else np.stack([bo[b] for b, _ in sel]))
        if kind == "step_not_slot" and inp.eta is not None:
            et = inp.eta[t].astype(np.float64)  # t instead of t mod P
            et = et if sel is None else np.array([et[b, h] for b, h in sel])
            out["beta"] = oracle.kaczmarz_beta(et, out["k"], inp.eps)
        if kind == "eps_dropped" and inp.eta is not None:
            et = inp.eta[inp.slot(t)].astype(np.float64)
            et = et if sel is None else np.array([et[b, h] for b, h in sel])
            out["beta"] = oracle.kaczmarz_beta(et, out["k"], 0.0)
        return out
    return step_arrays


@pytest.mark.parametrize("kind", ["bits_as_integers", "bits_as_half", "sel_swapped", "bonus_per_sequence",
                                  "step_not_slot", "eps_dropped"])
def test_step_arrays_mutant_is_caught(kind):
    with pytest.raises((AssertionError, IndexError)):
        P.pin_step_arrays(_step_arrays_mutant(kind))


def _run_eager_mutant(kind):
    from oracle.drive import step_arrays
    from oracle.recurrences import eager_step

    def run_eager(inp, steps, sel=None, keep_outputs=True, check_every=None, s0=None):
        if s0 is None or kind == "s0_ignored":
            order = sorted(sel) if (kind == "sel_sorted" and sel is not None) else sel
            s0 = inp.s0 if sel is None else np.stack([inp.s0[b, h] for b, h in order])
        S = np.array(s0, dtype=np.float64)
        outs = [] if keep_outputs else None
        snaps = {}
        marks = set(check_every or ())
        prev_o = None
        for t in range(steps - 1 if kind == "one_step_short" else steps):
            a = step_arrays(inp, t, sel)
            if kind == "snapshot_before_step" and t in marks:
                snaps[t] = S.copy()
            S, o = eager_step(inp.variant, S, a["q"], a["k"], a["v"], a["decay"], a["beta"], a["bonus"])
            if keep_outputs:
                outs.append(o if kind != "previous_output" or prev_o is None else prev_o)
            prev_o = o
            if t in marks and kind != "snapshot_before_step":
                snaps[t] = S.copy()
        res = (S, None if outs is None else np.stack(outs))
        return res + (snaps,) if check_every is not None else res
    return run_eager


@pytest.mark.parametrize("kind", ["one_step_short", "snapshot_before_step", "previous_output", "sel_sorted",
                                  "s0_ignored"])
def test_run_eager_mutant_is_caught(kind):
    with pytest.raises(AssertionError):
        P.pin_run_eager(_run_eager_mutant(kind))


def _run_deferred_mutant(kind):
    from oracle.drive import deferred_tiles, step_arrays

    def run_deferred(inp, steps, sel, log_len=None, low_bit_base=False):
        if kind == "fill0_ignored":
            saved = inp.fill0
            inp.fill0 = np.zeros_like(saved)
        try:
            tiles = deferred_tiles(inp, sel, None if kind == "log_len_ignored" else log_len, low_bit_base)
        finally:
            if kind == "fill0_ignored":
                inp.fill0 = saved
        outs, fills, slots = [], [], []
        for t in range(steps):
            a = step_arrays(inp, t, sel)
            row_o, row_f, row_s = [], [], []
            for i, tile in enumerate(tiles):
                before = tile.fill
                beta = None if a["beta"] is None else a["beta"][i]
                row_o.append(tile.step(a["q"][i], a["k"][i], a["v"][i], a["decay"][i], beta))
                row_f.append(before if kind == "fill_before_step" else tile.fill)
                row_s.append(tile.fill if kind == "slot_after_step" else tile.last_slot)
            outs.append(np.stack(row_o))
            fills.append(row_f)
            slots.append(row_s)
        return tiles, np.stack(outs), np.array(fills), np.array(slots)
    return run_deferred


@pytest.mark.parametrize("kind", ["fill0_ignored", "log_len_ignored", "fill_before_step", "slot_after_step"])
def test_run_deferred_mutant_is_caught(kind):
    with pytest.raises(AssertionError):
        P.pin_run_deferred(_run_deferred_mutant(kind))
