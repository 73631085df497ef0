"""The derived drift bound of a bf16-base run, checked on the oracle itself (CPU only).

The bf16-base oracle, run from the start state with no restarts, must stay within
the bound that tests/bf16_bound.py derives from the rounding (2^-8 of each value
rounded, carried through the decay, into the outputs through ||q||), at every
output element and in every state column, for every variant.  The bound is a
worst case; to show it is not vacuous, a quantiser four times coarser (6
significant bits) must break it.
"""
import numpy as np
import pytest

import bf16_bound as BB
import oracle
import oracle.deferred as OD
from inputs import make_inputs

CASES = [(1, 64, 64), (2, 16, 8), (3, 16, 8), (4, 16, 8), (6, 16, 8)]


def _run(w, dk, dv, T=1024):
    inp = make_inputs(w, T, batch=2, heads=2, pool=T, dk=dk, dv=dv, fill0=np.array([0, 5], np.int32))
    sel = [(b, h) for b in range(2) for h in range(2)]
    outs, tiles, ob, eb, fc = BB.drift_bound(inp, T, sel)
    S, eo = oracle.run_eager(inp, T, sel)
    return outs, tiles, ob, eb, fc, S, eo


@pytest.mark.parametrize("w,dk,dv", CASES)
def test_bf16_oracle_stays_within_the_derived_bound(w, dk, dv):
    outs, tiles, ob, eb, fc, S, eo = _run(w, dk, dv)
    ratio = np.abs(outs - eo) / ob
    assert np.all(np.isfinite(ob)) and np.all(ob > 0)
    assert ratio.max() <= 1.0, ratio.max()
    for t in tiles:
        if t.fill:
            t.merge()
    col = np.linalg.norm(np.stack([t.base for t in tiles]) - S, axis=-2)
    assert np.all(col <= eb + BB.UNIT * (fc + 2 * eb))


def test_a_coarser_quantiser_breaks_the_bound(monkeypatch):
    six_bits = lambda x: (lambda m, e: np.ldexp(np.rint(m * 64.0) / 64.0, e))(*np.frexp(np.asarray(x, np.float64)))
    monkeypatch.setattr(OD, "round_to_bf16", six_bits)
    broken = 0
    for w, dk, dv in CASES:
        outs, _, ob, _, _, _, eo = _run(w, dk, dv)
        broken += int(np.any(np.abs(outs - eo) > ob))
    assert broken >= 3, broken
