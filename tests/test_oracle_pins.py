"""The fp64 oracle against its pins (CPU only)."""
import numpy as np

import oracle
import oracle_pins as P


def test_golden_eager():
    P.pin_golden_eager(oracle.eager_step)


def test_golden_deferred():
    P.pin_golden_deferred(oracle.DeferredTile)


def test_transition_form():
    P.pin_transition_form(oracle.eager_step)


def test_rwkv6_unrolled():
    P.pin_rwkv6_unrolled(oracle.eager_step)


def test_closed_forms():
    P.pin_closed_forms(oracle.eager_step)


def test_projection_invariant():
    P.pin_projection(oracle.eager_step)


def test_kda_reduces_to_gdn():
    P.pin_kda_reduces_to_gdn(oracle.eager_step)


def test_deferred_equals_eager():
    P.pin_deferred_equals_eager(oracle.DeferredTile, oracle.eager_step)


def test_kaczmarz_step_size():
    P.pin_kaczmarz_step_size(oracle.eager_step, oracle.kaczmarz_beta)


def test_round_to_bf16_matches_the_format():
    """The oracle's bf16 rounding agrees with torch's float32 -> bfloat16 conversion
    (round to nearest, ties to even) on float32 inputs, including exact ties, is
    idempotent and stays within half a unit in the 8th significant bit."""
    import torch
    g = np.random.default_rng(5)
    x32 = np.concatenate([g.standard_normal(50000).astype(np.float32) * 3,
                          np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 0.0, 0.015625,
                                    1.00390625, 255.5, 1e-20], np.float32)])
    ref = torch.from_numpy(x32).to(torch.bfloat16).double().numpy()
    got = oracle.round_to_bf16(x32.astype(np.float64))
    assert np.array_equal(got, ref)
    assert np.array_equal(oracle.round_to_bf16(got), got)
    _, e = np.frexp(x32.astype(np.float64))
    assert np.all(np.abs(got - x32) <= np.ldexp(1.0, e - 9))  # half a unit in the 8th bit


def test_low_bit_base_deferred_model():
    """With a bf16 base the deferred model rounds exactly where the base is written:
    the start state, and at each merge the exact fp64 materialisation of the rounded
    base plus the log; every step's output is the fp64 model's on that base."""
    import copy
    S0, steps, _ = P._random_run(0, 900, T=10, dk=6, dv=4, unit_k=True)
    low = oracle.DeferredTile(0, S0, 4, low_bit_base=True)
    assert np.array_equal(low.base, oracle.round_to_bf16(S0))
    assert not np.array_equal(low.base, S0)
    for st in steps:
        twin = copy.deepcopy(low)
        twin.low_bit_base = False   # the same tile carried on in fp64 for this one step
        args = (st["q"], st["k"], st["v"], st["decay"], st["beta"])
        o_low, o_twin = low.step(*args), twin.step(*args)
        assert np.array_equal(o_low, o_twin)
        assert np.array_equal(low.base, oracle.round_to_bf16(twin.base))
        assert np.array_equal(oracle.round_to_bf16(low.base), low.base)
    assert low.merges == 2


# ------------------------------------------------------ the seeded driver ----
def test_rel_err():
    P.pin_rel_err(oracle.rel_err)


def test_elem_rel_err():
    P.pin_elem_rel_err(oracle.elem_rel_err)


def test_step_arrays():
    P.pin_step_arrays(oracle.step_arrays)


def test_run_eager():
    P.pin_run_eager(oracle.run_eager)


def test_run_deferred():
    P.pin_run_deferred(oracle.run_deferred)
