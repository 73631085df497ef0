"""The fp64 oracle against its pins (CPU only)."""
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
