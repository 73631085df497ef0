"""Low-bit (bf16) base against the oracle with the same quantisation (GPU).

The base is stored in bf16 and rounded to nearest even wherever it is written
(at init and at each fold); the log, the reads and the fold arithmetic stay in
fp32.  The oracle runs the same schedule in fp64 and rounds its base at the
same points, so the only differences left are fp32-vs-fp64 arithmetic and the
few values that fp32 puts on the other side of a bf16 rounding midpoint.

Two kinds of check: per fold period, against the oracle restarted from the base
the GPU holds (tight: the fp32 tolerance and bit equality of the folded base);
and over a whole run, against the exact oracle and the bf16-base oracle, both
started from the workload's own start state and never from GPU values, within
the drift bound derived from the rounding in tests/bf16_bound.py.
"""
import ctypes

import numpy as np
import pytest
import torch

import bf16_bound
import oracle
from gpu_harness import Uploaded, dev, materialized_state, new_pool, run_deltalog
from inputs import make_inputs
from linear_attention_recurrent_amd import deltalog as dl

pytestmark = pytest.mark.gpu

BF = dl.BASE_BF16
TOL_EXACT_BASE = 1e-4   # fp32 reads of a base both sides hold bit for bit


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("a GPU is required for the gpu-marked tests")
    dl.load_library()


def _ulps(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """|a - b| in bf16 units in the last place, less the fp32 arithmetic slack.

    A folded value is a sum of terms as large as the tile's largest entries;
    fp32 leaves it an absolute error of a few 2^-24 of that scale, which is many
    bf16 ulps of a value that cancels to near zero.  That slack (2^-18 of the
    tile's largest magnitude, last two axes) is taken off before counting ulps
    of the larger of the two magnitudes (8 significant bits).
    """
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    slack = 2.0 ** -18 * np.max(np.abs(b), axis=(-2, -1), keepdims=True)
    _, e = np.frexp(np.maximum(np.abs(a), np.abs(b)))
    return np.maximum(np.abs(a - b) - slack, 0.0) / np.ldexp(1.0, e - 8)


def _all_tiles(inp):
    return [(b, h) for b in range(inp.batch) for h in range(inp.heads)]


@pytest.mark.parametrize("w", [1, 3, 4])
def test_init_rounds_and_first_fold_matches(w):
    inp = make_inputs(w, 16, batch=2, heads=4, log_len=16, pool=16, fill0=np.zeros(2, np.int32))
    sel = _all_tiles(inp)
    up = Uploaded(inp)
    pool = new_pool(inp, up=up, base_dtype=BF)
    assert pool.base.dtype == torch.bfloat16
    init = pool.base.float().cpu().numpy()
    assert np.array_equal(init, oracle.round_to_bf16(inp.s0.astype(np.float64)))
    outs = []
    for t in range(15):
        dl.dl_decode_step(pool, up.io(t))
        outs.append(up.out.cpu().numpy().reshape(len(sel), inp.dv))
        assert torch.equal(pool.base.float().cpu(), torch.from_numpy(init))  # appends leave the base alone
    dl.dl_decode_step(pool, up.io(15))  # the 16th entry fills the log: this step folds
    outs.append(up.out.cpu().numpy().reshape(len(sel), inp.dv))
    assert int(pool.fill.max().item()) == 0
    tiles, ref_o, _, _ = oracle.run_deferred(inp, 16, sel, low_bit_base=True)
    err = oracle.rel_err(np.stack(outs), ref_o, (-1,))
    print(f"outputs before and at the fold: {err:.3e}", flush=True)
    assert err <= TOL_EXACT_BASE
    got = pool.base.float().cpu().numpy().reshape(len(sel), inp.dk, inp.dv)
    ref = np.stack([t.base for t in tiles])
    same = np.mean(got == ref)
    print(f"folded base: {same:.5%} bit-equal, max {_ulps(got, ref).max():g} ulp apart", flush=True)
    assert same >= 0.999
    assert np.all(_ulps(got, ref) <= 1)


@pytest.mark.parametrize("w,batch,heads", [(1, 1, 1), (2, 2, 4), (3, 2, 4), (4, 4, 4), (6, 2, 4)])
def test_every_fold_period_of_a_long_run(w, batch, heads):
    """Over a long run, each fold period is checked against the oracle started from
    the bf16 base the GPU holds at the period's start: the outputs to the fp32
    tolerance, the folded base bit for bit up to rounding-midpoint cases.

    Two trajectories that once rounded one value differently drift apart by
    bf16-sized amounts, so a whole-run comparison can only be as tight as the
    quantisation itself; restarting the oracle at each fold keeps every check
    tight.  test_whole_run_within_the_rounding_bound checks whole runs.
    """
    steps = 4096 if w != 1 else 1024
    inp = make_inputs(w, steps, batch=batch, heads=heads, pool=steps, fill0=np.zeros(batch, np.int32))
    L = inp.log_len
    sel = _all_tiles(inp)
    n = len(sel)
    up = Uploaded(inp)
    pool = new_pool(inp, up=up, base_dtype=BF)
    outs = np.empty((steps, n, inp.dv), np.float32)
    worst_o, worst_same, worst_ulp = 0.0, 1.0, 0.0
    for p0 in range(0, steps, L):
        start = pool.base.float().cpu().numpy().reshape(n, inp.dk, inp.dv).astype(np.float64)
        tiles = [oracle.DeferredTile(inp.variant, start[i], L, 0, None if inp.bonus is None else inp.bonus[h],
                                     low_bit_base=True) for i, (_, h) in enumerate(sel)]
        ref_o = []
        for t in range(p0, p0 + L):
            dl.dl_decode_step(pool, up.io(t))
            outs[t] = up.out.cpu().numpy().reshape(n, inp.dv)
            a = oracle.step_arrays(inp, t, sel)
            ref_o.append([tile.step(a["q"][i], a["k"][i], a["v"][i], a["decay"][i],
                                    None if a["beta"] is None else a["beta"][i]) for i, tile in enumerate(tiles)])
        assert int(pool.fill.max().item()) == 0 and all(tile.fill == 0 for tile in tiles)
        worst_o = max(worst_o, oracle.rel_err(outs[p0:p0 + L], np.array(ref_o), (-1,)))
        got = pool.base.float().cpu().numpy().reshape(n, inp.dk, inp.dv)
        ref = np.stack([tile.base for tile in tiles])
        worst_same = min(worst_same, float(np.mean(got == ref)))
        worst_ulp = max(worst_ulp, float(_ulps(got, ref).max()))
    print(f"per fold period: outputs {worst_o:.3e}, folded base >= {worst_same:.5%} bit-equal, "
          f"max {worst_ulp:.3f} ulp apart", flush=True)
    assert worst_o <= TOL_EXACT_BASE
    assert worst_same >= 0.999 and worst_ulp <= 1.0


@pytest.mark.parametrize("w,batch,heads,steps", [(1, 1, 1, 4096), (2, 2, 4, 2048), (3, 2, 4, 2048),
                                                 (4, 4, 4, 2048), (6, 2, 4, 2048)])
def test_whole_run_within_the_rounding_bound(w, batch, heads, steps):
    """A whole bf16-base run, unseeded: the GPU's outputs and final state against the
    exact fp64 oracle, element by element, within the bound derived from the rounding
    (tests/bf16_bound.py: 2^-8 of every value rounded at the start and at each fold,
    carried through the decay, into each output through ||q||), plus the fp32 path's
    own tolerance.  The bf16-base oracle, from the same start state, is held to the
    same bound (no fp32 slack), and the GPU's distance to it is reported."""
    inp = make_inputs(w, steps, batch=batch, heads=heads, pool=steps, fill0=np.arange(batch, dtype=np.int32) % 5)
    sel = _all_tiles(inp)
    n = len(sel)
    pool, outs = run_deltalog(inp, steps, base_dtype=BF)
    outs = outs.reshape(steps, n, inp.dv).astype(np.float64)
    q_o, tiles, bound_o, bound_col, fold_cols = bf16_bound.drift_bound(inp, steps, sel)
    exact_S, exact_o = oracle.run_eager(inp, steps)
    exact_o = exact_o.reshape(steps, n, inp.dv)
    exact_S = exact_S.reshape(n, inp.dk, inp.dv)
    slack_o = TOL_EXACT_BASE * np.max(np.abs(exact_o), axis=-1, keepdims=True)
    assert np.all(np.abs(q_o - exact_o) <= bound_o)
    ratio = np.abs(outs - exact_o) / (bound_o + slack_o)
    print(f"outputs vs the exact oracle: worst {ratio.max():.3f} of the bound; per tensor "
          f"{oracle.rel_err(outs, exact_o, (-1,)):.3e}, element-wise {oracle.elem_rel_err(outs, exact_o, (-1,)):.3e}; "
          f"vs the bf16-base oracle: per tensor {oracle.rel_err(outs, q_o, (-1,)):.3e}", flush=True)
    assert ratio.max() <= 1.0
    S = materialized_state(pool).reshape(n, inp.dk, inp.dv)
    folded = np.array([t.fill > 0 for t in tiles])
    for t in tiles:
        if t.fill:
            t.merge()
    col_bound = bound_col + bf16_bound.UNIT * (fold_cols + 2 * bound_col) * folded[:, None]
    col_slack = TOL_EXACT_BASE * np.linalg.norm(exact_S, axis=-2)
    col_err = np.linalg.norm(S - exact_S, axis=-2)
    print(f"state columns vs the exact oracle: worst {np.max(col_err / (col_bound + col_slack)):.3f} of the bound; "
          f"per tensor {oracle.rel_err(S, exact_S, (-2, -1)):.3e}; vs the bf16-base oracle "
          f"{oracle.rel_err(S, np.stack([t.base for t in tiles]), (-2, -1)):.3e}", flush=True)
    assert np.all(col_err <= col_bound + col_slack)


def test_merge_and_reruns_with_bf16_base():
    """dl_merge folds every log at or above min_fill into the bf16 base; reruns are bit-identical."""
    inp = make_inputs(2, 40, batch=3, heads=2, log_len=16, pool=40, fill0=np.array([0, 5, 11], np.int32))
    sel = _all_tiles(inp)
    up = Uploaded(inp)
    runs = []
    for _ in range(2):
        pool = new_pool(inp, up=up, base_dtype=BF)
        for t in range(9):
            dl.dl_decode_step(pool, up.io(t))
        fill = pool.fill.cpu().numpy().copy()
        before = pool.base.clone()
        dl.dl_merge(pool, 6)
        torch.cuda.synchronize()
        runs.append(pool)
    assert all(torch.equal(a, b) for a, b in zip(runs[0].tensors().values(), runs[1].tensors().values()))
    pool = runs[0]
    tiles, _, _, _ = oracle.run_deferred(inp, 9, sel, low_bit_base=True)
    after = pool.base.float().cpu().numpy().reshape(len(sel), inp.dk, inp.dv)
    for i, (b, h) in enumerate(sel):
        if fill[b, h] >= 6:
            assert pool.fill[b, h].item() == 0
            tiles[i].merge()
            ref = tiles[i].base
            assert np.mean(after[i] == ref) >= 0.999 and np.all(_ulps(after[i], ref) <= 1)
        else:
            assert pool.fill[b, h].item() == fill[b, h]
            assert torch.equal(pool.base[b, h], before[b, h])


def test_eager_rejects_a_bf16_base_and_bad_dtype_is_rejected():
    state = torch.zeros((1, 1, 64, 64), dtype=torch.float32, device=dev())
    inp = make_inputs(1, 1, batch=1, heads=1, pool=1, dk=64, dv=64)
    up = Uploaded(inp)
    lib = dl.load_library()
    dims = dl.Dims(0, 1, 1, 64, 64, 1, BF)
    rc = lib.dl_eager_step(ctypes.byref(dims), ctypes.c_void_p(state.data_ptr()), ctypes.byref(up.io(0)), None)
    assert rc == dl.DL_EUNSUPPORTED
    assert torch.count_nonzero(state).item() == 0
    bad = dl.DeltaLogPool(0, 1, 1, 64, 64, 8, dev(), base_dtype=7)
    with pytest.raises(dl.DeltaLogError) as ei:
        dl.dl_init_state(bad)
    assert ei.value.status == dl.DL_EINVAL
