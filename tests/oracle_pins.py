"""Pins for the fp64 oracle: checks against what the pages and the mathematics fix.

Each pin takes the implementation under test as an argument, so the same
checks run on the real oracle (test_oracle_pins.py) and on copies of it with a
planted mistake (test_oracle_mutations.py), which must each fail a pin.

`step` has the signature of oracle.eager_step:
    step(variant, S, q, k, v, decay, beta, bonus) -> (S_new, o)
`tile_cls` has the interface of oracle.DeferredTile.

Shapes use dk != dv wherever possible so that a transposed operand fails.
"""
from __future__ import annotations

import glob
import json
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
VARIANTS = {"gdn": 0, "kda": 1, "rwkv6": 2}


def _rng(seed):
    return np.random.default_rng(seed)


def load_golden():
    out = []
    for path in sorted(glob.glob(os.path.join(GOLDEN, "*_three_steps.json"))):
        with open(path) as f:
            out.append(json.load(f))
    return out


def _golden_step_args(g, st):
    bonus = np.array(g["bonus"], float) if "bonus" in g else None
    beta = np.array(st["beta"], float) if "beta" in st else None
    return (np.array(st["q"], float), np.array(st["k"], float), np.array(st["v"], float),
            np.array(st["decay"], float), beta, bonus)


# ------------------------------------------------------------------- P1 ----
def pin_golden_eager(step):
    """Hand-worked dyadic examples: every value exact, so equality is exact."""
    for g in load_golden():
        var = VARIANTS[g["variant"]]
        S = np.array(g["S0"], float)
        for st in g["steps"]:
            q, k, v, d, beta, bonus = _golden_step_args(g, st)
            S, o = step(var, S, q, k, v, d, beta, bonus)
            assert np.array_equal(S, np.array(st["S"], float)), (g["variant"], st["derivation"])
            assert np.array_equal(o, np.array(st["o"], float)), (g["variant"], st["derivation"])


def pin_golden_deferred(tile_cls):
    """The hand-worked examples through base + log, for every short log length and start fill."""
    for g in load_golden():
        var = VARIANTS[g["variant"]]
        bonus = np.array(g["bonus"], float) if "bonus" in g else None
        for L in (1, 2, 3, 4):
            for n0 in range(L):
                tile = tile_cls(var, np.array(g["S0"], float), L, n0, bonus)
                for t, st in enumerate(g["steps"], start=1):
                    q, k, v, d, beta, _ = _golden_step_args(g, st)
                    o = tile.step(q, k, v, d, beta)
                    assert np.array_equal(o, np.array(st["o"], float)), (g["variant"], L, n0, t)
                    assert np.array_equal(tile.materialize(), np.array(st["S"], float)), \
                        (g["variant"], L, n0, t)
                    assert tile.fill == (n0 + t) % L


# ------------------------------------------------------------------- P2 ----
def _random_run(variant, seed, T=12, dk=5, dv=3, unit_k=False):
    g = _rng(seed)
    S0 = g.standard_normal((dk, dv))
    steps = []
    for _ in range(T):
        k = g.standard_normal(dk)
        if unit_k:
            k /= np.linalg.norm(k)
        d = g.uniform(0.5, 1.0) if variant == 0 else g.uniform(0.3, 1.0, dk)
        steps.append(dict(q=g.standard_normal(dk), k=k, v=g.standard_normal(dv), decay=np.asarray(d),
                          beta=np.asarray(g.uniform(0.1, 1.0)) if variant != 2 else None))
    bonus = g.standard_normal(dk) if variant == 2 else None
    return S0, steps, bonus


def pin_transition_form(step):
    """GDN/KDA: the delta-rule step equals S_t = (I - beta k k^T) D S_{t-1} + beta k v^T.

    The transition form is an independent algebraic statement of the rule
    (gated decay, then a write that first subtracts the current read).
    """
    for variant in (0, 1):
        S0, steps, _ = _random_run(variant, 100 + variant)
        S = S0.copy()
        X = S0.copy()
        dk = S0.shape[0]
        for st in steps:
            S, o = step(variant, S, st["q"], st["k"], st["v"], st["decay"], st["beta"], None)
            Dm = np.eye(dk) * st["decay"] if variant == 0 else np.diag(st["decay"])
            A = np.eye(dk) - st["beta"] * np.outer(st["k"], st["k"])
            X = A @ Dm @ X + st["beta"] * np.outer(st["k"], st["v"])
            np.testing.assert_allclose(S, X, rtol=0, atol=1e-12)
            np.testing.assert_allclose(o, X.T @ st["q"], rtol=0, atol=1e-12)


def pin_rwkv6_unrolled(step):
    """RWKV6 outputs against the unrolled sum, built from scratch at each step (O(T^2)).

    o_t = r_t^T [diag(prod_{i<t} w_i) S_0 + sum_{j<t} diag(prod_{j<i<t} w_i) k_j v_j^T]
          + (sum_m r_t[m] bonus[m] k_t[m]) v_t
    """
    S0, steps, bonus = _random_run(2, 7)
    S = S0.copy()
    for t, st in enumerate(steps):
        S, o = step(2, S, st["q"], st["k"], st["v"], st["decay"], None, bonus)
        prev = np.prod([steps[i]["decay"] for i in range(t)], axis=0) if t else np.ones(S0.shape[0])
        Sprev = prev[:, None] * S0
        for j in range(t):
            w = np.ones(S0.shape[0])
            for i in range(j + 1, t):
                w = w * steps[i]["decay"]
            Sprev = Sprev + np.outer(w * steps[j]["k"], steps[j]["v"])
        ref = Sprev.T @ st["q"] + np.sum(st["q"] * bonus * st["k"]) * st["v"]
        np.testing.assert_allclose(o, ref, rtol=0, atol=1e-11)


# ------------------------------------------------------------------- P3 ----
def pin_closed_forms(step):
    """beta = 0 leaves pure decay; decay 1 and beta 0 keeps the state; RWKV6 with
    w = 1 and S_0 = 0 is causal linear attention plus the bonus diagonal."""
    for variant in (0, 1):
        S0, steps, _ = _random_run(variant, 200 + variant)
        S = S0.copy()
        cum = np.ones(S0.shape[0])
        for st in steps:
            S, o = step(variant, S, st["q"], st["k"], st["v"], st["decay"], np.asarray(0.0), None)
            cum = cum * st["decay"]
            np.testing.assert_allclose(S, cum[:, None] * S0, rtol=1e-13, atol=0)
            np.testing.assert_allclose(o, (cum[:, None] * S0).T @ st["q"], rtol=0, atol=1e-12)
        S = S0.copy()
        one = np.asarray(1.0) if variant == 0 else np.ones(S0.shape[0])
        for st in steps:
            S, _ = step(variant, S, st["q"], st["k"], st["v"], one, np.asarray(0.0), None)
        assert np.array_equal(S, S0)
    S0, steps, bonus = _random_run(2, 300)
    S = np.zeros_like(S0)
    for t, st in enumerate(steps):
        S, o = step(2, S, st["q"], st["k"], st["v"], np.ones(S0.shape[0]), None, bonus)
        att = sum((np.dot(st["q"], steps[j]["k"]) * steps[j]["v"] for j in range(t)),
                  np.zeros(S0.shape[1]))
        ref = att + np.sum(st["q"] * bonus * st["k"]) * st["v"]
        np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)
        kv = sum(np.outer(steps[j]["k"], steps[j]["v"]) for j in range(t + 1))
        np.testing.assert_allclose(S, kv, rtol=0, atol=1e-12)


# ------------------------------------------------------------------- P4 ----
def pin_projection(step):
    """Kaczmarz projection (Kaczmarz Linear Attention abstract): with the step size
    beta = 1/||k||^2 the written state maps k onto v exactly: S_t^T k_t = v_t,
    whatever the decay.  Unit k with beta = 1 is the special case."""
    for variant in (0, 1):
        for unit in (True, False):
            S0, steps, _ = _random_run(variant, 400 + 2 * variant + unit, unit_k=unit)
            S = S0.copy()
            for st in steps:
                beta = np.asarray(1.0 / np.dot(st["k"], st["k"]))
                S, _ = step(variant, S, st["q"], st["k"], st["v"], st["decay"], beta, None)
                np.testing.assert_allclose(S.T @ st["k"], st["v"], rtol=0, atol=1e-12)


# ------------------------------------------------------------------- P5 ----
def pin_kda_reduces_to_gdn(step):
    """KDA with a_t = alpha_t * 1 equals Gated DeltaNet (Gated DeltaNet-2 abstract)."""
    S0, steps, _ = _random_run(0, 500)
    Sg = S0.copy()
    Sk = S0.copy()
    for st in steps:
        Sg, og = step(0, Sg, st["q"], st["k"], st["v"], st["decay"], st["beta"], None)
        a = np.full(S0.shape[0], float(st["decay"]))
        Sk, ok = step(1, Sk, st["q"], st["k"], st["v"], a, st["beta"], None)
        np.testing.assert_allclose(Sk, Sg, rtol=0, atol=1e-13)
        np.testing.assert_allclose(ok, og, rtol=0, atol=1e-13)


# ------------------------------------------------------------------- P6/P7 -
def pin_deferred_equals_eager(tile_cls, step, log_lens=(1, 2, 3, 8, 16, 64), T=150):
    """Deferred base + log equals the eager recurrence at every step (DeltaLog
    Abstract: the deferred form leaves the dense state the model sees unchanged),
    and the merge schedule is the closed form (n0 + t) mod L."""
    for variant in (0, 1, 2):
        for L in log_lens:
            for n0 in sorted({0, L // 2, L - 1}):
                S0, steps, bonus = _random_run(variant, 600 + 7 * variant + L + n0, T=T, dk=6, dv=4,
                                               unit_k=True)
                S = S0.copy()
                tile = tile_cls(variant, S0, L, n0, bonus)
                base = tile.base.copy()
                merges = tile.merges
                for t, st in enumerate(steps, start=1):
                    S, o = step(variant, S, st["q"], st["k"], st["v"], st["decay"], st["beta"], bonus)
                    od = tile.step(st["q"], st["k"], st["v"], st["decay"], st["beta"])
                    scale = max(1.0, float(np.max(np.abs(S))))
                    assert np.max(np.abs(od - o)) <= 1e-12 * scale, (variant, L, n0, t)
                    assert np.max(np.abs(tile.materialize() - S)) <= 1e-12 * scale, (variant, L, n0, t)
                    assert tile.fill == (n0 + t) % L, (variant, L, n0, t)
                    assert tile.last_slot == (n0 + t - 1) % L
                    if (n0 + t) % L == 0:
                        assert tile.merges == merges + 1, (variant, L, n0, t)
                    else:
                        assert tile.merges == merges and np.array_equal(tile.base, base), (variant, L, n0, t)
                    base = tile.base.copy()
                    merges = tile.merges


# ------------------------------------------------------------ Kaczmarz ----
def pin_kaczmarz_step_size(step, kbeta):
    """Kaczmarz step size (Kaczmarz Linear Attention abstract), beta = eta / (||k||^2 + eps):
    the delta write then moves S^T k from the decayed read D^T k towards v by the
    fraction rho = eta ||k||^2 / (||k||^2 + eps); eta = 1, eps = 0 lands on v exactly."""
    for variant in (0, 1):
        S0, steps, _ = _random_run(variant, 800 + variant, unit_k=False)
        S = S0.copy()
        for i, st in enumerate(steps):
            eta = 1.0 if i % 2 == 0 else 0.3 + 0.05 * i
            eps = 0.0 if i % 3 == 0 else 0.25
            k = st["k"] * (1.0 + i)  # norms far from 1
            d = st["decay"]
            read_before = ((np.eye(S.shape[0]) * d if variant == 0 else np.diag(d)) @ S).T @ k
            beta = kbeta(np.asarray(eta), k, eps)
            S, _ = step(variant, S, st["q"], k, st["v"], d, beta, None)
            kk = float(np.dot(k, k))
            rho = eta * kk / (kk + eps)
            np.testing.assert_allclose(S.T @ k, (1 - rho) * read_before + rho * st["v"],
                                       rtol=0, atol=1e-10 * max(1.0, kk))


# ------------------------------------------------------ the seeded driver ----
# The driver (oracle/drive.py) turns a seeded workload into steps of the recurrence and
# measures the distance between two runs.  Every GPU parity assertion goes through it,
# so it is pinned here on hand-worked values: the per-tensor error on dyadic cases, the
# widening of bf16 bits on chosen bit patterns, and whole runs on the worked examples of
# tests/golden (every value exact, so runs must reproduce them bit for bit).

def pin_rel_err(rel_err):
    """Per-tensor relative error max|got - ref| / max|ref| (the reading of "max relative
    error": one tensor is a state or an output vector), worst tensor returned; a tensor
    whose reference is all zeros is measured in absolute terms.  Values worked by hand."""
    ref = np.array([[100.0, 0.0], [1.0, 1.0]])
    assert rel_err(np.array([[100.0, 0.0], [1.5, 1.0]]), ref, (-1,)) == 0.5   # 0.5 / 1, not / 100
    assert rel_err(np.array([[100.0, 0.0], [0.5, 1.0]]), ref, (-1,)) == 0.5   # error below the reference
    assert rel_err(np.array([[100.0, 0.0], [1.5, 1.0]]), ref) == 0.005        # one tensor: 0.5 / 100
    assert rel_err(np.array([[100.0, 0.0], [1.5, 1.0]]), ref, (-2, -1)) == 0.005
    # the scale is the largest magnitude, not the largest value
    assert rel_err(np.array([[-4.0, 3.0]]), np.array([[-4.0, 2.0]]), (-1,)) == 0.25
    # an all-zero reference: absolute error
    assert rel_err(np.array([[0.0, 0.25], [2.0, 4.0]]), np.array([[0.0, 0.0], [2.0, 4.0]]), (-1,)) == 0.25
    # states, axes (-2, -1): the second state's error is half its scale
    ref = np.array([[[1, 2], [3, 4]], [[0.5, 0], [0, 0]]], float)
    got = np.array([[[1, 2], [3, 4.5]], [[0.5, 0.25], [0, 0]]], float)
    assert rel_err(got, ref, (-2, -1)) == 0.5
    assert rel_err(got[:1], ref[:1], (-2, -1)) == 0.125
    assert rel_err(ref, ref, (-2, -1)) == 0.0


def pin_elem_rel_err(elem_rel_err):
    """Element-wise relative error |got - ref| / max(|ref|, 1e-6 max|ref|), the floor taken
    per tensor (the companion figure of the per-tensor error).  Worked by hand."""
    ref = np.array([4.0, 2.0 ** -30, 0.0, -2.0])
    got = np.array([4.0, 2.0 ** -29, 2.0 ** -20, -2.25])
    # elements: 0; 2^-30 / 4e-6; 2^-20 / 4e-6 (the floor); 0.25 / 2
    np.testing.assert_allclose(elem_rel_err(got, ref), 2.0 ** -20 / 4e-6, rtol=1e-14, atol=0)
    # a second tensor of scale 2^-10: its floor is 1e-6 2^-10, so 2^-30 off is 2^-20 / 1e-6
    ref2 = np.stack([ref, [2.0 ** -10, 0.0, 0.0, 0.0]])
    got2 = np.stack([got, [2.0 ** -10, 2.0 ** -30, 0.0, 0.0]])
    np.testing.assert_allclose(elem_rel_err(got2, ref2, (-1,)), 2.0 ** -20 / 1e-6, rtol=1e-14, atol=0)
    np.testing.assert_allclose(elem_rel_err(got2, ref2), 2.0 ** -20 / 4e-6, rtol=1e-14, atol=0)
    # exact agreement, and an all-zero reference (absolute error)
    assert elem_rel_err(ref, ref) == 0.0
    assert elem_rel_err(np.array([[0.0, 0.125]]), np.array([[0.0, 0.0]]), (-1,)) == 0.125
    # a relative error well above the floor is the plain |d| / |ref|
    assert elem_rel_err(np.array([1.0, 3.0]), np.array([1.0, 2.0])) == 0.5


# bf16 bit patterns and the values they encode (bf16 is the top half of an fp32)
BF16_CASES = [(0x3F80, 1.0), (0xC000, -2.0), (0x3FC0, 1.5), (0x0001, 2.0 ** -133),
              (0x7F7F, (2.0 - 2.0 ** -7) * 2.0 ** 127), (0x8000, -0.0), (0x3E80, 0.25), (0xBF40, -0.75)]


def _hand_inputs(variant, kla=False):
    """A 2-slot, 2 x 2-tile workload (dk = 2, dv = 3) whose every value is chosen by hand."""
    from inputs import DecodeInputs
    P, B, H, dk, dv = 2, 2, 2, 2, 3
    nc = len(BF16_CASES)
    idx = lambda p, b, h, i, off: (off + 5 * p + 3 * b + 2 * h + i) % nc
    bits = lambda d, off: np.array([[[[BF16_CASES[idx(p, b, h, i, off)][0] for i in range(d)]
                                      for h in range(H)] for b in range(B)] for p in range(P)], np.uint16)
    vals = lambda d, off: np.array([[[[BF16_CASES[idx(p, b, h, i, off)][1] for i in range(d)]
                                      for h in range(H)] for b in range(B)] for p in range(P)], np.float64)
    q, k, v = bits(dk, 0), bits(dk, 3), bits(dv, 6)
    want = dict(q=vals(dk, 0), k=vals(dk, 3), v=vals(dv, 6))
    dshape = (P, B, H) if variant == 0 else (P, B, H, dk)
    decay = (np.arange(np.prod(dshape), dtype=np.float32).reshape(dshape) + 1) / 64
    beta = None if variant == 2 else (np.arange(P * B * H, dtype=np.float32).reshape(P, B, H) + 1) / 32
    bonus = np.array([[0.5, -1.0], [2.0, 0.25]], np.float32) if variant == 2 else None
    eta = eps = None
    if kla:
        # tile (b, h) keys: slot 0 (b=0,h=0) is (1, -2) by construction of the table
        eta, beta, eps = beta, None, 0.75
    inp = DecodeInputs(variant, B, H, dk, dv, 4, 8, np.zeros((B, H, dk, dv), np.float32), q, k, v, decay, beta,
                       bonus, np.zeros(B, np.int32), eta, 0.0 if eps is None else eps)
    return inp, want


def pin_step_arrays(step_arrays):
    """Step t's inputs: bf16 bits widened exactly, pool slot t mod P, tiles in `sel`
    order, the RWKV6 bonus taken per head, and the Kaczmarz step size
    eta / (||k||^2 + eps) formed from the bf16 key as the kernels see it."""
    for variant in (0, 1, 2):
        inp, want = _hand_inputs(variant)
        for t in (0, 1, 2, 5):
            p = t % 2
            a = step_arrays(inp, t)
            for name in ("q", "k", "v"):
                assert a[name].dtype == np.float64
                assert np.array_equal(a[name], want[name][p]), (variant, name, t)
                assert np.array_equal(np.signbit(a[name]), np.signbit(want[name][p])), (variant, name, t)
            assert np.array_equal(a["decay"], inp.decay[p].astype(np.float64))
            if variant == 2:
                assert a["beta"] is None
                assert a["bonus"].shape == (2, 2, 2)
                for b in range(2):
                    assert np.array_equal(a["bonus"][b], inp.bonus.astype(np.float64))
            else:
                assert np.array_equal(a["beta"], inp.beta[p].astype(np.float64)) and a["bonus"] is None
            sel = [(1, 0), (0, 1), (1, 1)]
            s = step_arrays(inp, t, sel)
            for i, (b, h) in enumerate(sel):
                for name in ("q", "k", "v"):
                    assert np.array_equal(s[name][i], want[name][p, b, h]), (variant, name, t, b, h)
                assert np.array_equal(s["decay"][i], inp.decay[p, b, h])
                if variant == 2:
                    assert np.array_equal(s["bonus"][i], inp.bonus[h].astype(np.float64))
                else:
                    assert s["beta"][i] == inp.beta[p, b, h]
    # Kaczmarz step size, worked by hand from the table's keys
    for variant in (0, 1):
        inp, want = _hand_inputs(variant, kla=True)
        for t in (0, 3):
            p = t % 2
            a = step_arrays(inp, t)
            kk = np.sum(want["k"][p] ** 2, axis=-1)
            assert np.array_equal(a["beta"], inp.eta[p].astype(np.float64) / (kk + 0.75))
        # slot 0, tile (0, 1): k = (-0, 0.25) -> ||k||^2 = 1/16; eta = 2/32, eps = 3/4
        k01 = want["k"][0, 0, 1]
        assert k01[1] == 0.25 and k01[0] == 0.0 and np.signbit(k01[0])
        assert inp.eta[0, 0, 1] == 2.0 / 32
        assert step_arrays(inp, 0)["beta"][0, 1] == 0.0625 / 0.8125
        assert step_arrays(inp, 2, [(0, 1)])["beta"][0] == 0.0625 / 0.8125
        # the extremes of the table: k = (2^-133, largest bf16) at tile (0, 0)
        k00 = want["k"][0, 0, 0]
        assert k00[0] == 2.0 ** -133 and k00[1] == (2.0 - 2.0 ** -7) * 2.0 ** 127


def golden_inputs(g, scale2: bool = True):
    """A worked example as a seeded-workload object: batch 1, head 0 the example and, when
    `scale2`, head 1 the same run with S0 and every v doubled (each of the three rules is
    linear in (S0, v) jointly, so every state and output doubles, exactly)."""
    from inputs import DecodeInputs, f32_to_bf16_bits
    var = VARIANTS[g["variant"]]
    H = 2 if scale2 else 1
    steps = g["steps"]
    T = len(steps)
    S0 = np.array(g["S0"], np.float32)
    dk, dv = S0.shape
    mul = np.array([1.0, 2.0][:H], np.float32)
    s0 = (mul[:, None, None] * S0)[None].astype(np.float32)
    vec = lambda name, m: np.stack([np.stack([np.array(st[name], np.float32) * (mul[h] if m else 1)
                                              for h in range(H)])[None] for st in steps])
    q, k, v = (f32_to_bf16_bits(vec(n, n == "v")) for n in ("q", "k", "v"))
    for n, arr in (("q", q), ("k", k), ("v", v)):  # the examples' values are exact in bf16
        from inputs import bf16_bits_to_f32
        assert np.array_equal(bf16_bits_to_f32(arr), vec(n, n == "v")), n
    if var == 0:
        decay = np.array([[[st["decay"]] * H] for st in steps], np.float32)
    else:
        decay = np.stack([np.stack([np.array(st["decay"], np.float32)] * H)[None] for st in steps])
    beta = None if var == 2 else np.array([[[st["beta"]] * H] for st in steps], np.float32)
    bonus = np.stack([np.array(g["bonus"], np.float32)] * H) if var == 2 else None
    inp = DecodeInputs(var, 1, H, dk, dv, 4, T, s0, q, k, v, decay, beta, bonus, np.zeros(1, np.int32))
    want_S = np.array([np.array(st["S"], float) for st in steps])
    want_o = np.array([np.array(st["o"], float) for st in steps])
    return inp, want_S, want_o


def pin_run_eager(run_eager):
    """Whole eager runs over the worked examples reproduce them bit for bit: the final
    state, every output, the snapshots after chosen steps, and the order of `sel`."""
    for g in load_golden():
        inp, wS, wo = golden_inputs(g)
        T = len(wo)
        S, outs = run_eager(inp, T)
        assert S.shape == (1, 2) + wS.shape[1:] and outs.shape == (T, 1, 2, wo.shape[1])
        assert np.array_equal(S[0, 0], wS[-1]) and np.array_equal(S[0, 1], 2 * wS[-1]), g["variant"]
        assert np.array_equal(outs[:, 0, 0], wo) and np.array_equal(outs[:, 0, 1], 2 * wo), g["variant"]
        S, outs = run_eager(inp, T, sel=[(0, 1), (0, 0)])
        assert np.array_equal(S, np.stack([2 * wS[-1], wS[-1]]))
        assert np.array_equal(outs, np.stack([2 * wo, wo], axis=1))
        S, none, snaps = run_eager(inp, T, sel=[(0, 0)], keep_outputs=False, check_every={0, 1})
        assert none is None and sorted(snaps) == [0, 1]
        assert np.array_equal(snaps[0][0], wS[0]) and np.array_equal(snaps[1][0], wS[1])
        S, outs = run_eager(inp, 2, sel=[(0, 0)])
        assert np.array_equal(S[0], wS[1]) and np.array_equal(outs[:, 0], wo[:2])
        if g["variant"] == "rwkv6":
            # An explicit start state replaces the workload's.  RWKV6 is linear in S0 alone:
            # from 2 S0 with head 0's inputs the run adds diag(prod w) S0 to the state and
            # r_t^T diag(prod_{i<t} w_i) S0 to output t.  Worked by hand: prod w over the
            # three steps = (1/4, 1/16); the outputs gain (1, 2), (1.25, 2), (0.375, 0.5).
            S, outs = run_eager(inp, T, sel=[(0, 0)], s0=inp.s0[0, 1][None])
            assert np.array_equal(S[0], np.array([[4.0, 5.0], [2.625, 4.0]]))
            assert np.array_equal(outs[:, 0], np.array([[4.5, 7.0], [13.5, 18.0], [5.25, 8.0]]))


def pin_run_deferred(run_deferred):
    """Base + log runs over the worked examples: outputs and the dense state bit for bit
    for every short log length and start fill, the fill after each step (n0 + t) mod L,
    the slot each step wrote (n0 + t - 1) mod L, and a log length given explicitly."""
    for g in load_golden():
        inp, wS, wo = golden_inputs(g)
        T = len(wo)
        for L in (1, 2, 3, 4):
            for n0 in range(L):
                inp.fill0 = np.array([n0], np.int32)
                tiles, outs, fills, slots = run_deferred(inp, T, [(0, 1), (0, 0)], log_len=L)
                assert np.array_equal(outs, np.stack([2 * wo, wo], axis=1)), (g["variant"], L, n0)
                assert np.array_equal(tiles[0].materialize(), 2 * wS[-1])
                assert np.array_equal(tiles[1].materialize(), wS[-1])
                for t in range(T):
                    assert list(fills[t]) == [(n0 + t + 1) % L] * 2, (g["variant"], L, n0, t)
                    assert list(slots[t]) == [(n0 + t) % L] * 2, (g["variant"], L, n0, t)
        inp.fill0 = np.array([1], np.int32)
        inp.log_len = 3
        _, _, fills, _ = run_deferred(inp, T, [(0, 0)])
        assert [int(f[0]) for f in fills] == [2, 0, 1]
