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
    Abstract: the model observes the same dense state as in eager decoding),
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
