"""Seeded synthetic decode inputs shared by the oracle side and the HIP side.

This module holds no arithmetic of the recurrences: it only draws random
numbers, shapes them, rounds fp32 to bf16 bits and says which pool slot a step
uses.  Both the CPU oracle and the GPU harness read the arrays it returns, so
the two sides see bit-identical inputs.

Workloads (shapes and value distributions) stand in for the activations of
trained GDN / KDA / RWKV6 layers, which the DeltaLog page ("DeltaLog: Deferred
Materialization of Recurrent States for Linear Attention Decoding", Abstract)
evaluates on but does not print.  Readings taken where the recipe is silent:

* N(mu, sigma): sigma is the standard deviation.
* The initial state S0 ~ N(0, 0.02) for every workload.
* Only k is L2-normalised in the large GDN/KDA workloads; q is normalised
  only in the single-head smoke workload, which names both.
* The RWKV6 bonus u is one dk-vector per head, constant over time.
* Ragged initial log fills are per sequence and shared by all its heads.

Every (step, sequence) block is drawn from its own PCG64 stream keyed by
(seed, step, sequence), so a batch slice [0, B') of a workload is exactly the
first B' sequences of the full workload, and any single tile can be rebuilt
without drawing the rest.  Long runs may cycle a pool of P drawn steps: step t
uses pool slot t % P.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

GDN, KDA, RWKV6 = 0, 1, 2
VARIANT_NAMES = {GDN: "gdn", KDA: "kda", RWKV6: "rwkv6"}

# Workload table: shapes and distributions of the five decode workloads.
WORKLOADS = {
    1: dict(name="gdn-smoke", variant=GDN, batch=1, heads=1, dk=64, dv=64,
            log_len=8, steps=64, decay="softplus05", q_norm=True, ragged=False),
    2: dict(name="gdn-b64-h32-d128", variant=GDN, batch=64, heads=32, dk=128, dv=128,
            log_len=16, steps=1024, decay="uniform09", q_norm=False, ragged=False),
    3: dict(name="kda-b128-h32-d128", variant=KDA, batch=128, heads=32, dk=128, dv=128,
            log_len=16, steps=1024, decay="softplus002", q_norm=False, ragged=False),
    4: dict(name="rwkv6-b256-h64-d64", variant=RWKV6, batch=256, heads=64, dk=64, dv=64,
            log_len=32, steps=2048, decay="rwkv", q_norm=False, ragged=False),
    5: dict(name="gdn-serve-48l-b512-h32-d128", variant=GDN, batch=512, heads=32, dk=128,
            dv=128, log_len=16, steps=4096, decay="uniform09", q_norm=False, ragged=True,
            layers=48),
    # Kaczmarz step size (beta = eta / (||k||^2 + eps)) on the GDN B=64 shape; keys are not
    # normalised here, so the key norm actually sets the step.
    6: dict(name="gdn-kla-b64-h32-d128", variant=GDN, batch=64, heads=32, dk=128, dv=128,
            log_len=16, steps=1024, decay="uniform09", q_norm=False, k_norm=False, ragged=False,
            kla=True, eps=1e-6),
}


# ---------------------------------------------------------------- bf16 bits --
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (round to nearest, ties to even); return uint16 bits."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (b >> np.uint64(16)) & np.uint64(1)
    r = (b + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bits to the fp32 values they encode (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ------------------------------------------------------------------- inputs --
@dataclasses.dataclass
class DecodeInputs:
    """Inputs of one decode run.  Arrays are C-contiguous numpy arrays.

    s0:    fp32 [B][H][dk][dv]  initial state (rows are key channels)
    q,k,v: uint16 bf16 bits [P][B][H][dk|dv]  (q is RWKV6's receptance r)
    decay: fp32 [P][B][H] (GDN) or [P][B][H][dk] (KDA, RWKV6), in (0, 1]
    beta:  fp32 [P][B][H] (GDN, KDA) or None (RWKV6)
    bonus: fp32 [H][dk] (RWKV6) or None
    fill0: int32 [B] initial log fills, each in [0, log_len)
    eta:   fp32 [P][B][H] or None: when set (GDN/KDA), beta is None and the step
           size is the Kaczmarz one, eta / (||k||^2 + eps)
    """
    variant: int
    batch: int
    heads: int
    dk: int
    dv: int
    log_len: int
    steps: int
    s0: np.ndarray
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    decay: np.ndarray
    beta: Optional[np.ndarray]
    bonus: Optional[np.ndarray]
    fill0: np.ndarray
    eta: Optional[np.ndarray] = None
    eps: float = 0.0

    @property
    def pool(self) -> int:
        return self.q.shape[0]

    def slot(self, t: int) -> int:
        """Pool slot holding the inputs of step t (0-based)."""
        return t % self.pool

    def step(self, t: int) -> dict:
        """The inputs of step t as a dict of arrays [B][H][...]."""
        p = self.slot(t)
        return dict(q=self.q[p], k=self.k[p], v=self.v[p], decay=self.decay[p],
                    beta=None if self.beta is None else self.beta[p],
                    eta=None if self.eta is None else self.eta[p])


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(x) for x in key])))


def _softplus(x: np.ndarray) -> np.ndarray:
    return np.logaddexp(0.0, x)


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-x))


def _draw_decay(g: np.random.Generator, kind: str, variant: int, heads: int, dk: int) -> np.ndarray:
    shape = (heads,) if variant == GDN else (heads, dk)
    if kind == "softplus05":
        d = np.exp(-_softplus(g.standard_normal(shape)) * 0.05)
    elif kind == "uniform09":
        # alpha = 0.9 + 0.1*(1 - U), U in [0, 1): never reaches 0.9.
        d = 0.9 + 0.1 * (1.0 - g.random(shape))
    elif kind == "softplus002":
        d = np.exp(-_softplus(g.standard_normal(shape)) * 0.02)
    elif kind == "rwkv":
        d = np.exp(-np.exp(g.normal(-1.0, 0.5, shape)))
    else:
        raise ValueError(kind)
    return d.astype(np.float32)


def _l2n(x: np.ndarray) -> np.ndarray:
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def make_inputs(workload: int, steps: Optional[int] = None, *, batch: Optional[int] = None,
                heads: Optional[int] = None, log_len: Optional[int] = None,
                pool: Optional[int] = None, seed: Optional[int] = None,
                fill0: Optional[np.ndarray] = None, layer: int = 0, dk: Optional[int] = None,
                dv: Optional[int] = None, kla: Optional[bool] = None) -> DecodeInputs:
    """Draw the inputs of a decode workload (see WORKLOADS).

    steps:   number of decode steps the run will take (default: the workload's).
    batch, heads, log_len: override the workload's (a batch override is a slice).
    pool:    number of distinct drawn steps; step t uses slot t % pool
             (default: min(steps, 256)).
    seed:    stream seed (default: the workload number).
    fill0:   explicit initial fills [batch]; default zeros, or U{0..L-1} per
             sequence for ragged workloads.
    layer:   layer index for multi-layer workloads (separate streams per layer).
    dk, dv:  override the head sizes (edge-case shapes; distributions unchanged).
    kla:     GDN/KDA only: draw eta ~ sigmoid(N(0,1)) in place of beta (Kaczmarz step size).
    """
    w = WORKLOADS[workload]
    variant = w["variant"]
    B = w["batch"] if batch is None else int(batch)
    H = w["heads"] if heads is None else int(heads)
    dk = w["dk"] if dk is None else int(dk)
    dv = w["dv"] if dv is None else int(dv)
    L = w["log_len"] if log_len is None else int(log_len)
    T = w["steps"] if steps is None else int(steps)
    P = min(T, 256) if pool is None else int(pool)
    P = max(P, 1)
    seed = workload if seed is None else int(seed)
    kla = bool(w.get("kla", False)) if kla is None else bool(kla)
    if kla and variant == RWKV6:
        raise ValueError("the Kaczmarz step size applies to GDN and KDA")
    k_norm = w.get("k_norm", variant != RWKV6)

    s0 = np.empty((B, H, dk, dv), np.float32)
    for b in range(B):
        s0[b] = _rng(seed, layer, 0xB45E, b).standard_normal((H, dk, dv), dtype=np.float32)
        s0[b] *= np.float32(0.02)

    q = np.empty((P, B, H, dk), np.uint16)
    k = np.empty((P, B, H, dk), np.uint16)
    v = np.empty((P, B, H, dv), np.uint16)
    dshape = (P, B, H) if variant == GDN else (P, B, H, dk)
    decay = np.empty(dshape, np.float32)
    beta = None if variant == RWKV6 else np.empty((P, B, H), np.float32)
    for p in range(P):
        for b in range(B):
            g = _rng(seed, layer, p, b)
            qq = g.standard_normal((H, dk))
            kk = g.standard_normal((H, dk))
            vv = g.standard_normal((H, dv))
            if k_norm:
                kk = _l2n(kk)
            if w["q_norm"]:
                qq = _l2n(qq)
            q[p, b] = f32_to_bf16_bits(qq.astype(np.float32))
            k[p, b] = f32_to_bf16_bits(kk.astype(np.float32))
            v[p, b] = f32_to_bf16_bits(vv.astype(np.float32))
            decay[p, b] = _draw_decay(g, w["decay"], variant, H, dk)
            if beta is not None:
                beta[p, b] = _sigmoid(g.standard_normal(H)).astype(np.float32)

    bonus = None
    if variant == RWKV6:
        bonus = _rng(seed, layer, 0xB0, 0).normal(0.0, 0.1, (H, dk)).astype(np.float32)

    if fill0 is None:
        if w["ragged"]:
            fill0 = np.array([_rng(seed, 0xF111, b).integers(0, L) for b in range(B)], np.int32)
        else:
            fill0 = np.zeros(B, np.int32)
    fill0 = np.ascontiguousarray(fill0, dtype=np.int32)
    assert fill0.shape == (B,)

    eta = None
    if kla:
        # eta takes beta's draw (sigmoid of a standard normal) and beta goes away
        eta, beta = beta, None
    return DecodeInputs(variant, B, H, dk, dv, L, T, s0, q, k, v, decay, beta, bonus, fill0, eta,
                        float(w.get("eps", 1e-6)) if kla else 0.0)


def tile_inputs(inp: DecodeInputs, b: int, h: int) -> DecodeInputs:
    """The same run restricted to the single tile (b, h): batch 1, head 1."""
    sl = lambda a: None if a is None else np.ascontiguousarray(a[:, b:b + 1, h:h + 1])
    return DecodeInputs(inp.variant, 1, 1, inp.dk, inp.dv, inp.log_len, inp.steps,
                        np.ascontiguousarray(inp.s0[b:b + 1, h:h + 1]),
                        sl(inp.q), sl(inp.k), sl(inp.v), sl(inp.decay), sl(inp.beta),
                        None if inp.bonus is None else np.ascontiguousarray(inp.bonus[h:h + 1]),
                        np.ascontiguousarray(inp.fill0[b:b + 1]), sl(inp.eta), inp.eps)
