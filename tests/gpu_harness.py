"""Helpers for the GPU parity tests: upload seeded inputs, drive the C ABI, gather results.

Only marshalling and bookkeeping live here; every decode step runs in
libdeltalog.so through the Python binding.
"""
from __future__ import annotations

import numpy as np
import torch

from linear_attention_recurrent_amd import deltalog as dl


def dev():
    return torch.device("cuda", 0)


def to_bf16(bits: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device).view(torch.bfloat16)


class Uploaded:
    """A DecodeInputs copied to the device, with one StepIO per pool slot."""

    def __init__(self, inp, device=None, out=None):
        self.inp = inp
        self.device = device or dev()
        d = self.device
        self.q = to_bf16(inp.q, d)
        self.k = to_bf16(inp.k, d)
        self.v = to_bf16(inp.v, d)
        self.decay = torch.from_numpy(inp.decay).to(d)
        self.beta = None if inp.beta is None else torch.from_numpy(inp.beta).to(d)
        self.eta = None if inp.eta is None else torch.from_numpy(inp.eta).to(d)
        self.bonus = None if inp.bonus is None else torch.from_numpy(inp.bonus).to(d)
        self.s0 = torch.from_numpy(inp.s0).to(d)
        self.out = out if out is not None else torch.empty((inp.batch, inp.heads, inp.dv), dtype=torch.float32,
                                                           device=d)
        self.ios = [dl.make_step_io(inp.variant, inp.batch, inp.heads, inp.dk, inp.dv, d,
                                    self.q[p], self.k[p], self.v[p], self.decay[p],
                                    None if self.beta is None else self.beta[p], self.bonus, self.out,
                                    None if self.eta is None else self.eta[p], inp.eps)
                    for p in range(inp.pool)]

    def io(self, t: int):
        return self.ios[t % self.inp.pool]


def new_pool(inp, log_len=None, fill0=None, up: Uploaded = None, base_dtype=dl.BASE_F32):
    L = inp.log_len if log_len is None else log_len
    pool = dl.DeltaLogPool(inp.variant, inp.batch, inp.heads, inp.dk, inp.dv, L, dev(), base_dtype)
    dl.dl_init_state(pool, up.s0 if up is not None else torch.from_numpy(inp.s0).to(dev()),
                     inp.fill0 if fill0 is None else fill0)
    return pool


def run_deltalog(inp, steps, log_len=None, sel=None, up: Uploaded = None, every_step=None,
                 base_dtype=dl.BASE_F32):
    """Run `steps` decode steps; return (pool, outputs) with outputs float32 numpy
    [steps][tiles][dv] for the tiles in `sel` (list of (b, h)), or all tiles if None.
    every_step(t, pool) is called after each step when given."""
    up = up or Uploaded(inp)
    pool = new_pool(inp, log_len, up=up, base_dtype=base_dtype)
    if sel is None:
        idx = None
        outs = torch.empty((steps, inp.batch * inp.heads, inp.dv), dtype=torch.float32, device=dev())
    else:
        idx = torch.tensor([b * inp.heads + h for b, h in sel], device=dev())
        outs = torch.empty((steps, len(sel), inp.dv), dtype=torch.float32, device=dev())
    flat = up.out.view(inp.batch * inp.heads, inp.dv)
    for t in range(steps):
        dl.dl_decode_step(pool, up.io(t))
        if idx is None:
            outs[t].copy_(flat)
        else:
            outs[t].copy_(flat.index_select(0, idx))
        if every_step is not None:
            every_step(t, pool)
    torch.cuda.synchronize()
    o = outs.cpu().numpy()
    if sel is None:
        o = o.reshape(steps, inp.batch, inp.heads, inp.dv)
    return pool, o


def run_eager_gpu(inp, steps, up: Uploaded = None):
    up = up or Uploaded(inp)
    state = up.s0.clone()
    outs = torch.empty((steps, inp.batch, inp.heads, inp.dv), dtype=torch.float32, device=dev())
    for t in range(steps):
        dl.dl_eager_step(inp.variant, state, up.io(t))
        outs[t].copy_(up.out)
    torch.cuda.synchronize()
    return state.cpu().numpy(), outs.cpu().numpy()


def materialized_state(pool) -> np.ndarray:
    """The dense state of every tile: fold every non-empty log of a copy of the pool."""
    c = pool.clone()
    dl.dl_merge(c, 1)
    torch.cuda.synchronize()
    assert int(c.fill.max().item()) == 0
    return c.base.float().cpu().numpy()
