"""GPU parity of the fold's two arithmetic units (dl_merge_on): vector FMAs on a
streamed tile, and v_mfma_f32_4x4x1_16b_f32 on a register-resident tile.

Each case decodes from ragged start fills, then merges a copy of the pool with
each unit.  Integer results are exact: the fills of merged tiles become 0, the
others keep theirs, and untouched bases and every log array are bit-identical.
Merged fp32 bases match the fp64 oracle's dense state within 1e-4 per tensor
(max |gpu - ref| / max |ref|), and the two units agree bit for bit: both scale
the base, then add the entries one at a time in log order with a fused
multiply-add per element (the 4 x 4 x 1 MFMA adds one product to each element
it holds), from identically formed weights.  A bf16 base is rounded once by the
MFMA fold and once per stage by the vector fold (16 entries at 128 x 128, 32 at
64 x 64); with one stage, as in the bf16 cases here, at least 99 % of the merged
values must be bit-equal (measured: all) and the rest within one bf16 ulp.
Decoding then continues from the MFMA-merged pool and is held to the oracle
again.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_harness import Uploaded, materialized_state, new_pool
from inputs import make_inputs
from linear_attention_recurrent_amd import deltalog as dl

pytestmark = pytest.mark.gpu
TOL = 1e-4
UNITS = (dl.UNIT_VALU, dl.UNIT_MFMA)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("a GPU is required for the gpu-marked tests")
    dl.load_library()  # raises if the HIP library is missing: no fallback


def _close(what, got, ref, axes, tol=TOL):
    err = oracle.rel_err(got, ref, axes)
    print(f"{what}: max per-tensor rel err {err:.3e}, element-wise (floor 1e-6 of the tensor's scale) "
          f"{oracle.elem_rel_err(got, ref, axes):.3e}", flush=True)
    assert err <= tol, (what, err)
    return err


def _spread_fills(batch, L):
    """Start fills spread evenly over [0, L), the last one L - 1."""
    f = (np.arange(batch) * L // batch).astype(np.int32)
    f[-1] = L - 1
    return f


def _decoded_pool(inp, steps, base_dtype=dl.BASE_F32):
    up = Uploaded(inp)
    pool = new_pool(inp, up=up, base_dtype=base_dtype)
    for t in range(steps):
        dl.dl_decode_step(pool, up.io(t))
    torch.cuda.synchronize()
    return up, pool


def _merge_copies(pool, min_fill):
    """Merge one copy of `pool` with each unit; check the integer side exactly."""
    fill = pool.fill.cpu().numpy()
    base = pool.base.cpu()
    logs = [t.clone() for t in (pool.log_k, pool.log_u, pool.log_c)]
    merged = {}
    for unit in UNITS:
        c = pool.clone()
        dl.dl_merge_on(c, min_fill, unit)
        torch.cuda.synchronize()
        f = c.fill.cpu().numpy()
        hit = fill >= min_fill
        assert np.array_equal(f[hit], np.zeros(int(hit.sum()), np.int32)), unit
        assert np.array_equal(f[~hit], fill[~hit]), unit
        b = c.base.cpu()
        assert torch.equal(b[torch.from_numpy(~hit)], base[torch.from_numpy(~hit)]), unit
        for before, after in zip(logs, (c.log_k, c.log_u, c.log_c)):
            assert torch.equal(before, after), unit
        merged[unit] = (c, b)
    return fill >= min_fill, merged


CASES = [
    # workload (2 GDN, 3 KDA, 4 RWKV6), dk, dv, L, min_fill
    (2, 128, 128, 16, 1),
    (2, 128, 128, 64, 1),   # four staged passes for the vector unit, four stages of 16 entries here
    (2, 64, 64, 8, 3),
    (2, 64, 128, 20, 1),    # a partly filled last stage
    (3, 128, 128, 32, 1),
    (3, 64, 128, 16, 5),
    (3, 128, 64, 7, 1),
    (4, 64, 64, 32, 1),
    (4, 128, 64, 128, 1),   # the longest log: up to 127 entries
    (4, 64, 128, 12, 9),
]


@pytest.mark.parametrize("w,dk,dv,L,min_fill", CASES)
def test_units_match_the_oracle(w, dk, dv, L, min_fill):
    batch, heads = 6, 2
    steps = L + 7
    inp = make_inputs(w, steps + 12, batch=batch, heads=heads, log_len=L, dk=dk, dv=dv, pool=steps + 12,
                      seed=100 + w * 7 + L, fill0=_spread_fills(batch, L))
    up, pool = _decoded_pool(inp, steps)
    hit, merged = _merge_copies(pool, min_fill)
    assert hit.any() and (min_fill == 1 or (~hit).any())  # both kinds of tile occur
    ref_S, _ = oracle.run_eager(inp, steps, keep_outputs=False)
    m = torch.from_numpy(hit)
    got = {u: merged[u][1][m].numpy() for u in UNITS}
    for u in UNITS:
        _close(f"merged bases, unit {u}", got[u], ref_S[hit], (-2, -1))
    assert np.array_equal(got[dl.UNIT_MFMA], got[dl.UNIT_VALU])  # bit for bit
    # decoding continues from the MFMA-merged pool
    c = merged[dl.UNIT_MFMA][0]
    outs = []
    for t in range(steps, steps + 12):
        dl.dl_decode_step(c, up.io(t))
        outs.append(up.out.cpu().numpy())
    ref_S2, ref_o2 = oracle.run_eager(inp, steps + 12)
    _close("outputs after the MFMA merge", np.stack(outs), ref_o2[steps:], (-1,))
    _close("state after the MFMA merge", materialized_state(c), ref_S2, (-2, -1))


@pytest.mark.parametrize("w,L", [(2, 16), (3, 16), (4, 32)])
def test_units_on_a_bf16_base(w, L):
    batch, heads = 6, 2
    steps = L + 5
    dk = dv = 64 if w == 4 else 128
    inp = make_inputs(w, steps, batch=batch, heads=heads, log_len=L, pool=steps, seed=300 + w,
                      fill0=_spread_fills(batch, L))
    _, pool = _decoded_pool(inp, steps, base_dtype=dl.BASE_BF16)
    hit, merged = _merge_copies(pool, 1)
    m = torch.from_numpy(hit)
    a = merged[dl.UNIT_VALU][1][m].float().numpy()
    b = merged[dl.UNIT_MFMA][1][m].float().numpy()
    assert a.shape == (int(hit.sum()), dk, dv)
    same = np.mean(a == b)
    print(f"bf16 merged bases bit-equal between units: {same:.5f}", flush=True)
    assert same >= 0.99
    mag = np.maximum(np.abs(a), np.abs(b))
    ulp = np.exp2(np.floor(np.log2(np.where(mag > 0, mag, 1.0))) - 7)  # bf16: 8 significant bits
    assert np.all(np.abs(a - b) <= ulp)


@pytest.mark.parametrize("w", [2, 3, 4])
def test_full_size_units_agree_and_match_sampled_tiles(w):
    """The benchmark shapes (GDN B = 64 H = 32 128/128 L = 16, KDA B = 128 H = 32
    128/128 L = 16, RWKV6 B = 256 H = 64 64/64 L = 32) from ragged fills: the two
    units agree bit for bit on every tile; sampled tiles match the oracle."""
    probe = make_inputs(w, 1, pool=1)
    L = probe.log_len
    steps = L + 3
    inp = make_inputs(w, steps, pool=steps, seed=500 + w, fill0=_spread_fills(probe.batch, L))
    _, pool = _decoded_pool(inp, steps)
    hit, merged = _merge_copies(pool, 1)
    a = merged[dl.UNIT_VALU][1]
    b = merged[dl.UNIT_MFMA][1]
    assert torch.equal(a, b)  # every tile, bit for bit
    rng = np.random.default_rng(w)
    sel = [(int(rng.integers(inp.batch)), int(rng.integers(inp.heads))) for _ in range(6)]
    sel += [(0, 0), (inp.batch - 1, inp.heads - 1)]
    ref_S, _ = oracle.run_eager(inp, steps, sel=sel, keep_outputs=False)
    got = np.stack([b[bb, hh].numpy() for bb, hh in sel])
    _close("MFMA-merged sampled tiles", got, ref_S, (-2, -1))


# dl_merge's choice of unit (dl_merge_unit reports the library's measured table).  With a
# bf16 base and more than 16 entries per 128 x 128 tile the units round differently (the
# vector fold once per stage of 16 entries, the matrix fold once), so dl_merge's bits show
# which unit ran; the cases sit on both sides of the 128 x 128 bf16 thresholds.
AUTO_CASES = [
    # workload, dk, dv, L, expected unit
    (2, 128, 128, 32, dl.UNIT_MFMA),   # GDN, bf16 base: matrix cores from L = 32
    (3, 128, 128, 32, dl.UNIT_VALU),   # KDA, bf16 base: vector fold below L = 64
    (3, 128, 128, 64, dl.UNIT_MFMA),
]


@pytest.mark.parametrize("w,dk,dv,L,unit", AUTO_CASES)
def test_dl_merge_takes_the_measured_unit(w, dk, dv, L, unit):
    """dl_merge's result is bit-identical to the unit its table names and differs from the
    other unit's, on bf16 bases whose folds take more than one vector stage."""
    batch, heads = 4, 2
    steps = L - 1
    inp = make_inputs(w, steps, batch=batch, heads=heads, log_len=L, dk=dk, dv=dv, pool=steps, seed=700 + L,
                      fill0=np.zeros(batch, np.int32))
    _, pool = _decoded_pool(inp, steps, base_dtype=dl.BASE_BF16)
    assert int(pool.fill.min()) == L - 1
    assert dl.dl_merge_unit(pool.c_dims) == unit
    _, merged = _merge_copies(pool, 1)
    other = dl.UNIT_VALU if unit == dl.UNIT_MFMA else dl.UNIT_MFMA
    assert not torch.equal(merged[dl.UNIT_VALU][1], merged[dl.UNIT_MFMA][1])
    auto = pool.clone()
    dl.dl_merge(auto, 1)
    torch.cuda.synchronize()
    got = auto.base.cpu()
    assert torch.equal(got, merged[unit][1])
    assert not torch.equal(got, merged[other][1])
