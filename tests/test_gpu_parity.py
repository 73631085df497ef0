"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Tolerance: the largest per-tensor relative error max|gpu - ref| / max|ref|,
over every tile's state (dk x dv) and every (step, tile) output vector, must be
<= 1e-4.  Integer work (fills, log slots, which bases change) must be exact.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_harness import Uploaded, dev, materialized_state, new_pool, run_deltalog, run_eager_gpu
from inputs import GDN, KDA, RWKV6, make_inputs
from linear_attention_recurrent_amd import deltalog as dl

pytestmark = pytest.mark.gpu
TOL = 1e-4


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("a GPU is required for the gpu-marked tests")
    dl.load_library()  # raises if the HIP library is missing: no fallback


def _close(what, got, ref, axes):
    err = oracle.rel_err(got, ref, axes)
    print(f"{what}: max per-tensor rel err {err:.3e}, element-wise (floor 1e-6 of the tensor's scale) "
          f"{oracle.elem_rel_err(got, ref, axes):.3e}", flush=True)
    assert err <= TOL, (what, err)
    return err


def _compare(inp, steps, pool, outs, sel=None, log_len=None):
    ref_S, ref_o = oracle.run_eager(inp, steps, sel=sel)
    S = materialized_state(pool)
    if sel is not None:
        S = np.stack([S[b, h] for b, h in sel])
    _close("outputs", outs, ref_o, (-1,))
    _close("state", S, ref_S, (-2, -1))


# ---------------------------------------------------------------- workload 1 --
def test_workload1_64_steps_with_schedule():
    inp = make_inputs(1)
    L = inp.log_len
    fills, slots_ok, base_kept = [], [], []
    prev_base = {}

    def every(t, pool):
        f = pool.fill.cpu().numpy()
        fills.append(int(f[0, 0]))
        n_before = (int(inp.fill0[0]) + t) % L
        merged = (int(inp.fill0[0]) + t + 1) % L == 0
        if not merged:
            got = pool.log_k[0, 0, n_before].view(torch.int16).cpu().numpy().view(np.uint16)
            slots_ok.append(np.array_equal(got, inp.k[inp.slot(t), 0, 0]))
        b = pool.base.cpu().numpy()
        if "b" in prev_base:
            base_kept.append(np.array_equal(b, prev_base["b"]) != merged)
        prev_base["b"] = b

    pool, outs = run_deltalog(inp, inp.steps, every_step=every)
    assert fills == [(int(inp.fill0[0]) + t + 1) % L for t in range(inp.steps)]
    assert all(slots_ok) and len(slots_ok) == inp.steps - inp.steps // L
    assert all(base_kept)
    _compare(inp, inp.steps, pool, outs)
    # the deferred oracle's schedule agrees with the closed form used above
    _, _, dfills, dslots = oracle.run_deferred(inp, inp.steps, [(0, 0)])
    assert list(dfills[:, 0]) == fills


def test_workload1_4096_steps():
    inp = make_inputs(1, 4096, pool=4096)
    pool, outs = run_deltalog(inp, 4096)
    _compare(inp, 4096, pool, outs)


# ------------------------------------------------------- reduced-batch runs --
@pytest.mark.parametrize("w,batch,heads", [(2, 2, 4), (3, 2, 4), (4, 4, 4)])
def test_reduced_batch_4096_steps(w, batch, heads):
    inp = make_inputs(w, 4096, batch=batch, heads=heads, pool=4096)
    pool, outs = run_deltalog(inp, 4096)
    _compare(inp, 4096, pool, outs)


@pytest.mark.parametrize("w,batch,heads", [(1, 1, 1), (2, 2, 4), (3, 2, 4), (4, 4, 4)])
def test_eager_kernel(w, batch, heads):
    inp = make_inputs(w, 1024, batch=batch, heads=heads, pool=1024)
    S, outs = run_eager_gpu(inp, 1024)
    ref_S, ref_o = oracle.run_eager(inp, 1024)
    _close("eager outputs", outs, ref_o, (-1,))
    _close("eager state", S, ref_S, (-2, -1))


# ------------------------------------------ ragged serving slice, L sweep ----
@pytest.mark.parametrize("L,steps", [(4, 512), (8, 512), (16, 4096), (32, 512), (64, 512)])
def test_ragged_fills_log_length_sweep(L, steps):
    inp = make_inputs(5, steps, batch=16, heads=2, log_len=L, pool=min(steps, 512))
    assert len(set(inp.fill0.tolist())) > 1
    n0 = inp.fill0.astype(np.int64)
    state = {"base": None}
    bad = []

    def every(t, pool):
        f = pool.fill.cpu().numpy()
        expect = (n0 + t + 1) % L
        if not np.array_equal(f, np.repeat(expect[:, None], inp.heads, 1)):
            bad.append(("fill", t))
        base = pool.base.cpu().numpy()
        if state["base"] is not None:
            merged = expect == 0
            same = np.array([np.array_equal(base[b], state["base"][b]) for b in range(inp.batch)])
            if np.any(same[~merged] == False) or np.any(same[merged]):  # noqa: E712
                bad.append(("base", t))
            slot = (n0 + t) % L
            lk = pool.log_k.view(torch.int16).cpu().numpy().view(np.uint16)
            for b in range(inp.batch):
                if not merged[b] and not np.array_equal(lk[b, :, slot[b]], inp.k[inp.slot(t), b]):
                    bad.append(("slot", t, b))
        state["base"] = base

    check_every = every if steps <= 512 else None
    pool, outs = run_deltalog(inp, steps, every_step=check_every)
    assert not bad, bad[:5]
    _compare(inp, steps, pool, outs)


# ------------------------------------------------- full sizes, sampled tiles --
@pytest.mark.parametrize("w", [2, 3, 4])
def test_full_size_sampled_tiles_4096_steps(w):
    inp = make_inputs(w, 4096, pool=64)
    B, H = inp.batch, inp.heads
    sel = [(0, 0), (0, H - 1), (B // 3, H // 2), (B // 2, 1), (B - 1, 0), (B - 1, H - 1)]
    pool, outs = run_deltalog(inp, 4096, sel=sel)
    fill = pool.fill.cpu().numpy()
    assert np.all(fill == (inp.fill0[:, None] + 4096) % inp.log_len)
    _compare(inp, 4096, pool, outs, sel=sel)


def test_serving_shape_full_size_ragged_fills():
    """One layer of the 48-layer serving pool at its full size: GDN, B = 512, H = 32,
    128/128, L = 16, start fills ragged per sequence, the largest single launch the
    bench times (16,384 tiles).  512 steps (32 fold periods); fills checked everywhere,
    states and outputs on tiles across the batch and the heads."""
    steps = 512
    inp = make_inputs(5, steps, pool=16, log_len=16)
    B, H = inp.batch, inp.heads
    assert B * H == 16384 and len(set(inp.fill0.tolist())) > 1
    sel = [(0, 0), (1, H - 1), (B // 4, 3), (B // 2, H // 2), (3 * B // 4, 7), (B - 1, 0), (B - 1, H - 1)]
    pool, outs = run_deltalog(inp, steps, sel=sel)
    fill = pool.fill.cpu().numpy()
    assert np.all(fill == (inp.fill0[:, None] + steps) % inp.log_len)
    _compare(inp, steps, pool, outs, sel=sel)


# ------------------------------------------------------------- edge cases ----
@pytest.mark.parametrize("variant_w", [1, 3, 4])
@pytest.mark.parametrize("L", [1, 2, 3, 128])
def test_extreme_log_lengths(variant_w, L):
    steps = 300 if L == 128 else 64
    inp = make_inputs(variant_w, steps, batch=3, heads=2, log_len=L, pool=steps,
                      fill0=np.array([0, L // 2, L - 1], np.int32))
    pool, outs = run_deltalog(inp, steps)
    assert np.all(pool.fill.cpu().numpy() == ((inp.fill0 + steps) % L)[:, None])
    _compare(inp, steps, pool, outs)


@pytest.mark.parametrize("w", [1, 3, 4])
@pytest.mark.parametrize("dk,dv", [(64, 128), (128, 64), (64, 64), (128, 128)])
def test_head_size_combinations(w, dk, dv):
    inp = make_inputs(w, 80, batch=2, heads=3, log_len=16, pool=80, dk=dk, dv=dv,
                      fill0=np.array([0, 9], np.int32))
    pool, outs = run_deltalog(inp, 80)
    _compare(inp, 80, pool, outs)
    S, eo = run_eager_gpu(inp, 80)
    ref_S, ref_o = oracle.run_eager(inp, 80)
    _close("eager outputs", eo, ref_o, (-1,))
    _close("eager state", S, ref_S, (-2, -1))


@pytest.mark.parametrize("w", [1, 3, 4])
@pytest.mark.parametrize("dk,dv", [(64, 128), (128, 64), (64, 64), (128, 128)])
@pytest.mark.parametrize("L", [24, 40])
def test_log_entries_loaded_ahead(w, dk, dv, L):
    """Logs longer than the fold stage: the decode step loads up to 32 or 64 entries ahead of
    the base (chosen from L) and folds in several staged passes; ragged fills cover every
    depth of the log."""
    steps = 2 * L + 5
    inp = make_inputs(w, steps, batch=3, heads=2, log_len=L, pool=steps, dk=dk, dv=dv,
                      fill0=np.array([0, L // 3, L - 2], np.int32))
    pool, outs = run_deltalog(inp, steps)
    assert np.all(pool.fill.cpu().numpy() == ((inp.fill0 + steps) % L)[:, None])
    _compare(inp, steps, pool, outs)


@pytest.mark.parametrize("w", [1, 3, 4])
@pytest.mark.parametrize("L", [17, 18])
def test_log_length_at_the_prefetch_boundary(w, L):
    """L = 17 is the longest log the decode step's first variant covers (16 entries loaded
    ahead of the base, the fold in two staged passes; 512 threads per workgroup for GDN and
    KDA with an fp32 base at 128 x 128); L = 18 is the first that takes the 32-entry variant
    (512 threads for KDA as well, 256 for RWKV6).  Ragged fills put tiles at both ends of
    the log."""
    steps = 2 * L + 5
    inp = make_inputs(w, steps, batch=3, heads=2, log_len=L, pool=steps, dk=128, dv=128,
                      fill0=np.array([0, L // 2, L - 2], np.int32))
    pool, outs = run_deltalog(inp, steps)
    assert np.all(pool.fill.cpu().numpy() == ((inp.fill0 + steps) % L)[:, None])
    _compare(inp, steps, pool, outs)


@pytest.mark.parametrize("w", [1, 3, 4])
def test_unit_zero_and_tiny_decay(w):
    inp = make_inputs(w, 48, batch=2, heads=2, log_len=8, pool=48)
    d = inp.decay
    d[5] = 1.0
    d[11] = 1e-30
    d[17] = 0.0
    if d.ndim == 4:
        d[23, :, :, ::2] = 0.0
        d[29, :, :, 1::3] = 1e-20
    pool, outs = run_deltalog(inp, 48)
    _compare(inp, 48, pool, outs)


def test_merge_min_fill_then_continue():
    inp = make_inputs(3, 120, batch=6, heads=2, log_len=16, pool=120,
                      fill0=np.array([0, 3, 7, 9, 12, 15], np.int32))
    up = Uploaded(inp)
    pool = new_pool(inp, up=up)
    for t in range(50):
        dl.dl_decode_step(pool, up.io(t))
    ref_S, _ = oracle.run_eager(inp, 50, keep_outputs=False)
    fill = pool.fill.cpu().numpy()
    base_before = pool.base.cpu().numpy()
    log_k_before = pool.log_k.clone()
    m = 8
    dl.dl_merge(pool, m)
    torch.cuda.synchronize()
    fill_after = pool.fill.cpu().numpy()
    base_after = pool.base.cpu().numpy()
    for b in range(inp.batch):
        for h in range(inp.heads):
            if fill[b, h] >= m:
                assert fill_after[b, h] == 0
                _close(f"merged base ({b},{h})", base_after[b, h], ref_S[b, h], (-2, -1))
            else:
                assert fill_after[b, h] == fill[b, h]
                assert np.array_equal(base_after[b, h], base_before[b, h])
    assert torch.equal(pool.log_k, log_k_before)
    outs = []
    for t in range(50, 120):
        dl.dl_decode_step(pool, up.io(t))
        outs.append(up.out.cpu().numpy())
    _, ref_o = oracle.run_eager(inp, 120)
    _close("outputs after partial merge", np.stack(outs), ref_o[50:], (-1,))
    _close("state after partial merge", materialized_state(pool), oracle.run_eager(inp, 120)[0], (-2, -1))


@pytest.mark.parametrize("w", [2, 3, 4])
def test_reruns_are_bit_identical(w):
    """Every cross-lane and cross-wave sum of the step (512 threads for GDN and KDA at
    128 x 128) adds in a fixed order: the same steps twice give the same bits."""
    inp = make_inputs(w, 200, batch=3, heads=4, pool=200, fill0=np.array([0, 5, 11], np.int32))
    up = Uploaded(inp)
    p1, o1 = run_deltalog(inp, 200, up=up)
    p2, o2 = run_deltalog(inp, 200, up=up)
    assert np.array_equal(o1, o2)
    for name, t in p1.tensors().items():
        assert torch.equal(t, p2.tensors()[name]), name


def test_batch_zero_is_a_no_op():
    for variant in (GDN, KDA, RWKV6):
        pool = dl.DeltaLogPool(variant, 0, 2, 128, 128, 16, dev())
        dl.dl_init_state(pool)
        dl.dl_merge(pool, 1)
        e = torch.empty(0, device=dev())
        io = dl.StepIO(None, None, None, None, None, None, None)
        dl.dl_decode_step(pool, io)
        dl.dl_eager_step(variant, torch.empty((0, 2, 128, 128), device=dev()), io)
        assert e.numel() == 0


def test_bad_fill_is_rejected_before_any_work():
    inp = make_inputs(1, 4, pool=4)
    pool = dl.DeltaLogPool(GDN, 1, 1, 64, 64, 8, dev())
    with pytest.raises(dl.DeltaLogError) as ei:
        dl.dl_init_state(pool, torch.from_numpy(inp.s0).to(dev()), [8])
    assert ei.value.status == dl.DL_EINVAL
    with pytest.raises(dl.DeltaLogError) as ei:
        dl.dl_merge(pool, -1)
    assert ei.value.status == dl.DL_EINVAL


def test_merge_due_changes_nothing_and_merge_all_folds():
    """DL_MERGE_DUE (0) folds only full logs, and a decode step never leaves one, so the
    pool is unchanged; DL_MERGE_ALL (1) folds every non-empty log."""
    inp = make_inputs(2, 7, batch=2, heads=2, pool=7, fill0=np.array([0, 3], np.int32))
    up = Uploaded(inp)
    pool = new_pool(inp, up=up)
    for t in range(7):
        dl.dl_decode_step(pool, up.io(t))
    before = {k: v.clone() for k, v in pool.tensors().items()}
    dl.dl_merge(pool, dl.MERGE_DUE)
    torch.cuda.synchronize()
    assert all(torch.equal(before[k], v) for k, v in pool.tensors().items())
    dl.dl_merge(pool, dl.MERGE_ALL)
    torch.cuda.synchronize()
    assert int(pool.fill.abs().max()) == 0
    ref_S, _ = oracle.run_eager(inp, 7)
    _close("state after DL_MERGE_ALL", pool.base.cpu().numpy(), ref_S, (-2, -1))


# ------------------------------------------------- Kaczmarz step size (KLA) --
@pytest.mark.parametrize("w,kla", [(6, None), (3, True)])
def test_kaczmarz_step_size(w, kla):
    inp = make_inputs(w, 2048, batch=2, heads=4, pool=2048, kla=kla)
    assert inp.eta is not None and inp.beta is None
    pool, outs = run_deltalog(inp, 2048)
    _compare(inp, 2048, pool, outs)
    S, eo = run_eager_gpu(inp, 512)
    ref_S, ref_o = oracle.run_eager(inp, 512)
    _close("eager outputs", eo, ref_o, (-1,))
    _close("eager state", S, ref_S, (-2, -1))


def test_kaczmarz_projection_on_gpu():
    """eta = 1, eps = 0, decay 1: after each step the state maps k_t onto v_t."""
    inp = make_inputs(6, 24, batch=2, heads=2, pool=24)
    inp.eta[:] = 1.0
    inp.eps = 0.0
    inp.decay[:] = 1.0
    up = Uploaded(inp)
    pool = new_pool(inp, up=up)
    kf = oracle.step_arrays  # reuse only to widen the bf16 inputs exactly
    for t in range(24):
        dl.dl_decode_step(pool, up.io(t))
        S = materialized_state(pool).astype(np.float64)
        a = kf(inp, t)
        got = np.einsum("bhij,bhi->bhj", S, a["k"])
        np.testing.assert_allclose(got, a["v"], rtol=0, atol=2e-4 * np.abs(a["v"]).max())


# ------------------------------------------------------------- HIP graphs ----
def test_hip_graph_replays_match_direct_launches():
    """Capture one fold period of decode steps in a HIP graph and replay it several
    times, with other work and synchronisation in between; every replay must give
    bit-identical outputs and pool to the same steps launched directly."""
    inp = make_inputs(2, 16, batch=4, heads=4, pool=16, fill0=np.array([0, 3, 9, 15], np.int32))
    up = Uploaded(inp)
    ref_pool = new_pool(inp, up=up)
    ref = []
    for t in range(48):
        dl.dl_decode_step(ref_pool, up.io(t % 16))
        ref.append(up.out.clone())
    torch.cuda.synchronize()

    pool = new_pool(inp, up=up)
    outbuf = torch.empty((16,) + tuple(up.out.shape), dtype=torch.float32, device=dev())
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            for t in range(16):
                dl.dl_decode_step(pool, up.io(t))
                outbuf[t].copy_(up.out)
    torch.cuda.synchronize()
    # capture recorded the launches without running them: start from the same pool state
    dl.dl_init_state(pool, up.s0, inp.fill0)
    for r in range(3):
        g.replay()
        torch.cuda.synchronize()
        _ = (torch.ones(1 << 20, device=dev()) * 2).sum().item()  # unrelated work between replays
        for t in range(16):
            assert torch.equal(outbuf[t], ref[16 * r + t]), (r, t)
    for name, tnsr in pool.tensors().items():
        assert torch.equal(tnsr, ref_pool.tensors()[name]), name
