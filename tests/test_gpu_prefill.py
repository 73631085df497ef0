"""dl_prefill (chunkwise GDN, KDA and RWKV6 prefill on MFMA) against the fp64 eager oracle (GPU).

A prompt of T tokens is the workload's first T drawn steps; the oracle runs the
same T eager steps.  Outputs (one per token) and the final state (the base,
log empty) must be within 1e-4 per tensor.  Chunks are 32 tokens, so T covers
a single token, one token short of and past a chunk, several chunks and a long
prompt.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_harness import Uploaded, dev, materialized_state, new_pool
from inputs import make_inputs
from linear_attention_recurrent_amd import deltalog as dl

pytestmark = pytest.mark.gpu
TOL = 1e-4


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("a GPU is required for the gpu-marked tests")
    dl.load_library()


def _close(what, got, ref, axes, tol=TOL):
    err = oracle.rel_err(got, ref, axes)
    print(f"{what}: max per-tensor rel err {err:.3e}, element-wise (floor 1e-6 of the tensor's scale) "
          f"{oracle.elem_rel_err(got, ref, axes):.3e}", flush=True)
    assert err <= tol, (what, err)
    return err


def prompt(up: Uploaded, t0: int, T: int):
    """Steps t0 .. t0+T-1 of an uploaded workload as [batch][T][heads][...] prompt tensors."""
    sl = slice(t0, t0 + T)
    tm = lambda x: None if x is None else x[sl].transpose(0, 1).contiguous()
    return dict(q=tm(up.q), k=tm(up.k), v=tm(up.v), decay=tm(up.decay), beta=tm(up.beta), eta=tm(up.eta))


def run_prefill(pool, up, t0, T, eps=0.0):
    p = prompt(up, t0, T)
    inp = up.inp
    out = torch.full((inp.batch, T, inp.heads, inp.dv), float("nan"), dtype=torch.float32, device=dev())
    io = dl.make_prefill_io(pool, p["q"], p["k"], p["v"], p["decay"], p["beta"], out, p["eta"], eps, bonus=up.bonus)
    dl.dl_prefill(pool, io)
    torch.cuda.synchronize()
    return out.cpu().numpy().transpose(1, 0, 2, 3)  # [T][batch][heads][dv]


def check_prefill(inp, T, base_dtype=dl.BASE_F32):
    up = Uploaded(inp)
    pool = new_pool(inp, up=up, base_dtype=base_dtype)
    outs = run_prefill(pool, up, 0, T, inp.eps)
    assert int(pool.fill.max().item()) == 0
    ref_S, ref_o = oracle.run_eager(inp, T)
    _close(f"outputs T={T}", outs, ref_o, (-1,))
    _close(f"state T={T}", pool.base.float().cpu().numpy(), ref_S, (-2, -1))
    return pool, up


@pytest.mark.parametrize("T", [1, 31, 32, 33, 100, 4096])
def test_gdn_prefill_lengths(T):
    inp = make_inputs(2, T, batch=2, heads=4, pool=T)
    check_prefill(inp, T)


def test_gdn_smoke_shape():
    inp = make_inputs(1, 64, pool=64)
    check_prefill(inp, 64)


@pytest.mark.parametrize("dk,dv", [(64, 64), (64, 128), (128, 64)])
def test_head_size_combinations(dk, dv):
    inp = make_inputs(2, 97, batch=2, heads=3, pool=97, dk=dk, dv=dv)
    check_prefill(inp, 97)


def test_kaczmarz_step_size():
    inp = make_inputs(6, 300, batch=2, heads=4, pool=300)
    assert inp.eta is not None
    check_prefill(inp, 300)


def test_zero_and_unit_decay_tokens():
    inp = make_inputs(2, 70, batch=2, heads=2, pool=70)
    inp.decay[5] = 0.0          # a token that resets every state
    inp.decay[40:45] = 1.0      # no decay
    inp.beta[50:52] = 0.0       # no write
    check_prefill(inp, 70)


def test_decode_continues_after_prefill():
    """Prefill 100 tokens, then 40 decode steps (two folds at L = 16): same as 140 eager steps."""
    inp = make_inputs(2, 140, batch=2, heads=4, pool=140)
    up = Uploaded(inp)
    pool = new_pool(inp, up=up)
    run_prefill(pool, up, 0, 100)
    outs = []
    for t in range(100, 140):
        dl.dl_decode_step(pool, up.io(t))
        outs.append(up.out.cpu().numpy())
    ref_S, ref_o = oracle.run_eager(inp, 140)
    _close("decode outputs after prefill", np.stack(outs), ref_o[100:], (-1,))
    _close("state after prefill + decode", materialized_state(pool), ref_S, (-2, -1))


def test_prefill_folds_a_pending_log_first():
    """Decode steps from ragged fills leave logs non-empty; prefill folds them, then runs the prompt."""
    inp = make_inputs(2, 90, batch=3, heads=2, pool=90, log_len=16, fill0=np.array([0, 5, 11], np.int32))
    up = Uploaded(inp)
    pool = new_pool(inp, up=up)
    for t in range(10):
        dl.dl_decode_step(pool, up.io(t))
    assert int(pool.fill.max().item()) > 0
    outs = run_prefill(pool, up, 10, 80)
    assert int(pool.fill.max().item()) == 0
    ref_S, ref_o = oracle.run_eager(inp, 90)
    _close("prompt outputs after decode", outs, ref_o[10:], (-1,))
    _close("state", pool.base.cpu().numpy(), ref_S, (-2, -1))
    # an empty prompt only folds
    for t in range(10):
        dl.dl_decode_step(pool, up.io(t))
    want = materialized_state(pool)
    out = torch.empty((inp.batch, 0, inp.heads, inp.dv), dtype=torch.float32, device=dev())
    p = prompt(up, 0, 0)
    dl.dl_prefill(pool, dl.make_prefill_io(pool, p["q"], p["k"], p["v"], p["decay"], p["beta"], out,
                                           bonus=up.bonus))
    torch.cuda.synchronize()
    assert int(pool.fill.max().item()) == 0
    assert np.array_equal(pool.base.cpu().numpy(), want)


def test_bf16_base_prefill():
    """With a bf16 base the prompt starts from the rounded state and the final state is rounded once."""
    T = 200
    inp = make_inputs(2, T, batch=2, heads=4, pool=T)
    up = Uploaded(inp)
    pool = new_pool(inp, up=up, base_dtype=dl.BASE_BF16)
    outs = run_prefill(pool, up, 0, T)
    s0 = oracle.round_to_bf16(inp.s0.astype(np.float64))
    ref_S, ref_o = oracle.run_eager(inp, T, s0=s0)
    _close("outputs, bf16 base", outs, ref_o, (-1,))
    got = pool.base.float().cpu().numpy().astype(np.float64)
    ref = oracle.round_to_bf16(ref_S)
    same = float(np.mean(got == ref))
    print(f"final base: {same:.4%} bit-equal to the rounded oracle state", flush=True)
    assert same >= 0.99
    _, e = np.frexp(np.maximum(np.abs(got), np.abs(ref)))
    slack = 1e-5 * np.max(np.abs(ref), axis=(-2, -1), keepdims=True)
    assert np.all(np.abs(got - ref) <= np.ldexp(1.0, e - 8) + slack)


def test_reruns_are_bit_identical():
    inp = make_inputs(2, 77, batch=2, heads=2, pool=77)
    up = Uploaded(inp)
    res = []
    for _ in range(2):
        pool = new_pool(inp, up=up)
        res.append((run_prefill(pool, up, 0, 77), pool.base.cpu().numpy()))
    assert np.array_equal(res[0][0], res[1][0]) and np.array_equal(res[0][1], res[1][1])


# --------------------------------------------------------------------- KDA --
@pytest.mark.parametrize("T", [1, 31, 33, 100, 4096])
def test_kda_prefill_lengths(T):
    inp = make_inputs(3, T, batch=2, heads=4, pool=T)
    check_prefill(inp, T)


@pytest.mark.parametrize("dk,dv", [(64, 64), (64, 128), (128, 64)])
def test_kda_head_size_combinations(dk, dv):
    inp = make_inputs(3, 97, batch=2, heads=3, pool=97, dk=dk, dv=dv)
    check_prefill(inp, 97)


def test_kda_kaczmarz_step_size():
    inp = make_inputs(3, 200, batch=2, heads=4, pool=200, kla=True)
    assert inp.eta is not None
    check_prefill(inp, 200)


def test_kda_strong_zero_and_unit_channel_decays():
    """Per-channel extremes inside one chunk: some channels decay to zero, some by 2^-40
    per token (far below what a factorised 2^(c_i - r) 2^(r - c_j) could hold), some not
    at all; the decay-weighted products are formed pair by pair, so all stay exact."""
    inp = make_inputs(3, 70, batch=2, heads=2, pool=70)
    inp.decay[5, :, :, :16] = 0.0
    inp.decay[10:30, :, :, 16:32] = 2.0 ** -40
    inp.decay[40:45, :, :, 32:] = 1.0
    inp.beta[50:52] = 0.0
    check_prefill(inp, 70)


def test_kda_strong_decays_within_the_matrix_path():
    """Channels decaying by 2^-3 per token: 2^-48 over half a chunk, inside the range where
    the decay-weighted products run on MFMA with column factors up to 2^48."""
    inp = make_inputs(3, 96, batch=2, heads=2, pool=96)
    inp.decay[:, :, :, :40] = 2.0 ** -3
    check_prefill(inp, 96)


def test_kda_decode_continues_after_prefill():
    inp = make_inputs(3, 140, batch=2, heads=4, pool=140)
    up = Uploaded(inp)
    pool = new_pool(inp, up=up)
    run_prefill(pool, up, 0, 100)
    outs = []
    for t in range(100, 140):
        dl.dl_decode_step(pool, up.io(t))
        outs.append(up.out.cpu().numpy())
    ref_S, ref_o = oracle.run_eager(inp, 140)
    _close("decode outputs after prefill", np.stack(outs), ref_o[100:], (-1,))
    _close("state after prefill + decode", materialized_state(pool), ref_S, (-2, -1))


def test_kda_bf16_base_prefill():
    T = 120
    inp = make_inputs(3, T, batch=2, heads=4, pool=T)
    up = Uploaded(inp)
    pool = new_pool(inp, up=up, base_dtype=dl.BASE_BF16)
    outs = run_prefill(pool, up, 0, T)
    s0 = oracle.round_to_bf16(inp.s0.astype(np.float64))
    ref_S, ref_o = oracle.run_eager(inp, T, s0=s0)
    _close("outputs, bf16 base", outs, ref_o, (-1,))
    got = pool.base.float().cpu().numpy().astype(np.float64)
    ref = oracle.round_to_bf16(ref_S)
    assert float(np.mean(got == ref)) >= 0.99


# ------------------------------------------------------------------- RWKV6 --
@pytest.mark.parametrize("T", [1, 31, 33, 100, 2048])
def test_rwkv6_prefill_lengths(T):
    inp = make_inputs(4, T, batch=2, heads=4, pool=T)
    check_prefill(inp, T)


@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 128), (128, 64)])
def test_rwkv6_head_size_combinations(dk, dv):
    inp = make_inputs(4, 97, batch=2, heads=3, pool=97, dk=dk, dv=dv)
    check_prefill(inp, 97)


def test_rwkv6_strong_and_zero_decays():
    """Channels decaying to zero, by 2^-40 per token (pairwise path) or by 2^-3 per token
    (matrix path), and channels that do not decay."""
    for variant_decay in ("pairwise", "matrix"):
        inp = make_inputs(4, 70, batch=2, heads=2, pool=70)
        if variant_decay == "pairwise":
            inp.decay[5, :, :, :16] = 0.0
            inp.decay[10:30, :, :, 16:32] = 2.0 ** -40
        else:
            inp.decay[:, :, :, :24] = 2.0 ** -3
        inp.decay[40:45, :, :, 40:] = 1.0
        check_prefill(inp, 70)


def test_rwkv6_decode_continues_after_prefill():
    inp = make_inputs(4, 140, batch=2, heads=4, pool=140)
    up = Uploaded(inp)
    pool = new_pool(inp, up=up)
    run_prefill(pool, up, 0, 100)
    outs = []
    for t in range(100, 140):
        dl.dl_decode_step(pool, up.io(t))
        outs.append(up.out.cpu().numpy())
    ref_S, ref_o = oracle.run_eager(inp, 140)
    _close("decode outputs after prefill", np.stack(outs), ref_o[100:], (-1,))
    _close("state after prefill + decode", materialized_state(pool), ref_S, (-2, -1))


# ------------------------------------------- full sizes, sampled tiles ------
@pytest.mark.parametrize("w", [2, 3, 4, 6])
def test_long_prompts(w):
    """Prompts of 16,384 tokens (512 chunks; the bench's are 2,048-4,096), every tile
    of a small batch, prompt rows cycling over 512 drawn steps: the carried state's error
    must not grow with the number of chunks."""
    T = 16384
    inp = make_inputs(w, T, batch=2, heads=2, pool=512)
    up = Uploaded(inp)
    pool = new_pool(inp, up=up)
    idx = torch.arange(T, device=dev()) % inp.pool
    tm = lambda x: None if x is None else x.index_select(0, idx).transpose(0, 1).contiguous()
    out = torch.empty((inp.batch, T, inp.heads, inp.dv), dtype=torch.float32, device=dev())
    io = dl.make_prefill_io(pool, tm(up.q), tm(up.k), tm(up.v), tm(up.decay), tm(up.beta), out, tm(up.eta),
                            inp.eps, bonus=up.bonus)
    dl.dl_prefill(pool, io)
    torch.cuda.synchronize()
    got_o = out.cpu().numpy().transpose(1, 0, 2, 3)  # [T][batch][heads][dv]
    ref_S, ref_o = oracle.run_eager(inp, T)
    _close(f"outputs, workload {w}, T={T}", got_o, ref_o, (-1,))
    _close(f"state, workload {w}, T={T}", pool.base.cpu().numpy(), ref_S, (-2, -1))


@pytest.mark.parametrize("w,T", [(2, 4096), (3, 4096), (4, 2048)])
def test_full_size_prefill_sampled_tiles(w, T):
    """The shapes the bench times (every tile of the workload, prompt rows cycling over
    64 drawn steps); six tiles spread over batch and heads are checked against the oracle."""
    inp = make_inputs(w, T, pool=64)
    B, H = inp.batch, inp.heads
    up = Uploaded(inp)
    pool = new_pool(inp, up=up)
    idx = torch.arange(T, device=dev()) % inp.pool
    tm = lambda x: None if x is None else x.index_select(0, idx).transpose(0, 1).contiguous()
    out = torch.empty((B, T, H, inp.dv), dtype=torch.float32, device=dev())
    io = dl.make_prefill_io(pool, tm(up.q), tm(up.k), tm(up.v), tm(up.decay), tm(up.beta), out, tm(up.eta),
                            inp.eps, bonus=up.bonus)
    dl.dl_prefill(pool, io)
    torch.cuda.synchronize()
    sel = [(0, 0), (0, H - 1), (B // 3, H // 2), (B // 2, 1), (B - 1, 0), (B - 1, H - 1)]
    bi = torch.tensor([b for b, _ in sel], device=dev())
    hi = torch.tensor([h for _, h in sel], device=dev())
    got_o = out[bi, :, hi].cpu().numpy().transpose(1, 0, 2)   # [T][tiles][dv]
    got_S = pool.base[bi, hi].cpu().numpy()
    del out, io
    ref_S, ref_o = oracle.run_eager(inp, T, sel=sel)
    _close(f"outputs, workload {w}, T={T}", got_o, ref_o, (-1,))
    _close(f"state, workload {w}, T={T}", got_S, ref_S, (-2, -1))


def test_hip_graph_replays_of_prefill_and_decode():
    """A prefill followed by decode steps, captured in a HIP graph and replayed with
    unrelated work and synchronisation in between, gives bit-identical outputs and
    pools to the same calls launched directly (no memset nodes are involved)."""
    inp = make_inputs(2, 80, batch=2, heads=4, pool=80)
    up = Uploaded(inp)
    T = 45
    p = prompt(up, 0, T)
    ref_pool = new_pool(inp, up=up)
    out_ref = torch.empty((inp.batch, T, inp.heads, inp.dv), dtype=torch.float32, device=dev())
    dl.dl_prefill(ref_pool, dl.make_prefill_io(ref_pool, p["q"], p["k"], p["v"], p["decay"], p["beta"], out_ref))
    dec_ref = []
    for t in range(T, T + 20):
        dl.dl_decode_step(ref_pool, up.io(t))
        dec_ref.append(up.out.clone())
    torch.cuda.synchronize()

    pool = new_pool(inp, up=up)
    out = torch.empty_like(out_ref)
    io = dl.make_prefill_io(pool, p["q"], p["k"], p["v"], p["decay"], p["beta"], out)
    dec = torch.empty((20,) + tuple(up.out.shape), dtype=torch.float32, device=dev())
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            dl.dl_prefill(pool, io)
            for i, t in enumerate(range(T, T + 20)):
                dl.dl_decode_step(pool, up.io(t))
                dec[i].copy_(up.out)
    torch.cuda.synchronize()
    for r in range(3):
        dl.dl_init_state(pool, up.s0, None)
        g.replay()
        torch.cuda.synchronize()
        _ = (torch.ones(1 << 20, device=dev()) * 3).sum().item()
        assert torch.equal(out, out_ref), r
        for i in range(20):
            assert torch.equal(dec[i], dec_ref[i]), (r, i)
        for name, tnsr in pool.tensors().items():
            assert torch.equal(tnsr, ref_pool.tensors()[name]), (r, name)


# ------------------------------------------- seeded mixed configurations ------
def _mixed_case(i):
    """Case i: a variant (GDN with normalised keys, KDA, RWKV6, GDN with the Kaczmarz step
    size), head sizes, batch, heads, log length and ragged start fills, decode steps, a
    prompt, then decode steps again, all drawn from one seeded generator."""
    g = np.random.default_rng(1000 + i)
    w = int(g.choice([1, 3, 4, 6]))
    dk, dv = int(g.choice([64, 128])), int(g.choice([64, 128]))
    B, H = int(g.integers(1, 4)), int(g.integers(1, 4))
    L = int(g.choice([1, 2, 4, 8, 16, 32]))
    d0, T, d1 = int(g.integers(0, 21)), int(g.integers(0, 101)), int(g.integers(0, 21))
    kla = True if w == 6 else (bool(g.integers(0, 2)) if w == 3 else None)
    fill0 = g.integers(0, L, size=B).astype(np.int32)
    return dict(w=w, dk=dk, dv=dv, B=B, H=H, L=L, d0=d0, T=T, d1=d1, kla=kla, fill0=fill0)


@pytest.mark.parametrize("i", range(12))
def test_seeded_mixed_decode_prefill_decode(i):
    """Decode steps from ragged fills, a prompt (which folds the pending logs first), more
    decode steps: every output and the final state against one eager oracle run."""
    c = _mixed_case(i)
    steps = c["d0"] + c["T"] + c["d1"]
    print(f"case {i}: {c}", flush=True)
    inp = make_inputs(c["w"], max(steps, 1), batch=c["B"], heads=c["H"], log_len=c["L"], pool=max(steps, 1),
                      fill0=c["fill0"], dk=c["dk"], dv=c["dv"], kla=c["kla"])
    up = Uploaded(inp)
    pool = new_pool(inp, up=up)
    outs = []
    for t in range(c["d0"]):
        dl.dl_decode_step(pool, up.io(t))
        outs.append(up.out.cpu().numpy())
    po = run_prefill(pool, up, c["d0"], c["T"], inp.eps)
    assert int(pool.fill.max().item()) == 0
    outs.extend(list(po))
    for t in range(c["d0"] + c["T"], steps):
        dl.dl_decode_step(pool, up.io(t))
        outs.append(up.out.cpu().numpy())
    ref_S, ref_o = oracle.run_eager(inp, steps)
    if steps:
        _close(f"outputs, case {i}", np.stack(outs), ref_o[:steps], (-1,))
    _close(f"state, case {i}", materialized_state(pool), ref_S, (-2, -1))
