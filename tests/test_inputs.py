"""The seeded input generator (CPU only)."""
import numpy as np
import pytest
import torch

from inputs import (GDN, KDA, RWKV6, WORKLOADS, bf16_bits_to_f32, f32_to_bf16_bits, make_inputs,
                    tile_inputs)


def test_bf16_rounding_matches_torch_rne():
    g = np.random.default_rng(0)
    x = np.concatenate([g.standard_normal(100000).astype(np.float32),
                        g.standard_normal(1000).astype(np.float32) * 1e-30,
                        np.array([0.0, -0.0, 1.0, -2.5, 65504.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8,
                                  3.0e38], np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(f32_to_bf16_bits(x), ref)
    back = bf16_bits_to_f32(ref)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_ties_round_to_even():
    # 1 + 2^-8 lies halfway between bf16 neighbours 1 and 1 + 2^-7: ties go to the even one (1).
    assert bf16_bits_to_f32(f32_to_bf16_bits(np.array([1 + 2 ** -8], np.float32)))[0] == 1.0
    assert bf16_bits_to_f32(f32_to_bf16_bits(np.array([1 + 3 * 2 ** -8], np.float32)))[0] == 1 + 2 ** -6


def test_batch_slice_is_prefix_of_full_workload():
    full = make_inputs(2, 3, batch=6, heads=4)
    part = make_inputs(2, 3, batch=2, heads=4)
    assert np.array_equal(full.s0[:2], part.s0)
    for name in ("q", "k", "v", "decay", "beta"):
        assert np.array_equal(getattr(full, name)[:, :2], getattr(part, name)), name


def test_tile_view_and_determinism():
    a = make_inputs(4, 4, batch=3, heads=2)
    b = make_inputs(4, 4, batch=3, heads=2)
    for name in ("s0", "q", "k", "v", "decay", "bonus"):
        assert np.array_equal(getattr(a, name), getattr(b, name))
    t = tile_inputs(a, 2, 1)
    assert np.array_equal(t.s0[0, 0], a.s0[2, 1])
    assert np.array_equal(t.k[:, 0, 0], a.k[:, 2, 1])
    assert np.array_equal(t.bonus[0], a.bonus[1])


@pytest.mark.parametrize("w", [1, 2, 3, 4, 5])
def test_distributions(w):
    inp = make_inputs(w, 8, batch=min(WORKLOADS[w]["batch"], 8), heads=min(WORKLOADS[w]["heads"], 4))
    assert np.all(inp.decay > 0) and np.all(inp.decay <= 1)
    if w == 2:
        assert inp.decay.min() > 0.9
    if inp.variant in (GDN, KDA):
        k = bf16_bits_to_f32(inp.k).astype(np.float64)
        assert np.allclose(np.linalg.norm(k, axis=-1), 1.0, atol=1e-2)
        assert np.all((inp.beta > 0) & (inp.beta < 1))
        assert inp.decay.ndim == (3 if inp.variant == GDN else 4)
    else:
        assert inp.variant == RWKV6 and inp.beta is None and inp.bonus.shape == (inp.heads, inp.dk)
    assert np.all((inp.fill0 >= 0) & (inp.fill0 < inp.log_len))
    if WORKLOADS[w]["ragged"]:
        assert len(set(inp.fill0.tolist())) > 1
    assert abs(float(inp.s0.std()) - 0.02) < 0.002
