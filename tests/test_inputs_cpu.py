"""The seeded synthetic input recipes (CPU): seeds, draw order, variants, masks and the sweep's
case list, as the workload descriptions state them."""
import numpy as np
import pytest
import torch

import seeded_inputs as si


def test_generator_is_pcg64_seeded_by_config_and_case():
    a = si.rng_for(3, 0).standard_normal(8, dtype=np.float32)
    b = np.random.Generator(np.random.PCG64(np.random.SeedSequence([3, 0]))).standard_normal(8, dtype=np.float32)
    np.testing.assert_array_equal(a, b)
    assert not np.array_equal(a, si.rng_for(3, 1).standard_normal(8, dtype=np.float32))
    assert not np.array_equal(a, si.rng_for(4, 0).standard_normal(8, dtype=np.float32))


def test_chunked_normal_equals_one_draw():
    x = si._normal(si.rng_for(9, 9), (5, 7), chunk=4)
    np.testing.assert_array_equal(x.reshape(-1), si.rng_for(9, 9).standard_normal(35, dtype=np.float32))


def test_draw_order_q_then_k_then_v():
    q, k, v = si.draw_qkv(si.rng_for(8, 1), (1, 3, 2, 4), (1, 5, 2, 4))
    flat = si.rng_for(8, 1).standard_normal(24 + 40 + 40, dtype=np.float32)
    np.testing.assert_array_equal(q.reshape(-1), flat[:24])
    np.testing.assert_array_equal(k.reshape(-1), flat[24:64])
    np.testing.assert_array_equal(v.reshape(-1), flat[64:])


def test_sweep_has_every_combination_once():
    cases = si.sweep_cases()
    assert len(cases) == 5 * 3 * 2 * 2 * 2 * 3 == 360
    keys = {(c["N"], c["D"], c["dtype"], c["causal"], c["BN"], c["variant"]) for c in cases}
    assert len(keys) == 360
    assert {c["N"] for c in cases} == {1, 17, 1000, 2047, 2048} and {c["D"] for c in cases} == {16, 32, 64}


def test_sweep_variants_share_draws_and_act_on_q_only():
    cases = [c for c in si.sweep_cases() if c["N"] == 17 and c["D"] == 32 and c["dtype"] == "f16"
             and not c["causal"] and c["BN"] == 32]
    by = {c["variant"]: si.sweep_inputs(c) for c in cases}
    qn, kn, vn = by["normal"]
    ql, kl, vl = by["large"]
    qu, ku, vu = by["uniform"]
    assert torch.equal(kn, kl) and torch.equal(kn, ku) and torch.equal(vn, vl) and torch.equal(vn, vu)
    assert bool((qu == 0).all())
    q32, _, _ = si.draw_qkv(si.rng_for(si.CFG_SWEEP, 1 * 3 + 1), (1, 17, 1, 32), (1, 17, 1, 32))
    assert torch.equal(ql, torch.from_numpy(q32 * np.float32(30.0)).to(torch.float16))


def test_bernoulli_mask_half_visible_with_cleared_rows():
    mask, rows = si.bernoulli_mask(si.rng_for(5, 3), 256, 300, 4, row_block=64)
    assert mask.dtype == np.uint8 and set(np.unique(mask)) <= {0, 1}
    assert len(rows) == 4 and len(set(rows.tolist())) == 4
    assert not mask[rows].any()
    keep = np.setdiff1d(np.arange(256), rows)
    frac = mask[keep].mean()
    assert abs(frac - 0.5) < 0.01          # 76,800 draws: 5 standard deviations is 0.009
    # row blocks consume the stream in row-major order: the block size does not change the mask
    m2, r2 = si.bernoulli_mask(si.rng_for(5, 3), 256, 300, 4, row_block=1000)
    np.testing.assert_array_equal(mask, m2)
    np.testing.assert_array_equal(rows, r2)


def test_masked_workload_clears_one_row_in_64():
    q, k, v, mask, rows = si.masked_inputs(H=1, N=256)
    assert q.shape == (1, 256, 1, 256) and q.dtype == torch.bfloat16
    assert mask.shape == (256, 256) and len(rows) == 256 // 64
    assert not mask[rows].any()


def test_cast_is_round_to_nearest_even():
    """bf16: against round-to-nearest-even written on the float32 bits (add 0x7FFF plus the kept
    lowest bit, truncate); fp16: against numpy's conversion.  Ties are included."""
    x = si.rng_for(6, 6).standard_normal(4000, dtype=np.float32) * np.float32(100)
    bits = x.view(np.uint32).astype(np.uint64)
    ties = (np.arange(1, 65, dtype=np.uint64) << np.uint64(16)) | np.uint64(0x3F808000)   # exact halfway cases
    bits = np.concatenate([bits, ties, ties | np.uint64(1 << 31)])
    xs = bits.astype(np.uint32).view(np.float32)
    want = ((bits + np.uint64(0x7FFF) + ((bits >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)).astype(np.uint16)
    got = si.cast(xs, "bf16").view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(got, want)
    got16 = si.cast(x, "f16").view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(got16, x.astype(np.float16).view(np.uint16))
