"""Coordinate tests of the register and LDS layouts the attention kernels are built on, on the GPU
(Tylo.jl "Streaming attention and online state", section "Same-lane conversion": coordinate
tests enumerate every lane and value against an independent description, and a GPU test compares
the register path with a store / load through shared memory, consumed by a second product).

The written-down maps (the same ones the kernels' comments state) are checked with integer-valued
operands, so every product and sum is exact and the comparisons are bitwise:
  v_mfma_f32_32x32x16_bf16: A lane l element j = A[l % 32][8 (l / 32) + j];
      B lane l element j = B[8 (l / 32) + j][l % 32];
      C lane l register r = C[8 (r / 4) + 4 (l / 32) + r % 4][l % 32]
  v_mfma_f32_32x32x64_f8f6f4: byte j of lane l pairs A row l % 32 with B column l % 32 through
      reduction index 32 (l / 32) + j (any consistent labelling); C as above
  ds_read_b64_tr_b16: per 16-lane group, lane i element j = element i % 4 of the 8-byte chunk
      addressed by lane 4 j + i / 4 of the group
  ds_read_b64_tr_b8: per 16-lane group, lane i byte j = byte (i % 16) % 8 of the chunk addressed
      by lane 2 j + (i % 16) / 8 of the group
  permlane32 / permlane16 swaps: xor-32 / xor-16 partner; group_sum over all 64 lanes
"""
import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def probe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import probes
    return probes.lib()


def _p(t):
    return t.data_ptr()


def _bf16_words(vals):
    """[64, 8] integer-valued float -> [64, 4] u32 words (element 2i low, 2i+1 high)."""
    b = torch.from_numpy(np.asarray(vals, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    b = b.astype(np.uint32).reshape(64, 4, 2)
    return (b[:, :, 0] | (b[:, :, 1] << 16)).astype(np.uint32)


def _c_map(cmat):
    """Expected accumulator registers [64, 16] from a logical 32 x 32 matrix."""
    out = np.zeros((64, 16))
    for l in range(64):
        for r in range(16):
            out[l, r] = cmat[8 * (r // 4) + 4 * (l // 32) + r % 4, l % 32]
    return out


def test_mfma_bf16_operand_and_accumulator_maps(probe):
    rng = np.random.default_rng(21)
    A = rng.integers(-8, 9, (32, 16)).astype(np.float64)
    B = rng.integers(-8, 9, (16, 32)).astype(np.float64)
    a = np.zeros((64, 8)); b = np.zeros((64, 8))
    for l in range(64):
        for j in range(8):
            a[l, j] = A[l % 32, 8 * (l // 32) + j]
            b[l, j] = B[8 * (l // 32) + j, l % 32]
    da = torch.from_numpy(_bf16_words(a).view(np.int32)).to(DEV)
    db = torch.from_numpy(_bf16_words(b).view(np.int32)).to(DEV)
    c = torch.zeros(64 * 16, device=DEV)
    assert probe.probe_mfma_bf16(_p(da), _p(db), _p(c)) == 0
    got = c.cpu().numpy().reshape(64, 16)
    np.testing.assert_array_equal(got, _c_map(A @ B))


def test_mfma_f8f6f4_pairing_and_accumulator_map(probe):
    rng = np.random.default_rng(22)
    A = rng.integers(-4, 5, (32, 64)).astype(np.float32)
    B = rng.integers(-4, 5, (64, 32)).astype(np.float32)
    a = np.zeros((64, 32), np.float32); b = np.zeros((64, 32), np.float32)
    for l in range(64):
        for j in range(32):
            a[l, j] = A[l % 32, 32 * (l // 32) + j]
            b[l, j] = B[32 * (l // 32) + j, l % 32]
    da = torch.from_numpy(oracle.round_fp8_bits(a, "e4m3")).to(DEV)
    db = torch.from_numpy(oracle.round_fp8_bits(b, "e4m3")).to(DEV)
    c = torch.zeros(64 * 16, device=DEV)
    assert probe.probe_mfma_f8(_p(da), _p(db), _p(c)) == 0
    np.testing.assert_array_equal(c.cpu().numpy().reshape(64, 16), _c_map(A.astype(np.float64) @ B))


def _addr_patterns():
    return [8 * np.arange(64), (72 * np.arange(64)) % 4088 // 8 * 8, np.random.default_rng(23).permutation(512)[:64] * 8]


def test_ds_read_tr16_lane_map(probe):
    fill = torch.arange(2048, dtype=torch.int32).to(torch.int16).to(DEV)     # element e holds e
    for addr in _addr_patterns():
        da = torch.from_numpy(addr.astype(np.int32)).to(DEV)
        out = torch.zeros(256, dtype=torch.int16, device=DEV)
        assert probe.probe_tr16(_p(fill), _p(da), _p(out)) == 0
        got = out.cpu().numpy().astype(np.int64).reshape(64, 4)
        want = np.zeros((64, 4), np.int64)
        for i in range(64):
            g, ii = i // 16, i % 16
            for j in range(4):
                want[i, j] = addr[16 * g + 4 * j + ii // 4] // 2 + ii % 4
        np.testing.assert_array_equal(got, want)


def test_ds_read_tr8_lane_map(probe):
    for addr in _addr_patterns():
        da = torch.from_numpy(addr.astype(np.int32)).to(DEV)
        got = np.zeros((64, 8), np.int64)
        for shift in (0, 8):                                  # byte index = low byte | high byte << 8
            fill = torch.from_numpy(((np.arange(4096) >> shift) & 0xFF).astype(np.uint8)).to(DEV)
            out = torch.zeros(512, dtype=torch.uint8, device=DEV)
            assert probe.probe_tr8(_p(fill), _p(da), _p(out)) == 0
            got |= out.cpu().numpy().astype(np.int64).reshape(64, 8) << shift
        want = np.zeros((64, 8), np.int64)
        for i in range(64):
            g, ii = i // 16, i % 16
            for j in range(8):
                want[i, j] = addr[16 * g + 2 * j + ii // 8] + ii % 8
        np.testing.assert_array_equal(got, want)


def test_cross_lane_helpers(probe):
    x = np.random.default_rng(24).integers(-1000, 1000, 64).astype(np.float32)
    out = torch.zeros(256, device=DEV)
    assert probe.probe_xlane(_p(torch.from_numpy(x).to(DEV)), _p(out)) == 0
    got = out.cpu().numpy().reshape(64, 4)
    lanes = np.arange(64)
    np.testing.assert_array_equal(got[:, 0], x + x[lanes ^ 32])
    np.testing.assert_array_equal(got[:, 1], np.maximum(x, x[lanes ^ 32]))
    np.testing.assert_array_equal(got[:, 2], x + x[lanes ^ 16])
    np.testing.assert_array_equal(got[:, 3], np.full(64, x.sum()))


def test_same_lane_conversion_matches_lds_round_trip(probe):
    """Scores of one 32-key block through the key permutation, packed in place, give bitwise the
    second product of the same scores stored to LDS at their logical coordinates and reloaded in
    the operand layout; both equal V^T S on the host (integer values: exact)."""
    rng = np.random.default_rng(25)
    K = rng.integers(-2, 3, (32, 16)).astype(np.float32)
    Q = rng.integers(-2, 3, (32, 16)).astype(np.float32)
    V = rng.integers(-2, 3, (32, 32)).astype(np.float32)
    to16 = lambda m: torch.from_numpy(m).to(torch.bfloat16).view(torch.int16).to(DEV)
    o_reg = torch.zeros(1024, device=DEV)
    o_lds = torch.zeros(1024, device=DEV)
    s = torch.zeros(1024, device=DEV)
    assert probe.probe_same_lane(_p(to16(K)), _p(to16(Q)), _p(to16(V)), _p(o_reg), _p(o_lds), _p(s)) == 0
    S = K.astype(np.float64) @ Q.T.astype(np.float64)             # [key, query]
    np.testing.assert_array_equal(s.cpu().numpy().reshape(32, 32), S)
    a, b = o_reg.cpu().numpy(), o_lds.cpu().numpy()
    np.testing.assert_array_equal(a, b)
    OT = V.T.astype(np.float64) @ S                               # O^T [d, query]
    np.testing.assert_array_equal(a.reshape(64, 16), _c_map(OT))
