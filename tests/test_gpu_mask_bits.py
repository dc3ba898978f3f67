"""The packed mask (attn_mask_pack, attn_fwd_packed) through the C ABI.

attn_mask_pack is checked word by word against the encoding the header defines, rebuilt here in
numpy from its formula: word (g * ceil(Nkv / 64) + c) * 64 + l, bit b, is the byte at row
32 g + l % 32 and key 64 c + 32 (b // 16) + 16 ((b % 16) // 8) + 8 (l // 32) + b % 8 being nonzero
(0 outside the mask).  The forward with packed bits must give bit for bit the outputs of the
forward with the byte mask (the same visible set, the same arithmetic) and match the oracle to
the tolerances of the other parity tests (the visibility rule: triton-cuda-lab workshop "A3. Tiled
attention with online normalization", section "Masks that preserve the recurrence").
"""
import numpy as np
import pytest
import torch

import oracle
import seeded_inputs as si

pytestmark = pytest.mark.gpu

DEV = "cuda"
TOL = {"bf16": 2e-2, "f16": 5e-3}
SENTINEL = 0x5A5A5A5A


@pytest.fixture(scope="module")
def sa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import streaming_online_softmax_amd as mod
    return mod


def ref_pack(mask):
    """uint32 [ceil(Nq/32), ceil(Nkv/64), 64] from the header's formula."""
    Nq, Nkv = mask.shape
    ng, nkg = -(-Nq // 32), -(-Nkv // 64)
    vis = np.zeros((ng * 32, nkg * 64), bool)
    vis[:Nq, :Nkv] = mask != 0
    lane = np.arange(64)[:, None]
    b = np.arange(32)[None, :]
    key = 32 * (b // 16) + 16 * ((b % 16) // 8) + 8 * (lane // 32) + b % 8      # [64, 32]
    row = np.broadcast_to(lane % 32, key.shape)
    grid = vis.reshape(ng, 32, nkg, 64).transpose(0, 2, 1, 3)                  # [g, c, row, key]
    sel = grid[:, :, row, key]                                                  # [g, c, lane, bit]
    return (sel.astype(np.uint64) << b.astype(np.uint64)).sum(-1).astype(np.uint32)


def test_reference_encoding_by_hand():
    """The test's own encoder on hand-placed bytes: (row 0, key 0) is lane 0 bit 0; key 8 of row
    0 belongs to lane 32; key 16 of row 5 is lane 5 bit 8; key 32 is bit 16; key 63 of row 31 is
    lane 63 bit 31; key 64 starts the next key group."""
    m = np.zeros((32, 128), np.uint8)
    for r, kk in ((0, 0), (0, 8), (5, 16), (5, 32), (31, 63), (2, 64)):
        m[r, kk] = 7
    w = ref_pack(m)
    assert w.shape == (1, 2, 64)
    expect = np.zeros((1, 2, 64), np.uint32)
    expect[0, 0, 0] |= 1 << 0
    expect[0, 0, 32] |= 1 << 0
    expect[0, 0, 5] |= (1 << 8) | (1 << 16)
    expect[0, 0, 63] |= 1 << 31
    expect[0, 1, 2] |= 1 << 0
    assert np.array_equal(w, expect)


def _byte_mask(rng, Nq, Nkv):
    """Visible with probability 1/2, the visible bytes drawn from several nonzero values (the
    rule is 'nonzero', not 'equal to 1')."""
    vals = np.array([1, 2, 0x7F, 0x80, 0xFF], np.uint8)
    m = vals[rng.integers(0, len(vals), (Nq, Nkv))]
    m[rng.random((Nq, Nkv)) < 0.5] = 0
    return m


@pytest.mark.parametrize("Nq,Nkv,causal,offset", [
    (1, 1, 0, 0), (33, 65, 0, 0), (33, 65, 0, 1), (64, 128, 0, 0), (200, 77, 0, 3), (129, 1000, 0, 0),
    (1, 1, 1, 0), (64, 64, 1, 0), (203, 203, 1, 0), (400, 400, 1, 8), (400, 400, 1, 5), (400, 400, 0, 0)])
def test_pack_matches_encoding(sa, Nq, Nkv, causal, offset):
    """Every word against the reference encoding; a causal packing writes exactly the groups with
    64 c <= 32 g + 31 and leaves the others as they were.  offset shifts the mask start off
    8-byte alignment (the byte-by-byte read)."""
    rng = si.rng_for(95, Nq * 7 + Nkv * 3 + causal + offset)
    m = _byte_mask(rng, Nq, Nkv)
    buf = torch.zeros(Nq * Nkv + offset, dtype=torch.uint8, device=DEV)
    md = buf[offset:].view(Nq, Nkv)
    md.copy_(torch.from_numpy(m).to(DEV))
    bits = torch.full((sa.mask_bits_words(Nq, Nkv),), SENTINEL, dtype=torch.int32, device=DEV)
    sa.attn_mask_pack(md, bits, causal=bool(causal))
    torch.cuda.synchronize()
    got = bits.cpu().numpy().view(np.uint32).reshape(-1, -(-Nkv // 64), 64)
    ref = ref_pack(m)
    if not causal:
        assert np.array_equal(got, ref)
        return
    g = np.arange(got.shape[0])[:, None]
    c = np.arange(got.shape[1])[None, :]
    written = 64 * c <= 32 * g + 31
    assert np.array_equal(got[written], ref[written])
    assert np.all(got[~written] == SENTINEL)


FWD_CASES = [(D, BN, N, causal, dt) for (D, BN) in [(16, 32), (32, 64), (64, 32), (64, 64), (128, 64), (256, 64)]
             for N in (203, 400) for causal in (False, True) for dt in ("bf16", "f16")
             if not (dt == "f16" and N == 203)]


@pytest.mark.parametrize("D,BN,N,causal,dtype", FWD_CASES)
def test_packed_forward_matches_bytes_and_oracle(sa, D, BN, N, causal, dtype):
    """Packed bits give bitwise the byte-mask results (ragged last key tile, partial query
    block, all-masked rows), which match the oracle.  D = 128 causal with N = 400 runs the
    paired-block launch."""
    rng = si.rng_for(96, D * 1000 + BN * 10 + N + int(causal))
    H = 2
    q, k, v = (si.cast(x, dtype) for x in si.draw_qkv(rng, (1, N, H, D), (1, N, H, D)))
    mask, _ = si.bernoulli_mask(rng, N, N, 4)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    md = torch.from_numpy(mask).to(DEV)
    bits = sa.pack_mask(md, causal=causal)
    o1, l1 = sa.fwd(qd, kd, vd, causal=causal, mask=md, block_n=BN)
    o2, l2 = sa.fwd(qd, kd, vd, causal=causal, mask_bits=bits, block_n=BN)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2), "packed != bytes"
    ref, ref_lse = oracle.attn_dense(q, k, v, causal=causal, mask=mask)
    o = o2.float().cpu().numpy().reshape(ref.shape).astype(np.float64)
    assert np.abs(o - ref).max() <= TOL[dtype]
    empty = ref_lse == -np.inf
    assert np.all(o[empty] == 0.0)
    lg = l2.cpu().numpy().reshape(ref_lse.shape).astype(np.float64)
    assert np.all(lg[empty] == -np.inf)
    fin = ~empty
    assert np.all(np.abs(lg[fin] - ref_lse[fin]) <= 1e-3 * np.maximum(1.0, np.abs(ref_lse[fin])))


def test_packed_entry_point_and_all_masked(sa):
    """attn_fwd_packed on a mask with no visible key at all: every output 0, every LSE -inf; and
    on a full mask the unmasked result bit for bit."""
    rng = si.rng_for(97, 0)
    N, H, D = 300, 2, 64
    q, k, v = (si.cast(x, "bf16").to(DEV) for x in si.draw_qkv(rng, (1, N, H, D), (1, N, H, D)))
    out = torch.empty_like(q)
    lse = torch.empty((1, N, H), dtype=torch.float32, device=DEV)
    zeros = sa.pack_mask(torch.zeros((N, N), dtype=torch.uint8, device=DEV))
    sa.attn_fwd_packed(q, k, v, out, lse, causal=False, mask_bits=zeros)
    torch.cuda.synchronize()
    assert bool((out == 0).all()) and bool((lse == -float("inf")).all())
    for causal in (False, True):
        ones = sa.pack_mask(torch.ones((N, N), dtype=torch.uint8, device=DEV), causal=causal)
        sa.attn_fwd_packed(q, k, v, out, lse, causal=causal, mask_bits=ones)
        o0, l0 = sa.fwd(q, k, v, causal=causal)
        torch.cuda.synchronize()
        assert torch.equal(out, o0) and torch.equal(lse, l0)


def test_packed_rejects_without_enqueueing(sa):
    """Reject paths with real buffers: nothing written."""
    N, H, D = 64, 1, 64
    q = torch.zeros((1, N, H, D), dtype=torch.bfloat16, device=DEV)
    out = torch.full_like(q, 3.0)
    bits = torch.zeros(sa.mask_bits_words(N, N), dtype=torch.int32, device=DEV)
    md = torch.ones((N, N), dtype=torch.uint8, device=DEV)
    with pytest.raises(sa.AttnError):
        sa.attn_fwd(q, q, q, out, None, mask=md, mask_bits=bits)
    with pytest.raises(sa.AttnError):
        sa.attn_mask_pack(md[:, :63].contiguous(), bits, causal=True)
    torch.cuda.synchronize()
    assert bool((out == 3.0).all()) and bool((bits == 0).all())


def test_masked_long_context_packed_matches_bytes(sa):
    """The masked long-context workload (B1 H16 N16384 D256, causal AND a Bernoulli(1/2) mask,
    1/64 rows all-masked) packed causally: outputs and LSE bit for bit those of the byte mask,
    which test_gpu_parity compares with the oracle on every row-head."""
    q, k, v, mask, _ = si.masked_inputs()
    qd, kd, vd, md = q.to(DEV), k.to(DEV), v.to(DEV), torch.from_numpy(mask).to(DEV)
    del q, k, v, mask
    o1, l1 = sa.fwd(qd, kd, vd, causal=True, mask=md)
    bits = sa.pack_mask(md, causal=True)
    o2, l2 = sa.fwd(qd, kd, vd, causal=True, mask_bits=bits)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def _random_cases(n):
    rng = si.rng_for(99, 0)
    cases = []
    for _ in range(n):
        D = int(rng.choice([16, 32, 64, 128, 256]))
        BN = int(rng.choice([32, 64])) if D <= 64 else 64
        cases.append((int(rng.integers(1, 1500)), D, BN, bool(rng.integers(0, 2)), int(rng.integers(1, 3)),
                      int(rng.integers(1, 4)), float(rng.choice([0.1, 0.5, 0.9]))))
    return cases


RANDOM_CASES = _random_cases(40)


@pytest.mark.parametrize("N,D,BN,causal,B,H,density", RANDOM_CASES,
                         ids=[f"N{c[0]}-D{c[1]}-BN{c[2]}-{'c' if c[3] else 'nc'}-B{c[4]}H{c[5]}-p{c[6]}"
                              for c in RANDOM_CASES])
def test_packed_matches_bytes_random_shapes(sa, N, D, BN, causal, B, H, density):
    """Seeded random sizes (tile tails, partial query blocks and 32-row groups, paired causal
    blocks at D = 128, both tile widths) and mask densities: the packed forward equals the
    byte-mask forward bit for bit; the byte path is the one compared with the oracle elsewhere."""
    rng = si.rng_for(99, N * 7 + D + BN + int(causal))
    q, k, v = (si.cast(x, "bf16").to(DEV) for x in si.draw_qkv(rng, (B, N, H, D), (B, N, H, D)))
    mask = (rng.random((N, N)) < density).astype(np.uint8)
    md = torch.from_numpy(mask).to(DEV)
    bits = sa.pack_mask(md, causal=causal)
    o1, l1 = sa.fwd(q, k, v, causal=causal, mask=md, block_n=BN)
    o2, l2 = sa.fwd(q, k, v, causal=causal, mask_bits=bits, block_n=BN)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
