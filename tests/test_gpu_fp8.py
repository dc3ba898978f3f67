"""attn_fwd_fp8v (E4M3 or E5M2 V, probabilities rounded to E4M3 for the FP8 matrix cores) and the
E4M3 conversion, through the C ABI, against the oracle (O1 with V decoded exactly, O6).

Tolerance, per output element, derived from the arithmetic (the pages give none for 8-bit
operands).  With w_j = exp(s_j - M) the exact weights of row i (M its maximum, L = sum w_j) and
V_j the exact values decode(v_j) * v_scale:
  * each probability the kernel feeds the FP8 product is its FP32 weight p_j = 2^delta w_j
    (delta >= 0: the kernel's reference maximum is never above M) rounded to E4M3: the error is at
    most 2^-4 p_j (3 fraction bits, normal range) or 2^-10 absolute (half the subnormal spacing);
    divided by the FP32 denominator 2^delta L the 2^-10 term only shrinks, so it is bounded with
    delta = 0;
  * the FP8 matrix instruction accumulates with reduced internal precision: measured on gfx950 at
    most 2^-13.3 of the sum of |products| per instruction; 2^-11 of sum w_j |V_j| / L is used;
  * the output is rounded to bf16 (2^-8 relative) or fp16 (2^-11), plus FP32 slop (2^-20).
So |O - ref| <= (sum_j max(2^-4 w_j, 2^-10) |V_j| + 2^-11 sum_j w_j |V_j|) / L + u_out |ref| + 2^-20.
The LSE does not see the rounding (l sums the unrounded weights): |dLSE| <= 1e-3 max(1, |LSE|).
"""
import numpy as np
import pytest
import torch

import oracle
import seeded_inputs as si

pytestmark = pytest.mark.gpu
DEV = "cuda"
CHUNK = 1 << 28


@pytest.fixture(scope="module")
def sa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import streaming_online_softmax_amd as mod
    return mod


def _bound(q, k, v_codes, v_scale, causal, mask, rows, ref, dtype, v_format="e4m3", exact_weights=False):
    """Per-element bound for the selected row-heads rh = (b*N + i)*H + h.  exact_weights: every
    weight the kernel rounds is exactly representable in E4M3 (Q = 0: all weights 1), so the
    rounding term drops out."""
    qd = q.double().numpy()
    kd = k.double().numpy()
    vd = oracle.decode_bits(v_codes.numpy(), v_format) * v_scale
    B, N, H, D = qd.shape
    u_out = 2.0 ** -8 if dtype == "bf16" else 2.0 ** -11
    rows = np.asarray(rows)
    out = np.zeros((rows.size, D))
    vis = np.ones((N, N), bool)
    if causal:
        vis &= np.tri(N, dtype=bool)
    if mask is not None:
        vis &= mask != 0
    for b in range(B):
        for h in range(H):
            sel = np.nonzero((rows // (H * N) == b) & (rows % H == h))[0]
            if sel.size == 0:
                continue
            i = (rows[sel] // H) % N
            s = (qd[b, i, h, :] @ kd[b, :, h, :].T) / np.sqrt(D)          # [rows, N]
            v_ok = vis[i]
            s = np.where(v_ok, s, -np.inf)
            m = s.max(axis=1, keepdims=True)
            w = np.where(v_ok, np.exp(s - np.where(np.isfinite(m), m, 0.0)), 0.0)
            L = w.sum(axis=1, keepdims=True)
            av = np.abs(vd[b, :, h, :])
            rnd = 0.0 if exact_weights else np.where(v_ok, np.maximum(2.0 ** -4 * w, 2.0 ** -10), 0.0) @ av
            num = rnd + 2.0 ** -11 * (w @ av)
            out[sel] = np.where(L > 0, num / np.where(L > 0, L, 1.0), 0.0)
    return out + u_out * np.abs(ref) + 2.0 ** -20


def _check(sa, q, k, v, v_scale, causal, mask, dtype, rows=None, what="", v_format="e4m3", exact_weights=False):
    B, N, H, D = q.shape
    md = None if mask is None else torch.from_numpy(mask).to(DEV)
    out, lse = sa.fwd_fp8v(q.to(DEV), k.to(DEV), v.to(DEV), v_scale, causal=causal, mask=md, v_format=v_format)
    torch.cuda.synchronize()
    if rows is None:
        rows = np.arange(B * N * H)
    ref, ref_lse = oracle.attn_dense_fp8v(q, k, v, v_scale, causal=causal, mask=mask, rows=rows, v_format=v_format)
    rt = torch.from_numpy(np.asarray(rows)).to(DEV)
    o = out.reshape(-1, D)[rt].float().cpu().numpy().astype(np.float64)
    l = lse.reshape(-1)[rt].cpu().numpy().astype(np.float64)
    assert not np.isnan(o).any(), f"{what}: NaN"
    bnd = _bound(q, k, v, v_scale, causal, mask, rows, ref, dtype, v_format, exact_weights)
    excess = np.abs(o - ref) - bnd
    worst = np.unravel_index(np.argmax(excess), excess.shape)
    assert excess.max() <= 0, (f"{what}: |dO| {abs(o - ref)[worst]:.3e} > bound {bnd[worst]:.3e} at {worst}; "
                               f"max |dO| {np.abs(o - ref).max():.3e}")
    empty = ref_lse == -np.inf
    assert np.all(o[empty] == 0.0) and np.all(l[empty] == -np.inf), f"{what}: empty rows"
    fin = ~empty
    lerr = np.abs(l[fin] - ref_lse[fin]) / np.maximum(1.0, np.abs(ref_lse[fin]))
    assert (lerr.max() if lerr.size else 0.0) <= 1e-3, f"{what}: LSE"
    return np.abs(o - ref).max()


CASES = [(N, causal, masked, dtype, scale)
         for N in (1, 17, 64, 200, 1000)
         for causal in (False, True)
         for masked in (False, True)
         for dtype in ("bf16", "f16")
         for scale in (1.0, 0.25)
         if not (masked and N == 1)]


@pytest.mark.parametrize("N,causal,masked,dtype,scale", CASES,
                         ids=[f"N{n}-{'c' if c else 'nc'}-{'m' if m else 'nm'}-{d}-s{s}" for n, c, m, d, s in CASES])
def test_fp8v_against_oracle(sa, N, causal, masked, dtype, scale):
    """Every row of B=2, H=2 shapes (ragged tiles, a partial query block, masks with fully
    masked rows) against O1 on the exact E4M3 values."""
    case = CASES.index((N, causal, masked, dtype, scale))
    q, k, v = si.fp8v_inputs(B=2, H=2, N=N, case=case, dtype=dtype)
    mask = None
    if masked:
        mask, _ = si.bernoulli_mask(si.rng_for(si.CFG_FP8V, 100 + case), N, N, max(1, N // 64))
    _check(sa, q, k, v, scale, causal, mask, dtype, what=f"N={N} causal={causal} mask={masked} {dtype}")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_fp8v_staged_mask_full_tiles(sa, causal, dtype):
    """N = 768: six full 128-key tiles, so the byte mask is staged through LDS (rows 16-byte
    aligned) tile after tile, over several query blocks (paired when causal); every row against
    O1, and bitwise equal to the same mask read from global memory (a copy 8 bytes off 16-byte
    alignment)."""
    N = 768
    case = 300 + 2 * int(causal) + (dtype == "f16")
    q, k, v = si.fp8v_inputs(B=2, H=2, N=N, case=case, dtype=dtype)
    mask, _ = si.bernoulli_mask(si.rng_for(si.CFG_FP8V, 100 + case), N, N, N // 64)
    _check(sa, q, k, v, 1.0, causal, mask, dtype, what=f"staged mask N={N} causal={causal} {dtype}")
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    m16 = torch.from_numpy(mask).to(DEV)
    buf = torch.zeros(N * N + 8, dtype=torch.uint8, device=DEV)
    m8 = buf[8:].view(N, N)
    m8.copy_(m16)
    assert m16.data_ptr() % 16 == 0 and m8.data_ptr() % 16 == 8
    o1, l1 = sa.fwd_fp8v(qd, kd, vd, 1.0, causal=causal, mask=m16)
    o2, l2 = sa.fwd_fp8v(qd, kd, vd, 1.0, causal=causal, mask=m8)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2), "staged != direct"


E5M2_CASES = [(N, causal, masked, dtype) for N in (17, 200, 1000) for causal in (False, True)
              for masked in (False, True) for dtype in ("bf16", "f16")]


@pytest.mark.parametrize("N,causal,masked,dtype", E5M2_CASES,
                         ids=[f"N{n}-{'c' if c else 'nc'}-{'m' if m else 'nm'}-{d}" for n, c, m, d in E5M2_CASES])
def test_fp8v_e5m2_against_oracle(sa, N, causal, masked, dtype):
    """V as E5M2 codes (the FP8 instruction's A operand in its E5M2 form; P stays E4M3)."""
    case = 200 + E5M2_CASES.index((N, causal, masked, dtype))
    q, k, v = si.fp8v_inputs(B=2, H=2, N=N, case=case, dtype=dtype, v_format="e5m2")
    mask = None
    if masked:
        mask, _ = si.bernoulli_mask(si.rng_for(si.CFG_FP8V, 100 + case), N, N, max(1, N // 64))
    _check(sa, q, k, v, 0.5, causal, mask, dtype, what=f"e5m2 N={N} causal={causal} mask={masked} {dtype}",
           v_format="e5m2")


def test_fp8v_single_key_and_uniform(sa):
    """One key: O = V_0 * v_scale up to the output rounding (its weight is 1, exact in E4M3).
    Q = 0: every visible weight is 1 (exact), so O is the mean of the visible V rows."""
    q, k, v = si.fp8v_inputs(B=1, H=2, N=1, case=50)
    out, lse = sa.fwd_fp8v(q.to(DEV), k.to(DEV), v.to(DEV), 0.5)
    ref = torch.from_numpy(oracle.decode_bits(v.numpy(), "e4m3") * 0.5).to(torch.bfloat16)
    assert torch.equal(out.cpu(), ref.reshape(out.shape))
    q, k, v = si.fp8v_inputs(B=1, H=2, N=300, case=51)
    q = torch.zeros_like(q)
    for causal in (False, True):
        _check(sa, q, k, v, 1.0, causal, None, "bf16", what=f"uniform causal={causal}", exact_weights=True)


def _block_rows(B, N, H, seed):
    """One seeded row in each (batch, head, 256-row query block) unit -- every workgroup of the
    launch -- plus the first and last rows and rows at tile boundaries."""
    rng = si.rng_for(si.CFG_FP8V, seed)
    nb = (N + 255) // 256
    b = np.repeat(np.arange(B), nb * H)
    blk = np.tile(np.repeat(np.arange(nb), H), B)
    h = np.tile(np.arange(H), B * nb)
    tok = np.minimum(blk * 256 + rng.integers(0, 256, blk.size), N - 1)
    extra = np.array([0, 1, 63, 64, 255, 256, N - 1])
    rows = np.concatenate([(b * N + tok) * H + h, (rng.integers(0, B, extra.size) * N + extra) * H
                           + rng.integers(0, H, extra.size)])
    return np.unique(rows)


def test_fp8v_full_size(sa):
    """The benchmark shape (B4 H32 N4096 D128 causal, bf16 Q/K, E4M3 V): a row of every
    workgroup (2048 (batch, head, query block) units) within the per-element bound."""
    s = si.FP8V
    q, k, v = si.fp8v_inputs()
    rows = _block_rows(s["B"], s["N"], s["H"], 999)
    _check(sa, q, k, v, 1.0, True, None, "bf16", rows=rows, what="full size")


def test_fp8v_full_size_uniform_logits(sa):
    """The same shape with Q = 0: every visible weight is exactly 1 (exact in E4M3), so the bound
    reduces to the FP8 accumulation and output rounding terms (2^-11 of the mean |V| plus half
    an output ulp, ~4.5e-4 at 4096 keys).  A key dropped from a row of n keys moves that row's
    output by (O - V_j) / (n - 1), which exceeds the bound in the element where |V_j| is largest
    (~2.6 among 128 normal draws) for every n up to 4096."""
    s = si.FP8V
    q, k, v = si.fp8v_inputs()
    q = torch.zeros_like(q)
    rows = _block_rows(s["B"], s["N"], s["H"], 998)
    _check(sa, q, k, v, 1.0, True, None, "bf16", rows=rows, what="full size, uniform logits", exact_weights=True)


@pytest.mark.parametrize("fmt_dtype", ["e4m3"])
def test_round_e4m3_every_float32_bit_pattern(sa, fmt_dtype):
    """The kernels' E4M3 conversion (attn_round) equals O6 on every non-NaN float32 input
    (nearest even, subnormals kept, saturation to +-448 and for infinities); NaN -> a NaN code."""
    y = torch.empty(CHUNK, dtype=torch.uint8, device=DEV)
    base = np.arange(CHUNK, dtype=np.uint32)
    for c in range((1 << 32) // CHUNK):
        bits = base + np.uint32(c * CHUNK)
        x = bits.view(np.float32)
        sa.attn_round(torch.from_numpy(x).to(DEV), y)
        got = y.cpu().numpy()
        want = oracle.round_fp8_bits(x, fmt_dtype)
        nan_in = np.isnan(x)
        bad = np.nonzero((got != want) & ~nan_in)[0]
        assert bad.size == 0, (f"{bad.size} mismatches in chunk {c}; first x=0x{int(bits[bad[0]]):08x} "
                               f"got 0x{int(got[bad[0]]):02x} want 0x{int(want[bad[0]]):02x}")
        assert np.all((got[nan_in] & 0x7F) == 0x7F), f"a NaN input did not give a NaN code (chunk {c})"
        print(f"  e4m3 chunk {c:2d}/16 equal", flush=True)


def test_fp8v_rejects(sa):
    q = torch.zeros(1, 64, 1, 64, dtype=torch.bfloat16, device=DEV)
    v = torch.zeros(1, 64, 1, 64, dtype=torch.uint8, device=DEV)
    with pytest.raises(sa.AttnError) as e:
        sa.fwd_fp8v(q, q, v, 1.0)                    # D = 64
    assert e.value.code == 3
    q = torch.zeros(1, 64, 1, 128, dtype=torch.bfloat16, device=DEV)
    v = torch.zeros(1, 64, 1, 128, dtype=torch.uint8, device=DEV)
    with pytest.raises(sa.AttnError):
        sa.fwd_fp8v(q, q, v, float("inf"))
    with pytest.raises(sa.AttnError):
        sa.fwd_fp8v(q, q, v.view(torch.int8), 1.0)   # not 8-bit float codes
    with pytest.raises(sa.AttnError):
        sa.fwd_fp8v(q, q, v, 1.0, v_format="e3m4")
