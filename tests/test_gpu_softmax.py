"""Parity of attn_softmax_rows (through the C ABI) with the oracle's O5 row softmax.

Tolerance, per element, derived from the arithmetic.  A weight is 2^((x - m) * log2e): the
difference and the product are each rounded (relative 2^-24 of an argument of magnitude
|log2 w|), so the weight carries a relative error up to ln2 * 2^-23 * |log2 w| plus one unit
of the exp2 result; |log2 w| is bounded by |log2 ref| + log2(n).  A row sum takes at most
n/64 + 8 sequential FP32 additions per value (2^-24 relative each), and the division adds one
rounding.  The output type adds at most half a unit in the last place: 2^-8 relative for bf16
(7 fraction bits), 2^-11 for fp16 (and 2^-25 absolute below fp16's normal range).  So
    |y - ref| <= ((|log2 ref| + log2 n + 4) * 2^-23 + (n/64 + 8) * 2^-24 + u_out) * ref + 1e-30,
where 1e-30 absorbs weights below FP32's normal range.  Masked entries (-inf) must be exactly 0
and all-masked rows exactly 0; every method and dtype is compared element by element with the
oracle fed the exact input values.
"""
import numpy as np
import pytest
import torch

import oracle
import seeded_inputs as si

pytestmark = pytest.mark.gpu
DEV = "cuda"
METHODS = {"streaming": 0, "registers": 1, "three_pass": 2}


@pytest.fixture(scope="module")
def sa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import streaming_online_softmax_amd as mod
    return mod


def _check(y, x_dev, ref, dtype):
    yv = y.float().cpu().numpy().astype(np.float64)
    assert not np.isnan(yv).any(), "NaN in output"
    n = ref.shape[-1]
    with np.errstate(divide="ignore"):
        lg = np.where(ref > 0, np.abs(np.log2(np.where(ref > 0, ref, 1.0))), 0.0)
    u_out = {"f32": 0.0, "bf16": 2.0 ** -8, "f16": 2.0 ** -11}[dtype]
    rtol = (lg + np.log2(n) + 4) * 2.0 ** -23 + (n / 64 + 8) * 2.0 ** -24 + u_out
    atol = 1e-30 + (2.0 ** -25 if dtype == "f16" else 0.0)
    err = np.abs(yv - ref) - (rtol * np.abs(ref) + atol)
    i = np.unravel_index(np.argmax(err), err.shape)
    assert err.max() <= 0, f"excess {err.max():.3e} at {i}: y={yv[i]:.9e} ref={ref[i]:.9e}"
    masked = torch.isneginf(x_dev.float()).cpu().numpy()
    assert np.all(yv[masked] == 0.0), "masked entries not exactly 0"
    empty = masked.all(axis=-1)
    assert np.all(yv[empty] == 0.0), "all-masked rows not exactly 0"


CASES = []
for method in METHODS:
    for dtype in ("f32", "bf16", "f16"):
        for n in (1, 3, 64, 255, 256, 257, 1000, 4096, 4097, 5003, 40000, 65536):
            CASES.append((method, dtype, n))


@pytest.mark.parametrize("method,dtype,n", CASES, ids=[f"{m}-{d}-n{n}" for m, d, n in CASES])
def test_softmax_rows_against_oracle(sa, method, dtype, n):
    """37 rows (not a multiple of the four rows of a workgroup): normal logits, x30 logits, a
    third of the entries masked, and two all-masked rows."""
    rows = 37
    case = CASES.index((method, dtype, n))
    for variant, frac, full in (("normal", 0.0, 0), ("large", 0.0, 0), ("normal", 0.3, 2)):
        x32 = si.softmax_inputs(rows, n, case=case, variant=variant, masked_frac=frac, full_rows=full)
        x = si.cast(x32, dtype).to(DEV)
        y = sa.softmax_rows(x, METHODS[method])
        torch.cuda.synchronize()
        _check(y, x, oracle.softmax_rows(x.cpu()), dtype)


@pytest.mark.parametrize("method", list(METHODS))
def test_softmax_rows_in_place_and_unaligned(sa, method):
    """x == y is allowed; a row start that is not 16-byte aligned takes the scalar path."""
    x32 = si.softmax_inputs(9, 1024, case=7, masked_frac=0.1, full_rows=1)
    x = torch.from_numpy(x32).to(DEV)
    ref = oracle.softmax_rows(x.cpu())
    sa.attn_softmax_rows(x, x, METHODS[method])
    torch.cuda.synchronize()
    _check(x, torch.from_numpy(x32).to(DEV), ref, "f32")
    buf = torch.zeros(9 * 1024 + 1, device=DEV)
    xs = buf[1:].view(9, 1024)
    xs.copy_(torch.from_numpy(x32))
    ys = torch.zeros(9 * 1024 + 1, device=DEV)[1:].view(9, 1024)
    sa.attn_softmax_rows(xs, ys, METHODS[method])
    torch.cuda.synchronize()
    _check(ys, xs, ref, "f32")


def test_softmax_rows_full_size_sampled(sa):
    """The benchmark workload (32768 rows x 4096 fp32) by every method: sampled rows against the
    oracle, and every row sums to 1 within the FP32 bound."""
    s = si.SOFTMAX
    x32 = si.softmax_inputs(s["rows"], s["n"], case=0)
    x = torch.from_numpy(x32).to(DEV)
    rows = np.unique(si.rng_for(91, 0).integers(0, s["rows"], 64))
    ref = oracle.softmax_rows(torch.from_numpy(x32[rows]))
    for name, m in METHODS.items():
        y = sa.softmax_rows(x, m)
        torch.cuda.synchronize()
        _check(y[torch.from_numpy(rows).to(DEV)], x[torch.from_numpy(rows).to(DEV)], ref, "f32")
        tot = y.double().sum(dim=1)
        assert float((tot - 1).abs().max()) <= (s["n"] / 64 + 8) * 2.0 ** -24 + 4e-6, name


def test_softmax_rows_methods_agree_wide(sa):
    """64 rows of 32768 (a workgroup per row for the registers method): every method against the
    oracle."""
    x32 = si.softmax_inputs(64, 32768, case=1, variant="large", masked_frac=0.05, full_rows=1)
    x = torch.from_numpy(x32).to(DEV)
    ref = oracle.softmax_rows(torch.from_numpy(x32))
    for m in (0, 1, 2):
        y = sa.softmax_rows(x, m)
        torch.cuda.synchronize()
        _check(y, x, ref, "f32")


def test_softmax_rows_rejects(sa):
    x = torch.zeros(2, 65537, device=DEV)
    with pytest.raises(sa.AttnError) as e:
        sa.attn_softmax_rows(x, x, 1)            # registers method: n <= 65536
    assert e.value.code == 3
    with pytest.raises(sa.AttnError):
        sa.attn_softmax_rows(x, x, 9)
