"""Parity of the HIP path (through the C ABI) with the FP64 oracle on every workload.

Tolerances: max |O_gpu - O_oracle| <= 2e-2 (bf16) / 5e-3 (fp16) over all compared elements;
|LSE_gpu - LSE_oracle| <= 1e-3 * max(1, |LSE|); an all-masked row must give O exactly 0 and
LSE exactly -inf; split-K combined must match the unsplit result to 1e-3.  The oracle is fed the
exact bf16/fp16 values the kernels read.  The full-size workloads (causal prefill, split-K decode
at every split count, masked long context) compare every row-head with the oracle, in chunks of
rows; each such test prints its largest error over all rows (and, when ATTN_PARITY_REPORT names a
file, appends it there as one JSON line).
"""
import json
import math
import os
import time

import numpy as np
import pytest
import torch

import oracle
import seeded_inputs as si

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "f16": 5e-3}
DEV = "cuda"


@pytest.fixture(scope="module")
def sa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import streaming_online_softmax_amd as mod
    return mod


def _compare(out, lse, ref, ref_lse, dtype, what=""):
    """out: [rows, D] GPU result (any float dtype), lse: [rows] natural log."""
    o = out.float().cpu().numpy().reshape(ref.shape).astype(np.float64)
    assert not np.isnan(o).any(), f"{what}: NaN in output"
    err = np.abs(o - ref).max() if o.size else 0.0
    assert err <= TOL[dtype], f"{what}: max|dO|={err:.3e} > {TOL[dtype]}"
    empty = ref_lse == -np.inf
    assert np.all(o[empty] == 0.0), f"{what}: all-masked rows not exactly 0"
    if lse is not None:
        l = lse.float().cpu().numpy().reshape(ref_lse.shape).astype(np.float64)
        assert np.all(l[empty] == -np.inf), f"{what}: all-masked rows LSE not -inf"
        fin = ~empty
        lerr = np.abs(l[fin] - ref_lse[fin]) / np.maximum(1.0, np.abs(ref_lse[fin]))
        assert (lerr.max() if lerr.size else 0.0) <= 1e-3, f"{what}: LSE rel err {lerr.max():.3e}"
    return err


def _report(name, **fields):
    line = {"test": name, **fields}
    print("parity:", json.dumps(line), flush=True)
    path = os.environ.get("ATTN_PARITY_REPORT")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps(line) + "\n")


def _full_compare(out, lse, q, k, v, dtype, name, causal=False, mask=None, chunk=1 << 16):
    """Every row-head of out [B, N, H, D] / lse [B, N, H] (GPU tensors) against O1, the oracle
    run over contiguous chunks of row-heads.  Returns the worst errors and where they occur."""
    D = q.shape[-1]
    o_all = out.reshape(-1, D).float().cpu().numpy()
    l_all = lse.reshape(-1).cpu().numpy()
    n = o_all.shape[0]
    worst = {"rows": n, "max_abs_err": 0.0, "at_row": -1, "abs_O_there": 0.0, "max_lse_rel_err": 0.0,
             "empty_rows": 0}
    t0 = time.perf_counter()
    for r0 in range(0, n, chunk):
        rows = np.arange(r0, min(n, r0 + chunk), dtype=np.int64)
        ref, ref_lse = oracle.attn_dense(q, k, v, causal=causal, mask=mask, rows=rows)
        o = o_all[rows].astype(np.float64)
        l = l_all[rows].astype(np.float64)
        assert not np.isnan(o).any(), f"{name}: NaN in rows {r0}.."
        e = np.abs(o - ref)
        i = int(np.argmax(e.max(axis=1)))
        if e[i].max() > worst["max_abs_err"]:
            worst.update(max_abs_err=float(e[i].max()), at_row=int(rows[i]),
                         abs_O_there=float(np.abs(ref[i]).max()))
        empty = ref_lse == -np.inf
        worst["empty_rows"] += int(empty.sum())
        assert np.all(o[empty] == 0.0), f"{name}: all-masked rows not exactly 0"
        assert np.all(l[empty] == -np.inf), f"{name}: all-masked rows LSE not -inf"
        fin = ~empty
        if fin.any():
            lerr = np.abs(l[fin] - ref_lse[fin]) / np.maximum(1.0, np.abs(ref_lse[fin]))
            worst["max_lse_rel_err"] = max(worst["max_lse_rel_err"], float(lerr.max()))
    worst["oracle_s"] = round(time.perf_counter() - t0, 1)
    _report(name, dtype=dtype, **worst)
    assert worst["max_abs_err"] <= TOL[dtype], f"{name}: max|dO|={worst['max_abs_err']:.3e} at row {worst['at_row']}"
    assert worst["max_lse_rel_err"] <= 1e-3, f"{name}: LSE rel err {worst['max_lse_rel_err']:.3e}"
    return worst


# ---------------------------------------------------------------------------------------------
# single-head N64 D16 (fp32 draws, run on the bf16 and fp16 casts), BN = 32
# ---------------------------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_small_fp32_drawn(sa, dtype):
    q32, k32, v32 = si.small_inputs()
    q, k, v = si.cast(q32, dtype), si.cast(k32, dtype), si.cast(v32, dtype)
    out, lse = sa.fwd(q.to(DEV), k.to(DEV), v.to(DEV), block_n=32)
    ref, ref_lse = oracle.attn_dense(q, k, v)
    _compare(out, lse, ref, ref_lse, dtype, f"small {dtype}")


# ---------------------------------------------------------------------------------------------
# single-head sweep: N x D x dtype x causal x BN x variant (360 cases)
# ---------------------------------------------------------------------------------------------
_ORACLE_CACHE = {}


def _sweep_ref(case, q, k, v):
    key = (case["N"], case["D"], case["dtype"], case["causal"], case["variant"])
    if key not in _ORACLE_CACHE:
        _ORACLE_CACHE.clear()
        _ORACLE_CACHE[key] = oracle.attn_dense(q, k, v, causal=case["causal"])
    return _ORACLE_CACHE[key]


CASES = si.sweep_cases()


def _case_id(c):
    return f"N{c['N']}-D{c['D']}-{c['dtype']}-{'causal' if c['causal'] else 'full'}-BN{c['BN']}-{c['variant']}"


@pytest.mark.parametrize("case", sorted(CASES, key=lambda c: (c["N"], c["D"], c["dtype"], c["causal"], c["variant"], c["BN"])),
                         ids=_case_id)
def test_sweep(sa, case):
    q, k, v = si.sweep_inputs(case)
    out, lse = sa.fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal=case["causal"], block_n=case["BN"])
    ref, ref_lse = _sweep_ref(case, q, k, v)
    _compare(out, lse, ref, ref_lse, case["dtype"], _case_id(case))
    if case["variant"] == "uniform":
        # p = 1 for every visible key: l is an exact integer, LSE = ln |vis|
        N = case["N"]
        cnt = np.arange(1, N + 1) if case["causal"] else np.full(N, N)
        np.testing.assert_allclose(lse.cpu().numpy().reshape(-1), np.log(cnt), rtol=1e-6)


def test_single_key_is_exact(sa):
    """N = 1: the only weight is 1, so O equals v0 bit for bit (bf16 in, bf16 out)."""
    for D in (16, 32, 64, 128, 256):
        rng = si.rng_for(80, D)
        q, k, v = (si.cast(x, "bf16") for x in si.draw_qkv(rng, (2, 1, 3, D), (2, 1, 3, D)))
        out, lse = sa.fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal=True)
        assert torch.equal(out.cpu(), v)


# ---------------------------------------------------------------------------------------------
# D = 128 (the two-group kernel): ragged lengths, several heads, both dtypes, split path
# ---------------------------------------------------------------------------------------------
@pytest.mark.parametrize("N", [1, 63, 333, 600])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True])
def test_d128_ragged(sa, N, dtype, causal):
    rng = si.rng_for(79, N)
    q, k, v = (si.cast(x, dtype) for x in si.draw_qkv(rng, (2, N, 3, 128), (2, N, 3, 128)))
    out, lse = sa.fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal)
    ref, ref_lse = oracle.attn_dense(q, k, v, causal=causal)
    _compare(out.reshape(-1, 128), lse.reshape(-1), ref, ref_lse, dtype, f"D128 N={N} {dtype} causal={causal}")


@pytest.mark.parametrize("P", [2, 5])
@pytest.mark.parametrize("causal", [False, True])
def test_d128_split(sa, P, causal):
    rng = si.rng_for(78, P)
    N = 517
    q, k, v = (si.cast(x, "bf16") for x in si.draw_qkv(rng, (1, N, 2, 128), (1, N, 2, 128)))
    o_p, l_p, out, lse = sa.splitk(q.to(DEV), k.to(DEV), v.to(DEV), P, causal=causal)
    torch.cuda.synchronize()
    ref_op, ref_lp = oracle.splitk(q, k, v, P, causal=causal)
    for pp in range(P):
        _compare(o_p[pp].reshape(-1, 128), None, ref_op[pp], ref_lp[pp], "bf16", f"o_partial p={pp}")
        lp = l_p[pp].reshape(-1).cpu().numpy().astype(np.float64)
        fin = np.isfinite(ref_lp[pp])
        assert np.all(lp[~fin] == -np.inf)
        np.testing.assert_allclose(lp[fin], ref_lp[pp][fin], rtol=1e-4, atol=1e-4)
    ref, ref_lse = oracle.attn_dense(q, k, v, causal=causal)
    _compare(out.reshape(-1, 128), lse.reshape(-1), ref, ref_lse, "bf16", f"D128 split P={P}")


# ---------------------------------------------------------------------------------------------
# D = 256 without a mask: the unmasked two-stage tile body and the lazy-rescale weight-sum test
# on fully visible tiles (a mask always forces the exact test), ragged lengths, both dtypes
# ---------------------------------------------------------------------------------------------
D256_CASES = [(N, dt, causal, var) for N in (333, 1000, 2048) for dt in ("bf16", "f16")
              for causal in (False, True) for var in ("normal",)] + \
             [(1000, dt, causal, "large") for dt in ("bf16", "f16") for causal in (False, True)]


@pytest.mark.parametrize("N,dtype,causal,variant", D256_CASES,
                         ids=[f"N{n}-{d}-{'causal' if c else 'full'}-{v}" for n, d, c, v in D256_CASES])
def test_d256_unmasked(sa, N, dtype, causal, variant):
    rng = si.rng_for(93, N)
    q, k, v = (si.cast(x, dtype) for x in si.draw_qkv(rng, (1, N, 2, 256), (1, N, 2, 256), variant))
    out, lse = sa.fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal)
    ref, ref_lse = oracle.attn_dense(q, k, v, causal=causal)
    _compare(out.reshape(-1, 256), lse.reshape(-1), ref, ref_lse, dtype, f"D256 N={N} {dtype} causal={causal} {variant}")


def test_d256_causal_long_context_sampled(sa):
    """The masked long-context tensors (B1 H16 N16384 D256) without the mask: causal only, the
    unmasked D = 256 kernel at full size.  Four rows of every (128-row query block, head) unit, one
    in each wave's 32 rows at a seeded lane, so every workgroup and every wave is checked."""
    s = si.MASKED
    q, k, v, _, _ = si.masked_inputs()
    N, H, D = s["N"], s["H"], s["D"]
    out, lse = sa.fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal=True)
    torch.cuda.synchronize()
    rng = si.rng_for(94, 0)
    blocks = np.arange(N // 128)
    i = (blocks[:, None, None] * 128 + np.arange(4)[None, :, None] * 32
         + rng.integers(0, 32, (blocks.size, 4, H))).reshape(-1)
    h = np.broadcast_to(np.arange(H)[None, None, :], (blocks.size, 4, H)).reshape(-1)
    rows = np.unique(i * H + h)
    ref, ref_lse = oracle.attn_dense(q, k, v, causal=True, rows=rows)
    rt = torch.from_numpy(rows).to(DEV)
    err = _compare(out.reshape(-1, D)[rt], lse.reshape(-1)[rt], ref, ref_lse, "bf16", "D256 causal long context")
    _report("d256_causal_long_context_sampled", dtype="bf16", rows=int(rows.size), max_abs_err=float(err))


# ---------------------------------------------------------------------------------------------
# split-K with several queries and a different key length (the matrix-core split producer on
# rectangular shapes): per-partition key ranges, ragged partitions, mask rows of [Nq, Nkv]
# staged through LDS (Nkv and the partition length multiples of 16), read 8 bytes at a time or
# bytewise
# ---------------------------------------------------------------------------------------------
RECT_CASES = [(3, 2000, 64, 5, False), (3, 2000, 64, 5, True), (77, 1000, 128, 3, False),
              (77, 2048, 128, 8, True), (300, 1000, 64, 8, True), (300, 2000, 128, 3, False),
              (77, 1000, 256, 3, True), (130, 777, 32, 4, True)]


@pytest.mark.parametrize("Nq,Nkv,D,P,masked", RECT_CASES,
                         ids=[f"Nq{a}-Nkv{b}-D{c}-P{d}-{'mask' if m else 'nomask'}" for a, b, c, d, m in RECT_CASES])
def test_splitk_rectangular(sa, Nq, Nkv, D, P, masked):
    rng = si.rng_for(95, Nq * 7 + Nkv + D + P)
    B, H = 2, 3
    q, k, v = (si.cast(x, "bf16") for x in si.draw_qkv(rng, (B, Nq, H, D), (B, Nkv, H, D)))
    mask = None
    md = None
    if masked:
        mask, _ = si.bernoulli_mask(rng, Nq, Nkv, 1)
        md = torch.from_numpy(mask).to(DEV)
    o_p, l_p, out, lse = sa.splitk(q.to(DEV), k.to(DEV), v.to(DEV), P, mask=md)
    torch.cuda.synchronize()
    ref_op, ref_lp = oracle.splitk(q, k, v, P, mask=mask)
    for pp in range(P):
        _compare(o_p[pp].reshape(-1, D), None, ref_op[pp], ref_lp[pp], "bf16", f"o_partial p={pp}")
        lp = l_p[pp].reshape(-1).cpu().numpy().astype(np.float64)
        fin = np.isfinite(ref_lp[pp])
        assert np.all(lp[~fin] == -np.inf)
        np.testing.assert_allclose(lp[fin], ref_lp[pp][fin], rtol=1e-4, atol=1e-4)
    ref, ref_lse = oracle.attn_dense(q, k, v, mask=mask)
    _compare(out.reshape(-1, D), lse.reshape(-1), ref, ref_lse, "bf16", f"rectangular Nq={Nq} Nkv={Nkv} P={P}")


# ---------------------------------------------------------------------------------------------
# causal future-V perturbation (workshop checker)
# ---------------------------------------------------------------------------------------------
@pytest.mark.parametrize("D", [64, 128])
def test_future_perturbation_bitwise(sa, D):
    N, i0 = 1000, 437
    rng = si.rng_for(81, D)
    q, k, v = (si.cast(x, "bf16") for x in si.draw_qkv(rng, (1, N, 2, D), (1, N, 2, D)))
    out1, lse1 = sa.fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal=True)
    _, k_new, v_new = si.draw_qkv(si.rng_for(82, D), (1, 1, 1, 1), (1, N - i0 - 1, 2, D))
    k2, v2 = k.clone(), v.clone()
    k2[:, i0 + 1:] = si.cast(k_new, "bf16")
    v2[:, i0 + 1:] = si.cast(v_new, "bf16")
    out2, lse2 = sa.fwd(q.to(DEV), k2.to(DEV), v2.to(DEV), causal=True)
    assert torch.equal(out1[:, : i0 + 1], out2[:, : i0 + 1])
    assert torch.equal(lse1[:, : i0 + 1], lse2[:, : i0 + 1])
    changed = (out1[:, i0 + 1:] != out2[:, i0 + 1:]).flatten(2).any(dim=2)
    assert bool(changed.all())


# ---------------------------------------------------------------------------------------------
# multi-head causal prefill B4 H32 N4096 D128 bf16 (the benchmark's launch configuration)
# ---------------------------------------------------------------------------------------------
def test_prefill_full_size(sa):
    """Every one of the 524,288 row-heads of the benchmark's launch against the oracle."""
    q, k, v = si.prefill_inputs()
    out, lse = sa.fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal=True)
    torch.cuda.synchronize()
    _full_compare(out, lse, q, k, v, "bf16", "prefill_B4H32N4096D128_causal_all_rows", causal=True)


# ---------------------------------------------------------------------------------------------
# split-K decode B8 H32 Nq1 Nkv32768 D128 bf16, P in {4, 8, 16, 37}
# ---------------------------------------------------------------------------------------------
@pytest.fixture(scope="module")
def decode_data(sa):
    q, k, v = si.decode_inputs()
    ref, ref_lse = oracle.attn_dense(q, k, v)          # every one of the 256 row-heads
    return q, k, v, q.to(DEV), k.to(DEV), v.to(DEV), ref, ref_lse


@pytest.mark.parametrize("P", [4, 8, 16, 37])
def test_decode_splitk_full_size(sa, decode_data, P):
    """Every row-head and every partition: o_partial and lse_partial against the oracle's
    per-partition definition, the merged output against O1, and the split result against the
    unsplit one (a single partition) to 1e-3 in FP32."""
    s = si.DECODE
    q, k, v, qd, kd, vd, ref, ref_lse = decode_data
    o_p, l_p, out, lse = sa.splitk(qd, kd, vd, P)
    # unsplit reference on the GPU: one partition (the combine is then the identity)
    o1, l1, _, _ = sa.splitk(qd, kd, vd, 1, combine=False)
    out_f32, lse_f32 = sa.combine(o_p, l_p, torch.float32)
    torch.cuda.synchronize()
    RH = s["B"] * s["H"]
    d = (out_f32.reshape(RH, -1) - o1.reshape(RH, -1)).abs().max().item()
    assert d <= 1e-3, f"split vs unsplit {d:.3e}"
    ref_op, ref_lp = oracle.splitk(q, k, v, P)
    worst_p = 0.0
    for p in range(P):
        worst_p = max(worst_p, _compare(o_p[p].reshape(RH, -1), None, ref_op[p], ref_lp[p], "bf16", f"o_partial p={p}"))
        lp = l_p[p].reshape(-1).cpu().numpy().astype(np.float64)
        np.testing.assert_allclose(lp, ref_lp[p], rtol=1e-4, atol=1e-4)
    err = _compare(out.reshape(RH, -1), lse.reshape(-1), ref, ref_lse, "bf16", f"combined P={P}")
    _report(f"decode_B8H32Nkv32768D128_P{P}_all_rows", dtype="bf16", rows=RH, max_abs_err_o_partial=float(worst_p),
            max_abs_err_combined=float(err), split_vs_unsplit_fp32=float(d))


def test_decode_empty_partitions(sa):
    """More partitions than keys: empty partitions give o_partial exactly 0 and lse -inf, and the
    combine ignores them."""
    rng = si.rng_for(85, 0)
    q, k, v = (si.cast(x, "bf16") for x in si.draw_qkv(rng, (2, 1, 3, 128), (2, 17, 3, 128)))
    o_p, l_p, out, lse = sa.splitk(q.to(DEV), k.to(DEV), v.to(DEV), 37)
    torch.cuda.synchronize()
    ref_op, ref_lp = oracle.splitk(q, k, v, 37)
    empty = ref_lp == -np.inf
    assert empty.sum() > 0
    assert np.all(l_p.cpu().numpy().reshape(37, -1)[empty] == -np.inf)
    assert np.all(o_p.cpu().numpy().reshape(37, 6, -1)[empty] == 0.0)
    ref, ref_lse = oracle.attn_dense(q, k, v)
    _compare(out.reshape(6, -1), lse.reshape(-1), ref, ref_lse, "bf16", "decode P>Nkv")


@pytest.mark.parametrize("P", [4, 8, 16, 37])
def test_decode_fused_full_size(sa, decode_data, P):
    """attn_fwd_splitk_fused: one launch; the workspace equals the unfused producer's bit for
    bit (same code); the merged output matches the two-launch path to one bf16 unit in the last
    place (their FP32 merge orders differ, so the two FP32 values may round to neighbouring bf16
    numbers) and the oracle on every row-head; tickets end at 0."""
    s = si.DECODE
    q, k, v, qd, kd, vd, ref, ref_lse = decode_data
    tk = sa.tickets(qd)
    out, lse, o_p, l_p = sa.splitk_fused(qd, kd, vd, P, tk=tk)
    o_u, l_u, out_u, lse_u = sa.splitk(qd, kd, vd, P)
    torch.cuda.synchronize()
    assert int(tk.abs().sum()) == 0
    assert torch.equal(o_p, o_u) and torch.equal(l_p, l_u)
    RH = s["B"] * s["H"]
    a, b = out.reshape(-1), out_u.reshape(-1)
    same_sign = torch.signbit(a.float()) == torch.signbit(b.float())
    ulps = (a.view(torch.int16).int() - b.view(torch.int16).int()).abs()
    assert bool((same_sign & (ulps <= 1)).all()), f"max {int(ulps.max())} bf16 ulps apart"
    assert int((ulps > 0).sum()) < a.numel() // 100
    assert torch.allclose(lse, lse_u, rtol=1e-6, atol=1e-6)
    _compare(out.reshape(RH, -1), lse.reshape(-1), ref, ref_lse, "bf16", f"fused P={P}")


def test_decode_fused_reuses_tickets(sa):
    """Two fused calls in a row on one ticket array, the second smaller (fewer partitions, other
    data, fp16): both match the oracle and the tickets are 0 after each."""
    rng = si.rng_for(88, 0)
    tk = torch.zeros(2 * 1 * 8 * sa.TICKET_STRIDE, dtype=torch.int32, device=DEV)
    for P, n, dt in ((13, 3000, "bf16"), (5, 700, "f16")):
        q, k, v = (si.cast(x, dt) for x in si.draw_qkv(rng, (2, 1, 8, 64), (2, n, 8, 64)))
        out, lse, _, _ = sa.splitk_fused(q.to(DEV), k.to(DEV), v.to(DEV), P, tk=tk)
        torch.cuda.synchronize()
        assert int(tk.abs().sum()) == 0
        ref, ref_lse = oracle.attn_dense(q, k, v)
        _compare(out.reshape(16, -1), lse.reshape(-1), ref, ref_lse, dt, f"fused P={P} n={n}")


@pytest.mark.parametrize("D,P,Nkv", [(32, 255, 2049), (256, 256, 4100), (256, 7, 1000), (128, 64, 64 * 40 + 3)])
def test_decode_fused_depths_and_split_bounds(sa, D, P, Nkv):
    """Fused decode at the largest split count (every lane of the merging wave holds four
    partitions' LSEs), ragged counts, depths below one wave (lanes past D idle in the merge) and
    at 256 (four depth slices per lane); the workspace equals the two-launch producer's, the
    output matches the oracle, the tickets end at 0."""
    rng = si.rng_for(90, D * 1000 + P)
    B, H = 2, 4
    q, k, v = (si.cast(x, "f16") for x in si.draw_qkv(rng, (B, 1, H, D), (B, Nkv, H, D)))
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    tk = sa.tickets(qd)
    out, lse, o_p, l_p = sa.splitk_fused(qd, kd, vd, P, tk=tk)
    o_u, l_u, _, _ = sa.splitk(qd, kd, vd, P)
    torch.cuda.synchronize()
    assert int(tk.abs().sum()) == 0
    assert torch.equal(o_p, o_u) and torch.equal(l_p, l_u)
    ref, ref_lse = oracle.attn_dense(q, k, v)
    _compare(out.reshape(B * H, -1), lse.reshape(-1), ref, ref_lse, "f16", f"fused D={D} P={P} Nkv={Nkv}")


def test_decode_fused_empty_and_masked(sa):
    """Fused decode with more partitions than keys, and with a byte mask that hides every key of
    one row-head's query (output 0, lse -inf), and with a few queries per head (Nq = 3)."""
    rng = si.rng_for(89, 0)
    q, k, v = (si.cast(x, "bf16") for x in si.draw_qkv(rng, (2, 1, 3, 128), (2, 17, 3, 128)))
    out, lse, _, _ = sa.splitk_fused(q.to(DEV), k.to(DEV), v.to(DEV), 37)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.attn_dense(q, k, v)
    _compare(out.reshape(6, -1), lse.reshape(-1), ref, ref_lse, "bf16", "fused P>Nkv")
    Nq, Nkv = 3, 500
    q, k, v = (si.cast(x, "bf16") for x in si.draw_qkv(rng, (1, Nq, 4, 64), (1, Nkv, 4, 64)))
    mask, _ = si.bernoulli_mask(rng, Nq, Nkv, 0)
    mask[1, :] = 0
    out, lse, _, _ = sa.splitk_fused(q.to(DEV), k.to(DEV), v.to(DEV), 6, mask=torch.from_numpy(mask).to(DEV))
    torch.cuda.synchronize()
    ref, ref_lse = oracle.attn_dense(q, k, v, mask=mask)
    _compare(out.reshape(Nq * 4, -1), lse.reshape(-1), ref, ref_lse, "bf16", "fused masked Nq=3")
    assert bool((out[0, 1] == 0).all()) and bool(torch.isneginf(lse[0, 1]).all())


@pytest.mark.parametrize("P,D", [(1, 64), (200, 128), (256, 16)])
def test_decode_fused_partition_extremes(sa, P, D):
    """Fused decode at one partition (the merge is the identity) and at up to 256 partitions
    (four per lane of the merging wave), with causal square shapes (Nq = Nkv = 3) too."""
    rng = si.rng_for(92, P)
    q, k, v = (si.cast(x, "bf16") for x in si.draw_qkv(rng, (2, 1, 4, D), (2, 3000, 4, D)))
    out, lse, _, _ = sa.splitk_fused(q.to(DEV), k.to(DEV), v.to(DEV), P)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.attn_dense(q, k, v)
    _compare(out.reshape(8, -1), lse.reshape(-1), ref, ref_lse, "bf16", f"fused P={P} D={D}")
    q, k, v = (si.cast(x, "f16") for x in si.draw_qkv(rng, (1, 3, 2, D), (1, 3, 2, D)))
    out, lse, _, _ = sa.splitk_fused(q.to(DEV), k.to(DEV), v.to(DEV), min(P, 5), causal=True)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.attn_dense(q, k, v, causal=True)
    _compare(out.reshape(6, -1), lse.reshape(-1), ref, ref_lse, "f16", f"fused causal P={min(P, 5)}")


def _weighted_abs_v(q, k, v, causal):
    """E[rh, d] = sum_j (w_j / L) |v_jd| with the exact weights w_j = exp(s_j - M) of each row
    (float64, numpy; the sensitivity of O to relative perturbations of the weights)."""
    qd, kd, vd = (t.double().numpy() for t in (q, k, v))
    B, N, H, D = qd.shape
    E = np.zeros((B, N, H, D))
    for b in range(B):
        for h in range(H):
            s = qd[b, :, h, :] @ kd[b, :, h, :].T / np.sqrt(D)
            if causal:
                s = np.where(np.tri(N, dtype=bool), s, -np.inf)
            w = np.exp(s - s.max(axis=1, keepdims=True))
            E[b, :, h, :] = (w / w.sum(axis=1, keepdims=True)) @ np.abs(vd[b, :, h, :])
    return E.reshape(B * N * H, D)


@pytest.mark.parametrize("P", [1, 3, 7])
def test_square_causal_split_matches_unsplit(sa, P):
    """Square causal shapes through the matrix-core split path, split (P partitions merged in
    FP32) against unsplit (one partition, FP32 workspace: no output rounding on either side).
    Each side rounds every weight p_j to bf16 before the P.V product against its own reference
    maximum (relative error <= u = 2^-8, 8 significand bits) while l sums the unrounded weights,
    so O_x - O = sum_j (p_j / l) d_j v_j with |d_j| <= u, and per element
        |O_split - O_unsplit| <= 2 u E[rh, d] + 2^-14 E[rh, d] + 1e-6,
    E = sum_j (w_j / L) |v_jd| (exact weights; 2^-14 E covers FP32 accumulation and the merge's
    exponentials).  Here |O| reaches ~3 (rows with few keys), so the benchmark spec's 1e-3 applies to
    the decode workload (|O| ~ 1e-2), where it is checked directly.  Both sides and attn_fwd are
    also compared with the oracle."""
    rng = si.rng_for(86, P)
    N, D = 1000, 64
    q, k, v = (si.cast(x, "bf16") for x in si.draw_qkv(rng, (2, N, 4, D), (2, N, 4, D)))
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    o_p, l_p, _, _ = sa.splitk(qd, kd, vd, P, causal=True, combine=False)
    out32, lse32 = sa.combine(o_p, l_p, torch.float32)
    o1, l1, _, _ = sa.splitk(qd, kd, vd, 1, causal=True, combine=False)
    out, lse = sa.fwd(qd, kd, vd, causal=True)
    torch.cuda.synchronize()
    o_split = out32.reshape(-1, D).cpu().numpy().astype(np.float64)
    o_unsplit = o1.reshape(-1, D).cpu().numpy().astype(np.float64)
    E = _weighted_abs_v(q, k, v, causal=True)
    bound = (2 * 2.0 ** -8 + 2.0 ** -14) * E + 1e-6
    d = np.abs(o_split - o_unsplit)
    ratio = float((d / bound).max())
    assert ratio <= 1.0, f"split vs unsplit {d.max():.3e}; worst element at {ratio:.2f} of its bound"
    if P == 1:
        assert d.max() == 0.0, "one partition is the unsplit computation"
    _report(f"square_causal_split_vs_unsplit_P{P}", max_abs_diff=float(d.max()), worst_fraction_of_bound=ratio,
            median_bound=float(np.median(bound)))
    lse_split = lse32.reshape(-1).cpu().numpy().astype(np.float64)
    lse_unsplit = l1.reshape(-1).cpu().numpy().astype(np.float64) * math.log(2.0)
    np.testing.assert_allclose(lse_split, lse_unsplit, rtol=1e-5, atol=1e-4)
    ref, ref_lse = oracle.attn_dense(q, k, v, causal=True)
    _compare(out32.reshape(-1, D), lse32.reshape(-1), ref, ref_lse, "bf16", f"split P={P}")
    _compare(out.reshape(-1, D), lse.reshape(-1), ref, ref_lse, "bf16", "unsplit")


# ---------------------------------------------------------------------------------------------
# masked long context B1 H16 N16384 D256: causal AND Bernoulli(0.5) mask, 1/64 rows all-masked
# ---------------------------------------------------------------------------------------------
def test_masked_long_context_full_size(sa):
    s = si.MASKED
    q, k, v, mask, cleared = si.masked_inputs()
    qd, kd, vd, md = q.to(DEV), k.to(DEV), v.to(DEV), torch.from_numpy(mask).to(DEV)
    out, lse = sa.fwd(qd, kd, vd, causal=True, mask=md)
    torch.cuda.synchronize()
    N, H = s["N"], s["H"]
    assert not torch.isnan(out).any()
    # every all-masked row (the cleared ones and any naturally empty causal prefix row)
    vis_any = np.zeros(N, bool)
    tri_rows = np.nonzero(mask.any(axis=1))[0]
    for i in tri_rows:
        vis_any[i] = mask[i, : i + 1].any()
    empty = np.nonzero(~vis_any)[0]
    assert set(cleared.tolist()) <= set(empty.tolist())
    o = out.reshape(N, H, -1)[torch.from_numpy(empty).to(DEV)]
    l = lse.reshape(N, H)[torch.from_numpy(empty).to(DEV)]
    assert bool((o == 0).all()) and bool((l == -math.inf).all())
    assert bool(torch.isfinite(lse.reshape(N, H)[torch.from_numpy(np.nonzero(vis_any)[0]).to(DEV)]).all())
    _full_compare(out, lse, q, k, v, "bf16", "masked_B1H16N16384D256_causal_and_mask_all_rows", causal=True,
                  mask=mask, chunk=1 << 15)


def test_long_sequence_mask_past_32_bit_offsets(sa):
    """N = 65536: a 4 GiB mask (row offsets beyond 2^32, so read from global memory with 64-bit
    offsets) ANDed with causal; sampled rows, the first and the last among them, against the
    oracle.  The mask is a fixed pattern (visible unless (i + 3 j) % 7 == 0, every 5000th row
    fully masked) so that building it stays cheap."""
    N, D = 65536, 64
    rng = si.rng_for(90, 0)
    q, k, v = (si.cast(x, "bf16") for x in si.draw_qkv(rng, (1, N, 1, D), (1, N, 1, D)))
    j3 = (3 * np.arange(N, dtype=np.int64)) % 7
    pattern = np.stack([((r + j3) % 7 != 0) for r in range(7)]).astype(np.uint8)   # row i uses i % 7
    mask = np.empty((N, N), np.uint8)
    for r0 in range(0, N, 4096):
        mask[r0:r0 + 4096] = pattern[np.arange(r0, r0 + 4096) % 7]
    mask[::5000] = 0
    md = torch.from_numpy(mask).to(DEV)
    out, lse = sa.fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal=True, mask=md)
    torch.cuda.synchronize()
    del md
    rows = np.unique(np.concatenate([si.rng_for(90, 1).integers(0, N, 48), [0, 1, 5000, 40000, N - 1]]))
    ref, ref_lse = oracle.attn_dense(q, k, v, causal=True, mask=mask, rows=rows)
    rt = torch.from_numpy(rows).to(DEV)
    _compare(out.reshape(-1, D)[rt], lse.reshape(-1)[rt], ref, ref_lse, "bf16", "N=65536 masked")


@pytest.mark.parametrize("D,BN", [(16, 32), (64, 64), (128, 64), (256, 64)])
def test_mask_ragged_small(sa, D, BN):
    """Arbitrary masks with ragged N (odd lengths, unaligned mask rows) against the oracle."""
    rng = si.rng_for(88, D)
    N = 203
    q, k, v = (si.cast(x, "f16") for x in si.draw_qkv(rng, (1, N, 2, D), (1, N, 2, D)))
    mask, _ = si.bernoulli_mask(rng, N, N, 3)
    for causal in (False, True):
        out, lse = sa.fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal, mask=torch.from_numpy(mask).to(DEV), block_n=BN)
        ref, ref_lse = oracle.attn_dense(q, k, v, causal=causal, mask=mask)
        _compare(out.reshape(-1, D), lse.reshape(-1), ref, ref_lse, "f16", f"mask D={D} causal={causal}")


@pytest.mark.parametrize("D,BN", [(16, 32), (32, 64), (64, 32), (64, 64), (128, 64), (256, 64)])
def test_mask_staged_matches_direct(sa, D, BN):
    """Mask tiles staged through LDS (rows 16-byte aligned) give bitwise the results of the mask
    read straight from global memory (the same bytes 8 bytes off alignment), for attn_fwd and the
    split producer, and match the oracle; N = 400 leaves a ragged last key tile and a partial
    query block."""
    rng = si.rng_for(89, D + BN)
    N, H = 400, 2
    q, k, v = (si.cast(x, "bf16") for x in si.draw_qkv(rng, (1, N, H, D), (1, N, H, D)))
    mask, _ = si.bernoulli_mask(rng, N, N, 4)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    m16 = torch.from_numpy(mask).to(DEV)
    buf = torch.zeros(N * N + 8, dtype=torch.uint8, device=DEV)
    m8 = buf[8:].view(N, N)
    m8.copy_(m16)
    assert m16.data_ptr() % 16 == 0 and m8.data_ptr() % 16 == 8
    for causal in (False, True):
        o1, l1 = sa.fwd(qd, kd, vd, causal=causal, mask=m16, block_n=BN)
        o2, l2 = sa.fwd(qd, kd, vd, causal=causal, mask=m8, block_n=BN)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2), f"staged != direct (causal={causal})"
        ref, ref_lse = oracle.attn_dense(q, k, v, causal=causal, mask=mask)
        _compare(o1.reshape(-1, D), l1.reshape(-1), ref, ref_lse, "bf16", f"staged mask D={D} causal={causal}")
    if BN == 64:
        # five partitions of 80 keys (a multiple of 16: staged) against the same unaligned
        p1 = sa.splitk(qd, kd, vd, 5, causal=True, mask=m16, combine=False)
        p2 = sa.splitk(qd, kd, vd, 5, causal=True, mask=m8, combine=False)
        torch.cuda.synchronize()
        assert torch.equal(p1[0], p2[0]) and torch.equal(p1[1], p2[1]), "split: staged != direct"
        ref_op, ref_lp = oracle.splitk(q, k, v, 5, causal=True, mask=mask)
        for pp in range(5):
            _compare(p1[0][pp].reshape(-1, D), None, ref_op[pp], ref_lp[pp], "bf16", f"staged mask o_partial p={pp}")
            lp = p1[1][pp].reshape(-1).cpu().numpy().astype(np.float64)
            fin = np.isfinite(ref_lp[pp])
            assert np.all(lp[~fin] == -np.inf)
            np.testing.assert_allclose(lp[fin], ref_lp[pp][fin], rtol=1e-4, atol=1e-4)


# ---------------------------------------------------------------------------------------------
# the combine on its own: static-P and runtime-P instantiations, every output dtype
# ---------------------------------------------------------------------------------------------
@pytest.mark.parametrize("P", [1, 2, 4, 8, 16, 37, 64, 65, 200, 256])
@pytest.mark.parametrize("depth", [16, 64, 128, 256])
def test_combine_against_oracle(sa, P, depth):
    rng = np.random.default_rng(P * 1000 + depth)
    rows, heads = 5, 3
    o_p = rng.standard_normal((P, rows, heads, depth)).astype(np.float32)
    l_p = (rng.standard_normal((P, rows, heads)) * 4).astype(np.float32)
    l_p[rng.random((P, rows, heads)) < 0.2] = -np.inf
    l_p[:, 0, 0] = -np.inf                           # one row-head with every partition empty
    o_p[l_p == -np.inf] = 0.0
    ref, G = oracle.combine_log2(o_p.reshape(P, rows * heads, depth).astype(np.float64),
                                 l_p.reshape(P, -1).astype(np.float64))
    for out_dtype, tol in ((torch.float32, 1e-5), (torch.bfloat16, 2e-2), (torch.float16, 5e-3)):
        out, lse = sa.combine(torch.from_numpy(o_p).to(DEV), torch.from_numpy(l_p).to(DEV), out_dtype)
        o = out.float().cpu().numpy().reshape(rows * heads, depth)
        err = np.abs(o - ref).max()
        assert err <= tol * max(1.0, np.abs(ref).max()), (out_dtype, err)
        l = lse.cpu().numpy().reshape(-1).astype(np.float64)
        fin = np.isfinite(G)
        assert np.all(l[~fin] == -np.inf) and np.all(o[~fin] == 0)
        np.testing.assert_allclose(l[fin], G[fin] * math.log(2.0), rtol=1e-5, atol=1e-5)


# ---------------------------------------------------------------------------------------------
# reject paths with real buffers: nothing is written
# ---------------------------------------------------------------------------------------------
def test_reject_paths_write_nothing(sa):
    q = torch.randn(1, 64, 2, 64, device=DEV).to(torch.bfloat16)
    out = torch.full_like(q, 7.0)
    o_p = torch.full((4, 64, 2, 64), 7.0, device=DEV)
    l_p = torch.full((4, 64, 2), 7.0, device=DEV)
    with pytest.raises(sa.AttnError):
        sa.attn_fwd_splitk(q, q[:, :32], q[:, :32], 4, o_p, l_p, causal=True)   # rectangular causal
    with pytest.raises(sa.AttnError):
        sa.attn_fwd_splitk(q, q, q, 0, o_p, l_p)
    with pytest.raises(sa.AttnError):
        sa.attn_fwd(q, q, q, out, block_n=48)
    q48 = torch.zeros(1, 64, 2, 48, device=DEV, dtype=torch.bfloat16)
    with pytest.raises(sa.AttnError):
        sa.attn_fwd(q48, q48, q48, torch.zeros_like(q48))
    q1 = q[:, :1]
    with pytest.raises(sa.AttnError) as e:   # tickets are required
        sa.attn_fwd_splitk_fused(q1, q, q, 4, o_p, l_p, None, torch.zeros_like(q1))
    assert e.value.code == 5
    torch.cuda.synchronize()
    assert bool((out == 7.0).all()) and bool((o_p == 7.0).all()) and bool((l_p == 7.0).all())
