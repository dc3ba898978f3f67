"""Pins of the FP64 oracle to facts fixed outside the oracle itself.

Each test names the passage or the mathematical fact it checks.  The pins are chosen so that a
plausible slip in the oracle (a dropped rescale, exp instead of exp2, a wrong index or a
transposed operand, a missing mask guard) fails at least one of them.  CPU only.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import seeded_inputs as si

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _num(x):
    return math.log(2.0) if x == "ln2" else float(x)


# ------------------------------------------------------------------------------------------
# Worked examples printed on the pages
# ------------------------------------------------------------------------------------------
def test_worked_trace_gives_six():
    """Workshop page, 'Trace one query before writing the kernel': (m,l,a) after each tile,
    output 6, LSE = ln 4 (the total of the weights 1 + 1 + 2)."""
    g = _golden("worked_trace.json")
    s = [_num(x) for tile in g["logits"] for x in tile]
    v = [x for tile in g["values"] for x in tile]
    out, lse, trace = oracle.online_from_logits(s, v, BN=2)
    t1, t2 = g["after_tile_1"], g["after_tile_2"]
    assert trace[0][0] == t1["m"] and trace[0][1] == t1["l"] and trace[0][2] == t1["a"]
    assert trace[1][0] == pytest.approx(_num(t2["m"]), abs=0, rel=1e-15)
    assert trace[1][3] == pytest.approx(t2["alpha"], rel=1e-15)
    assert trace[1][1] == pytest.approx(t2["l"], rel=1e-15)
    assert trace[1][2] == pytest.approx(t2["a"], rel=1e-15)
    assert out[0] == pytest.approx(g["output"], rel=1e-15)
    assert lse == pytest.approx(math.log(4.0), rel=1e-15)


def test_worked_trace_bug_gives_seven():
    """Same passage: rescaling l but not the numerator gives 7 -- the switch must reproduce it,
    which shows the numerator rescale is load-bearing in the oracle's recurrence."""
    g = _golden("worked_trace.json")
    s = [_num(x) for tile in g["logits"] for x in tile]
    v = [x for tile in g["values"] for x in tile]
    out, _, _ = oracle.online_from_logits(s, v, BN=2, no_numerator_rescale=True)
    assert out[0] == pytest.approx(g["output_without_numerator_rescale"], rel=1e-15)


def test_worked_trace_dense_and_weights():
    """Same passage: softmax over all three logits at once weighs the keys 1/4, 1/4 and 1/2, and
    the weighted value is again 6.  The dense
    definition is fed D=1, q=1, k = logits so that q.k/sqrt(1) reproduces the logits; the
    weights are read out by giving V the identity rows."""
    g = _golden("worked_trace.json")
    s = np.array([_num(x) for tile in g["logits"] for x in tile], np.float32)
    q = np.ones((1, 1, 1, 1), np.float32)
    k = s.reshape(1, 3, 1, 1)
    v = np.array([x for tile in g["values"] for x in tile], np.float32).reshape(1, 3, 1, 1)
    # q must have Nq rows; broadcast the single query over a 1-row problem with Nkv = 3
    out, lse = oracle.attn_dense(q, k, v)
    assert out[0, 0] == pytest.approx(6.0, rel=1e-7)  # ln 2 rounded to float32
    # weights through an identity V with D = 3 (q, k padded with zero columns)
    q3 = np.zeros((1, 1, 1, 3), np.float32); q3[..., 0] = 1.0
    k3 = np.zeros((1, 3, 1, 3), np.float32); k3[0, :, 0, 0] = s * np.float32(math.sqrt(3.0))
    v3 = np.eye(3, dtype=np.float32).reshape(1, 3, 1, 3)
    w, _ = oracle.attn_dense(q3, k3, v3)
    np.testing.assert_allclose(w[0], g["full_softmax_weights"], rtol=1e-6)


def test_softmax_state_example():
    """Tylo 'Streaming attention and online state', Online statistics: from the empty state,
    an update with scores (0, 0) gives max 0, sum 2, rescale 0, normalised weights (0.5, 0.5)."""
    g = _golden("softmax_state_example.json")
    out, lse, trace = oracle.online_from_logits(g["scores"], np.eye(2), BN=2)
    m, l, _, alpha = trace[0]
    assert m == g["state_max"] and l == g["state_sum"] and alpha == g["rescale"]
    assert list(out) == g["normalized_weights"]
    assert lse == pytest.approx(math.log(2.0), rel=1e-15)


# ------------------------------------------------------------------------------------------
# Merge and split-K combine
# ------------------------------------------------------------------------------------------
def test_log2_combine_of_the_trace():
    """fa4_splitk_combine formulas on the worked trace split as A = {key 0}, B = {keys 1, 2}:
    o_partial = [1, 23/3], lse2 = [0, log2 3] must give 6 with G = 2.  A combine that mixed
    in the natural exponential would give about 6.5327 here (computed below), so this pin
    separates the two bases; equal LSEs (the tile-boundary split) could not."""
    o_p = np.array([[[1.0]], [[23.0 / 3.0]]])
    l_p = np.array([[0.0], [math.log2(3.0)]])
    out, G = oracle.combine_log2(o_p, l_p)
    assert out[0, 0] == pytest.approx(6.0, rel=1e-14)
    assert G[0] == pytest.approx(2.0, rel=1e-15)
    # the mixed-base mistake, written out, lands far from 6
    ms = max(l_p[:, 0])
    Gn = math.log(sum(math.exp(x - ms) for x in l_p[:, 0])) + ms
    wrong = sum(math.exp(l_p[p, 0] - Gn) * o_p[p, 0, 0] for p in range(2))
    assert wrong == pytest.approx(6.5327, abs=1e-4)
    # tile-boundary split: o = [2, 10], lse2 = [1, 1]
    out2, G2 = oracle.combine_log2(np.array([[[2.0]], [[10.0]]]), np.array([[1.0], [1.0]]))
    assert out2[0, 0] == pytest.approx(6.0, rel=1e-15) and G2[0] == pytest.approx(2.0, rel=1e-15)


def test_merge_nat_of_the_trace():
    """Tylo softmax_merge: summaries A = (0, 1, 1) and B = (ln 2, 1.5, 11.5) of the trace merge
    to (ln 2, 2, 12) with rescale factors (1/2, 1), i.e. output 6."""
    m, l, a, al1, al2 = oracle.merge_nat(0.0, 1.0, [1.0], math.log(2.0), 1.5, [11.5])
    assert m == pytest.approx(math.log(2.0), rel=1e-15)
    assert (al1, al2) == (pytest.approx(0.5, rel=1e-15), 1.0)
    assert l == pytest.approx(2.0, rel=1e-15) and a[0] == pytest.approx(12.0, rel=1e-15)
    # two empty summaries stay empty, with no NaN
    m, l, a, al1, al2 = oracle.merge_nat(-math.inf, 0.0, [0.0], -math.inf, 0.0, [0.0])
    assert m == -math.inf and l == 0.0 and a[0] == 0.0 and al1 == 0.0 and al2 == 0.0


def test_combine_special_cases():
    rng = np.random.default_rng(7)
    o = rng.standard_normal((1, 5, 8))
    lse = rng.standard_normal((1, 5))
    out, G = oracle.combine_log2(o, lse)           # P = 1: identity, scale exactly 1
    np.testing.assert_allclose(out, o[0], rtol=1e-15)
    np.testing.assert_allclose(G, lse[0], rtol=1e-15)
    o = rng.standard_normal((4, 3, 8))             # equal LSEs: plain mean
    out, G = oracle.combine_log2(o, np.full((4, 3), 1.25))
    np.testing.assert_allclose(out, o.mean(axis=0), rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(G, 1.25 + 2.0, rtol=1e-15)
    o = np.zeros((3, 2, 4))                        # all empty: 0 and -inf
    out, G = oracle.combine_log2(o, np.full((3, 2), -np.inf))
    assert np.all(out == 0) and np.all(G == -np.inf)
    o = rng.standard_normal((3, 2, 4))             # one empty partition contributes nothing
    o[1] = 0.0
    l = rng.standard_normal((3, 2)); l[1] = -np.inf
    out, _ = oracle.combine_log2(o, l)
    out2, _ = oracle.combine_log2(o[[0, 2]], l[[0, 2]])
    np.testing.assert_allclose(out, out2, rtol=1e-14)


def test_natural_merge_equals_log2_combine():
    """Tylo's natural-base merge and the base-2 combine are the same operator: random
    summaries (m, l, a) merged pairwise must equal the combine of (a/l, (m + ln l)/ln 2)."""
    rng = np.random.default_rng(11)
    for _ in range(20):
        m = rng.standard_normal(2) * 5
        l = rng.uniform(0.5, 40, 2)
        a = rng.standard_normal((2, 6)) * 3
        mm, ll, aa, _, _ = oracle.merge_nat(m[0], l[0], a[0], m[1], l[1], a[1])
        o_p = (a / l[:, None])[:, None, :]
        lse2 = ((m + np.log(l)) / math.log(2.0))[:, None]
        out, G = oracle.combine_log2(o_p, lse2)
        np.testing.assert_allclose(out[0], aa / ll, rtol=1e-12, atol=1e-14)
        assert G[0] * math.log(2.0) == pytest.approx(mm + math.log(ll), rel=1e-12, abs=1e-12)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("P", [1, 3, 4, 8, 37])
def test_splitk_then_combine_equals_dense(P, causal):
    """Split-K workspace + base-2 combine reproduce the dense definition, including empty
    partitions (P > keys per row and causal rows whose later partitions lie in the future)."""
    rng = si.rng_for(90, P)
    B, N, H, D = 2, 29, 3, 16
    q, k, v = si.draw_qkv(rng, (B, N, H, D), (B, N, H, D))
    q, k, v = si.cast(q, "bf16"), si.cast(k, "bf16"), si.cast(v, "bf16")
    ref, ref_lse = oracle.attn_dense(q, k, v, causal=causal)
    o_p, l_p = oracle.splitk(q, k, v, P, causal=causal)
    assert not np.isnan(o_p).any()
    empty = l_p == -np.inf
    assert np.all(o_p[empty] == 0.0)
    if P == 37:
        assert empty.any()
    out, G = oracle.combine_log2(o_p, l_p)
    np.testing.assert_allclose(out, ref, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(G * math.log(2.0), ref_lse, rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------------------------------------
# Chunking invariance and the dense definition against library routines
# ------------------------------------------------------------------------------------------
def _numpy_attention(q, k, v, causal=False, mask=None):
    """The definition through numpy library calls (einsum, max, exp, sum) in float64: a second,
    independent spelling used only to pin the C dense oracle on small shapes."""
    q = q.double().numpy() if isinstance(q, torch.Tensor) else q.astype(np.float64)
    k = k.double().numpy() if isinstance(k, torch.Tensor) else k.astype(np.float64)
    v = v.double().numpy() if isinstance(v, torch.Tensor) else v.astype(np.float64)
    B, Nq, H, D = q.shape
    Nkv = k.shape[1]
    s = np.einsum("bihd,bjhd->bhij", q, k) / np.sqrt(D)
    vis = np.ones((Nq, Nkv), bool)
    if causal:
        vis &= np.tril(np.ones((Nq, Nkv), bool))
    if mask is not None:
        vis &= mask.astype(bool)
    s = np.where(vis[None, None], s, -np.inf)
    rowmax = s.max(axis=-1, keepdims=True)
    empty = ~vis.any(axis=-1)                                   # [Nq]
    rowmax = np.where(np.isinf(rowmax), 0.0, rowmax)
    w = np.exp(s - rowmax)
    L = w.sum(axis=-1, keepdims=True)
    o = np.einsum("bhij,bjhd->bihd", w, v) / np.where(L == 0, 1.0, L).transpose(0, 2, 1, 3)
    lse = (np.log(np.where(L == 0, 1.0, L)) + rowmax)[..., 0].transpose(0, 2, 1)  # [B, Nq, H]
    o[:, empty] = 0.0
    lse[:, empty] = -np.inf
    return o.reshape(-1, D), lse.reshape(-1)


@pytest.mark.parametrize("causal", [False, True])
def test_dense_matches_numpy_expression(causal):
    """Non-square B, H, D and distinct sizes catch a transposed operand or a wrong stride."""
    rng = si.rng_for(91, int(causal))
    B, N, H, D = 2, 7, 3, 5
    q, k, v = si.draw_qkv(rng, (B, N, H, D), (B, N, H, D))
    ref, ref_lse = _numpy_attention(q, k, v, causal=causal)
    out, lse = oracle.attn_dense(q, k, v, causal=causal)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-12, atol=1e-14)


def test_dense_rectangular_and_row_selection():
    rng = si.rng_for(92, 0)
    B, Nq, Nkv, H, D = 2, 3, 11, 2, 8
    q, k, v = si.draw_qkv(rng, (B, Nq, H, D), (B, Nkv, H, D))
    ref, ref_lse = _numpy_attention(q, k, v)
    rows = np.array([5, 0, 11, 7])
    out, lse = oracle.attn_dense(q, k, v, rows=rows)
    np.testing.assert_allclose(out, ref[rows], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse, ref_lse[rows], rtol=1e-12)


def test_every_mask_row_pattern_brute_force():
    """Tylo 'Attention as a consumer': an arbitrary Boolean M x N mask.  Every one of the 2^6
    row patterns over 6 keys (including all-masked) is one query row; the C oracle must match a
    pure-Python brute force, with all-masked rows giving exactly 0 and -inf."""
    Nkv, D = 6, 3
    patterns = np.array(list(itertools.product([0, 1], repeat=Nkv)), np.uint8)   # [64, 6]
    Nq = patterns.shape[0]
    rng = si.rng_for(93, 0)
    q, k, v = si.draw_qkv(rng, (1, Nq, 1, D), (1, Nkv, 1, D))
    out, lse = oracle.attn_dense(q, k, v, mask=patterns)
    for i in range(Nq):
        vis = [j for j in range(Nkv) if patterns[i, j]]
        if not vis:
            assert np.all(out[i] == 0.0) and lse[i] == -np.inf
            continue
        s = {j: sum(float(q[0, i, 0, d]) * float(k[0, j, 0, d]) for d in range(D)) / math.sqrt(D) for j in vis}
        M = max(s.values())
        w = {j: math.exp(s[j] - M) for j in vis}
        L = sum(w.values())
        for d in range(D):
            assert out[i, d] == pytest.approx(sum(w[j] * float(v[0, j, 0, d]) for j in vis) / L, rel=1e-12, abs=1e-14)
        assert lse[i] == pytest.approx(M + math.log(L), rel=1e-12, abs=1e-14)


@pytest.mark.parametrize("BN", [1, 2, 32, 64, 64 * 1024])
def test_chunking_does_not_change_the_result_small(BN):
    """Tylo Online statistics: chunked summaries equal the full softmax up to rounding order;
    the recurrence at any tile width reproduces the dense definition (FP64, 1e-12)."""
    q, k, v = si.small_inputs()
    ref, ref_lse = oracle.attn_dense(q, k, v)
    out, lse = oracle.attn_online(q, k, v, BN)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("case_idx", list(range(0, 360, 7)))
def test_chunking_on_the_sweep(case_idx):
    case = si.sweep_cases()[case_idx]
    q, k, v = si.sweep_inputs(case)
    N = case["N"]
    rows = np.unique(np.linspace(0, N - 1, min(N, 24)).astype(np.int64))
    ref, ref_lse = oracle.attn_dense(q, k, v, causal=case["causal"], rows=rows)
    out, lse = oracle.attn_online(q, k, v, case["BN"], causal=case["causal"], rows=rows)
    np.testing.assert_allclose(out, ref, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------------------------------------
# Closed forms and special cases
# ------------------------------------------------------------------------------------------
@pytest.mark.parametrize("causal", [False, True])
def test_uniform_logits_closed_form(causal):
    """Q = 0: every visible key has weight 1/|vis|, so O_i is the mean of the visible V rows
    (a prefix mean under causal) and LSE_i = ln |vis(i)|."""
    case = dict(N=1000, D=32, dtype="bf16", causal=causal, BN=64, variant="uniform")
    q, k, v = si.sweep_inputs(case)
    out, lse = oracle.attn_dense(q, k, v, causal=causal)
    vv = v.double().numpy()[0, :, 0, :]
    if causal:
        ref = np.cumsum(vv, axis=0) / np.arange(1, 1001)[:, None]
        ref_lse = np.log(np.arange(1, 1001))
    else:
        ref = np.broadcast_to(vv.mean(axis=0), (1000, 32))
        ref_lse = np.full(1000, math.log(1000))
    np.testing.assert_allclose(out, ref, rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-14)


def test_single_element_closed_form():
    """N = 1: the only key has weight 1, O = v0 and LSE = q.k / sqrt(D)."""
    for D in (16, 32, 64):
        case = dict(N=1, D=D, dtype="f16", causal=True, BN=32, variant="normal")
        q, k, v = si.sweep_inputs(case)
        out, lse = oracle.attn_dense(q, k, v, causal=True)
        np.testing.assert_array_equal(out[0], v.double().numpy().reshape(-1))
        ref = float(np.dot(q.double().numpy().reshape(-1), k.double().numpy().reshape(-1))) / math.sqrt(D)
        assert lse[0] == pytest.approx(ref, rel=1e-14, abs=1e-15)


def test_large_logits_match_library_expression():
    """Q x 30 (logit spread ~30): exp without the max shift overflows in float32 but the oracle
    must still equal the definition; compared with the numpy spelling."""
    case = dict(N=17, D=64, dtype="bf16", causal=True, BN=32, variant="large")
    q, k, v = si.sweep_inputs(case)
    ref, ref_lse = _numpy_attention(q, k, v, causal=True)
    out, lse = oracle.attn_dense(q, k, v, causal=True)
    assert np.abs(lse).max() > 88.8   # past the float32 exp overflow point
    np.testing.assert_allclose(out, ref, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-13)


def test_future_v_perturbation_leaves_causal_rows_unchanged():
    """Workshop page, checker: changing V (and K) rows after i0 must leave causal rows <= i0
    bitwise unchanged and must change later rows."""
    case = dict(N=1000, D=64, dtype="bf16", causal=True, BN=64, variant="normal")
    q, k, v = si.sweep_inputs(case)
    i0 = 400
    out1, lse1 = oracle.attn_dense(q, k, v, causal=True)
    rng = si.rng_for(94, 0)
    k2, v2 = k.clone(), v.clone()
    fresh_k, fresh_v = si.draw_qkv(rng, (1, 1000 - i0 - 1, 1, 64), (1, 1000 - i0 - 1, 1, 64))[1:]
    k2[:, i0 + 1:] = si.cast(fresh_k, "bf16")
    v2[:, i0 + 1:] = si.cast(fresh_v, "bf16")
    out2, lse2 = oracle.attn_dense(q, k2, v2, causal=True)
    np.testing.assert_array_equal(out1[: i0 + 1], out2[: i0 + 1])
    np.testing.assert_array_equal(lse1[: i0 + 1], lse2[: i0 + 1])
    assert np.all(np.any(out1[i0 + 1:] != out2[i0 + 1:], axis=1))


def test_fully_masked_rows_give_zero_and_minus_inf():
    """Tylo Online statistics and Worked softmax: an all-masked row has output 0 and LSE -inf,
    in the dense definition and in the recurrence, with no NaN."""
    rng = si.rng_for(95, 0)
    N, D = 40, 16
    q, k, v = si.draw_qkv(rng, (1, N, 2, D), (1, N, 2, D))
    mask, rows = si.bernoulli_mask(rng, N, N, 5)
    out, lse = oracle.attn_dense(q, k, v, causal=True, mask=mask)
    on, ln = oracle.attn_online(q, k, v, 8, causal=True, mask=mask)
    vis = (np.tril(np.ones((N, N), bool)) & mask.astype(bool)).any(axis=1)
    assert not vis[rows].any()
    for o, l in ((out, lse), (on, ln)):
        o = o.reshape(N, 2, D)
        l = l.reshape(N, 2)
        assert not np.isnan(o).any()
        assert np.all(o[~vis] == 0.0) and np.all(l[~vis] == -np.inf)
        assert np.all(np.isfinite(l[vis]))


def test_same_boundary_mode_stays_close():
    """Rounding p to bf16 before p.v (l unrounded) moves the output by at most u * max|v|
    relative to the exact definition, with u the unit roundoff of round-to-nearest-even: 2^-8 for
    bf16 (8 significand bits), 2^-11 for fp16 (11); and the rounding does move it."""
    q, k, v = si.small_inputs()
    ref, _ = oracle.attn_dense(q, k, v)
    vmax = float(np.abs(v).max())
    for mode, bound in (("bf16", 2.0 ** -8), ("f16", 2.0 ** -11)):
        out, _ = oracle.attn_online(q, k, v, 32, same_boundary=mode)
        err = np.abs(out - ref).max()
        assert 0 < err <= bound * vmax


# ------------------------------------------------------------------------------------------
# Conversion (O4) and decoding against torch's library conversions
# ------------------------------------------------------------------------------------------
def test_pack_word_example():
    """Tylo 'Register fragments and logical axes': packing (1, -2) as Float16 gives the word
    0xc0003c00 with the lowest element in the low half; the bf16 analogue is 0xc0003f80."""
    g = _golden("pack_word.json")
    for fmt, key in (("f16", "f16_word"), ("bf16", "bf16_word_derived")):
        bits = oracle.round_bits(np.array(g["values"], np.float32), fmt).astype(np.uint32)
        assert int(bits[0] | (bits[1] << 16)) == int(g[key], 16)


def _torch_bits(x, fmt):
    t = torch.from_numpy(x).to(torch.bfloat16 if fmt == "bf16" else torch.float16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _compare_rounding(x, fmt):
    got = oracle.round_bits(x, fmt)
    ref = _torch_bits(x, fmt)
    nan = np.isnan(x)
    if fmt == "bf16":
        isnan_bits = lambda b: ((b & 0x7F80) == 0x7F80) & ((b & 0x7F) != 0)
    else:
        isnan_bits = lambda b: ((b & 0x7C00) == 0x7C00) & ((b & 0x3FF) != 0)
    assert np.all(isnan_bits(got[nan]))
    bad = np.nonzero(got[~nan] != ref[~nan])[0]
    assert bad.size == 0, (fmt, x[~nan][bad[:5]], got[~nan][bad[:5]], ref[~nan][bad[:5]])


def test_rne_bf16_every_exponent_and_rounding_class():
    """bf16 rounding depends on the high 16 bits and on how the low 16 compare with 0x8000:
    all 65536 high halves x {0, 1, 0x7fff, 0x8000, 0x8001, 0xffff, 3 random} covers every
    exponent, sign, tie (both parities), overflow to inf and subnormal."""
    hi = np.arange(65536, dtype=np.uint32) << 16
    rng = np.random.default_rng(3)
    lows = [0, 1, 0x7FFF, 0x8000, 0x8001, 0xFFFF] + list(rng.integers(0, 65536, 3))
    u = (hi[:, None] | np.array(lows, np.uint32)[None, :]).reshape(-1)
    _compare_rounding(u.view(np.float32), "bf16")


def test_rne_f16_structured_and_random():
    """fp16: every float32 exponent/sign with mantissas at and around each rounding boundary
    (13 dropped bits: ties of both parities), plus 2^22 random patterns."""
    exps = np.arange(256, dtype=np.uint32) << 23
    rng = np.random.default_rng(4)
    kept = rng.integers(0, 1 << 10, 64).astype(np.uint32) << 13
    dropped = np.array([0, 1, 0xFFF, 0x1000, 0x1001, 0x1FFF], np.uint32)
    m = (kept[:, None] | dropped[None, :]).reshape(-1)
    u = (exps[:, None] | m[None, :]).reshape(-1)
    u = np.concatenate([u, u | 0x80000000])
    # subnormal-result range: float32 exponents 100..113 with every low-bit boundary
    sub_e = np.arange(100, 114, dtype=np.uint32) << 23
    sub_m = rng.integers(0, 1 << 23, 4096).astype(np.uint32)
    u = np.concatenate([u, (sub_e[:, None] | sub_m[None, :]).reshape(-1)])
    u = np.concatenate([u, rng.integers(0, 1 << 32, 1 << 22, dtype=np.uint64).astype(np.uint32)])
    specials = np.array([65504.0, 65519.996, 65520.0, 65535.0, 6.1035156e-05, 5.9604645e-08,
                         2.9802322e-08, 2.9802326e-08, -0.0, np.inf, -np.inf], np.float32)
    _compare_rounding(np.concatenate([u.view(np.float32), specials]), "f16")


def test_decode_every_pattern():
    bits = np.arange(65536, dtype=np.uint16)
    for fmt, tdt in (("bf16", torch.bfloat16), ("f16", torch.float16)):
        got = oracle.decode_bits(bits, fmt)
        ref = torch.from_numpy(bits.view(np.int16)).view(tdt).double().numpy()
        nan = np.isnan(ref)
        assert np.array_equal(np.isnan(got), nan)
        np.testing.assert_array_equal(got[~nan], ref[~nan])
        np.testing.assert_array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


# ------------------------------------------------------------------------------------------
# O6: 8-bit floats (Tylo "Register fragments and logical axes", "Logical types and register
# packing": Float8E4M3 / Float8E5M2, nearest even rounding, out-of-range results clamped to the largest finite value)
# ------------------------------------------------------------------------------------------
_TORCH_FP8 = {"e4m3": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}
_FP8_MAX = {"e4m3": 448.0, "e5m2": 57344.0}


def test_fp8_decode_every_code_matches_library():
    """All 256 codes of each format widen exactly as torch's float8 types do."""
    codes = np.arange(256, dtype=np.uint8)
    for fmt, tdt in _TORCH_FP8.items():
        got = oracle.decode_bits(codes, fmt)
        ref = torch.from_numpy(codes).view(tdt).double().numpy()
        nan = np.isnan(ref)
        assert np.array_equal(np.isnan(got), nan)
        np.testing.assert_array_equal(got[~nan], ref[~nan])
        np.testing.assert_array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))
    # format facts: E4M3 has one NaN pattern per sign and no infinities, so its largest finite
    # value is 1.75 * 2^8; E5M2 keeps IEEE infinities
    e4 = oracle.decode_bits(codes, "e4m3")
    assert e4[0x7E] == 448.0 and np.isnan(e4[0x7F]) and np.isnan(e4[0xFF]) and not np.isinf(e4).any()
    assert e4[0x01] == 2.0 ** -9 and e4[0x08] == 2.0 ** -6 and e4[0x38] == 1.0
    e5 = oracle.decode_bits(codes, "e5m2")
    assert e5[0x7B] == 57344.0 and e5[0x7C] == np.inf and e5[0xFC] == -np.inf and e5[0x01] == 2.0 ** -16


def _brute_force_fp8(x, fmt):
    """Nearest finite code by exhaustive search over the decoded table, ties to the code whose
    last fraction bit is 0, then saturation; NaN -> NaN."""
    codes = np.arange(256, dtype=np.uint8)
    vals = oracle.decode_bits(codes, fmt)
    fin = np.isfinite(vals)
    cand, cv = codes[fin], vals[fin]
    out = np.zeros(x.shape, np.float64)
    for i, xv in enumerate(x.astype(np.float64)):
        if np.isnan(xv):
            out[i] = np.nan
            continue
        xc = float(np.clip(xv, -_FP8_MAX[fmt], _FP8_MAX[fmt]))
        d = np.abs(cv - xc)
        best = np.nonzero(d == d.min())[0]
        if best.size > 1:
            best = best[(cand[best] & 1) == 0]
        out[i] = cv[best[0]] if cv[best[0]] != 0 else np.copysign(0.0, xv)   # a zero keeps the sign
    return out


def test_fp8_round_brute_force_nearest():
    """O6 against an exhaustive nearest search: random values over every binade of both formats
    (subnormal range and beyond the largest finite value included), exact ties, signed zero."""
    rng = np.random.default_rng(12)
    for fmt in ("e4m3", "e5m2"):
        vals = oracle.decode_bits(np.arange(256, dtype=np.uint8), fmt)
        fin = np.sort(np.unique(vals[np.isfinite(vals)]))
        mids = (fin[1:] + fin[:-1]) / 2                       # every exact tie (exact in float32)
        x = np.concatenate([
            np.exp2(rng.uniform(-20, 18, 3000)) * rng.choice([-1, 1], 3000),
            mids, np.nextafter(mids.astype(np.float32), np.float32(np.inf)),
            np.nextafter(mids.astype(np.float32), np.float32(-np.inf)),
            [0.0, -0.0, np.inf, -np.inf, np.nan, 1e30, -1e30]]).astype(np.float32)
        got = oracle.decode_bits(oracle.round_fp8_bits(x, fmt), fmt)
        ref = _brute_force_fp8(x, fmt)
        nan = np.isnan(ref)
        assert np.array_equal(np.isnan(got), nan)
        np.testing.assert_array_equal(got[~nan], ref[~nan])
        np.testing.assert_array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_fp8_round_in_range_matches_library_and_saturates():
    """Within the finite range O6 equals torch's float8 conversion (which rounds to nearest even
    but does not saturate); beyond it, and for infinities, the result is the largest finite value
    of the input's sign (E4M3: 464 is the tie between 448 and the missing 480 and goes to 448)."""
    rng = np.random.default_rng(13)
    for fmt, tdt in _TORCH_FP8.items():
        mx = _FP8_MAX[fmt]
        u = rng.integers(0, 1 << 32, 1 << 20, dtype=np.uint64).astype(np.uint32).view(np.float32)
        x = u[np.isfinite(u) & (np.abs(u) <= mx)]
        got = oracle.round_fp8_bits(x, fmt)
        ref = torch.from_numpy(x).to(tdt).view(torch.uint8).numpy()
        np.testing.assert_array_equal(got, ref)
        big = np.array([np.inf, 1e30, 2 * mx, mx * 1.0625, -np.inf, -1e30, -2 * mx], np.float32)
        dec = oracle.decode_bits(oracle.round_fp8_bits(big, fmt), fmt)
        np.testing.assert_array_equal(dec, np.where(big > 0, mx, -mx))
    tie = oracle.decode_bits(oracle.round_fp8_bits(np.array([464.0, 464.01, -464.0], np.float32), "e4m3"), "e4m3")
    assert tie.tolist() == [448.0, 448.0, -448.0]


def test_attn_dense_fp8v_definition():
    """O1 with V as 8-bit codes times a scale: (a) equals O1 on the same values stored as bf16
    (every E4M3 and E5M2 value is a bf16 value), through a different decoder; (b) is linear
    in the scale (out halves, LSE unchanged); (c) equals a numpy float64 softmax-weighted sum with
    V decoded by torch's float8 type."""
    rng = np.random.default_rng(14)
    B, N, H, D = 1, 37, 2, 16
    q = torch.from_numpy(rng.standard_normal((B, N, H, D)).astype(np.float32)).to(torch.bfloat16)
    k = torch.from_numpy(rng.standard_normal((B, N, H, D)).astype(np.float32)).to(torch.bfloat16)
    codes = oracle.round_fp8_bits(rng.standard_normal((B, N, H, D)).astype(np.float32), "e4m3")
    v_bf16 = torch.from_numpy(oracle.decode_bits(codes, "e4m3").astype(np.float32)).to(torch.bfloat16)
    for causal in (False, True):
        o8, l8 = oracle.attn_dense_fp8v(q, k, codes, 1.0, causal=causal)
        ob, lb = oracle.attn_dense(q, k, v_bf16, causal=causal)
        np.testing.assert_allclose(o8, ob, rtol=0, atol=1e-14)
        np.testing.assert_allclose(l8, lb, rtol=0, atol=1e-14)
        oh, lh = oracle.attn_dense_fp8v(q, k, codes, 0.5, causal=causal)
        np.testing.assert_allclose(oh, 0.5 * o8, rtol=0, atol=1e-15)
        np.testing.assert_array_equal(lh, l8)
    c5 = oracle.round_fp8_bits(rng.standard_normal((B, N, H, D)).astype(np.float32), "e5m2")
    v5 = torch.from_numpy(oracle.decode_bits(c5, "e5m2").astype(np.float32)).to(torch.bfloat16)
    o5, l5 = oracle.attn_dense_fp8v(q, k, c5, 1.0, causal=True, v_format="e5m2")
    ob5, lb5 = oracle.attn_dense(q, k, v5, causal=True)
    np.testing.assert_allclose(o5, ob5, rtol=0, atol=1e-14)
    vt = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    qd, kd = q.double().numpy(), k.double().numpy()
    s = np.einsum("bihd,bjhd->bhij", qd, kd) / np.sqrt(D)
    w = np.exp(s - s.max(-1, keepdims=True))
    ref = np.einsum("bhij,bjhd->bihd", w / w.sum(-1, keepdims=True), vt * 0.25)
    o, _ = oracle.attn_dense_fp8v(q, k, codes, 0.25)
    np.testing.assert_allclose(o, ref.reshape(-1, D), rtol=1e-12, atol=1e-13)


# ------------------------------------------------------------------------------------------
# O5: standalone row softmax (Tylo "Register fragments and logical axes", "Worked softmax";
# Tylo "Streaming attention and online state", "Online statistics")
# ------------------------------------------------------------------------------------------
def test_row_softmax_state_example():
    """The SoftmaxState example printed on the page: scores (0, 0) normalise to (0.5, 0.5)."""
    g = _golden("softmax_state_example.json")
    y = oracle.softmax_rows(np.array([g["scores"]], np.float32))
    assert y[0].tolist() == g["normalized_weights"]


def test_row_softmax_all_masked_conventions():
    """'Worked softmax': -inf logits get weight exactly 0, the other entries are the softmax of
    the visible ones alone, and a row with every logit -inf normalises to zeros (not NaN)."""
    rng = si.rng_for(90, 0)
    x = rng.standard_normal((6, 37)).astype(np.float32)
    x[0, :] = -np.inf
    x[1, 5] = -np.inf
    x[2, ::2] = -np.inf
    x[3, 1:] = -np.inf
    y = oracle.softmax_rows(x)
    assert np.all(y[0] == 0.0)
    assert y[3, 0] == 1.0 and np.all(y[3, 1:] == 0.0)
    for r in (1, 2, 4, 5):
        vis = np.isfinite(x[r])
        assert np.all(y[r, ~vis] == 0.0)
        w = [math.exp(float(t) - max(x[r, vis].astype(np.float64))) for t in x[r, vis].astype(np.float64)]
        s = math.fsum(w)
        np.testing.assert_allclose(y[r, vis], [t / s for t in w], rtol=1e-14, atol=0)


def test_row_softmax_closed_forms():
    """Uniform logits give 1/n; two logits give the logistic function; adding a constant to a
    row (a power of two, exact in float32) or permuting its entries changes nothing but the
    order."""
    for n in (1, 2, 3, 64, 1000):
        y = oracle.softmax_rows(np.full((2, n), 1.75, np.float32))
        np.testing.assert_allclose(y, 1.0 / n, rtol=1e-15)
    a, b = 0.25, -1.5
    y = oracle.softmax_rows(np.array([[a, b]], np.float32))[0]
    np.testing.assert_allclose(y, [1 / (1 + math.exp(b - a)), 1 / (1 + math.exp(a - b))], rtol=1e-15)
    rng = si.rng_for(90, 1)
    x = (np.round(rng.standard_normal((4, 300)) * 1024) / 1024).astype(np.float32)   # x + 64 exact
    y = oracle.softmax_rows(x)
    np.testing.assert_allclose(oracle.softmax_rows(x + np.float32(64.0)), y, rtol=1e-12)
    perm = rng.permutation(300)
    np.testing.assert_allclose(oracle.softmax_rows(x[:, perm]), y[:, perm], rtol=1e-13)   # sum order


def test_row_softmax_matches_library_routine():
    """The textbook definition as an independent library computes it (scipy.special.softmax,
    float64), on normal and x30 large logits: natural exponent, max-shifted, rows sum to 1."""
    from scipy.special import softmax as sp_softmax
    rng = si.rng_for(90, 2)
    for scale in (1.0, 30.0):
        x = (rng.standard_normal((8, 513)) * scale).astype(np.float32)
        y = oracle.softmax_rows(x)
        np.testing.assert_allclose(y, sp_softmax(x.astype(np.float64), axis=1), rtol=1e-12, atol=1e-300)
        np.testing.assert_allclose(y.sum(axis=1), 1.0, rtol=1e-13)


def test_row_softmax_reads_16_bit_inputs_exactly():
    """bfloat16 and float16 logits are widened exactly: the result equals the float32 path on
    the same (representable) values."""
    rng = si.rng_for(90, 3)
    x = rng.standard_normal((3, 77)).astype(np.float32)
    for dt in ("bf16", "f16"):
        xt = si.cast(x, dt)
        np.testing.assert_array_equal(oracle.softmax_rows(xt), oracle.softmax_rows(xt.float()))
