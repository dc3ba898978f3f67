"""Seeded synthetic inputs shared by the tests, the benchmark and the smoke check.

This module holds none of the attention arithmetic: it only draws random numbers and lays
them out.  Both the HIP path and the oracle are fed from here, so they see identical values.

Recipe (the same everywhere):
  * generator: numpy PCG64 seeded with SeedSequence([config, case]);
  * draw order: Q, then K, then V, each standard_normal float32 in [B, N, H, D] order, then the
    mask (if any);
  * variants act on the float32 Q before the cast: 'large' multiplies Q by 30, 'uniform' sets
    Q to zero (both leave the K and V draws untouched);
  * the float32 arrays are cast to the kernel dtype by torch's round-to-nearest-even conversion;
    the oracle then reads the cast values, so input quantisation is not charged to a kernel;
  * the masked workload's mask is a Bernoulli(0.5) draw per (query, key) in row-major order
    (uniform < 0.5 means visible), after which N/64 query rows chosen by the same generator
    (uniformly, without replacement) are cleared to all-masked.
"""
import numpy as np
import torch

DTYPES = {"bf16": torch.bfloat16, "f16": torch.float16, "fp16": torch.float16, "f32": torch.float32}

# The five workloads by what they are.
SMALL_F32 = dict(name="single-head N64 D16 fp32-drawn, BN32", B=1, H=1, N=64, D=16, causal=False)
PREFILL = dict(name="causal prefill B4 H32 N4096 D128 bf16", B=4, H=32, N=4096, D=128, causal=True)
DECODE = dict(name="split-K decode B8 H32 Nq1 Nkv32768 D128 bf16", B=8, H=32, Nq=1, Nkv=32768, D=128,
              P_list=(4, 8, 16, 37))
MASKED = dict(name="masked causal B1 H16 N16384 D256 bf16", B=1, H=16, N=16384, D=256, causal=True)
# standalone row softmax: rows of attention-score logits (a second workload on the same primitives)
SOFTMAX = dict(name="row softmax 32768 rows x 4096 logits fp32", rows=32768, n=4096, dtype="f32")
SOFTMAX_WIDE = dict(name="row softmax 4096 rows x 32768 logits fp32", rows=4096, n=32768, dtype="f32")

FP8V = dict(name="causal prefill B4 H32 N4096 D128, bf16 Q/K, E4M3 V", B=4, H=32, N=4096, D=128, causal=True)

SWEEP_N = (1, 17, 1000, 2047, 2048)
SWEEP_D = (16, 32, 64)
SWEEP_DTYPES = ("bf16", "f16")
SWEEP_BN = (32, 64)
SWEEP_VARIANTS = ("normal", "large", "uniform")

CFG_SMALL, CFG_SWEEP, CFG_PREFILL, CFG_DECODE, CFG_MASKED, CFG_SOFTMAX, CFG_FP8V = 1, 2, 3, 4, 5, 6, 7


def rng_for(cfg, case):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(cfg), int(case)])))


def _normal(rng, shape, chunk=1 << 24):
    """standard_normal float32 drawn in chunks (the stream is consumed in order, so the values
    equal one large draw) to bound the float64 temporaries numpy makes."""
    n = int(np.prod(shape))
    out = np.empty(n, np.float32)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        out[s:e] = rng.standard_normal(e - s, dtype=np.float32)
    return out.reshape(shape)


def draw_qkv(rng, q_shape, kv_shape, variant="normal"):
    """float32 Q, K, V in draw order; the variant acts on Q only."""
    q = _normal(rng, q_shape)
    k = _normal(rng, kv_shape)
    v = _normal(rng, kv_shape)
    if variant == "large":
        q = q * np.float32(30.0)
    elif variant == "uniform":
        q = np.zeros_like(q)
    elif variant != "normal":
        raise ValueError(variant)
    return q, k, v


def cast(x, dtype):
    """float32 numpy -> torch CPU tensor of the kernel dtype (round to nearest even)."""
    t = torch.from_numpy(np.ascontiguousarray(x))
    return t.to(DTYPES[dtype]) if dtype != "f32" else t.clone()


def cast_e4m3(x):
    """float32 numpy -> uint8 torch CPU tensor of E4M3 codes (torch's float8_e4m3fn conversion,
    round to nearest even; the draws here stay far inside its finite range)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8)


def cast_e5m2(x):
    """float32 numpy -> uint8 torch CPU tensor of E5M2 codes (torch's float8_e5m2 conversion,
    round to nearest even)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.float8_e5m2).view(torch.uint8)


def fp8v_inputs(B=None, H=None, N=None, case=0, dtype="bf16", v_format="e4m3"):
    """q, k in dtype and v as 8-bit codes (E4M3 or E5M2), all [B, N, H, D], drawn like the
    prefill workload."""
    s = FP8V
    B, H, N = B or s["B"], H or s["H"], N or s["N"]
    rng = rng_for(CFG_FP8V, case)
    q, k, v = draw_qkv(rng, (B, N, H, s["D"]), (B, N, H, s["D"]))
    return cast(q, dtype), cast(k, dtype), (cast_e4m3(v) if v_format == "e4m3" else cast_e5m2(v))


def bernoulli_mask(rng, Nq, Nkv, n_full_rows, row_block=1024):
    """uint8 [Nq, Nkv]: 1 = visible with probability 1/2, drawn row-major in row blocks;
    then n_full_rows seeded rows set to all-masked.  Returns (mask, cleared_rows)."""
    mask = np.empty((Nq, Nkv), np.uint8)
    for r0 in range(0, Nq, row_block):
        r1 = min(Nq, r0 + row_block)
        mask[r0:r1] = rng.random((r1 - r0, Nkv)) < 0.5
    rows = np.sort(rng.choice(Nq, size=n_full_rows, replace=False)) if n_full_rows else np.zeros(0, np.int64)
    mask[rows] = 0
    return mask, rows


def sweep_cases():
    """The single-head sweep: every (N, D, dtype, causal, BN, variant) combination, in a fixed
    order; the index is the case number of the seed."""
    cases = []
    for N in SWEEP_N:
        for D in SWEEP_D:
            for dt in SWEEP_DTYPES:
                for causal in (False, True):
                    for BN in SWEEP_BN:
                        for var in SWEEP_VARIANTS:
                            cases.append(dict(N=N, D=D, dtype=dt, causal=causal, BN=BN, variant=var))
    return cases


def sweep_inputs(case):
    """Inputs of one sweep case.  Variants of the same (N, D) share the Q, K, V draws: the seed
    depends on (N, D) only, and the variant is applied after the draw."""
    N, D = case["N"], case["D"]
    seed_case = SWEEP_N.index(N) * len(SWEEP_D) + SWEEP_D.index(D)
    rng = rng_for(CFG_SWEEP, seed_case)
    q, k, v = draw_qkv(rng, (1, N, 1, D), (1, N, 1, D), case["variant"])
    dt = case["dtype"]
    return cast(q, dt), cast(k, dt), cast(v, dt)


def small_inputs():
    rng = rng_for(CFG_SMALL, 0)
    s = SMALL_F32
    return draw_qkv(rng, (1, s["N"], 1, s["D"]), (1, s["N"], 1, s["D"]))


def prefill_inputs(dtype="bf16", B=None, H=None, N=None):
    s = PREFILL
    B, H, N = B or s["B"], H or s["H"], N or s["N"]
    rng = rng_for(CFG_PREFILL, 0)
    q, k, v = draw_qkv(rng, (B, N, H, s["D"]), (B, N, H, s["D"]))
    return cast(q, dtype), cast(k, dtype), cast(v, dtype)


def decode_inputs(dtype="bf16", B=None, H=None, Nkv=None):
    s = DECODE
    B, H, Nkv = B or s["B"], H or s["H"], Nkv or s["Nkv"]
    rng = rng_for(CFG_DECODE, 0)
    q, k, v = draw_qkv(rng, (B, 1, H, s["D"]), (B, Nkv, H, s["D"]))
    qt = cast(q, dtype)
    del q
    kt = cast(k, dtype)
    del k
    vt = cast(v, dtype)
    return qt, kt, vt


def masked_inputs(dtype="bf16", H=None, N=None):
    """Masked long-context workload; returns (q, k, v, mask, cleared_rows)."""
    s = MASKED
    H, N = H or s["H"], N or s["N"]
    rng = rng_for(CFG_MASKED, 0)
    q, k, v = draw_qkv(rng, (s["B"], N, H, s["D"]), (s["B"], N, H, s["D"]))
    mask, rows = bernoulli_mask(rng, N, N, N // 64)
    return cast(q, dtype), cast(k, dtype), cast(v, dtype), mask, rows


def softmax_inputs(rows, n, case=0, variant="normal", masked_frac=0.0, full_rows=0):
    """float32 [rows, n] logits for the row softmax: standard_normal (x30 for 'large'); then, if
    masked_frac > 0, each entry is masked (-inf) with that probability (uniform < masked_frac,
    row-major); then full_rows seeded rows (without replacement) are set to all -inf."""
    rng = rng_for(CFG_SOFTMAX, case)
    x = _normal(rng, (rows, n))
    if variant == "large":
        x = x * np.float32(30.0)
    if masked_frac > 0:
        x[rng.random((rows, n)) < masked_frac] = -np.inf
    if full_rows:
        x[rng.choice(rows, size=full_rows, replace=False)] = -np.inf
    return x
