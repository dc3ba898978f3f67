"""FP64 CPU oracle for streaming online-softmax attention (test infrastructure only).

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may
import this package.  It shares no code with the HIP path and the HIP path never calls it.

The arithmetic lives in ``oracle.c`` (plain C, double precision, OpenMP over query rows); this
module only marshals arguments through ctypes.  Every function names the page passage it
follows in the C source.  Inputs are torch CPU tensors (float32, bfloat16, float16 or float64) or numpy
float32 arrays; they are widened to double exactly inside the C code.  Outputs are numpy float64.

Functions:
    attn_dense         O1  the dense definition (pass criterion)
    attn_online        O2  the chunked online recurrence (self-check, trace, bug switch)
    online_from_logits O2  logits-in form for the worked trace
    merge_nat          O3a softmax_merge of two summaries, natural base
    combine_log2       O3b the LSE-weighted split-K combine, base 2
    splitk             O3c split-K workspace (locally normalised O_p/l_p, base-2 LSE)
    round_bits         O4  round-to-nearest-even float32 -> bf16 / f16 bits
    round_fp8_bits     O6  round-to-nearest-even, saturating float32 -> E4M3 / E5M2 codes
    decode_bits            exact widening of bf16 / f16 bits and E4M3 / E5M2 codes
    attn_dense_fp8v    O1  with V given as E4M3 codes times a scale
"""
import ctypes
import os
import subprocess

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

F32, BF16, F16, E4M3, E5M2, F64 = 0, 1, 2, 3, 4, 5
NO_NUMERATOR_RESCALE, SAME_BOUNDARY_BF16, SAME_BOUNDARY_F16 = 1, 2, 4

_lib = None


def build(force=True):
    """Compile oracle.c with gcc (plain -O2, no fast-math) into liboracle.so."""
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall",
           "-o", _LIB_PATH + ".tmp", _SRC, "-lm"]
    if force or not os.path.exists(_LIB_PATH):
        subprocess.check_call(cmd)
        os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build(force=True)
        L = ctypes.CDLL(_LIB_PATH)
        vp, i32, i64, dp = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_void_p
        L.oracle_attn_dense.argtypes = [vp, vp, vp, i32, vp, i32, i32, i32, i32, i32, i32, vp, i64, dp, dp]
        L.oracle_attn_online.argtypes = [vp, vp, vp, i32, vp, i32, i32, i32, i32, i32, i32, i32, i32,
                                         vp, i64, dp, dp]
        L.oracle_online_from_logits.argtypes = [dp, dp, i32, i32, i32, i32, dp, dp, dp]
        L.oracle_online_from_logits.restype = None
        d = ctypes.c_double
        L.oracle_merge_nat.argtypes = [d, d, dp, d, d, dp, i32, dp, dp, dp, dp, dp]
        L.oracle_merge_nat.restype = None
        L.oracle_combine_log2.argtypes = [dp, dp, i32, i64, i32, dp, dp]
        L.oracle_combine_log2.restype = None
        L.oracle_splitk.argtypes = [vp, vp, vp, i32, vp, i32, i32, i32, i32, i32, i32, i32, vp, i64, dp, dp]
        L.oracle_round_array.argtypes = [vp, i64, i32, vp]
        L.oracle_round_array.restype = None
        L.oracle_round_fp8_array.argtypes = [vp, i64, i32, vp]
        L.oracle_round_fp8_array.restype = None
        L.oracle_decode.argtypes = [vp, i32, i64, dp]
        L.oracle_softmax_rows.argtypes = [vp, i32, i64, i64, dp]
        L.oracle_softmax_rows.restype = None
        L.oracle_decode.restype = None
        L.oracle_num_threads.restype = i32
        _lib = L
    return _lib


def _as_cpu_tensor(x):
    if isinstance(x, np.ndarray):
        x = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64 if x.dtype == np.float64 else np.float32))
    x = x.detach()
    if x.device.type != "cpu":
        x = x.cpu()
    return x.contiguous()


def _dtype_code(t):
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float16:
        return F16
    if t.dtype == torch.float64:
        return F64
    raise TypeError(f"oracle: unsupported element type {t.dtype}")


def _ptr(a):
    if isinstance(a, np.ndarray):
        return a.ctypes.data
    return a.data_ptr()


def _prep(q, k, v, mask, rows):
    q, k, v = _as_cpu_tensor(q), _as_cpu_tensor(k), _as_cpu_tensor(v)
    dt = _dtype_code(q)
    if _dtype_code(k) != dt or _dtype_code(v) != dt:
        raise TypeError("oracle: q, k, v must share one element type")
    B, Nq, H, D = q.shape
    Nkv = k.shape[1]
    if mask is not None:
        mask = np.ascontiguousarray(mask.cpu().numpy() if isinstance(mask, torch.Tensor) else mask,
                                    dtype=np.uint8)
        assert mask.shape == (Nq, Nkv)
    if rows is not None:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        nsel = rows.size
    else:
        nsel = B * Nq * H
    return q, k, v, dt, mask, rows, (B, H, Nq, Nkv, D), nsel


def attn_dense(q, k, v, causal=False, mask=None, rows=None):
    """O1 over the selected row-heads rh = (b*Nq + i)*H + h (all of them if rows is None).
    Returns (out [nsel, D] float64, lse [nsel] float64, natural log)."""
    q, k, v, dt, mask, rows, (B, H, Nq, Nkv, D), nsel = _prep(q, k, v, mask, rows)
    out = np.zeros((nsel, D), np.float64)
    lse = np.zeros(nsel, np.float64)
    rc = lib().oracle_attn_dense(_ptr(q), _ptr(k), _ptr(v), dt, None if mask is None else _ptr(mask),
                                 B, H, Nq, Nkv, D, int(causal), None if rows is None else _ptr(rows),
                                 nsel, _ptr(out), _ptr(lse))
    if rc:
        raise MemoryError("oracle_attn_dense failed")
    return out, lse


def attn_online(q, k, v, BN, causal=False, mask=None, rows=None, no_numerator_rescale=False,
                same_boundary=None):
    """O2 with BN-key tiles. same_boundary in (None, 'bf16', 'f16')."""
    q, k, v, dt, mask, rows, (B, H, Nq, Nkv, D), nsel = _prep(q, k, v, mask, rows)
    flags = NO_NUMERATOR_RESCALE if no_numerator_rescale else 0
    if same_boundary == "bf16":
        flags |= SAME_BOUNDARY_BF16
    elif same_boundary == "f16":
        flags |= SAME_BOUNDARY_F16
    out = np.zeros((nsel, D), np.float64)
    lse = np.zeros(nsel, np.float64)
    rc = lib().oracle_attn_online(_ptr(q), _ptr(k), _ptr(v), dt, None if mask is None else _ptr(mask),
                                  B, H, Nq, Nkv, D, int(causal), int(BN), flags,
                                  None if rows is None else _ptr(rows), nsel, _ptr(out), _ptr(lse))
    if rc:
        raise ValueError("oracle_attn_online failed")
    return out, lse


def online_from_logits(s, v, BN, no_numerator_rescale=False):
    """O2 on already-scaled logits s[n] (-inf = masked) and value rows v[n, D].
    Returns (out [D], lse, trace [tiles, 4] of (m, l, a[0], alpha) after each tile)."""
    s = np.ascontiguousarray(s, dtype=np.float64)
    v = np.ascontiguousarray(v, dtype=np.float64)
    if v.ndim == 1:
        v = v[:, None].copy()
    n, D = v.shape
    tiles = (n + BN - 1) // BN
    out = np.zeros(D, np.float64)
    lse = np.zeros(1, np.float64)
    trace = np.zeros((max(tiles, 1), 4), np.float64)
    lib().oracle_online_from_logits(_ptr(s), _ptr(v), n, D, int(BN),
                                    NO_NUMERATOR_RESCALE if no_numerator_rescale else 0,
                                    _ptr(out), _ptr(lse), _ptr(trace))
    return out, float(lse[0]), trace[:tiles]


def merge_nat(m1, l1, a1, m2, l2, a2):
    """O3a. Returns (m, l, a, alpha1, alpha2)."""
    a1 = np.ascontiguousarray(a1, dtype=np.float64)
    a2 = np.ascontiguousarray(a2, dtype=np.float64)
    D = a1.size
    a = np.zeros(D, np.float64)
    m, l, al1, al2 = (ctypes.c_double() for _ in range(4))
    lib().oracle_merge_nat(float(m1), float(l1), _ptr(a1), float(m2), float(l2), _ptr(a2), D,
                           ctypes.addressof(m), ctypes.addressof(l), _ptr(a),
                           ctypes.addressof(al1), ctypes.addressof(al2))
    return m.value, l.value, a, al1.value, al2.value


def combine_log2(o_partial, lse_partial):
    """O3b. o_partial [P, RH, D], lse_partial [P, RH] (base 2) -> (out [RH, D], G [RH] base 2)."""
    o_partial = np.ascontiguousarray(o_partial, dtype=np.float64)
    lse_partial = np.ascontiguousarray(lse_partial, dtype=np.float64)
    P, RH, D = o_partial.shape
    assert lse_partial.shape == (P, RH)
    out = np.zeros((RH, D), np.float64)
    g = np.zeros(RH, np.float64)
    lib().oracle_combine_log2(_ptr(o_partial), _ptr(lse_partial), P, RH, D, _ptr(out), _ptr(g))
    return out, g


def splitk(q, k, v, P, causal=False, mask=None, rows=None):
    """O3c. Returns (o_partial [P, nsel, D], lse_partial [P, nsel] base 2)."""
    q, k, v, dt, mask, rows, (B, H, Nq, Nkv, D), nsel = _prep(q, k, v, mask, rows)
    o_p = np.zeros((P, nsel, D), np.float64)
    l_p = np.zeros((P, nsel), np.float64)
    rc = lib().oracle_splitk(_ptr(q), _ptr(k), _ptr(v), dt, None if mask is None else _ptr(mask),
                             B, H, Nq, Nkv, D, int(causal), int(P), None if rows is None else _ptr(rows),
                             nsel, _ptr(o_p), _ptr(l_p))
    if rc:
        raise ValueError("oracle_splitk failed")
    return o_p, l_p


def softmax_rows(x):
    """O5. Row softmax of the last axis with the all-masked conventions (-inf = masked; an
    all-masked row gives zeros).  x: float32 / bfloat16 / float16 tensor or float32 array.
    Returns float64 array of x's shape."""
    x = _as_cpu_tensor(x)
    n = x.shape[-1]
    rows = x.numel() // n if n else 0
    y = np.zeros(tuple(x.shape), np.float64)
    lib().oracle_softmax_rows(_ptr(x), _dtype_code(x), rows, n, _ptr(y))
    return y


def round_bits(x, target):
    """O4. float32 array -> uint16 bits of the RNE-rounded bf16 ('bf16') or float16 ('f16')."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.zeros(x.shape, np.uint16)
    lib().oracle_round_array(_ptr(x), x.size, BF16 if target == "bf16" else F16, _ptr(out))
    return out


def decode_bits(bits, dtype):
    """Exact widening to float64 of uint16 bf16 ('bf16') / float16 ('f16') bit patterns, or of
    uint8 E4M3 ('e4m3') / E5M2 ('e5m2') codes."""
    code = {"bf16": BF16, "f16": F16, "e4m3": E4M3, "e5m2": E5M2}[dtype]
    bits = np.ascontiguousarray(bits, dtype=np.uint8 if code in (E4M3, E5M2) else np.uint16)
    out = np.zeros(bits.shape, np.float64)
    lib().oracle_decode(_ptr(bits), code, bits.size, _ptr(out))
    return out


def round_fp8_bits(x, target):
    """O6. float32 array -> uint8 codes, round to nearest even with saturation to the largest
    finite value, E4M3 ('e4m3') or E5M2 ('e5m2')."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.zeros(x.shape, np.uint8)
    lib().oracle_round_fp8_array(_ptr(x), x.size, E4M3 if target == "e4m3" else E5M2, _ptr(out))
    return out


def attn_dense_fp8v(q, k, v_codes, v_scale, causal=False, mask=None, rows=None, v_format="e4m3"):
    """O1 with V given as 8-bit codes (E4M3 or E5M2) and a scale: the values the kernel consumes
    are decode(v_codes) * v_scale (exact in float64); q and k (bf16 / f16) widen exactly."""
    qd = _as_cpu_tensor(q).to(torch.float64)
    kd = _as_cpu_tensor(k).to(torch.float64)
    codes = v_codes.cpu().numpy() if isinstance(v_codes, torch.Tensor) else np.asarray(v_codes)
    vd = torch.from_numpy(decode_bits(codes, v_format) * float(v_scale))
    return attn_dense(qd, kd, vd, causal=causal, mask=mask, rows=rows)


def num_threads():
    return int(lib().oracle_num_threads())
