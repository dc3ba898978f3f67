"""Streaming (online-softmax) attention for AMD MI355X: Python binding of libattn.so.

The binding only marshals arguments: every step of the computation runs in the HIP kernels of
libattn.so (built from ``csrc/`` by ``build.py``).  torch supplies device memory and streams.
If the library has not been built, the first call raises -- there is no fallback.

Entry points (same names as the C ABI in include/attn.h):
    attn_fwd(q, k, v, out, lse=None, causal=False, mask=None, block_n=0, stream=None, mask_bits=None)
    attn_fwd_packed(q, k, v, out, lse=None, causal=False, mask_bits=..., stream=None)
    attn_mask_pack(mask, bits, causal=False, stream=None)
                    (mask uint8 [Nq, Nkv]; bits int32 of mask_bits_words(Nq, Nkv) elements)
    attn_fwd_splitk(q, k, v, P, o_partial, lse_partial, out=None, lse=None, causal=False,
                    mask=None, stream=None)
    attn_fwd_splitk_fused(q, k, v, P, o_partial, lse_partial, tickets, out, lse=None, causal=False,
                          mask=None, stream=None)
    attn_fwd_splitk_noalloc(q, k, v, P, out, lse=None, causal=False, mask=None, stream=None)
                    (the workspace in the library's static device memory; nothing allocated)
    attn_combine(o_partial, lse_partial, out, lse_out=None, stream=None)
    attn_softmax_rows(x, y, method=SOFTMAX_STREAMING, stream=None)   (x, y: [..., n])
    attn_fwd_fp8v(q, k, v, v_scale, out, lse=None, causal=False, mask=None, v_format=None, stream=None)
    attn_round(x, y, stream=None)    (x float32, y bf16/fp16/E4M3, same number of elements)
    attn_last_error(), attn_abi_version()
Tensors are torch tensors on the GPU, contiguous, laid out as the header states
(q/out [B, Nq, H, D]; k/v [B, Nkv, H, D]; o_partial [P, B*Nq, H, D]; lse_partial [P, B*Nq, H];
tickets int32 [B*Nq*H*TICKET_STRIDE], zero before the first call and left zero by every call).
Allocating helpers fwd(), fwd_fp8v(), splitk(), splitk_fused(), combine() and pack_mask() return
fresh outputs.
"""
import ctypes
import os
import re

import torch  # noqa: F401  (loads the HIP runtime that libattn.so then binds to)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libattn.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "attn.h")

ATTN_BF16, ATTN_FP16, ATTN_FP32, ATTN_FP8_E4M3, ATTN_FP8_E5M2 = 0, 1, 2, 3, 4
STATUS = {0: "ATTN_OK", 1: "ATTN_E_NULL", 2: "ATTN_E_SHAPE", 3: "ATTN_E_UNSUPPORTED",
          4: "ATTN_E_ALIGN", 5: "ATTN_E_WORKSPACE", 6: "ATTN_E_HIP"}
P_MAX = 256
TICKET_STRIDE = 32          # int32 slots per row-head in a fused-decode ticket array
NOALLOC_SCRATCH_BYTES = 64 << 20   # per-GPU static workspace of attn_fwd_splitk_noalloc
SOFTMAX_STREAMING, SOFTMAX_REGISTERS, SOFTMAX_THREE_PASS = 0, 1, 2


class AttnError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"{STATUS.get(code, code)}: {msg}")
        self.code = code


class FwdArgs(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("out", ctypes.c_void_p), ("lse", ctypes.c_void_p), ("mask", ctypes.c_void_p),
                ("B", ctypes.c_int), ("H", ctypes.c_int), ("N", ctypes.c_int), ("D", ctypes.c_int),
                ("causal", ctypes.c_int), ("dtype", ctypes.c_int), ("block_n", ctypes.c_int),
                ("mask_bits", ctypes.c_void_p)]


_LIB = None


def lib():
    """The loaded libattn.so (ctypes).  Raises if it is missing or fails to load."""
    global _LIB
    if _LIB is None:
        _LIB = _load()
    return _LIB


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built: run `python -m streaming_online_softmax_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32 = ctypes.c_void_p, ctypes.c_int
    L.attn_fwd.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, vp, i32, vp]
    L.attn_fwd.restype = i32
    L.attn_fwd_splitk.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, vp, i32, vp, vp, i32, vp]
    L.attn_fwd_splitk.restype = i32
    L.attn_fwd_splitk_fused.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, vp, i32, vp, vp, vp, i32, vp]
    L.attn_fwd_splitk_fused.restype = i32
    L.attn_fwd_splitk_noalloc.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, vp, i32, i32, vp]
    L.attn_fwd_splitk_noalloc.restype = i32
    L.attn_softmax_rows.argtypes = [vp, vp, ctypes.c_int64, i32, i32, i32, vp]
    L.attn_softmax_rows.restype = i32
    L.attn_round.argtypes = [vp, vp, ctypes.c_int64, i32, vp]
    L.attn_fwd_fp8v.argtypes = [vp, vp, vp, i32, ctypes.c_float, vp, vp, i32, i32, i32, i32, i32, vp, i32, vp]
    L.attn_fwd_fp8v.restype = i32
    L.attn_round.restype = i32
    L.attn_combine.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, vp]
    L.attn_combine.restype = i32
    L.attn_fwd_packed.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, vp, i32, vp]
    L.attn_fwd_packed.restype = i32
    L.attn_mask_pack.argtypes = [vp, i32, i32, i32, vp, vp]
    L.attn_mask_pack.restype = i32
    L.attn_fwd_ex.argtypes = [ctypes.POINTER(FwdArgs), vp]
    L.attn_fwd_ex.restype = i32
    L.attn_last_error.restype = ctypes.c_char_p
    L.attn_abi_version.restype = i32
    return L



def declared_symbols():
    """Function names the public header declares."""
    with open(HEADER) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(attn_\w+)\s*\(", text, re.M)))


def attn_last_error():
    return lib().attn_last_error().decode()


def attn_abi_version():
    return int(lib().attn_abi_version())


def _check(rc):
    if rc != 0:
        raise AttnError(rc, attn_last_error())


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    if t.dtype == torch.float16:
        return ATTN_FP16
    if t.dtype == torch.float32:
        return ATTN_FP32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError("tensors must be contiguous GPU tensors")
    return t.data_ptr()


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def attn_fwd(q, k, v, out, lse=None, causal=False, mask=None, block_n=0, stream=None, mask_bits=None):
    B, N, H, D = q.shape
    a = FwdArgs(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(mask),
                B, H, N, D, int(causal), _dtype_code(q), int(block_n), _ptr(mask_bits))
    _check(lib().attn_fwd_ex(ctypes.byref(a), _stream(stream)))


def attn_fwd_packed(q, k, v, out, lse=None, causal=False, mask_bits=None, stream=None):
    B, N, H, D = q.shape
    _check(lib().attn_fwd_packed(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, N, D, int(causal),
                                 _ptr(mask_bits), _dtype_code(q), _stream(stream)))


def mask_bits_words(Nq, Nkv):
    """32-bit words of a packed Nq x Nkv mask (ATTN_MASK_BITS_WORDS)."""
    return ((Nq + 31) // 32) * ((Nkv + 63) // 64) * 64


def attn_mask_pack(mask, bits, causal=False, stream=None):
    Nq, Nkv = mask.shape
    if bits.numel() != mask_bits_words(Nq, Nkv) or bits.element_size() != 4:
        raise AttnError(2, f"bits must hold {mask_bits_words(Nq, Nkv)} 32-bit words")
    _check(lib().attn_mask_pack(_ptr(mask), Nq, Nkv, int(causal), _ptr(bits), _stream(stream)))


def attn_fwd_splitk(q, k, v, P, o_partial, lse_partial, out=None, lse=None, causal=False, mask=None,
                    stream=None):
    B, Nq, H, D = q.shape
    Nkv = k.shape[1]
    _check(lib().attn_fwd_splitk(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, Nq, Nkv, D,
                               int(causal), _ptr(mask), int(P), _ptr(o_partial), _ptr(lse_partial),
                               _dtype_code(q), _stream(stream)))


def attn_fwd_splitk_fused(q, k, v, P, o_partial, lse_partial, tickets, out, lse=None, causal=False,
                          mask=None, stream=None):
    B, Nq, H, D = q.shape
    Nkv = k.shape[1]
    _check(lib().attn_fwd_splitk_fused(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, Nq, Nkv, D,
                                     int(causal), _ptr(mask), int(P), _ptr(o_partial), _ptr(lse_partial),
                                     _ptr(tickets), _dtype_code(q), _stream(stream)))


def attn_fwd_splitk_noalloc(q, k, v, P, out, lse=None, causal=False, mask=None, stream=None):
    """attn_fwd_splitk with the combine, its workspace in the library's static device array
    (no allocation on any path; calls that overlap on one GPU race on that array)."""
    B, Nq, H, D = q.shape
    Nkv = k.shape[1]
    _check(lib().attn_fwd_splitk_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, Nq, Nkv, D,
                                         int(causal), _ptr(mask), int(P), _dtype_code(q), _stream(stream)))


def attn_combine(o_partial, lse_partial, out, lse_out=None, stream=None):
    P = o_partial.shape[0]
    depth = o_partial.shape[-1]
    heads = o_partial.shape[-2]
    rows = o_partial[0].numel() // (heads * depth)
    _check(lib().attn_combine(_ptr(o_partial), _ptr(lse_partial), _ptr(out), _ptr(lse_out), int(P),
                            rows, heads, depth, _dtype_code(out), _stream(stream)))


def attn_softmax_rows(x, y, method=SOFTMAX_STREAMING, stream=None):
    n = x.shape[-1]
    rows = x.numel() // n
    _check(lib().attn_softmax_rows(_ptr(x), _ptr(y), rows, n, _dtype_code(x), int(method), _stream(stream)))


def _fp8_code(t, fmt=None):
    """Format code of 8-bit data: float8_e4m3fn / float8_e5m2 tensors name their format; uint8
    codes take `fmt` ('e4m3' unless given)."""
    if t.dtype == torch.float8_e4m3fn or (t.dtype == torch.uint8 and fmt in (None, "e4m3")):
        return ATTN_FP8_E4M3
    if t.dtype == torch.float8_e5m2 or (t.dtype == torch.uint8 and fmt == "e5m2"):
        return ATTN_FP8_E5M2
    raise AttnError(3, f"8-bit data must be uint8 codes, float8_e4m3fn or float8_e5m2 (got {t.dtype}, {fmt})")


def attn_round(x, y, stream=None):
    """y = x (fp32) rounded to nearest even by the kernels' packed conversion: bf16 / fp16, or
    E4M3 (saturating) when y is uint8 or float8_e4m3fn."""
    if x.dtype != torch.float32 or x.numel() != y.numel():
        raise AttnError(2, "x must be float32 with as many elements as y")
    code = _fp8_code(y) if y.element_size() == 1 else _dtype_code(y)
    _check(lib().attn_round(_ptr(x), _ptr(y), x.numel(), code, _stream(stream)))


def attn_fwd_fp8v(q, k, v, v_scale, out, lse=None, causal=False, mask=None, v_format=None, stream=None):
    """attn_fwd with V as 8-bit codes ([B, N, H, D]: float8_e4m3fn, float8_e5m2, or uint8 with
    v_format 'e4m3' / 'e5m2') of value decode(code) * v_scale; P is rounded to E4M3 for the FP8
    second product.  D must be 128."""
    B, N, H, D = q.shape
    fmt = _fp8_code(v, v_format)
    if tuple(v.shape) != (B, N, H, D):
        raise AttnError(2, f"v must be [B, N, H, D] = {(B, N, H, D)} (got {tuple(v.shape)})")
    _check(lib().attn_fwd_fp8v(_ptr(q), _ptr(k), _ptr(v), fmt, float(v_scale), _ptr(out), _ptr(lse), B, H, N, D,
                               int(bool(causal)), _ptr(mask), _dtype_code(q), _stream(stream)))


# ---- allocating helpers -------------------------------------------------------------------
def fwd(q, k, v, causal=False, mask=None, block_n=0, with_lse=True, mask_bits=None):
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device) if with_lse else None
    attn_fwd(q, k, v, out, lse, causal=causal, mask=mask, block_n=block_n, mask_bits=mask_bits)
    return out, lse


def pack_mask(mask, causal=False):
    """attn_mask_pack into a fresh int32 tensor (words of a causal packing above the diagonal
    are left unset)."""
    bits = torch.empty(mask_bits_words(*mask.shape), dtype=torch.int32, device=mask.device)
    attn_mask_pack(mask, bits, causal=causal)
    return bits


def fwd_fp8v(q, k, v, v_scale=1.0, causal=False, mask=None, v_format=None):
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    attn_fwd_fp8v(q, k, v, v_scale, out, lse, causal=causal, mask=mask, v_format=v_format)
    return out, lse


def workspace(q, P):
    B, Nq, H, D = q.shape
    o_p = torch.empty((P, B * Nq, H, D), dtype=torch.float32, device=q.device)
    l_p = torch.empty((P, B * Nq, H), dtype=torch.float32, device=q.device)
    return o_p, l_p


def splitk(q, k, v, P, causal=False, mask=None, combine=True):
    o_p, l_p = workspace(q, P)
    out = lse = None
    if combine:
        out = torch.empty_like(q)
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    attn_fwd_splitk(q, k, v, P, o_p, l_p, out=out, lse=lse, causal=causal, mask=mask)
    return o_p, l_p, out, lse


def softmax_rows(x, method=SOFTMAX_STREAMING):
    y = torch.empty_like(x)
    attn_softmax_rows(x, y, method)
    return y


def tickets(q):
    """A zeroed ticket array for attn_fwd_splitk_fused (reusable: every call leaves it zero).
    One counter per row-head, TICKET_STRIDE slots apart (one 128-byte line each)."""
    B, Nq, H, _ = q.shape
    return torch.zeros(B * Nq * H * TICKET_STRIDE, dtype=torch.int32, device=q.device)


def splitk_fused(q, k, v, P, causal=False, mask=None, tk=None):
    o_p, l_p = workspace(q, P)
    tk = tickets(q) if tk is None else tk
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    attn_fwd_splitk_fused(q, k, v, P, o_p, l_p, tk, out, lse=lse, causal=causal, mask=mask)
    return out, lse, o_p, l_p


def combine(o_partial, lse_partial, out_dtype=torch.float32):
    P, RH = lse_partial.shape[0], lse_partial[0].numel()
    heads = o_partial.shape[-2]
    out = torch.empty(o_partial.shape[1:], dtype=out_dtype, device=o_partial.device)
    lse = torch.empty(o_partial.shape[1:-1], dtype=torch.float32, device=o_partial.device)
    attn_combine(o_partial, lse_partial, out, lse)
    return out, lse
