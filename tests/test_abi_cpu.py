"""The C ABI library loads, exports every declared symbol and rejects bad arguments before any
HIP call.  CPU only: the reject-path calls use fake, never-dereferenced pointer values, so they
run only where no GPU is visible (the GPU suite repeats them with real buffers)."""
import ctypes

import pytest
import torch

import streaming_online_softmax_amd as sa

E_NULL, E_SHAPE, E_UNSUP, E_ALIGN, E_WS = 1, 2, 3, 4, 5


def test_library_exports_every_declared_symbol():
    names = sa.declared_symbols()
    assert {"attn_fwd", "attn_fwd_splitk", "attn_fwd_splitk_fused", "attn_combine", "attn_softmax_rows",
            "attn_round", "attn_fwd_fp8v", "attn_fwd_ex", "attn_last_error", "attn_abi_version",
            "attn_fwd_splitk_noalloc", "attn_mask_pack", "attn_fwd_packed"} <= set(names)
    for n in names:
        assert hasattr(sa.lib(), n), n


@pytest.mark.parametrize("lang,std", [("c", "-std=c11"), ("c++", "-std=c++17")])
def test_header_is_plain_c_and_cpp(lang, std, tmp_path):
    """include/attn.h compiles on its own as C11 (no torch or C++ types in the boundary) and as
    C++17, warning-free; a C program that calls every entry point links against libattn.so."""
    import os
    import shutil
    import subprocess
    cc = shutil.which("gcc" if lang == "c" else "g++")
    if cc is None:
        pytest.skip("no host compiler")
    hdr = os.path.join(os.path.dirname(sa.LIB_PATH), "..", "include", "attn.h")
    r = subprocess.run([cc, std, "-Wall", "-Wextra", "-pedantic", "-Werror", "-fsyntax-only", "-x", lang, hdr],
                       stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert r.returncode == 0, r.stdout
    if lang == "c":
        src = tmp_path / "use.c"
        src.write_text('#include "attn.h"\n'
                       "int main(void) {\n"
                       "  return attn_abi_version() == ATTN_ABI_VERSION &&\n"
                       "         attn_fwd(0, 0, 0, 0, 0, 1, 1, 1, 64, 0, 0, ATTN_BF16, 0) == ATTN_E_NULL &&\n"
                       "         attn_fwd_splitk(0, 0, 0, 0, 0, 1, 1, 1, 1, 64, 0, 0, 1, 0, 0, ATTN_BF16, 0) == ATTN_E_NULL &&\n"
                       "         attn_fwd_splitk_fused(0, 0, 0, 0, 0, 1, 1, 1, 1, 64, 0, 0, 1, 0, 0, 0, ATTN_BF16, 0) == ATTN_E_NULL &&\n"
                       "         attn_fwd_splitk_noalloc(0, 0, 0, 0, 0, 1, 1, 1, 1, 64, 0, 0, 1, ATTN_BF16, 0) == ATTN_E_NULL &&\n"
                       "         attn_combine(0, 0, 0, 0, 1, 1, 1, 64, ATTN_FP32, 0) == ATTN_E_NULL &&\n"
                       "         attn_softmax_rows(0, 0, 1, 1, ATTN_FP32, ATTN_SOFTMAX_STREAMING, 0) == ATTN_E_NULL &&\n"
                       "         attn_fwd_fp8v(0, 0, 0, ATTN_FP8_E4M3, 1.0f, 0, 0, 1, 1, 1, 128, 0, 0, ATTN_BF16, 0) == ATTN_E_NULL &&\n"
                       "         attn_round(0, 0, 4, ATTN_BF16, 0) == ATTN_E_NULL &&\n"
                       "         attn_mask_pack(0, 1, 1, 0, 0, 0) == ATTN_E_NULL &&\n"
                       "         attn_fwd_packed(0, 0, 0, 0, 0, 1, 1, 1, 64, 0, 0, ATTN_BF16, 0) == ATTN_E_NULL &&\n"
                       "         ATTN_MASK_BITS_WORDS(33, 65) == 256 && ATTN_MASK_BITS_WORDS(32, 64) == 64 &&\n"
                       "         attn_fwd_ex(0, 0) == ATTN_E_NULL && attn_last_error()[0] != 0 ? 0 : 1;\n"
                       "}\n")
        exe = tmp_path / "use"
        libdir = os.path.dirname(sa.LIB_PATH)
        r = subprocess.run([cc, std, "-Wall", "-Werror", "-I", os.path.dirname(hdr), str(src), "-o", str(exe),
                            "-L", libdir, "-lattn", "-Wl,-rpath," + libdir],
                           stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
        assert r.returncode == 0, r.stdout
        r = subprocess.run([str(exe)], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=60)
        assert r.returncode == 0, r.stdout


def test_abi_version():
    assert sa.attn_abi_version() == 2


@pytest.mark.parametrize("nq,nkv", [(1, 1), (32, 64), (33, 64), (32, 65), (400, 400), (16384, 16384)])
def test_mask_bits_words(nq, nkv):
    """The binding's word count of a packed mask is the header's: one word per lane (64) per
    32-row group and 64-key group."""
    assert sa.mask_bits_words(nq, nkv) == -(-nq // 32) * -(-nkv // 64) * 64


def test_binding_constants_match_the_header():
    """The binding's copies of the header's sizes and codes are the header's values."""
    import re
    with open(sa.HEADER) as f:
        text = f.read()
    defines = dict((n, int(v)) for n, v in re.findall(r"^#define (ATTN_\w+) (\d+)", text, re.M))
    enums = dict((n, int(v)) for n, v in re.findall(r"\b(ATTN_[A-Z0-9_]+) = (\d+)", text))
    assert defines["ATTN_P_MAX"] == sa.P_MAX
    assert defines["ATTN_TICKET_STRIDE"] == sa.TICKET_STRIDE
    assert defines["ATTN_ABI_VERSION"] == sa.attn_abi_version()
    scratch = re.search(r"^#define ATTN_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text, re.M)
    assert int(scratch.group(1)) << int(scratch.group(2)) == sa.NOALLOC_SCRATCH_BYTES
    for name in ("ATTN_BF16", "ATTN_FP16", "ATTN_FP32", "ATTN_FP8_E4M3", "ATTN_FP8_E5M2",
                 "ATTN_SOFTMAX_STREAMING", "ATTN_SOFTMAX_REGISTERS", "ATTN_SOFTMAX_THREE_PASS"):
        binding = name[len("ATTN_"):] if name.startswith("ATTN_SOFTMAX") else name
        assert enums[name] == getattr(sa, binding), name


needs_no_gpu = pytest.mark.skipif(torch.cuda.is_available(),
                                  reason="fake-pointer reject paths run only where no GPU is visible")

A = 0x10000      # 16-byte aligned fake address (never dereferenced: every call below is rejected)
BAD = 0x10008    # 8-byte aligned only


def fwd(q=A, k=A, v=A, out=A, lse=None, B=1, H=1, N=64, D=64, causal=0, mask=None, dtype=0):
    return sa.lib().attn_fwd(q, k, v, out, lse, B, H, N, D, causal, mask, dtype, None)


def splitk(q=A, k=A, v=A, out=None, lse=None, B=1, H=1, Nq=1, Nkv=64, D=64, causal=0, mask=None, P=4,
           o_p=A, l_p=A, dtype=0):
    return sa.lib().attn_fwd_splitk(q, k, v, out, lse, B, H, Nq, Nkv, D, causal, mask, P, o_p, l_p, dtype, None)


def fused(q=A, k=A, v=A, out=A, lse=None, B=1, H=1, Nq=1, Nkv=64, D=64, causal=0, mask=None, P=4,
          o_p=A, l_p=A, tk=A, dtype=0):
    return sa.lib().attn_fwd_splitk_fused(q, k, v, out, lse, B, H, Nq, Nkv, D, causal, mask, P, o_p, l_p, tk,
                                          dtype, None)


def noalloc(q=A, k=A, v=A, out=A, lse=None, B=1, H=1, Nq=1, Nkv=64, D=64, causal=0, mask=None, P=4, dtype=0):
    return sa.lib().attn_fwd_splitk_noalloc(q, k, v, out, lse, B, H, Nq, Nkv, D, causal, mask, P, dtype, None)


def softmax(x=A, y=A, rows=1, n=64, dtype=2, method=0):
    return sa.lib().attn_softmax_rows(x, y, rows, n, dtype, method, None)


def fp8v(q=A, k=A, v=A, v_format=3, v_scale=1.0, out=A, lse=None, B=1, H=1, N=64, D=128, causal=0, mask=None,
         dtype=0):
    return sa.lib().attn_fwd_fp8v(q, k, v, v_format, v_scale, out, lse, B, H, N, D, causal, mask, dtype, None)


def rnd(x=A, y=A, n=64, dtype=0):
    return sa.lib().attn_round(x, y, n, dtype, None)


def combine(o_p=A, l_p=A, out=A, lse=None, P=4, rows=1, heads=1, depth=64, out_dtype=2):
    return sa.lib().attn_combine(o_p, l_p, out, lse, P, rows, heads, depth, out_dtype, None)


def pack(mask=A, Nq=64, Nkv=64, causal=0, bits=A):
    return sa.lib().attn_mask_pack(mask, Nq, Nkv, causal, bits, None)


def packed(q=A, k=A, v=A, out=A, lse=None, B=1, H=1, N=64, D=64, causal=0, bits=A, dtype=0):
    return sa.lib().attn_fwd_packed(q, k, v, out, lse, B, H, N, D, causal, bits, dtype, None)


def fwd_ex(mask=None, bits=None, block_n=0, D=64):
    a = sa.FwdArgs(A, A, A, A, None, mask, 1, 1, 64, D, 0, 0, block_n, bits)
    return sa.lib().attn_fwd_ex(ctypes.byref(a), None)


@needs_no_gpu
@pytest.mark.parametrize("call,code", [
    (lambda: fwd(q=None), E_NULL),
    (lambda: fwd(out=None), E_NULL),
    (lambda: fwd(B=0), E_SHAPE),
    (lambda: fwd(N=0), E_SHAPE),
    (lambda: fwd(H=-1), E_SHAPE),
    (lambda: fwd(D=48), E_UNSUP),
    (lambda: fwd(D=512), E_UNSUP),
    (lambda: fwd(dtype=2), E_UNSUP),
    (lambda: fwd(causal=2), E_SHAPE),
    (lambda: fwd(q=BAD), E_ALIGN),
    (lambda: fwd(out=BAD), E_ALIGN),
    (lambda: splitk(causal=1), E_SHAPE),            # rectangular causal is rejected
    (lambda: splitk(P=0), E_SHAPE),
    (lambda: splitk(P=257), E_UNSUP),
    (lambda: splitk(o_p=None), E_WS),
    (lambda: splitk(l_p=None), E_WS),
    (lambda: splitk(o_p=BAD), E_ALIGN),
    (lambda: splitk(D=8), E_UNSUP),
    (lambda: fused(tk=None), E_WS),
    (lambda: fused(out=None), E_NULL),
    (lambda: fused(tk=A + 2), E_ALIGN),
    (lambda: fused(P=300), E_UNSUP),
    (lambda: fused(causal=1), E_SHAPE),
    (lambda: noalloc(q=None), E_NULL),
    (lambda: noalloc(out=None), E_NULL),
    (lambda: noalloc(out=BAD), E_ALIGN),
    (lambda: noalloc(lse=A + 2), E_ALIGN),
    (lambda: noalloc(P=0), E_SHAPE),
    (lambda: noalloc(P=257), E_UNSUP),
    (lambda: noalloc(causal=1), E_SHAPE),
    (lambda: noalloc(D=48), E_UNSUP),
    # 256 * 300 * 256 * 4 B of o_partial = 78.6 MB > the 64 MiB scratch; then the smallest Nq past it
    (lambda: noalloc(P=256, H=300, D=256), E_WS),
    (lambda: noalloc(P=256, H=1, Nq=(64 << 20) // (256 * 129 * 4) + 1, D=128), E_WS),
    (lambda: softmax(x=None), E_NULL),
    (lambda: softmax(rows=0), E_SHAPE),
    (lambda: softmax(n=0), E_SHAPE),
    (lambda: softmax(dtype=5), E_UNSUP),
    (lambda: softmax(method=3), E_UNSUP),
    (lambda: softmax(method=1, n=65537), E_UNSUP),
    (lambda: softmax(x=A + 2), E_ALIGN),
    (lambda: fp8v(v=None), E_NULL),
    (lambda: fp8v(out=None), E_NULL),
    (lambda: fp8v(D=64), E_UNSUP),
    (lambda: fp8v(v_scale=float("inf")), E_UNSUP),
    (lambda: fp8v(v_scale=float("nan")), E_UNSUP),
    (lambda: fp8v(dtype=2), E_UNSUP),
    (lambda: fp8v(v=BAD), E_ALIGN),
    (lambda: fp8v(N=0), E_SHAPE),
    (lambda: fp8v(v_format=0), E_UNSUP),
    (lambda: fp8v(v_format=5), E_UNSUP),
    (lambda: rnd(n=-1), E_SHAPE),
    (lambda: rnd(dtype=4), E_UNSUP),
    (lambda: rnd(dtype=3, y=A + 1, x=A + 2), E_ALIGN),
    (lambda: rnd(x=None), E_NULL),
    (lambda: rnd(y=None), E_NULL),
    (lambda: rnd(dtype=2), E_UNSUP),
    (lambda: rnd(x=A + 2), E_ALIGN),
    (lambda: rnd(y=A + 1), E_ALIGN),
    (lambda: combine(P=0), E_SHAPE),
    (lambda: combine(P=300), E_UNSUP),
    (lambda: combine(depth=100), E_UNSUP),
    (lambda: combine(out_dtype=7), E_UNSUP),
    (lambda: combine(out=None), E_NULL),
    (lambda: combine(o_p=BAD), E_ALIGN),
    (lambda: combine(rows=0), E_SHAPE),
    (lambda: pack(mask=None), E_NULL),
    (lambda: pack(bits=None), E_NULL),
    (lambda: pack(Nq=0), E_SHAPE),
    (lambda: pack(Nkv=-1), E_SHAPE),
    (lambda: pack(causal=2), E_SHAPE),
    (lambda: pack(causal=1, Nkv=65), E_SHAPE),     # causal packing is square only
    (lambda: pack(bits=A + 2), E_ALIGN),
    (lambda: packed(bits=None), E_NULL),
    (lambda: packed(bits=A + 2), E_ALIGN),
    (lambda: packed(q=None), E_NULL),
    (lambda: packed(D=48), E_UNSUP),
    (lambda: packed(causal=3), E_SHAPE),
    (lambda: fwd_ex(mask=A, bits=A), E_SHAPE),      # one mask form at a time
    (lambda: fwd_ex(bits=A + 1), E_ALIGN),
    (lambda: fwd_ex(bits=A, block_n=48), E_UNSUP),
])
def test_reject_paths(call, code):
    rc = call()
    assert rc == code, (rc, sa.attn_last_error())
    assert sa.attn_last_error() != ""


@needs_no_gpu
def test_round_of_nothing_enqueues_nothing():
    assert rnd(x=None, y=None, n=0) == 0


def test_fwd_ex_rejects_bad_block_n():
    a = sa.FwdArgs(A, A, A, A, None, None, 1, 1, 64, 128, 0, 0, 32)
    assert sa.lib().attn_fwd_ex(ctypes.byref(a), None) == E_UNSUP
    a.block_n = 48
    assert sa.lib().attn_fwd_ex(ctypes.byref(a), None) == E_UNSUP
    assert sa.lib().attn_fwd_ex(None, None) == E_NULL


def test_binding_refuses_host_tensors():
    q = torch.zeros(1, 4, 1, 16, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        sa.attn_fwd(q, q, q, q)
