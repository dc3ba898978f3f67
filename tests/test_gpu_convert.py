"""The kernels' FP32 -> bf16 / fp16 conversion (probabilities before the second product, stored
output), through attn_round, against the oracle's independent round-to-nearest-even (O4).

Exhaustive: every one of the 2^32 float32 bit patterns, for each target type, in chunks of 2^28.
Every non-NaN input must give exactly the oracle's bits (ties to even, subnormals kept, signed
zeros and infinities kept, overflow to infinity, no saturation); every NaN input must give some
NaN (Tylo.jl "Streaming attention and online state", section "Same-lane conversion").  The
packed-word example of Tylo.jl "Register fragments and logical axes", section "Logical types and
register packing" is checked on the device as well.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu
DEV = "cuda"
CHUNK = 1 << 28


@pytest.fixture(scope="module")
def sa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import streaming_online_softmax_amd as mod
    return mod


def _is_nan16(bits, fmt):
    exp_mask, man_mask = (0x7f80, 0x007f) if fmt == "bf16" else (0x7c00, 0x03ff)
    return ((bits & exp_mask) == exp_mask) & ((bits & man_mask) != 0)


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
def test_round_every_float32_bit_pattern(sa, fmt):
    tdt = torch.bfloat16 if fmt == "bf16" else torch.float16
    y = torch.empty(CHUNK, dtype=tdt, device=DEV)
    base = np.arange(CHUNK, dtype=np.uint32)
    for c in range((1 << 32) // CHUNK):
        bits = base + np.uint32(c * CHUNK)
        x = bits.view(np.float32)
        sa.attn_round(torch.from_numpy(x).to(DEV), y)
        got = y.view(torch.int16).cpu().numpy().view(np.uint16)
        want = oracle.round_bits(x, fmt)
        nan_in = np.isnan(x)
        bad = np.nonzero((got != want) & ~nan_in)[0]
        assert bad.size == 0, (f"{fmt}: {bad.size} mismatches in chunk {c}; first x=0x{int(bits[bad[0]]):08x} "
                               f"got 0x{int(got[bad[0]]):04x} want 0x{int(want[bad[0]]):04x}")
        assert _is_nan16(got[nan_in], fmt).all(), f"{fmt}: a NaN input did not give a NaN (chunk {c})"
        print(f"  {fmt} chunk {c:2d}/16 equal", flush=True)


def test_round_packed_word_example(sa):
    """(1, -2) packs to 0xc0003c00 as fp16 (printed on the page) and 0xc0003f80 as bf16 (derived),
    the lower element in the low half; odd lengths convert the tail alone."""
    with open(os.path.join(os.path.dirname(__file__), "golden", "pack_word.json")) as f:
        g = json.load(f)
    x = torch.tensor(g["values"] + [0.5], dtype=torch.float32, device=DEV)
    for tdt, key in ((torch.float16, "f16_word"), (torch.bfloat16, "bf16_word_derived")):
        y = torch.full((3,), 7.0, dtype=tdt, device=DEV)
        sa.attn_round(x, y)
        b = y.view(torch.int16).cpu().numpy().view(np.uint16)
        assert (int(b[1]) << 16 | int(b[0])) == int(g[key], 16)
        assert float(y[2]) == 0.5


def test_round_empty_and_rejects(sa):
    x = torch.zeros(4, device=DEV)
    sa.attn_round(x[:0], torch.empty(0, dtype=torch.bfloat16, device=DEV))
    with pytest.raises(sa.AttnError):
        sa.attn_round(x, torch.empty(4, dtype=torch.float32, device=DEV))   # fp32 target
    with pytest.raises(sa.AttnError):
        sa.attn_round(x, torch.empty(3, dtype=torch.bfloat16, device=DEV))  # size mismatch
