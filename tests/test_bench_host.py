"""Host-side checks of bench.py (CPU): the algorithmic work behind every rate it reports, counted
independently, and its refusal of more than one GPU."""
import importlib.util
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_prefill_flops_counts_causal_pairs(bench):
    """4*D FLOP per visible (query, key) pair, diagonal included: the pair count against a brute
    force over small N, and the causal prefill B4 H32 N4096 D128 figure."""
    for n in (1, 2, 7, 64, 129):
        pairs = sum(1 for i in range(n) for j in range(n) if j <= i)
        assert bench.prefill_flops(1, 1, n, 16) == 4.0 * 16 * pairs
    assert bench.prefill_flops(3, 5, 100, 64) == 3 * 5 * bench.prefill_flops(1, 1, 100, 64)
    assert bench.prefill_flops(4, 32, 4096, 128) == 549_890_031_616


def test_decode_bytes(bench):
    """K and V read once (bf16), q read once, the fp32 workspace entry (O_p and its LSE) written
    once per partition and row-head; B8 H32 Nkv32768 D128 at P = 16 is 4,297,146,368 B."""
    B, H, Nkv, D, P = 2, 3, 50, 16, 5
    kv = np.zeros((B, Nkv, H, D), np.uint16).nbytes * 2
    q = np.zeros((B, 1, H, D), np.uint16).nbytes
    ws = np.zeros((P, B, H, D), np.float32).nbytes + np.zeros((P, B, H), np.float32).nbytes
    assert bench.decode_bytes(B, H, Nkv, D, P) == kv + q + ws
    assert bench.decode_bytes(8, 32, 32768, 128, 16) == 4_297_146_368


def test_combine_bytes(bench):
    """The workspace read once, the output (bf16) and its LSE (fp32) written once."""
    P, RH, D = 7, 11, 32
    read = np.zeros((P, RH, D), np.float32).nbytes + np.zeros((P, RH), np.float32).nbytes
    write = np.zeros((RH, D), np.uint16).nbytes + np.zeros(RH, np.float32).nbytes
    assert bench.combine_bytes(P, RH, D) == read + write
    assert bench.combine_bytes(P, RH, D, out_elem=4) == read + np.zeros((RH, D), np.float32).nbytes + RH * 4


def test_mask_pack_bytes(bench):
    """A causal pack of an N x N mask moves, for every 32-row group g and 64-key group c it
    writes (those holding a key at or below some row of the group: 64 c <= 32 g + 31), the 32 x 64
    mask bytes read and the 64 words written; counted here pair by pair over the mask instead."""
    for n in (1, 31, 32, 64, 65, 200, 1000):
        ng, nkg = -(-n // 32), -(-n // 64)
        groups = set()
        for i in range(ng * 32):
            for c in range(nkg):
                if 64 * c <= i:                 # some key of group c is visible to row i
                    groups.add((i // 32, c))
        assert bench.mask_pack_bytes(n) == len(groups) * (32 * 64 + 64 * 4), n
    assert bench.mask_pack_bytes(16384) == 151_584_768


def test_published_peaks(bench):
    assert bench.PEAK_BF16_TFLOPS == 2500.0 and bench.PEAK_HBM_GBS == 8000.0 and bench.PEAK_FP8_TFLOPS == 5000.0
    # a FLOP of the bf16 / FP8 half-and-half mix at both peaks
    assert abs(bench.PEAK_MIX_TFLOPS - 1.0 / (0.5 / 2500.0 + 0.5 / 5000.0)) < 1e-9


def test_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], cwd=ROOT,
                       stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""
