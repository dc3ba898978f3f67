"""Benchmark of the streaming-attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

One step is one pass over every kernel of the path, on resident synthetic inputs:
    1. attn_fwd          causal prefill B4 H32 N4096 D128 bf16      (tiled matrix-core kernel)
    2. attn_fwd_splitk   decode B8 H32 Nq1 Nkv32768 D128 bf16, P=16 (bandwidth kernel)
    3. attn_combine      merge of that P=16 workspace into the bf16 output
`value` is the prefill's throughput in TFLOP/s of algorithmic work (4*D per visible
query-key pair, causal diagonal included); the decode and combine bandwidths are reported
beside it, together with a decode sweep over P in {4, 8, 16, 37} (two launches, and the same
work fused into one attn_fwd_splitk_fused launch) and a combine measured on a workspace too large
for the caches, the standalone row softmax (three methods) on 32768 x 4096 and 4096 x 32768
fp32 rows, the masked long-context prefill (B1 H16 N16384 D256, causal AND a Bernoulli(0.5)
mask with 1/64 of the rows fully masked: the mask packed to bits, then the forward on the bits;
the forward on the byte mask and the same shape without the mask beside it), the prefill
with E4M3 V on the FP8 matrix cores (attn_fwd_fp8v), the decode-shape combine on cold workspaces
(cycling through more than 1 GiB of them), 32- vs 64-key tiles on a single-head N2048 D64 shape,
and the shader clock rocm-smi reports right after the timed region.  Every per-kernel time comes
from HIP events recorded on the stream the kernels are launched on, around each launch of the
timed region (default 50 steps after 5 warm-up steps): mean, median and minimum per kernel.
Rank 0 prints one JSON line.
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import seeded_inputs as si  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E, published
PEAK_FP8_TFLOPS = 5000.0      # MI355X dense FP8 MFMA, published
# attn_fwd_fp8v does half its work (Q K^T) on bf16 and half (P V) on FP8 matrix cores, so at
# both peaks one FLOP of the mix takes (1/2)/2500 + (1/2)/5000 ps: a mixed peak of 3333 TFLOP/s
PEAK_MIX_TFLOPS = 1.0 / (0.5 / PEAK_BF16_TFLOPS + 0.5 / PEAK_FP8_TFLOPS)
METRIC = "attn TFLOP/s (% bf16 MFMA peak) B4 H32 N4096 D128 causal; combine GB/s"


def prefill_flops(B, H, N, D):
    pairs = N * (N + 1) // 2                     # causal pairs, diagonal included
    return 4.0 * D * pairs * B * H


def decode_bytes(B, H, Nkv, D, P):
    kv = 2 * B * Nkv * H * D * 2                 # K and V, bf16
    q = B * H * D * 2
    egress = P * B * H * (D + 1) * 4             # o_partial + lse_partial, fp32
    return kv + q + egress


def softmax_figures(sa, dev, steps=10, warmup=3):
    """GB/s of algorithmic bytes (read x once, write y once) for each method."""
    res = {}
    for w in (si.SOFTMAX, si.SOFTMAX_WIDE):
        x = torch.from_numpy(si.softmax_inputs(w["rows"], w["n"], case=0)).to(dev)
        y = torch.empty_like(x)
        nbytes = 2 * x.numel() * 4
        fig = {}
        for name, m in (("streaming", 0), ("registers", 1), ("three_pass", 2)):
            _, ms = timed_events([lambda: sa.attn_softmax_rows(x, y, m)], steps, warmup)
            fig[name] = {"ms": ms[0], "GB/s": nbytes / (ms[0] * 1e-3) / 1e9,
                         "hbm_frac": nbytes / (ms[0] * 1e-3) / 1e9 / PEAK_HBM_GBS}
        res[w["name"]] = fig
        del x, y
    return res


def mask_pack_bytes(N):
    """Bytes a causal attn_mask_pack of an N x N mask moves: the mask bytes of the groups it
    writes (64-key groups c with 64 c <= 32 g + 31 for 32-row groups g), and their words."""
    ng, nkg = -(-N // 32), -(-N // 64)
    groups = sum(min(nkg, (32 * g + 31) // 64 + 1) for g in range(ng))
    return groups * (32 * 64 + 64 * 4)


def masked_figures(sa, dev, steps=10, warmup=3):
    """The masked long-context workload, and the same tensors without the mask.  The masked step
    is attn_mask_pack (the byte mask to packed bits, causal half) followed by the forward reading
    the bits; the forward reading the byte mask directly is timed beside it.  TFLOP/s counts 4*D
    per causal pair (the work the kernel does); 'useful' counts only the pairs the mask leaves
    visible."""
    s = si.MASKED
    qc, kc, vc, mask, _ = si.masked_inputs()
    vis = 0
    for r0 in range(0, s["N"], 2048):                  # visible pairs of causal AND mask, in row blocks
        blk = mask[r0:r0 + 2048]
        vis += int(np.count_nonzero(np.tril(blk, k=r0)))
    q, k, v = qc.to(dev), kc.to(dev), vc.to(dev)
    md = torch.from_numpy(mask).to(dev)
    del qc, kc, vc, mask
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    bits = torch.empty(sa.mask_bits_words(s["N"], s["N"]), dtype=torch.int32, device=dev)
    fl = prefill_flops(s["B"], s["H"], s["N"], s["D"])
    useful = 4.0 * s["D"] * vis * s["B"] * s["H"]

    def packed_step():
        sa.attn_mask_pack(md, bits, causal=True)
        sa.attn_fwd(q, k, v, out, lse, causal=True, mask_bits=bits)
    _, m = timed_events([packed_step,
                         lambda: sa.attn_mask_pack(md, bits, causal=True),
                         lambda: sa.attn_fwd(q, k, v, out, lse, causal=True, mask=md),
                         lambda: sa.attn_fwd(q, k, v, out, lse, causal=True)], steps, warmup)
    return {"B": s["B"], "H": s["H"], "N": s["N"], "D": s["D"],
            "step": "attn_mask_pack(causal) + attn_fwd(mask_bits)", "masked_ms": m[0],
            "masked_TFLOP/s": fl / (m[0] * 1e-3) / 1e12, "mfma_frac": fl / (m[0] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
            "useful_TFLOP/s": useful / (m[0] * 1e-3) / 1e12, "visible_pair_frac": vis / (s["N"] * (s["N"] + 1) / 2),
            "pack_ms": m[1], "pack_GB/s": mask_pack_bytes(s["N"]) / (m[1] * 1e-3) / 1e9,
            "byte_mask_ms": m[2], "byte_mask_TFLOP/s": fl / (m[2] * 1e-3) / 1e12,
            "causal_only_ms": m[3], "causal_only_TFLOP/s": fl / (m[3] * 1e-3) / 1e12,
            "masked_over_causal_only": m[0] / m[3]}


def fp8v_figures(sa, dev, steps=10, warmup=3, bf16_ms=None, bf16_fn=None):
    """attn_fwd_fp8v on the prefill shape (bf16 Q/K, E4M3 V, causal).  With bf16_fn (the bf16
    prefill of the same shape) both kernels run alternately in one timed loop, so the speedup
    compares them at the same clock and temperature; bf16_ms (the step loop's prefill mean) is
    reported beside it."""
    s = si.FP8V
    qc, kc, vc = si.fp8v_inputs()
    q, k, v = qc.to(dev), kc.to(dev), vc.to(dev)
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    fl = prefill_flops(s["B"], s["H"], s["N"], s["D"])
    fns = [lambda: sa.attn_fwd_fp8v(q, k, v, 1.0, out, lse, causal=True)]
    if bf16_fn is not None:
        fns.append(bf16_fn)
    _, m = timed_events(fns, steps, warmup)
    tf = fl / (m[0] * 1e-3) / 1e12
    r = {"workload": s["name"], "ms": m[0], "TFLOP/s": tf, "mixed_peak_TFLOP/s": PEAK_MIX_TFLOPS,
         "mixed_peak_frac": tf / PEAK_MIX_TFLOPS,
         "speedup_vs_bf16_step_loop": None if bf16_ms is None else bf16_ms / m[0]}
    if bf16_fn is not None:
        r["bf16_ms_same_loop"] = m[1]
        r["speedup_vs_bf16"] = m[1] / m[0]
    return r


def combine_large_figures(sa, dev, sd, steps=10, warmup=3):
    """attn_combine with P = 16 on rows 8192, the decode's heads and depth: a 2.2 GB workspace,
    larger than the caches."""
    Pc, rows_c = 16, 8192
    opc = torch.randn((Pc, rows_c, sd["H"], sd["D"]), dtype=torch.float32, device=dev)
    lpc = torch.randn((Pc, rows_c, sd["H"]), dtype=torch.float32, device=dev)
    obc = torch.empty((rows_c, sd["H"], sd["D"]), dtype=torch.bfloat16, device=dev)
    _, m = timed_events([lambda: sa.attn_combine(opc, lpc, obc)], steps, warmup)
    cb = combine_bytes(Pc, rows_c * sd["H"], sd["D"])
    return {"P": Pc, "rows": rows_c, "heads": sd["H"], "depth": sd["D"], "ms": m[0], "bytes": cb,
            "GB/s": cb / (m[0] * 1e-3) / 1e9, "hbm_frac": cb / (m[0] * 1e-3) / 1e9 / PEAK_HBM_GBS}


def combine_cold_figures(sa, dev, sd, replays=5):
    """attn_combine at the decode shape (rows B*Nq, heads H, depth D) for each P of the sweep,
    each call on a different workspace of a set larger than 1 GiB, so that every call reads its
    workspace from HBM.  The calls over the whole set are captured once in a HIP graph and the
    graph is replayed: the time per call then excludes the host's per-launch dispatch cost (a
    Python loop of launches measures that cost, ~9 us per call, rather than the kernel)."""
    res = {}
    RH = sd["B"] * sd["H"]
    for P in sd["P_list"]:
        one = P * RH * (sd["D"] + 1) * 4
        copies = max(8, (1 << 30) // one + 1)
        op = torch.randn((copies, P, sd["B"], sd["H"], sd["D"]), dtype=torch.float32, device=dev)
        lp = torch.randn((copies, P, sd["B"], sd["H"]), dtype=torch.float32, device=dev)
        ob = torch.empty((sd["B"], sd["H"], sd["D"]), dtype=torch.bfloat16, device=dev)
        for c in range(min(copies, 16)):
            sa.attn_combine(op[c], lp[c], ob)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for c in range(copies):
                sa.attn_combine(op[c], lp[c], ob)
        g.replay()
        torch.cuda.synchronize()
        per = []
        for _ in range(replays):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            per.append(e0.elapsed_time(e1) / copies)
        ms = float(np.median(per))
        cb = combine_bytes(P, RH, sd["D"])
        res[str(P)] = {"copies": copies, "us": ms * 1e3, "GB/s": cb / (ms * 1e-3) / 1e9,
                       "timing": f"HIP graph of {copies} launches, median of {replays} replays"}
        del g, op, lp
        torch.cuda.empty_cache()
    return res


def block_n_figures(sa, dev, steps=20, warmup=5):
    """Single-head attn_fwd, N 2048, D 64, bf16, causal and not: 32- vs 64-key tiles (context;
    launch-latency-sized work)."""
    q, k, v = (t.to(dev) for t in si.prefill_inputs(B=1, H=1, N=2048))
    q, k, v = (t[..., :64].contiguous() for t in (q, k, v))
    res = {}
    for causal in (False, True):
        out = torch.empty_like(q)
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
        _, m = timed_events([lambda: sa.attn_fwd(q, k, v, out, lse, causal=causal, block_n=32),
                             lambda: sa.attn_fwd(q, k, v, out, lse, causal=causal, block_n=64)], steps, warmup)
        res["causal" if causal else "full"] = {"BN32_us": m[0] * 1e3, "BN64_us": m[1] * 1e3}
    return res


def gpu_clock():
    """Shader clock reported by rocm-smi right after the timed region (None if unavailable)."""
    import subprocess
    try:
        r = subprocess.run(["rocm-smi", "--showclocks"], stdout=subprocess.PIPE, stderr=subprocess.DEVNULL,
                           text=True, timeout=20)
        for line in r.stdout.splitlines():
            if "sclk" in line:
                mhz = re.search(r"\((\d+)\s*Mhz\)", line, re.IGNORECASE)
                return f"{mhz.group(1)} MHz" if mhz else line.strip()
    except (OSError, subprocess.SubprocessError):
        return None
    return None


def combine_bytes(P, RH, D, out_elem=2):
    return P * RH * (D + 1) * 4 + RH * D * out_elem + RH * 4


KERNEL_SOURCES = ("attn_fwd_kernel.h", "attn_fwd.hip", "device.h", "launch.h")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_fwd_prefill_B4H32N4096D128_hbm_traffic.txt")


def kernel_source_hash():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "streaming_online_softmax_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per launch of the prefill kernel from the committed counter summary
    (FETCH_SIZE and WRITE_SIZE, each scaled by the same counter on a 1 GiB device copy), or
    None when that summary was taken on different kernel sources."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    with open(TRAFFIC_FILE) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256") != kernel_source_hash():
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def timed_events(fn_list, steps, warmup, stats=None):
    """Run the list of callables once per step; returns (wall seconds for `steps` steps,
    per-callable mean milliseconds from events on the current stream).  With a dict `stats`,
    also stores the per-callable median and minimum (ms) there under "median" and "min"."""
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        for fn in fn_list:
            fn()
    torch.cuda.synchronize()
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in fn_list]
          for _ in range(steps)]
    t0 = time.perf_counter()
    for s in range(steps):
        for j, fn in enumerate(fn_list):
            ev[s][j][0].record(stream)
            fn()
            ev[s][j][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = [[ev[s][j][0].elapsed_time(ev[s][j][1]) for s in range(steps)] for j in range(len(fn_list))]
    ms = [float(np.mean(x)) for x in per]
    if stats is not None:
        stats["median"] = [float(np.median(x)) for x in per]
        stats["min"] = [float(np.min(x)) for x in per]
    return wall, ms


def cpu_baseline(q, k, v, budget_s=15.0):
    """The FP64 oracle (dense definition, OpenMP over rows) on a seeded sample of the prefill
    workload's query rows, scaled to TFLOP/s of the same algorithmic work."""
    import oracle
    s = si.PREFILL
    B, N, H, D = s["B"], s["N"], s["H"], s["D"]
    rng = si.rng_for(99, 0)
    perm = rng.permutation(B * N * H)

    def run(rows):
        i = (rows // H) % N
        flops = float(np.sum(4.0 * D * (i + 1)))
        t0 = time.perf_counter()
        oracle.attn_dense(q, k, v, causal=True, rows=rows)
        return flops, time.perf_counter() - t0

    f0, t0 = run(perm[:512])                     # calibration
    n = int(min(len(perm) - 512, max(512, 512 * (budget_s / max(t0, 1e-3)))))
    rows = perm[512:512 + n]
    f, t = run(rows)
    return {"value": f / t / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"{n} seeded query rows (of {B * N * H} row-heads) of the causal prefill "
                      f"B4 H32 N4096 D128 bf16 workload, FP64 dense definition, {t:.1f} s wall"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=["prefill", "decode", "combine", "copy", "softmax", "fp8v", "masked", "combine_large",
                                       "combine_cold"],
                    default=None,
                    help="time a single kernel (for profiler runs); 'copy' times a plain 1 GiB device "
                         "copy, the calibration for the HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: the benchmark runs on one GPU; --gpus {args.gpus} is not supported "
              "(the library has no multi-GPU path: each GPU would run its own share)", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(2)
    import streaming_online_softmax_amd as sa

    dev = torch.device("cuda:0")
    if args.only == "copy":
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        _, ms = timed_events([lambda: dst.copy_(src)], args.steps, args.warmup)
        print(json.dumps({"calibration": "device copy", "bytes_read": 1 << 30, "bytes_written": 1 << 30,
                          "ms": ms[0], "GB/s": 2 * (1 << 30) / (ms[0] * 1e-3) / 1e9}), flush=True)
        return
    if args.only == "softmax":
        print(json.dumps({"softmax": softmax_figures(sa, dev, args.steps, args.warmup)}), flush=True)
        return
    if args.only == "combine_large":
        print(json.dumps({"combine_large": combine_large_figures(sa, dev, si.DECODE, args.steps, args.warmup)}), flush=True)
        return
    if args.only == "combine_cold":
        print(json.dumps({"combine_cold": combine_cold_figures(sa, dev, si.DECODE)}), flush=True)
        return
    if args.only == "masked":
        print(json.dumps({"masked_long_context": masked_figures(sa, dev, args.steps, args.warmup)}), flush=True)
        return
    if args.only == "fp8v":
        print(json.dumps({"fp8v_prefill": fp8v_figures(sa, dev, args.steps, args.warmup)}), flush=True)
        return
    # ---- inputs (seeded, synthetic, resident in HBM before timing) -----------------------
    sp = si.PREFILL
    qc, kc, vc = si.prefill_inputs()
    q, k, v = qc.to(dev), kc.to(dev), vc.to(dev)
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    sd = si.DECODE
    dq, dk, dv = (t.to(dev) for t in si.decode_inputs())
    P_STEP = 16
    RH = sd["B"] * sd["H"]
    o_p = torch.empty((P_STEP, RH, sd["D"]), dtype=torch.float32, device=dev)
    l_p = torch.empty((P_STEP, RH), dtype=torch.float32, device=dev)
    dout = torch.empty((RH, sd["D"]), dtype=torch.bfloat16, device=dev)
    dlse = torch.empty((RH,), dtype=torch.float32, device=dev)

    def k_prefill():
        sa.attn_fwd(q, k, v, out, lse, causal=True)

    def k_decode():
        sa.attn_fwd_splitk(dq, dk, dv, P_STEP, o_p.view(P_STEP, sd["B"], sd["H"], sd["D"]),
                           l_p.view(P_STEP, sd["B"], sd["H"]))

    def k_combine():
        sa.attn_combine(o_p.view(P_STEP, sd["B"], sd["H"], sd["D"]), l_p.view(P_STEP, sd["B"], sd["H"]),
                        dout.view(sd["B"], sd["H"], sd["D"]), dlse.view(sd["B"], sd["H"]))

    fns = {"prefill": [k_prefill], "decode": [k_decode], "combine": [k_decode, k_combine]}.get(
        args.only, [k_prefill, k_decode, k_combine])
    torch.cuda.synchronize()
    kstats = {}
    wall, ms = timed_events(fns, args.steps, args.warmup, stats=kstats)
    clock = gpu_clock()
    assert not torch.isnan(out).any() and not torch.isnan(dout).any(), "NaN in outputs"

    names = {"prefill": ["prefill"], "decode": ["decode"], "combine": ["decode", "combine"]}.get(
        args.only, ["prefill", "decode", "combine"])
    t = dict(zip(names, ms))
    fl = prefill_flops(sp["B"], sp["H"], sp["N"], sp["D"])
    res = {}
    if "prefill" in t:
        res["prefill_tflops"] = fl / (t["prefill"] * 1e-3) / 1e12
    if "decode" in t:
        res["decode_gbs"] = decode_bytes(sd["B"], sd["H"], sd["Nkv"], sd["D"], P_STEP) / (t["decode"] * 1e-3) / 1e9
    if "combine" in t:
        res["combine_gbs"] = combine_bytes(P_STEP, RH, sd["D"]) / (t["combine"] * 1e-3) / 1e9

    extra = {}
    if args.only is None:
        # ---- the prefill with E4M3 V and an FP8 second product (right after the bf16 prefill,
        #      in the same state of the GPU) ----------------------------------------------------
        extra["fp8v_prefill"] = fp8v_figures(sa, dev, steps=args.steps, warmup=args.warmup, bf16_ms=t.get("prefill"),
                                             bf16_fn=lambda: sa.attn_fwd(q, k, v, out, lse, causal=True))
        # ---- the same tensors without the causal mask (context): per-FLOP rate of causal vs full
        out_full = torch.empty_like(q)
        _, mfull = timed_events([lambda: sa.attn_fwd(q, k, v, out_full, None, causal=False)], args.steps, args.warmup)
        fl_full = 4.0 * sp["D"] * sp["N"] * sp["N"] * sp["B"] * sp["H"]
        extra["prefill_noncausal"] = {"ms": mfull[0], "TFLOP/s": fl_full / (mfull[0] * 1e-3) / 1e12,
                                      "causal_per_flop_rate_vs_full": (fl / t["prefill"]) / (fl_full / mfull[0])
                                      if "prefill" in t else None}
        del out_full
        # ---- decode sweep over P (context) -------------------------------------------------
        sweep = {}
        for P in sd["P_list"]:
            op = torch.empty((P, sd["B"], sd["H"], sd["D"]), dtype=torch.float32, device=dev)
            lp = torch.empty((P, sd["B"], sd["H"]), dtype=torch.float32, device=dev)
            ob = torch.empty((sd["B"], sd["H"], sd["D"]), dtype=torch.bfloat16, device=dev)
            _, m = timed_events([lambda: sa.attn_fwd_splitk(dq, dk, dv, P, op, lp),
                                 lambda: sa.attn_combine(op, lp, ob)], 10, 3)
            sweep[str(P)] = {"decode_ms": m[0], "decode_GB/s": decode_bytes(sd["B"], sd["H"], sd["Nkv"], sd["D"], P) / (m[0] * 1e-3) / 1e9,
                             "combine_ms": m[1], "combine_GB/s": combine_bytes(P, RH, sd["D"]) / (m[1] * 1e-3) / 1e9}
            # the same producer and merge in one launch (attn_fwd_splitk_fused)
            tk = torch.zeros(RH * sa.TICKET_STRIDE, dtype=torch.int32, device=dev)
            fl_ = torch.empty((sd["B"], sd["H"]), dtype=torch.float32, device=dev)
            _, mf = timed_events([lambda: sa.attn_fwd_splitk_fused(dq, dk, dv, P, op, lp, tk, ob, fl_)], 10, 3)
            fb = decode_bytes(sd["B"], sd["H"], sd["Nkv"], sd["D"], P) + combine_bytes(P, RH, sd["D"])
            sweep[str(P)].update({"fused_ms": mf[0], "fused_GB/s": fb / (mf[0] * 1e-3) / 1e9,
                                  "two_launch_ms": m[0] + m[1],
                                  "pipeline_GB/s": fb / ((m[0] + m[1]) * 1e-3) / 1e9})
        extra["decode_sweep"] = sweep
        # ---- the combine at the decode shape with its workspace cold: cycle through enough
        #      separate workspaces (> 1 GiB) that each call reads from HBM, not the caches
        extra["combine_cold"] = combine_cold_figures(sa, dev, sd)
        # ---- combine on a workspace larger than the caches (rows 8192, heads 32, depth 128) -
        extra["combine_large"] = combine_large_figures(sa, dev, sd)
        # ---- single-head shape, 32- vs 64-key tiles (context) --------------------------------
        extra["block_n_single_head_N2048_D64"] = block_n_figures(sa, dev)
        # ---- standalone row softmax (32768 rows x 4096 fp32; and 4096 x 32768) -------------
        extra["softmax"] = softmax_figures(sa, dev)
        # ---- masked long context B1 H16 N16384 D256, causal AND Bernoulli(0.5) mask ----------
        extra["masked_long_context"] = masked_figures(sa, dev)

    value = res.get("prefill_tflops")
    line = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "causal prefill B4 H32 N4096 D128 bf16 [B,N,H,D]",
                   "step": "attn_fwd(prefill) + attn_fwd_splitk(decode B8 H32 Nq1 Nkv32768 D128 bf16, P=16) + attn_combine",
                   "B": sp["B"], "H": sp["H"], "N": sp["N"], "D": sp["D"], "causal": True},
        "kernel_ms": t,
        "kernel_ms_median": dict(zip(names, kstats["median"])),
        "kernel_ms_min": dict(zip(names, kstats["min"])),
        "gpu_clock_after_timing": clock,
        "roofline": None,
        "decode": None if "decode" not in t else {
            "GB/s": res["decode_gbs"], "hbm_frac": res["decode_gbs"] / PEAK_HBM_GBS, "P": P_STEP},
        "combine": None if "combine" not in t else {
            "GB/s": res["combine_gbs"], "P": P_STEP,
            "note": "workspace just written by the decode producer (cache-resident at this size)"},
    }
    if value is not None:
        line["roofline"] = {"bound": "mfma", "achieved": value, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                            "frac": value / PEAK_BF16_TFLOPS, "traffic": measured_traffic(),
                            "traffic_unit": "bytes per launch (HBM, counter-measured)",
                            "kernel": "attn_fwd_kernel<bf16, D=128, BN=64, waves=8, stages=3>",
                            "work_per_launch": f"{fl:.4e} FLOP (4*D per causal pair)"}
    line.update(extra)
    if args.only is None and not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(qc, kc, vc)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
